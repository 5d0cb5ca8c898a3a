// Block dequantisation of one device payload into the logical row-major
// matrices (gate, up, down) — the weights every expert kernel computes with.
// Q8_0: w = d * q; Q4_0: w = d * (n - 8); both exact in fp32 (a 7-bit code
// times an 11-bit fp16 significand fits in 24 bits).  bf16 mode rounds that
// exact value to the nearest bf16, ties to even.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

template <int QT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ payload, int f, int d,
                                                      int nb_d, int nb_f, int64_t tile_bytes,
                                                      int64_t gu_tiles, int prec, float* __restrict__ out) {
    const int64_t gate_blocks = (int64_t)f * nb_d;
    const int64_t total = 2 * gate_blocks + (int64_t)d * nb_f;
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= total) return;
    int m;
    int64_t L;
    if (b < gate_blocks) { m = 0; L = b; }
    else if (b < 2 * gate_blocks) { m = 1; L = b - gate_blocks; }
    else { m = 2; L = b - 2 * gate_blocks; }
    const int64_t t = L / kTileBlocks;
    const int i = (int)(L % kTileBlocks);
    const int64_t toff = m == 0 ? 2 * t * tile_bytes
                       : m == 1 ? (2 * t + 1) * tile_bytes
                                : (2 * gu_tiles + t) * tile_bytes;
    const uint8_t* tile = payload + toff;
    float* o = out + (int64_t)m * f * d + L * kQK;
    if (QT == MOE_Q8_0) {
        const float s = f16_bits_to_f32(*(const uint16_t*)(tile + q8_scale(i)));
        const int8_t* lo = (const int8_t*)(tile + q8_lo(i));
        const int8_t* hi = (const int8_t*)(tile + q8_hi(i));
        for (int j = 0; j < 16; j++) {
            float a = (float)lo[j] * s, c = (float)hi[j] * s;
            o[j] = prec ? round_bf16(a) : a;
            o[16 + j] = prec ? round_bf16(c) : c;
        }
    } else {
        const float s = f16_bits_to_f32(*(const uint16_t*)(tile + q4_scale(i)));
        const uint8_t* nb = tile + q4_nib(i);
        for (int j = 0; j < 16; j++) {
            float a = (float)((int)(nb[j] & 15) - 8) * s, c = (float)((int)(nb[j] >> 4) - 8) * s;
            o[j] = prec ? round_bf16(a) : a;
            o[16 + j] = prec ? round_bf16(c) : c;
        }
    }
}

}  // namespace

hipError_t launch_dequant(const Geom& g, const uint8_t* payload, int prec, float* out, hipStream_t s) {
    const int64_t total = 2 * (int64_t)g.f * g.nb_d + (int64_t)g.d * g.nb_f;
    dim3 grid((unsigned)((total + 255) / 256));
    if (g.qtype == MOE_Q8_0)
        hipLaunchKernelGGL(dequant_kernel<MOE_Q8_0>, grid, dim3(256), 0, s, payload, g.f, g.d, g.nb_d, g.nb_f,
                           g.tile_bytes, g.gu_tiles, prec, out);
    else
        hipLaunchKernelGGL(dequant_kernel<MOE_Q4_0>, grid, dim3(256), 0, s, payload, g.f, g.d, g.nb_d, g.nb_f,
                           g.tile_bytes, g.gu_tiles, prec, out);
    return hipGetLastError();
}

}  // namespace moe
