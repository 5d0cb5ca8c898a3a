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
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ payload, Geom g, int prec,
                                                      float* __restrict__ out) {
    const int64_t gate_blocks = (int64_t)g.f * g.nb_d;
    const int64_t total = 2 * gate_blocks + (int64_t)g.d * g.nb_f;
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= total) return;
    // b enumerates logical blocks: gate rows, up rows, down rows, row-major
    int m;
    int64_t L;
    if (b < gate_blocks) { m = 0; L = b; }
    else if (b < 2 * gate_blocks) { m = 1; L = b - gate_blocks; }
    else { m = 2; L = b - 2 * gate_blocks; }
    const int nb = m < 2 ? g.nb_d : g.nb_f;
    const int64_t r = L / nb;
    const int cb = (int)(L % nb);
    int64_t t;
    int i;
    int64_t toff;
    if (m < 2) {
        g.gu_block(r, cb, &t, &i);
        toff = m == 0 ? g.gate_tile(t) : g.up_tile(t);
    } else {
        g.down_block(r, cb, &t, &i);
        toff = g.down_tile(t);
    }
    const uint8_t* tile = payload + toff;
    float* o = out + (int64_t)m * g.f * g.d + L * kQK;
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
        const uint8_t* nbp = tile + q4_nib(i);
        for (int j = 0; j < 16; j++) {
            float a = (float)((int)(nbp[j] & 15) - 8) * s, c = (float)((int)(nbp[j] >> 4) - 8) * s;
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
        hipLaunchKernelGGL(dequant_kernel<MOE_Q8_0>, grid, dim3(256), 0, s, payload, g, prec, out);
    else
        hipLaunchKernelGGL(dequant_kernel<MOE_Q4_0>, grid, dim3(256), 0, s, payload, g, prec, out);
    return hipGetLastError();
}

}  // namespace moe
