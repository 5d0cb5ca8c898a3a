/* CPU oracle for routed mixture-of-experts FFN execution.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg.  Shares no code with the HIP path.
 *
 * What is computed, and where the pages state it:
 *  - the router picks each token's experts and those decisions are final
 *    ("Nanite for Experts", §3.1 Authoritative routing); each token uses eight
 *    routed experts out of 256 plus one shared expert (same page, §1; "Paging
 *    the Experts", §3.1);
 *  - the routed tokens are unioned expert-major so each distinct expert is
 *    scheduled once ("Nanite for Experts", §5.3 and §11.3);
 *  - experts are GGUF-quantised (Q8_0 named in "MawForge", §V-B); their FFN
 *    results are merged back into the tokens' output positions ("Nanite for
 *    Experts", §5.5).
 * The pages do not write out the router, softmax, block formats or SwiGLU;
 * the readings taken here are:
 *  - router logits are x . W_r; the top-k is taken on the logits with ties to
 *    the lower expert index; the routing weights are the softmax over the k
 *    selected logits (or, with norm == 0, the full softmax probability);
 *  - Q8_0 block = fp16 scale d + 32 int8 codes q, value d*q; Q4_0 block =
 *    fp16 scale d + 16 bytes, element j < 16 in the low nibble of byte j and
 *    element j + 16 in its high nibble, value d*(n - 8) (the GGUF layouts);
 *  - expert: y = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + exp(-z));
 *    the shared expert has weight 1 and the routed layer output is the
 *    weighted sum of the selected experts plus the shared expert;
 *  - bf16 precision mode rounds the dequantised weights, the activations and
 *    the hidden state silu(g)*u to bf16 (nearest, ties to even) and keeps
 *    everything else exact.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)frac, -24);               /* subnormal: frac * 2^-14 * 2^-10 */
    else if (exp == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), exp - 25); /* (1 + frac/1024) * 2^(exp-15) */
    return sign ? -v : v;
}

/* bfloat16: 8 significant bits, same exponent range as binary32
 * (smallest normal 2^-126, smallest subnormal 2^-133, largest 255 * 2^120). */
double orc_bf16_round(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(fabs(v), &e);                 /* |v| = m * 2^e, 0.5 <= m < 1 */
    int qexp = (e < -125 ? -125 : e) - 8; /* weight of the last kept bit */
    double r = ldexp(nearbyint(ldexp(fabs(v), -qexp)), qexp); /* default mode: ties to even */
    if (r > ldexp(255.0, 120)) r = INFINITY;
    return copysign(r, v);
}

size_t orc_block_bytes(int qtype) {
    return qtype == ORC_Q8_0 ? 34 : qtype == ORC_Q4_0 ? 18 : 0;
}

static int block_code(int qtype, const uint8_t* blk, int j) {
    if (qtype == ORC_Q8_0) return (int)(int8_t)blk[2 + j];
    int byte = blk[2 + (j & 15)];
    return (j < 16 ? (byte & 0x0f) : (byte >> 4)) - 8;
}

/* Nearest bfloat16 of a value that binary32 holds exactly and that is zero or
 * normal in binary32 (every d*q: at most 18 significant bits, magnitude
 * between 2^-24 and 2^23): round-to-nearest-even on the binary32 bits, i.e.
 * add half of the dropped 16 bits' weight (minus one unless the kept last
 * bit is odd) and truncate.  Same results as orc_bf16_round on such values. */
static double bf16_round_exact_f32(double v) {
    float f = (float)v;
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &b, sizeof f);
    return (double)f;
}

void orc_dequant(int qtype, int prec, const uint8_t* blocks, int64_t n_elems, double* out) {
    size_t bb = orc_block_bytes(qtype);
    for (int64_t b = 0; b < n_elems / 32; b++) {
        const uint8_t* blk = blocks + (size_t)b * bb;
        double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int j = 0; j < 32; j++) {
            double w = d * (double)block_code(qtype, blk, j); /* exact: <= 18 significant bits */
            out[b * 32 + j] = prec == ORC_PREC_BF16 ? bf16_round_exact_f32(w) : w;
        }
    }
}

void orc_router_logits(const double* x, const float* w_r, int64_t T, int E, int d, float* logits) {
    for (int64_t t = 0; t < T; t++)
        for (int e = 0; e < E; e++) {
            double s = 0.0;
            for (int i = 0; i < d; i++) s += x[t * d + i] * (double)w_r[(int64_t)e * d + i];
            logits[t * E + e] = (float)s;
        }
}

int orc_topk(const float* logits, int64_t T, int E, int k, int norm, int32_t* ids, float* w) {
    if (k < 1 || k > E) return -1;
    char* taken = (char*)malloc((size_t)E);
    if (!taken) return -1;
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * E;
        for (int e = 0; e < E; e++)
            if (!isfinite(l[e])) { free(taken); return -1; }
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) /* strict '>' keeps the lower index on ties; +0 == -0 */
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double lmax = l[ids[t * k]];
        double z = 0.0;
        if (norm) {
            for (int j = 0; j < k; j++) z += exp((double)l[ids[t * k + j]] - lmax);
        } else {
            for (int e = 0; e < E; e++) z += exp((double)l[e] - lmax);
        }
        for (int j = 0; j < k; j++) w[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - lmax) / z);
    }
    free(taken);
    return 0;
}

int orc_plan_union(const int32_t* ids, int64_t T, int k, int E, int32_t* n_active,
                   int32_t* experts, int32_t* offsets, int32_t* entries) {
    int64_t n = T * k;
    int64_t* cursor = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!cursor) return -1;
    for (int64_t i = 0; i < n; i++) {
        if (ids[i] < 0 || ids[i] >= E) { free(cursor); return -1; }
        cursor[ids[i]]++;
    }
    int32_t a = 0;
    int64_t pos = 0;
    for (int e = 0; e < E; e++) {
        int64_t c = cursor[e];
        cursor[e] = pos;
        if (c) {
            experts[a] = e;
            offsets[a] = (int32_t)pos;
            a++;
        }
        pos += c;
    }
    offsets[a] = (int32_t)pos;
    *n_active = a;
    for (int64_t i = 0; i < n; i++) entries[cursor[ids[i]]++] = (int32_t)i; /* stable */
    free(cursor);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The hidden state of one SwiGLU expert, before any rounding of it:
 * h[r] = silu(g_r) * u_r with g = W_g x, u = W_u x (x rounded to bf16 first
 * in bf16 mode). */
void orc_expert_hidden(int qtype, int prec, const uint8_t* rec, int d, int f,
                       const double* x_in, double* h) {
    size_t bb = orc_block_bytes(qtype);
    size_t row_in_d = (size_t)(d / 32) * bb; /* bytes of one gate/up row */
    const uint8_t* gate = rec;
    const uint8_t* up = gate + (size_t)f * row_in_d;
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < d; i++) x[i] = prec == ORC_PREC_BF16 ? orc_bf16_round(x_in[i]) : x_in[i];
#pragma omp parallel
    {
        double* wg = (double*)malloc(sizeof(double) * (size_t)d);
        double* wu = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int r = 0; r < f; r++) {
            orc_dequant(qtype, prec, gate + (size_t)r * row_in_d, d, wg);
            orc_dequant(qtype, prec, up + (size_t)r * row_in_d, d, wu);
            double g = 0.0, u = 0.0;
            for (int i = 0; i < d; i++) {
                g += wg[i] * x[i];
                u += wu[i] * x[i];
            }
            h[r] = silu(g) * u;
        }
        free(wg);
        free(wu);
    }
    free(x);
}

/* The down projection of one expert on a given hidden state: y = W_d h. */
void orc_expert_down(int qtype, int prec, const uint8_t* rec, int d, int f,
                     const double* h, double* y) {
    size_t bb = orc_block_bytes(qtype);
    size_t row_in_d = (size_t)(d / 32) * bb;
    size_t row_in_f = (size_t)(f / 32) * bb; /* bytes of one down row */
    const uint8_t* down = rec + 2 * (size_t)f * row_in_d;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(static)
        for (int i = 0; i < d; i++) {
            orc_dequant(qtype, prec, down + (size_t)i * row_in_f, f, wd);
            double s = 0.0;
            for (int r = 0; r < f; r++) s += wd[r] * h[r];
            y[i] = s;
        }
        free(wd);
    }
}

/* The expert: its hidden state (rounded to bf16 in bf16 mode), then the down
 * projection. */
void orc_expert_ffn(int qtype, int prec, const uint8_t* rec, int d, int f,
                    const double* x_in, double* y) {
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
    orc_expert_hidden(qtype, prec, rec, d, f, x_in, h);
    if (prec == ORC_PREC_BF16)
        for (int r = 0; r < f; r++) h[r] = orc_bf16_round(h[r]);
    orc_expert_down(qtype, prec, rec, d, f, h, y);
    free(h);
}

void orc_bf16_round_array(const double* v, int64_t n, double* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_round(v[i]);
}

int orc_moe_layer(int qtype, int prec, const uint8_t* const* experts, int E,
                  const uint8_t* shared, int d, int f, int64_t T, int k,
                  const double* x, const int32_t* ids, const float* w, float* y) {
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    double* ye = (double*)malloc(sizeof(double) * (size_t)d);
    int rc = 0;
    for (int64_t t = 0; t < T && rc == 0; t++) {
        for (int i = 0; i < d; i++) acc[i] = 0.0;
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            if (e < 0 || e >= E || !experts[e]) { rc = -1; break; }
            orc_expert_ffn(qtype, prec, experts[e], d, f, x + t * d, ye);
            for (int i = 0; i < d; i++) acc[i] += (double)w[t * k + j] * ye[i];
        }
        if (rc) break;
        if (shared) {
            orc_expert_ffn(qtype, prec, shared, d, f, x + t * d, ye);
            for (int i = 0; i < d; i++) acc[i] += ye[i];
        }
        for (int i = 0; i < d; i++) y[t * d + i] = (float)acc[i];
    }
    free(acc);
    free(ye);
    return rc;
}
