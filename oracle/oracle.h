/* CPU oracle for routed mixture-of-experts FFN execution.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the product (the HIP path
 * behind include/moe.h) never includes, links or calls it, and this file
 * includes nothing of the product.
 *
 * Plain, slow, obviously correct: every quantity is accumulated in double
 * precision and rounded to float only where a result is defined as float.
 * OpenMP splits independent output rows across threads; each output element
 * is computed by one thread in one fixed order, so results do not depend on
 * the thread count.
 */
#ifndef ORC_ORACLE_H
#define ORC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_Q8_0 0
#define ORC_Q4_0 1
#define ORC_PREC_F32 0   /* exact block dequantisation, exact SwiGLU hidden state */
#define ORC_PREC_BF16 1  /* weights, activations and hidden state rounded to bf16 */

/* threads used by the row loops (<= 0: OpenMP default); returns the count in use */
int orc_set_threads(int n);

/* IEEE binary16 bit pattern -> value, decoded field by field */
double orc_f16_to_f64(uint16_t h);
/* round to the nearest bfloat16 value, ties to even (result returned exactly as a double) */
double orc_bf16_round(double v);
/* bytes of one 32-element block (34 for Q8_0, 18 for Q4_0), 0 for an unknown type */
size_t orc_block_bytes(int qtype);

/* Dequantise n_elems (a multiple of 32) consecutive block elements. */
void orc_dequant(int qtype, int prec, const uint8_t* blocks, int64_t n_elems, double* out);

/* logits[t,e] = sum_i x[t,i] * w_r[e,i], accumulated in double, rounded to float */
void orc_router_logits(const double* x, const float* w_r, int64_t T, int E, int d, float* logits);

/* Top-k experts per token on float logits, larger first, ties to the lower
 * expert index; weights are the softmax restricted to the selected experts
 * (norm != 0) or the full softmax probability of each selected expert
 * (norm == 0).  Returns 0, or -1 for k outside [1, E] or a non-finite logit. */
int orc_topk(const float* logits, int64_t T, int E, int k, int norm, int32_t* ids, float* w);

/* Expert-major union of the T*k assignments (stable counting sort by expert):
 * experts[0..n_active) ascending, bucket a holds entries[offsets[a]..offsets[a+1])
 * with entry value t*k + j, ascending within the bucket.  Returns 0 or -1 for
 * an expert id outside [0, E). */
int orc_plan_union(const int32_t* ids, int64_t T, int k, int E, int32_t* n_active,
                   int32_t* experts, int32_t* offsets, int32_t* entries);

/* One SwiGLU expert: y = W_d (silu(W_g x) * (W_u x)).  rec holds GGUF blocks:
 * gate [f rows x d], up [f rows x d], down [d rows x f], each row-major with
 * blocks along the row (the input dimension). */
void orc_expert_ffn(int qtype, int prec, const uint8_t* rec, int d, int f,
                    const double* x, double* y);
/* Its two halves: the hidden state h = silu(W_g x) * (W_u x) before any
 * rounding of h (x rounded to bf16 first in bf16 mode; f values), and the
 * down projection y = W_d h of a given hidden state.  orc_expert_ffn is the
 * first, then (bf16 mode) orc_bf16_round of each h, then the second. */
void orc_expert_hidden(int qtype, int prec, const uint8_t* rec, int d, int f,
                       const double* x, double* h);
void orc_expert_down(int qtype, int prec, const uint8_t* rec, int d, int f,
                     const double* h, double* y);
/* orc_bf16_round of each of n values */
void orc_bf16_round_array(const double* v, int64_t n, double* out);

/* Routed layer: y[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t]) + FFN_shared(x[t]),
 * summed in double in rank order j, shared expert last, rounded to float.
 * experts[e] points at expert e's record (may be NULL for experts no token
 * selects); shared may be NULL.  Returns 0 or -1 on an invalid or missing id. */
int orc_moe_layer(int qtype, int prec, const uint8_t* const* experts, int E,
                  const uint8_t* shared, int d, int f, int64_t T, int k,
                  const double* x, const int32_t* ids, const float* w, float* y);

#ifdef __cplusplus
}
#endif
#endif
