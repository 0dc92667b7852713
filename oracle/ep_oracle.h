/*
 * ep_oracle.h -- slow, single-threaded CPU oracle for MoE token dispatch and
 * combine.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it; the product path never does.  It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Pages cited (by title and section):
 *   [DeepEP overview]  "DeepSeek merilis library open source DeepEP untuk
 *                      pelatihan dan inferensi MoE" (GeekNews, Indonesian)
 *   [Perplexity blog]  "Lower latency and higher throughput with multi-node
 *                      DeepSeek deployment" (Perplexity, Icelandic rendering)
 *   [torchtitan PR]    "Integrate DeepEP to experimental torchtitan"
 *   [EPLB page]        "DeepSeek V3/R1 ... DualPipe, EPLB, Profile-Data"
 *                      (GeekNews, Turkish)
 *
 * Notation: T tokens, H hidden, k top-k, E experts, R simulated ranks,
 * El = E/R experts per rank, P = T*k (token, slot) pairs, p = t*k + j.
 * Rank r owns experts [r*El, (r+1)*El) ([Perplexity blog], "Sérfræðinga-
 * samsíðun": each GPU holds 256/EP routed experts).
 *
 * Data types: indices int32, weights and scales fp32, bf16 as uint16 bit
 * patterns, FP8 OCP E4M3 ("fn": bias 7, no infinity, max 448) as uint8.
 *
 * Every function is a direct transcription of the definition it cites; there
 * is no blocking, fusion or reordering.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return 0 when the shapes and every index are acceptable, else a nonzero
 * code: 1 bad shape (T,k,R<1, E%R, H%8, H%128 under FP8), 2 index outside
 * [0,E). */
int oracle_validate(int T, int H, int k, int E, int R, int fp8, const int32_t *idx);

/* Routing layout ([Perplexity blog], "MoE-beirari": dense dispatch/combine
 * need routing information summed per expert; [DeepEP overview], "Pola
 * penggunaan...": the handle's per-expert token counts feed the GEMM).
 * Outputs: cnt[E], off[E+1], rcnt[R], roff[R+1], slot[P], src[P], row[P].
 * Returns oracle_validate's code for (T,8,k,E,R,0,idx); outputs untouched on
 * error. */
int oracle_layout(int T, int k, int E, int R, const int32_t *idx,
                  int32_t *cnt, int32_t *off, int32_t *rcnt, int32_t *roff,
                  int32_t *slot, int32_t *src, int32_t *row);

/* BF16 dispatch: recv[r][row[p]][:] = x[t][:] bitwise. recv[r] has H-element
 * rows. */
void oracle_dispatch_bf16(int T, int H, int k, int E, int R, const int32_t *idx,
                          const int32_t *slot, const int32_t *roff,
                          const uint16_t *x, uint16_t *const *recv);

/* FP8 dispatch with per-128-channel scales ([Perplexity blog], "Magntölun":
 * activation scales over 128-element vectors, computed on the fly, a scale
 * tensor of M x ceil_div(K,128)).  recv_q[r] rows of H bytes, recv_s[r] rows
 * of H/128 floats. */
void oracle_dispatch_fp8(int T, int H, int k, int E, int R, const int32_t *idx,
                         const int32_t *slot, const int32_t *roff,
                         const uint16_t *x, uint8_t *const *recv_q,
                         float *const *recv_s);

/* Quantize one token row (H channels) to q[H] and s[H/128]. */
void oracle_quantize_row(int H, const uint16_t *xrow, uint8_t *q, float *s);

/* Un-permute: u[p][:] = recv_y[r(p)][row(p)][:], u is [P,H] in (t,j) order
 * ([torchtitan PR]: the token unpermute after the experts). */
void oracle_unpermute(int T, int H, int k, int E, int R, const int32_t *idx,
                      const int32_t *slot, const int32_t *roff,
                      const uint16_t *const *recv_y, uint16_t *u);

/* Weighted combine ([Perplexity blog], "Sérfræðinga-samsíðun": the routed
 * results are weighted and summed; [DeepEP overview], "Pola penggunaan...":
 * combine reduces expert outputs back to the source).  fp32 accumulation in
 * ascending j with a correctly rounded fused multiply-add, then bf16 RNE.
 * w == NULL means unit weights. */
void oracle_combine(int T, int H, int k, int E, int R, const int32_t *idx,
                    const int32_t *slot, const int32_t *roff,
                    const uint16_t *const *recv_y, const float *w, uint16_t *out);

/* Weighted combine plus the shared expert ([Perplexity blog], "Sérfræðinga-
 * samsíðun": every token also runs through the shared expert and that result
 * is added to the routed experts' result): acc as in oracle_combine, then
 * acc = acc + f32(shared[t][h]) (one binary32 addition), then bf16 RNE. */
void oracle_combine_shared(int T, int H, int k, int E, int R, const int32_t *idx,
                           const int32_t *slot, const int32_t *roff,
                           const uint16_t *const *recv_y, const float *w,
                           const uint16_t *shared, uint16_t *out);

/* Backward of combine ([DeepEP overview], "Pola penggunaan ...": the backward
 * of combine is a dispatch).  For every pair p = (t, j):
 *   grad_recv[r][row(p)][h] = BF16_RNE(RN32(w[p] * f32(grad_out[t][h])))
 *     (w == NULL: unit weights, an exact copy), and, when grad_w != NULL,
 *   grad_w[p] = RN32( sum_h f32(grad_out[t][h]) * f32(y[r][row(p)][h]) ),
 *     the sum taken in binary64 (each bf16 x bf16 product is exact there). */
void oracle_combine_backward(int T, int H, int k, int E, int R, const int32_t *idx,
                             const int32_t *slot, const int32_t *roff,
                             const uint16_t *grad_out, const float *w,
                             const uint16_t *const *recv_y, uint16_t *const *grad_recv,
                             float *grad_w);

/* Expert activation with block re-quantization ([Perplexity blog],
 * "Magntölun": the SiLU kernel splits the hidden dimension into blocks and
 * quantizes per 128 elements, with scales computed on the fly).  For one
 * row of 2I bf16 values (gate = row[0:I], up = row[I:2I]):
 *   a[h] = RN32( silu(g) * u ),  silu(v) = v / (1 + e^-v), all in binary64;
 * then per 128-element block of a exactly as oracle_quantize_row:
 *   s = RN32(amax/448), q = E4M3(RN32(a/s)); an all-zero block gives s = 0,
 *   q = 0x00.  oracle_silu_mul_row stops after a. */
void oracle_silu_mul_row(int I, const uint16_t *row, float *a);
void oracle_silu_mul_quant_row(int I, const uint16_t *row, uint8_t *q, float *s);
void oracle_quantize_f32_row(int n, const float *a, uint8_t *q, float *s);

/* Router ([Perplexity blog], "MoE-beirari": one router serves every MoE
 * model, DeepSeek's group-limited top-k with Mixtral as the case where the
 * top-k group is all experts, and it emits top-k indices and scores;
 * [EPLB page]: group-limited expert routing and redundant experts;
 * [torchtitan PR]: node-limited routing).  logits [T, El] binary32, El
 * logical experts in G groups of El/G consecutive ids.  Per token t:
 *   z[e] = logits[t][e] + bias[e]   (one binary32 add; bias may be NULL);
 *   s[e] = RN32(gate(z)) with the gate in binary64: softmax (gate 0,
 *          exp(z_e - max z) / sum_e exp(z_e - max z), sum in ascending e) or
 *          sigmoid (gate 1, 1 / (1 + exp(-z_e)));
 *   group score = best s in the group (group_topn 1) or the binary32 sum of
 *          the two best (group_topn 2); the TG best groups stay eligible;
 *   the k best eligible experts in descending order; ties of scores (compared
 *          as unsigned bit patterns) go to the lower id;
 *   w[t][j] = s of expert j, divided by the binary32 sum over j (ascending)
 *          when renorm and that sum is > 0;
 *   idx[t][j] = rep_slots[rep_off[l] + t mod n_l], n_l = rep_off[l+1] -
 *          rep_off[l] (-1 when n_l = 0), or l itself when rep_off is NULL.
 * Returns 1 (outputs untouched) unless 1 <= k <= El, G | El, 1 <= TG <= G,
 * k <= TG*El/G, gate in {0,1}, group_topn in {1,2}. */
/* The router's gate scores alone: scores [T, El] binary32, each the binary64
 * gate rounded once (the first step of oracle_route).  Returns nonzero for
 * T < 1, El < 1 or an unknown gate. */
int oracle_route_scores(int T, int El, int gate, const float *logits, const float *bias,
                        float *scores);
int oracle_route(int T, int El, int k, int gate, int G, int TG, int group_topn, int renorm,
                 const float *logits, const float *bias, const int32_t *rep_off,
                 const int32_t *rep_slots, int32_t *idx, float *w);

/* Codecs. */
uint8_t  oracle_e4m3_encode(float v);
float    oracle_e4m3_decode(uint8_t c);
uint16_t oracle_bf16_rne(float v);
float    oracle_bf16_to_f32(uint16_t b);
void     oracle_e4m3_encode_n(const float *v, uint8_t *out, int64_t n);
void     oracle_e4m3_decode_n(const uint8_t *c, float *out, int64_t n);
void     oracle_bf16_rne_n(const float *v, uint16_t *out, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
