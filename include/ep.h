/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE token dispatch / combine library.
 *
 * Pages cited (by title and section):
 *   [DeepEP overview]  "DeepSeek merilis library open source DeepEP untuk
 *                      pelatihan dan inferensi MoE" (GeekNews, Indonesian):
 *                      "Antarmuka berpusat pada ElasticBuffer" (buffers sized
 *                      from the MoE config, a size hint, SM counts computed
 *                      analytically with a per-call override) and "Pola
 *                      penggunaan untuk pelatihan, prefill, dan decoding"
 *                      (dispatch routes tokens to their experts' ranks and
 *                      returns a handle with per-expert token counts for the
 *                      GEMM; combine reduces expert outputs back; the handle
 *                      is reused while gating is unchanged; the backward of
 *                      dispatch is a combine and vice versa).
 *   [Perplexity blog]  "Lower latency and higher throughput with multi-node
 *                      DeepSeek deployment" (Icelandic rendering):
 *                      "Sérfræðinga-samsíðun" (each GPU holds 256/EP experts;
 *                      the 8 routed results are weighted and summed),
 *                      "Magntölun" (activation scales over 128-element
 *                      vectors, computed on the fly, M x ceil_div(K,128)),
 *                      "MoE-beirari" (dense dispatch/combine need routing
 *                      summed per expert), "CUDA-graf" and the persistent-
 *                      kernel paragraph of "Magntölun" (under graphs, kernels
 *                      read the token counts on the device instead of sizing
 *                      work from the upper-bound buffer).
 *   [torchtitan PR]    "Integrate DeepEP to experimental torchtitan" (the
 *                      token unpermute after the experts; index selection on
 *                      the host costs CPU time; node-limited routing).
 *   [EPLB page]        "DeepSeek V3/R1 ... DualPipe, EPLB, Profile-Data"
 *                      (GeekNews, Turkish): redundant (replicated) experts
 *                      and group-limited expert routing.
 *
 * Model.  One GPU.  The R expert-parallel "ranks" are R destination buffers in
 * the same HBM; rank r owns the experts [r*E/R, (r+1)*E/R).  A (token t, top-k
 * slot j) pair p = t*k + j is one received row.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  All memory belongs
 *     to the caller; the library allocates nothing, keeps no pointer after a
 *     call returns and has no global mutable state, so calls on distinct
 *     handles and streams are independent.  The one exception is
 *     ep_layout_noalloc, whose chunk table is a static device array shared
 *     by all its calls on one GPU (see there).
 *   - Work is enqueued on `stream` and never synchronizes; inputs must stay
 *     alive and unmodified until the stream has passed the call.  Every call
 *     can be captured into a hipGraph (no host sync, no allocation, no memset
 *     nodes).
 *   - Host-checkable problems (NULL pointers, bad sizes, too small a
 *     capacity, a misaligned row buffer) return a nonzero ep_status at once
 *     and enqueue nothing.
 *   - Row buffers must be 16-byte aligned (EP_ERR_INVALID_ARG otherwise):
 *     x, recv_x[r], recv_scales[r], recv_y[r], out, shared, grad_out,
 *     grad_recv[r], act_in[r], q_out[r], scales_out[r] and the layout
 *     workspace.  The kernels move rows with 16-byte vector loads and stores;
 *     every row pitch is a multiple of 16 bytes by the size rules above, so
 *     an aligned base aligns every row.  Any device allocation is aligned;
 *     a view that starts inside a row is not.  The index, weight and logit
 *     arrays need only their element alignment.
 *   - Data problems found on the device (a routing index outside [0,E), a
 *     row outside the capacity) set bits in the handle's error word.  Every
 *     call that reads a handle (dispatch, combine with or without the shared
 *     expert, combine backward, the SiLU re-quantization, unpermute) reads
 *     the word first and writes nothing when the layout flagged the handle
 *     (EP_DEVERR_INDEX or EP_DEVERR_INTERNAL).  A row outside the capacity
 *     (a stale handle) is checked per pair: the pair's token is skipped and
 *     EP_DEVERR_ROW set, and every other token is written, so what a call
 *     writes does not depend on the order its waves run in.
 *   - Output bytes do not depend on ep_config.num_workgroups.
 *   - Resources: the row kernels run single-wave workgroups.  Dispatch,
 *     combine and the large-batch combine backward launches of 16384 work
 *     units or more (a unit is one token's 1024-channel segment) reserve 11
 *     to 13 KiB of LDS per workgroup that the kernels never touch, which caps
 *     how many of their workgroups a CU holds (fewer waves in flight move
 *     their scattered rows faster); kernels running beside them on the same
 *     CUs see that LDS as taken.
 *
 * Data types: routing indices int32 [T,k] row-major; weights fp32 [T,k];
 * activations bf16 as 16-bit patterns; FP8 is OCP E4M3 ("fn", max 448) one
 * byte per channel; scales fp32.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 2u  /* 2: row buffers must be 16-byte aligned; ep_layout_noalloc */

/* Limits of this build. */
#define EP_MAX_RANKS 64    /* R: per-rank buffer pointers travel as kernel arguments */
#define EP_MAX_TOPK 32     /* k */
#define EP_MAX_EXPERTS 2048 /* E: the layout keeps per-expert counters in LDS */
#define EP_MAX_HIDDEN 65536 /* H */
#define EP_MAX_GROUPS 64    /* router expert groups: one per lane of a wave */

typedef int32_t ep_status;
#define EP_OK 0
#define EP_ERR_INVALID_ARG 1 /* NULL pointer or a size outside the limits */
#define EP_ERR_UNSUPPORTED 2 /* a valid request this build does not implement */
#define EP_ERR_CAPACITY 3    /* capacity_rows below ep_recv_capacity_rows() */
#define EP_ERR_HIP 4         /* a HIP launch failed (hipGetLastError) */

/* Bits of the device error word (ep_layout_t.error_flag[0]).  The layout
 * (ep_layout, ep_layout_dispatch, ep_route_layout) rewrites the word: it
 * clears it and sets EP_DEVERR_INDEX, in an order no other write of the same
 * layout can overtake (a two-launch layout clears it in its first launch; a
 * one-launch layout has one workgroup write it).  Later calls only OR bits
 * in. */
#define EP_DEVERR_INDEX 1u    /* ep_layout saw an index outside [0,E) */
#define EP_DEVERR_ROW 2u      /* a call saw a row outside [0,capacity) and skipped
                                 that row's token */
#define EP_DEVERR_INTERNAL 4u /* ep_layout computed a slot outside [0,T*k): a library
                                 bug.  Such a pair's slot_of is -1, so later calls on
                                 the handle report EP_DEVERR_ROW for its token even
                                 where the layout could not set this bit without a
                                 race (a one-launch layout's other workgroups). */

typedef int32_t ep_dtype;
#define EP_DTYPE_BF16 0     /* dispatch copies bf16 rows */
#define EP_DTYPE_FP8_E4M3 1 /* dispatch quantizes rows to E4M3 + fp32 scales */

typedef int32_t ep_gate;
#define EP_GATE_SOFTMAX 0 /* softmax over the token's logical experts */
#define EP_GATE_SIGMOID 1 /* independent sigmoid per expert */

typedef struct {
  int32_t num_tokens;     /* T >= 1 (cf. num_max_tokens_per_rank of the buffer) */
  int32_t hidden;         /* H, multiple of 8; of 128 under FP8 */
  int32_t num_topk;       /* k in [1, EP_MAX_TOPK] */
  int32_t num_experts;    /* E in [1, EP_MAX_EXPERTS], E % R == 0 */
  int32_t num_ranks;      /* R in [1, EP_MAX_RANKS] */
  int32_t dispatch_dtype; /* ep_dtype (cf. use_fp8_dispatch) */
  int32_t num_workgroups; /* 0 = analytic default; otherwise the grid size of
                             the per-row kernels: dispatch, combine (and with
                             the shared expert), combine backward, unpermute,
                             the SiLU re-quantization, the router and the
                             one-launch layout + dispatch (cf. the per-call
                             SM-count override).  The layout's kernels keep
                             their own grids. */
} ep_config;

/* The routing handle.  Caller-allocated device arrays; ep_layout fills them
 * and dispatch / combine / unpermute read them.  Reusing one handle across
 * calls with unchanged routing is the cached-handle path. */
typedef struct {
  int32_t *expert_counts;  /* [E]   rows routed to each expert */
  int32_t *expert_offsets; /* [E+1] exclusive prefix of expert_counts (global slot space) */
  int32_t *rank_counts;    /* [R]   rows valid in each rank buffer; sums to T*k */
  int32_t *rank_offsets;   /* [R+1] = expert_offsets[r*E/R]; rank_offsets[R] = T*k */
  int32_t *slot_of;        /* [T*k] pair p -> global slot; its row in rank r's
                              buffer is slot_of[p] - rank_offsets[r] */
  int32_t *src_of;         /* [T*k] global slot -> pair p (inverse of slot_of) */
  int32_t *error_flag;     /* [1]   EP_DEVERR_* bits, 0 = ok */
} ep_layout_t;

/* Router parameters (see ep_route).  Node-limited routing is group-limited
 * routing with one group per node's experts. */
typedef struct {
  int32_t num_logical;  /* El in [1, EP_MAX_EXPERTS]: experts the router scores */
  int32_t gate;         /* ep_gate */
  int32_t num_groups;   /* G in [1, EP_MAX_GROUPS], El % G == 0; 1 = plain top-k */
  int32_t topk_groups;  /* TG in [1, G]: groups a token may use; k <= TG * El/G */
  int32_t group_topn;   /* 1: a group scores its best expert; 2: its two best, summed */
  int32_t renormalize;  /* nonzero: weights divided by their sum over the k chosen */
} ep_router_t;

/* EP_ABI_VERSION of the loaded library. */
uint32_t ep_abi_version(void);

/* Static text for a status code. */
const char *ep_status_string(ep_status status);

/* Rows each rank buffer must hold: T*k, the worst case (every pair of every
 * token on one rank; a token may name one expert twice).  Cf. the buffer size
 * hint of [DeepEP overview] "Antarmuka berpusat pada ElasticBuffer".
 * Returns -1 for an invalid config. */
int64_t ep_recv_capacity_rows(const ep_config *cfg /*(host)*/);

/* Bytes of device workspace ep_layout, ep_layout_dispatch and ep_route_layout
 * need for this config (their per-chunk expert histograms; the larger of the
 * two table shapes).  Returns 0 for an invalid config. */
size_t ep_layout_workspace_bytes(const ep_config *cfg /*(host)*/);

/* Routing layout ([Perplexity blog] "MoE-beirari"; [DeepEP overview] "Pola
 * penggunaan ...").  From topk_idx [T,k] computes
 *   expert_counts[e] = #{p : topk_idx[p] = e},
 *   expert_offsets   = exclusive prefix over e,
 *   rank_counts[r], rank_offsets[r] over rank r's experts,
 *   slot_of[p] = expert_offsets[e] + #{p' < p : topk_idx[p'] = e}
 *     (a counting sort by expert that keeps ascending p inside each expert:
 *      the expert-contiguous "GEMM layout"), and src_of = slot_of^-1,
 * and writes error_flag (EP_DEVERR_INDEX when an index is outside [0,E); the
 * other handle arrays are then unspecified).  `workspace` must hold
 * ep_layout_workspace_bytes(cfg) bytes and be 16-byte aligned (any device
 * allocation is; otherwise EP_ERR_INVALID_ARG); its contents on entry do not
 * matter and are clobbered.  Launches one kernel for T*k <= 2048, or for
 * T*k <= 8192 with E <= 384, else two, on `stream`. */
ep_status ep_layout(const ep_config *cfg /*(host)*/, const int32_t *topk_idx,
                    const ep_layout_t *h /*(host struct of device pointers)*/,
                    void *workspace, hipStream_t stream);

/* ep_layout without a workspace argument, for callers that cannot allocate
 * device memory: code under hipGraph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus `workspace`), results and
 * errors as ep_layout.  The per-chunk table lives in a file-scope device
 * array of 288 KiB, which covers every valid config (EP_ERR_UNSUPPORTED if a
 * config ever needed more); each GPU the library runs on holds its own copy
 * until the process ends.  The first call on a device resolves the array's
 * address (hipGetSymbolAddress; make that first call outside a capture); no
 * call allocates.  All calls on one GPU share the array: calls that overlap
 * in time on one GPU (different streams, or concurrent host threads) race
 * and must be serialized by the caller. */
ep_status ep_layout_noalloc(const ep_config *cfg /*(host)*/, const int32_t *topk_idx,
                            const ep_layout_t *h /*(host struct of device pointers)*/,
                            hipStream_t stream);

/* Dispatch ([DeepEP overview] "Pola penggunaan ...": route each token to its
 * top-k experts' ranks; [Perplexity blog] "Magntölun" for FP8).  For every
 * pair p = (t, j), with r = topk_idx[p] / (E/R) and row = slot_of[p] -
 * rank_offsets[r]:
 *   BF16: recv_x[r] row `row` (H bf16) := x[t], bit for bit;
 *   FP8:  for each 128-channel block b of x[t]: a = max|x|, s = a/448 (fp32,
 *         correctly rounded), q = E4M3(x/s) (fp32 quotient, round to nearest
 *         even, saturating at 448); a = 0 gives s = 0 and q = 0x00; with
 *         non-finite values the same formulas in IEEE arithmetic: a NaN in
 *         the block makes a and s NaN and every code NaN, an infinity makes
 *         s = +inf (finite values -> signed zero codes, infinities -> NaN
 *         codes); the sign and payload of NaN codes and scales are
 *         unspecified;
 *         recv_x[r] row `row` (H bytes) := q, recv_scales[r] row `row`
 *         (H/128 fp32) := s.  Every copy of a token is byte-identical.
 * x is [T,H] bf16; recv_x / recv_scales are (host) arrays of R device
 * pointers to row-major buffers of capacity_rows rows (recv_scales is ignored
 * and may be NULL for BF16).  Rows past rank_counts[r] are not written. */
ep_status ep_dispatch(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                      const int32_t *topk_idx, const void *x,
                      void *const *recv_x /*(host)[R]*/, float *const *recv_scales /*(host)[R]*/,
                      int64_t capacity_rows, hipStream_t stream);

/* Layout and dispatch in one call, for small batches (decode): the same
 * handle and the same receive bytes as ep_layout followed by ep_dispatch
 * ([Perplexity blog] "CUDA-graf": a decode step is bound by launch overhead).
 * With T*k <= 2048 this is ONE kernel launch: every workgroup reads the
 * whole index array and derives the offsets itself, so none waits for
 * another.  Larger inputs run ep_layout's and ep_dispatch's kernels, so
 * `workspace` must hold ep_layout_workspace_bytes(cfg) bytes either way.
 * Arguments and errors as for ep_layout and ep_dispatch; an index outside
 * [0,E) sets EP_DEVERR_INDEX and nothing is dispatched. */
ep_status ep_layout_dispatch(const ep_config *cfg /*(host)*/, const int32_t *topk_idx,
                             const ep_layout_t *h /*(host)*/, void *workspace, const void *x,
                             void *const *recv_x /*(host)[R]*/,
                             float *const *recv_scales /*(host)[R]*/, int64_t capacity_rows,
                             hipStream_t stream);

/* Combine ([Perplexity blog] "Sérfræðinga-samsíðun": the routed results are
 * weighted and summed; [DeepEP overview] "Pola penggunaan ...": combine
 * reduces expert outputs back to the source).  For every token t and channel
 * h:  acc = +0;  for j = 0..k-1:  acc = fma(w[t][j], y_j[h], acc)  (fp32);
 * out[t][h] = bf16(acc) rounded to nearest even, where y_j is row
 * slot_of[t*k+j] - rank_offsets[r] of recv_y[r].  This fuses the un-permute.
 * topk_weights NULL means all weights 1 (the backward of dispatch).
 * recv_y is a (host) array of R device pointers to [capacity_rows, H] bf16;
 * out is [T,H] bf16 and is written exactly once per element. */
ep_status ep_combine(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                     const int32_t *topk_idx, const void *const *recv_y /*(host)[R]*/,
                     const float *topk_weights, void *out, int64_t capacity_rows,
                     hipStream_t stream);

/* Combine plus the shared expert ([Perplexity blog] "Sérfræðinga-samsíðun":
 * every token also goes through the shared expert, whose result is added to
 * the routed experts' result).  As ep_combine, except that after the routed
 * fold acc = acc + f32(shared[t][h]) (one fp32 addition) before the bf16
 * rounding.  shared is [T,H] bf16 and must not be NULL. */
ep_status ep_combine_shared(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                            const int32_t *topk_idx, const void *const *recv_y /*(host)[R]*/,
                            const float *topk_weights, const void *shared, void *out,
                            int64_t capacity_rows, hipStream_t stream);

/* Backward of combine ([DeepEP overview] "Pola penggunaan ...": the backward
 * of combine is a dispatch).  For every pair p = (t, j) with its row as in
 * ep_combine:
 *   grad_recv[r] row `row` (H bf16) := bf16(w[t][j] * grad_out[t][h]), the
 *     product one fp32 multiply, rounded to nearest even (topk_weights NULL:
 *     unit weights, an exact copy);
 *   grad_weights[t][j] := <grad_out[t], y row>, accumulated in fp32 in a
 *     fixed order (each thread's channels in order, a butterfly across the
 *     wave and, for T < 2048, where a token takes a workgroup of 8 waves,
 *     those waves in order), so it does not depend on num_workgroups, when
 *     recv_y / grad_weights are given; pass both or neither.
 * The backward of dispatch is ep_combine with topk_weights NULL applied to
 * the gradient rows.  grad_out is [T,H] bf16; grad_recv and recv_y are (host)
 * arrays of R device pointers to [capacity_rows, H] bf16; grad_weights is
 * [T,k] fp32. */
ep_status ep_combine_backward(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                              const int32_t *topk_idx, const void *grad_out,
                              const float *topk_weights, const void *const *recv_y /*(host)[R]*/,
                              void *const *grad_recv /*(host)[R]*/, float *grad_weights,
                              int64_t capacity_rows, hipStream_t stream);

/* Expert activation on the received rows ([Perplexity blog] "Magntölun":
 * SiLU with per-128-element block quantization, scales on the fly, work
 * split from device-side token counts under graphs).  For every received row
 * (the T*k slots, mapped to rank r and row with the handle's rank_offsets on
 * the device): gate = act_in row [0, I), up = [I, 2I) (bf16);
 *   a = g * rcp(1 + e^-g) * u in fp32, with e^-g from the hardware base-2
 *   exponential after a split-constant argument reduction and the hardware
 *   reciprocal (within 2.34 fp32 ulps of the binary64 value), then
 *   per 128-element block s = a_max/448 (correctly rounded) and
 *   q = E4M3(a * (1/s)) (one divide per block; exact a/s for blocks whose
 *   1/s overflows).
 * act_in: (host) R pointers to [capacity_rows, 2I] bf16; q_out: (host) R
 * pointers to [capacity_rows, I] bytes; scales_out: (host) R pointers to
 * [capacity_rows, I/128] fp32.  intermediate = I, a multiple of 128.  Rows
 * past rank_counts[r] are not read or written.  Results match a binary64
 * reference to E4M3 rounding (codes can differ where the fp32 activation
 * sits on a rounding boundary). */
ep_status ep_silu_mul_quant(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                            int32_t intermediate, const void *const *act_in /*(host)[R]*/,
                            void *const *q_out /*(host)[R]*/, float *const *scales_out /*(host)[R]*/,
                            int64_t capacity_rows, hipStream_t stream);

/* Router ([Perplexity blog] "MoE-beirari": one router for every MoE model,
 * DeepSeek's group-limited top-k with Mixtral's as the case of one group
 * holding all experts, emitting top-k indices and scores per token;
 * [EPLB page]: group-limited routing and redundant experts; [torchtitan PR]:
 * node-limited routing).  For each token t, with logits [T, El] fp32:
 *   z[e] = logits[t][e] + bias[e]  (one fp32 add; bias [El] may be NULL);
 *   s[e] = gate score evaluated in binary64 and rounded once to fp32:
 *          softmax exp(z_e - max z) / sum exp(z_i - max z), the sum taken
 *          in ascending i (one binary64 addition at a time), or sigmoid
 *          1 / (1 + exp(-z_e));
 *   each group of El/G consecutive experts scores its best s (group_topn 1)
 *          or the fp32 sum of its two best; the TG best groups stay eligible;
 *   topk_idx[t] = the k best eligible experts, best first; equal scores
 *          (compared as fp32 bit patterns) go to the lower id;
 *   topk_weights[t][j] = s of expert j, divided by the fp32 sum over j
 *          (ascending) when renormalize is set and that sum is > 0.
 * Redundant experts: with replica_offsets [El+1] and replica_slots (device
 * arrays, CSR), logical expert l is served by physical experts
 * replica_slots[replica_offsets[l] ..  replica_offsets[l+1]) and token t
 * takes the (t mod count)-th; a logical expert with no replica yields -1,
 * and a slot outside [0, E) is passed through, so ep_layout flags either with
 * EP_DEVERR_INDEX.  Without a table (both NULL) topk_idx holds logical ids and
 * cfg->num_experts must equal El.  Logits must be finite (otherwise the
 * choice is unspecified but still k distinct experts).  cfg->hidden and
 * num_ranks are checked as everywhere but not used.  One launch: one wave
 * per token, or four tokens per wave from 2048 tokens on (same results). */
ep_status ep_route(const ep_config *cfg /*(host)*/, const ep_router_t *router /*(host)*/,
                   const float *logits, const float *bias, const int32_t *replica_offsets,
                   const int32_t *replica_slots, int32_t *topk_idx, float *topk_weights,
                   hipStream_t stream);

/* ep_route followed by ep_layout on its output ([Perplexity blog]
 * "MoE-beirari": the dense dispatch and combine need the routing summed per
 * expert), so the handle is built from the logits with no host round trip.
 * Where ep_layout would take two launches and the router routes four tokens
 * per wave (E <= 512, num_workgroups 0), the router also counts the layout's
 * per-chunk expert histograms -- one router workgroup per chunk of tokens --
 * so only the layout's scatter kernel follows (two launches instead of
 * three); otherwise it runs the two calls' kernels in turn.  The results are
 * the same bytes either way.  Arguments as for the two calls; `workspace` as
 * for ep_layout. */
ep_status ep_route_layout(const ep_config *cfg /*(host)*/, const ep_router_t *router /*(host)*/,
                          const float *logits, const float *bias, const int32_t *replica_offsets,
                          const int32_t *replica_slots, int32_t *topk_idx, float *topk_weights,
                          const ep_layout_t *h /*(host)*/, void *workspace, hipStream_t stream);

/* Un-permute ([torchtitan PR]: the token unpermute after the experts) as a
 * standalone call for testing: out[p] (H bf16) := recv_y[r(p)] row row(p), so
 * out is [T*k, H] in (t, j) order.  Same arguments and errors as ep_combine. */
ep_status ep_unpermute(const ep_config *cfg /*(host)*/, const ep_layout_t *h /*(host)*/,
                       const int32_t *topk_idx, const void *const *recv_y /*(host)[R]*/,
                       void *out, int64_t capacity_rows, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* EP_H */
