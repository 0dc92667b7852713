// ep_dispatch.hip -- dispatch on gfx950: copy every token row into the
// receive buffers of its k experts' ranks, optionally quantized to FP8.
//
// Pages: [DeepEP overview] "DeepSeek merilis library open source DeepEP ...",
// "Pola penggunaan ..." (dispatch routes tokens to the experts' ranks, from
// BF16 or FP8) and "Hasil pengukuran performa" (the V3 config: FP8 dispatch);
// [Perplexity blog] "Lower latency and higher throughput with multi-node
// DeepSeek deployment", "Magntölun" (activation scales over 128-element
// vectors, computed on the fly; the horizontal amax is the awkward part).
//
// Design.  The work unit is one (token, segment) pair and one single-wave
// workgroup takes one unit at a time (grid-stride), so a token's row is spread
// over several short-lived waves.  Each unit's slice of the token row is read
// once and, for FP8, quantized once; lanes 0..k-1 form the k destination rows
// from the token's indices and slots and the per-lane rank tables (row_addr),
// and their base addresses are taken with readlane, so each of the k copies is
// a scalar-base + vector-offset 16-byte non-temporal store.
//   BF16: a segment is 128 chunks of 16 B (1024 channels), two chunks per lane
//         (c and c + 64), both loaded before the k copies are stored.
//   FP8:  a segment is 8 blocks of 128 channels; a lane holds 16 channels
//         (2 x 16 B of bf16 -> 16 B of E4M3), so 8 lanes form one block and
//         the block amax takes 3 xor-shuffles.  amax is taken on the bf16 bit
//         patterns (|x| is monotone in the low 15 bits), the scale is the
//         correctly rounded binary32 a/448 and every code is E4M3 of the
//         correctly rounded binary32 quotient x/s; the lane that holds a
//         block's first channels writes its scale into each copy.
// The gradient rows of combine's backward are the BF16 form with one multiply
// per copy (combine_backward_rows_kernel): the backward of combine is a
// dispatch of grad_out.
// (Measured on MI355X at T=8192, H=7168, k=8: one-wave units beat one wave per
// token, four-wave workgroups, token-per-workgroup with LDS-staged scales,
// copy-per-wave splits and plain stores; the scattered row stores, not the
// quantization arithmetic, bound this kernel.  Plain stores look faster per
// call but leave dirty lines in the MALL whose write-back the next kernel
// pays: slower in steady state.  BF16 at T=4096, H=2048, k=6: two chunks per
// lane take 1.5 us off one chunk, four add it back.  Issuing every load of a
// unit at once, instead of resolving index -> rank offset -> base pointer one
// dependent load at a time, is worth 13 % at decode (T=128) and nothing at
// T=8192, where the stores bound the kernel.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kThreads = kRowWaves * kWave;
constexpr int kFp8SegBlocks = 8;  // 128-channel blocks per FP8 work unit (= 64 lanes x 16 ch)
constexpr int kBf16SegChunks = 2 * kWave;  // 16-byte chunks per BF16 work unit (two per lane)

// Large dispatches keep fewer of their waves resident (resident_cap_lds): a
// CU holds at most 14 FP8 or 12 BF16 dispatch workgroups instead of the 32
// their registers allow.  With every wave's scattered row stores in flight at
// once the memory system queues more than it can schedule well; fewer waves
// write faster.  Measured on MI355X (same process, interleaved): FP8 at
// T=8192, H=7168, k=8 122.2 -> 116.4 us (dispatch + combine 301.2 -> 296.1
// us), Zipf-skewed routing 116.9 -> 111.2 us, BF16 at the same shape 215.9 ->
// 204.3 us; 12 to 16 workgroups per CU all gain, 8 lose.  Below two rounds of
// the GPU's resident waves a partly filled extra round can cost more than
// this gains (FP8 at T=512: 9.7 us uncapped, 12.1 us at 12 per CU), hence
// kResidentCapMinUnits.  (The SiLU re-quantization, with more arithmetic per
// byte, is slower with fewer waves: 116 -> 124 us at 16 per CU.)
constexpr int kFp8WgPerCu = 14, kBf16WgPerCu = 12;

// The loads of a unit do not wait for one another: the error word (read once
// per wave, checked before the first write), the per-lane rank tables, the
// unit's slice of x and the token's k indices and slots are all in flight
// together; the destination rows then come from row_addr's shuffles.  A row
// outside the capacity (a stale handle) raises EP_DEVERR_ROW and the token is
// skipped.
//
// The BF16 copies of a unit.  Scaled (combine's backward, whose gradient rows
// are a dispatch of grad_out): copy j is bf16(RN32(w_j * x)), one binary32
// multiply per element with w_j = w[t*k+j] (1 if w is NULL), loaded beside
// the token's indices.
template <bool Scaled>
__device__ inline void bf16_rows(const uint16_t *__restrict__ x, const int32_t *__restrict__ idx,
                                 const int32_t *__restrict__ slot_of,
                                 const int32_t *__restrict__ rank_offsets,
                                 int32_t *__restrict__ err, const float *__restrict__ w, int32_t T,
                                 int32_t H, int32_t k, int32_t E, int32_t El, int32_t R,
                                 int64_t cap, const RankPtrs &rx) {
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nch = H / 8;  // 16-byte chunks per row
  const int nseg = (nch + kBf16SegChunks - 1) / kBf16SegChunks;
  const int64_t units = (int64_t)T * nseg;
  const int64_t u0 = (int64_t)blockIdx.x * kRowWaves + wave;
  if (u0 >= units) return;
  int32_t err0 = 0;
  // One unit; false once the error word is found set (nothing is written).
  // The word is read once, by the first unit, after its other loads are out.
  auto unit = [&](int64_t u, bool first) -> bool {
    const int64_t t = u / nseg;
    const int c0 = (int)(u % nseg) * kBf16SegChunks + lane;
    const int c1 = c0 + kWave;
    const bool ok0 = c0 < nch, ok1 = c1 < nch;
    int32_t e = -1, sl = 0;
    float wj = 1.0f;
    if (lane < k) {
      e = idx[t * k + lane];
      sl = slot_of[t * k + lane];
      if (Scaled && w) wj = w[t * k + lane];
    }
    int32_t my_roff = 0;
    uint64_t my_base = 0;
    if (lane < R) {
      my_roff = rank_offsets[lane];
      my_base = (uint64_t)rx.p[lane];
    }
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + t * H);
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (ok0) v0 = __builtin_nontemporal_load(xrow + c0);
    if (ok1) v1 = __builtin_nontemporal_load(xrow + c1);
    if (first) err0 = *err;
    if (err0 & kLayoutErrBits) return false;
    int rank;
    int64_t row;
    uint64_t dst = row_addr(e, sl, E, El, cap, my_roff, my_base, (int64_t)H * 2, rank, row);
    if (lane >= k) dst = 0;
    else if (dst == 0) atomicOr(err, (int32_t)EP_DEVERR_ROW);
    if (__ballot(lane < k && dst == 0) != 0) return true;  // a bad row: write nothing for t
    for (int j = 0; j < k; ++j) {
      u32x4 *d = reinterpret_cast<u32x4 *>(readlane64(dst, j));
      u32x4 o0 = v0, o1 = v1;
      if (Scaled) {
        const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
        float p0[8], p1[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[2 * i] = wv * __uint_as_float(v0[i] << 16);
          p0[2 * i + 1] = wv * __uint_as_float(v0[i] & 0xFFFF0000u);
          p1[2 * i] = wv * __uint_as_float(v1[i] << 16);
          p1[2 * i + 1] = wv * __uint_as_float(v1[i] & 0xFFFF0000u);
        }
        o0 = pack8(p0);
        o1 = pack8(p1);
      }
      if (ok0) __builtin_nontemporal_store(o0, d + c0);
      if (ok1) __builtin_nontemporal_store(o1, d + c1);
    }
    return true;
  };
  // the first unit outside the loop, so that its loads and the error word's
  // are in flight together (one unit per wave by default)
  if (!unit(u0, true)) return;
  for (int64_t u = u0 + (int64_t)gridDim.x * kRowWaves; u < units;
       u += (int64_t)gridDim.x * kRowWaves)
    unit(u, false);
}

__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ err, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El, int32_t R,
    int64_t cap, RankPtrs rx) {
  bf16_rows<false>(x, idx, slot_of, rank_offsets, err, nullptr, T, H, k, E, El, R, cap, rx);
}

// Combine's backward: its gradient rows (ep_combine_backward).
__global__ __launch_bounds__(kThreads) void combine_backward_rows_kernel(
    const uint16_t *__restrict__ gout, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ err, const float *__restrict__ w, int32_t T, int32_t H, int32_t k,
    int32_t E, int32_t El, int32_t R, int64_t cap, RankPtrs rg) {
  bf16_rows<true>(gout, idx, slot_of, rank_offsets, err, w, T, H, k, E, El, R, cap, rg);
}

__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ err, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El, int32_t R,
    int64_t cap, RankPtrs rq, ScalePtrs rs) {
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nb = H / 128;  // 128-channel blocks per row
  const int nseg = (nb + kFp8SegBlocks - 1) / kFp8SegBlocks;
  const int64_t units = (int64_t)T * nseg;
  const int64_t u0 = (int64_t)blockIdx.x * kRowWaves + wave;
  if (u0 >= units) return;
  int32_t err0 = 0;
  auto unit = [&](int64_t u, bool first) -> bool {  // as in the BF16 kernel
    const int64_t t = u / nseg;
    const int blk = (int)(u % nseg) * kFp8SegBlocks + lane / 8;
    const bool valid = blk < nb;
    const int ch = blk * 128 + (lane % 8) * 16;
    int32_t e = -1, sl = 0;
    if (lane < k) {
      e = idx[t * k + lane];
      sl = slot_of[t * k + lane];
    }
    int32_t my_roff = 0;
    uint64_t my_q = 0, my_s = 0;
    if (lane < R) {
      my_roff = rank_offsets[lane];
      my_q = (uint64_t)rq.p[lane];
      my_s = (uint64_t)rs.p[lane];
    }
    const uint16_t *xrow = x + t * H;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (valid) {
      v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch));
      v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch + 8));
    }
    if (first) err0 = *err;
    if (err0 & kLayoutErrBits) return false;
    int rank;
    int64_t row;
    uint64_t qdst = row_addr(e, sl, E, El, cap, my_roff, my_q, (int64_t)H, rank, row);
    const uint64_t sbase = shfl64(my_s, rank);
    uint64_t sdst = 0;
    if (lane >= k) qdst = 0;
    else if (qdst == 0) atomicOr(err, (int32_t)EP_DEVERR_ROW);
    else sdst = sbase + (uint64_t)(row * nb * 4);
    if (__ballot(lane < k && qdst == 0) != 0) return true;  // a bad row: write nothing for t
    // 8 lanes per block: invalid lanes form whole groups of 8 and stay at 0
    float s;
    const u32x4 q = quant_block16(v0, v1, s);
    for (int j = 0; j < k; ++j) {
      uint8_t *d = reinterpret_cast<uint8_t *>(readlane64(qdst, j));
      float *sd = reinterpret_cast<float *>(readlane64(sdst, j));
      if (valid) {
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(d + ch));
        if ((lane % 8) == 0) sd[blk] = s;
      }
    }
    return true;
  };
  if (!unit(u0, true)) return;
  for (int64_t u = u0 + (int64_t)gridDim.x * kRowWaves; u < units;
       u += (int64_t)gridDim.x * kRowWaves)
    unit(u, false);
}

}  // namespace

hipError_t launch_combine_backward_rows(const ep_config &c, const ep_layout_t &h,
                                        const int32_t *topk_idx, const void *grad_out,
                                        const float *w, const RankPtrs &rg,
                                        int64_t capacity_rows, hipStream_t s) {
  const int64_t nseg = (c.hidden / 8 + kBf16SegChunks - 1) / kBf16SegChunks;
  const int64_t units = (int64_t)c.num_tokens * nseg;
  hipLaunchKernelGGL(combine_backward_rows_kernel, dim3(row_grid(c, units)), dim3(kThreads),
                     resident_cap_lds(units, kBf16WgPerCu), s,
                     static_cast<const uint16_t *>(grad_out), topk_idx, h.slot_of, h.rank_offsets,
                     h.error_flag, w, c.num_tokens, c.hidden, c.num_topk, c.num_experts,
                     c.num_experts / c.num_ranks, c.num_ranks, capacity_rows, rg);
  return hipGetLastError();
}

hipError_t launch_dispatch(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                           const void *x, const RankPtrs &rx, const ScalePtrs &rs,
                           int64_t capacity_rows, hipStream_t s) {
  const int32_t El = c.num_experts / c.num_ranks;
  if (c.dispatch_dtype == EP_DTYPE_FP8_E4M3) {
    const int64_t nseg = (c.hidden / 128 + kFp8SegBlocks - 1) / kFp8SegBlocks;
    const int64_t units = (int64_t)c.num_tokens * nseg;
    hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(row_grid(c, units)), dim3(kThreads),
                       resident_cap_lds(units, kFp8WgPerCu), s,
                       static_cast<const uint16_t *>(x), topk_idx, h.slot_of, h.rank_offsets,
                       h.error_flag, c.num_tokens, c.hidden, c.num_topk, c.num_experts, El,
                       c.num_ranks, capacity_rows, rx, rs);
  } else {
    const int64_t nseg = (c.hidden / 8 + kBf16SegChunks - 1) / kBf16SegChunks;
    const int64_t units = (int64_t)c.num_tokens * nseg;
    hipLaunchKernelGGL(dispatch_bf16_kernel, dim3(row_grid(c, units)), dim3(kThreads),
                       resident_cap_lds(units, kBf16WgPerCu), s,
                       static_cast<const uint16_t *>(x), topk_idx, h.slot_of, h.rank_offsets,
                       h.error_flag, c.num_tokens, c.hidden, c.num_topk, c.num_experts, El,
                       c.num_ranks, capacity_rows, rx);
  }
  return hipGetLastError();
}

}  // namespace ep
