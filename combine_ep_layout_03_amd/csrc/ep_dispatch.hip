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
// once and, for FP8, quantized once; lanes 0..k-1 resolve the k destination
// rows and their base addresses are taken with readlane, so each of the k
// copies is a scalar-base + vector-offset 16-byte non-temporal store.
//   BF16: a segment is 128 chunks of 16 B (1024 channels), two chunks per lane
//         (c and c + 64), both loaded before the k copies are stored.
//   FP8:  a segment is 8 blocks of 128 channels; a lane holds 16 channels
//         (2 x 16 B of bf16 -> 16 B of E4M3), so 8 lanes form one block and
//         the block amax takes 3 xor-shuffles.  amax is taken on the bf16 bit
//         patterns (|x| is monotone in the low 15 bits), the scale is the
//         correctly rounded binary32 a/448 and every code is E4M3 of the
//         correctly rounded binary32 quotient x/s; the lane that holds a
//         block's first channels writes its scale into each copy.
// (Measured on MI355X at T=8192, H=7168, k=8: one-wave units beat one wave per
// token, four-wave workgroups, token-per-workgroup with LDS-staged scales,
// copy-per-wave splits and plain stores; the scattered row stores, not the
// quantization arithmetic, bound this kernel.  Plain stores look faster per
// call but leave dirty lines in the MALL whose write-back the next kernel
// pays: slower in steady state.  BF16 at T=4096, H=2048, k=6: two chunks per
// lane take 1.5 us off one chunk, four add it back.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kThreads = kRowWaves * kWave;
constexpr int kFp8SegBlocks = 8;  // 128-channel blocks per FP8 work unit (= 64 lanes x 16 ch)
constexpr int kBf16SegChunks = 2 * kWave;  // 16-byte chunks per BF16 work unit (two per lane)

// Lane j < k: byte address of token t's destination row j (0 if unusable,
// which also raises EP_DEVERR_ROW).  `rowbytes` is the destination row pitch.
__device__ inline uint64_t dest_row(const int32_t *__restrict__ idx,
                                    const int32_t *__restrict__ slot_of,
                                    const int32_t *__restrict__ rank_offsets,
                                    int32_t *__restrict__ err, int64_t p, int32_t E, int32_t El,
                                    int64_t cap, const void *const *base, int64_t rowbytes,
                                    int32_t &rank, int64_t &row) {
  const int32_t e = idx[p];
  if ((uint32_t)e < (uint32_t)E) {
    const int32_t r = e / El;
    const int64_t rr = (int64_t)slot_of[p] - rank_offsets[r];
    if (rr >= 0 && rr < cap) {
      rank = r;
      row = rr;
      return (uint64_t)base[r] + (uint64_t)(rr * rowbytes);
    }
  }
  atomicOr(err, (int32_t)EP_DEVERR_ROW);
  return 0;
}

__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ err, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El, int64_t cap,
    RankPtrs rx) {
  if (*err != 0) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nch = H / 8;  // 16-byte chunks per row
  const int nseg = (nch + kBf16SegChunks - 1) / kBf16SegChunks;
  const int64_t units = (int64_t)T * nseg;
  for (int64_t u = (int64_t)blockIdx.x * kRowWaves + wave; u < units;
       u += (int64_t)gridDim.x * kRowWaves) {
    const int64_t t = u / nseg;
    const int c0 = (int)(u % nseg) * kBf16SegChunks + lane;
    const int c1 = c0 + kWave;
    uint64_t dst = 0;
    if (lane < k) {
      int32_t r;
      int64_t row;
      dst = dest_row(idx, slot_of, rank_offsets, err, t * k + lane, E, El, cap,
                     (const void *const *)rx.p, (int64_t)H * 2, r, row);
    }
    if (__ballot(lane < k && dst == 0) != 0) continue;  // a bad row: write nothing for t
    const bool ok0 = c0 < nch, ok1 = c1 < nch;
    const u32x4 *xrow = reinterpret_cast<const u32x4 *>(x + t * H);
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (ok0) v0 = __builtin_nontemporal_load(xrow + c0);
    if (ok1) v1 = __builtin_nontemporal_load(xrow + c1);
    for (int j = 0; j < k; ++j) {
      u32x4 *d = reinterpret_cast<u32x4 *>(readlane64(dst, j));
      if (ok0) __builtin_nontemporal_store(v0, d + c0);
      if (ok1) __builtin_nontemporal_store(v1, d + c1);
    }
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ err, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El, int64_t cap,
    RankPtrs rq, ScalePtrs rs) {
  if (*err != 0) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nb = H / 128;  // 128-channel blocks per row
  const int nseg = (nb + kFp8SegBlocks - 1) / kFp8SegBlocks;
  const int64_t units = (int64_t)T * nseg;
  for (int64_t u = (int64_t)blockIdx.x * kRowWaves + wave; u < units;
       u += (int64_t)gridDim.x * kRowWaves) {
    const int64_t t = u / nseg;
    const int blk = (int)(u % nseg) * kFp8SegBlocks + lane / 8;
    uint64_t qdst = 0, sdst = 0;
    if (lane < k) {
      int32_t r = 0;
      int64_t row = 0;
      qdst = dest_row(idx, slot_of, rank_offsets, err, t * k + lane, E, El, cap,
                      (const void *const *)rq.p, (int64_t)H, r, row);
      if (qdst) sdst = (uint64_t)(rs.p[r] + row * nb);
    }
    if (__ballot(lane < k && qdst == 0) != 0) continue;  // a bad row: write nothing for t
    const bool valid = blk < nb;
    const int ch = blk * 128 + (lane % 8) * 16;
    const uint16_t *xrow = x + t * H;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (valid) {
      v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch));
      v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch + 8));
    }
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
  }
}

}  // namespace

hipError_t launch_dispatch(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                           const void *x, const RankPtrs &rx, const ScalePtrs &rs,
                           int64_t capacity_rows, hipStream_t s) {
  const int32_t El = c.num_experts / c.num_ranks;
  if (c.dispatch_dtype == EP_DTYPE_FP8_E4M3) {
    const int64_t nseg = (c.hidden / 128 + kFp8SegBlocks - 1) / kFp8SegBlocks;
    const int grid = row_grid(c, (int64_t)c.num_tokens * nseg);
    hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const uint16_t *>(x), topk_idx, h.slot_of, h.rank_offsets,
                       h.error_flag, c.num_tokens, c.hidden, c.num_topk, c.num_experts, El,
                       capacity_rows, rx, rs);
  } else {
    const int64_t nseg = (c.hidden / 8 + kBf16SegChunks - 1) / kBf16SegChunks;
    const int grid = row_grid(c, (int64_t)c.num_tokens * nseg);
    hipLaunchKernelGGL(dispatch_bf16_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<const uint16_t *>(x), topk_idx, h.slot_of, h.rank_offsets,
                       h.error_flag, c.num_tokens, c.hidden, c.num_topk, c.num_experts, El,
                       capacity_rows, rx);
  }
  return hipGetLastError();
}

}  // namespace ep
