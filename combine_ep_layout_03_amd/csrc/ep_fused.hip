// ep_fused.hip -- routing layout and dispatch in ONE launch, for small
// batches (decode).
//
// Pages: [Perplexity blog] "Lower latency and higher throughput with
// multi-node DeepSeek deployment", "CUDA-graf" (one graph per batch size; a
// decode step is bound by launch overhead) and "MoE-beirari" (dense dispatch
// needs the routing summed per expert); [DeepEP overview] "DeepSeek merilis
// library open source DeepEP ...", "Pola penggunaan ..." (decode reuses the
// routing handle while gating is unchanged).
//
// Design.  With T*k <= kFusedMaxPairs the whole index array is 8 KB or less,
// so every single-wave workgroup reads all of it (coalesced, L2-resident) and
// computes the expert histogram and its exclusive scan in LDS itself: no
// workgroup waits for another, and the layout costs no launch of its own.  A
// workgroup then takes (token, segment) units like ep_dispatch; for its
// token's k pairs it finds each pair's rank among the earlier pairs of the
// same expert by counting matches in the register-held index array -- eight
// pairs at once, two counts per word, reduced by DPP row sums -- which gives
// exactly the stable slot of the two-pass layout.  The unit's payload and its
// token's k indices are loaded first, so their latency overlaps the layout
// work (reading the indices after the histogram's barriers cost 1.3 us).  Segment-0 units
// write their token's slot_of / src_of entries; unit 0 writes the per-expert
// and per-rank arrays and the error word.  The row payload is the same code
// as ep_dispatch.  (Measured on MI355X at 128 tokens x 8: counting one pair
// at a time, each a dependent load and a shuffle-based wave sum, took 5.8 of
// this kernel's 11.8 us.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kPL = kFusedMaxPairs / kWave;  // indices held per lane
constexpr int kFp8SegBlocks = 8;             // as in ep_dispatch

// One unit's slice of x: FP8 units take 16 channels per lane (two 16-byte
// vectors), BF16 units one 16-byte chunk per lane (v1 unused).
template <bool FP8>
__device__ inline void load_payload(const uint16_t *__restrict__ x, int64_t t, int seg, int H,
                                    int lane, u32x4 &v0, u32x4 &v1) {
  v0 = u32x4{0u, 0u, 0u, 0u};
  v1 = v0;
  const uint16_t *xrow = x + t * H;
  if (FP8) {
    const int blk = seg * kFp8SegBlocks + lane / 8;
    if (blk < H / 128) {
      const int ch = blk * 128 + (lane % 8) * 16;
      v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch));
      v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + ch + 8));
    }
  } else {
    const int c = seg * kWave + lane;
    if (c < H / 8) v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow) + c);
  }
}

template <bool FP8>
__global__ __launch_bounds__(kWave) void layout_dispatch_small_kernel(
    const int32_t *__restrict__ idx, const uint16_t *__restrict__ x, int32_t T, int32_t H,
    int32_t k, int32_t E, int32_t R, int64_t cap, RankPtrs rq, ScalePtrs rs, ep_layout_t h) {
  extern __shared__ int32_t off[];  // [E+1]: histogram, then exclusive offsets
  const int lane = threadIdx.x;
  const int64_t P = (int64_t)T * k;
  const int32_t El = E / R;
  const int nv = (int)((P + kWave - 1) / kWave);  // index registers in use
  const int nb = H / 128, nch = H / 8;
  const int nseg = FP8 ? (nb + kFp8SegBlocks - 1) / kFp8SegBlocks : (nch + kWave - 1) / kWave;
  const int64_t units = (int64_t)T * nseg;

  // the first unit's payload and its token's k indices, and the ranks'
  // buffer bases (lane r < R holds rank r's, taken later with a shuffle),
  // loaded now so that they overlap the layout work
  int64_t u = blockIdx.x;
  u32x4 pv0, pv1;
  int32_t e_first = 0;
  if (u < units) {
    load_payload<FP8>(x, u / nseg, (int)(u % nseg), H, lane, pv0, pv1);
    if (lane < k) e_first = idx[(u / nseg) * k + lane];
  }
  uint64_t my_q = 0, my_s = 0;
  if (lane < R) {
    my_q = (uint64_t)rq.p[lane];
    if (FP8) my_s = (uint64_t)rs.p[lane];
  }

  // every index, coalesced: value i of this lane is pair i*64 + lane
  int32_t ev[kPL];
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int64_t p = (int64_t)i * kWave + lane;
    ev[i] = (i < nv && p < P) ? idx[p] : 0;
    if (i < nv && p < P && (uint32_t)ev[i] >= (uint32_t)E) ++bad;
  }
  for (int e = lane; e <= E; e += kWave) off[e] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPL; ++i) {
    const int64_t p = (int64_t)i * kWave + lane;
    if (i < nv && p < P && (uint32_t)ev[i] < (uint32_t)E) atomicAdd(&off[ev[i]], 1);
  }
  bad = wave_sum_u32(bad);
  __syncthreads();
  {  // exclusive scan of off[0..E), off[E] = total
    const int per = (E + kWave - 1) / kWave;
    const int b = (lane * per < E) ? lane * per : E;
    const int end = (b + per < E) ? b + per : E;
    int32_t s = 0;
    for (int i = b; i < end; ++i) s += off[i];
    const int32_t incl = wave_inclusive_scan(s, lane);
    int32_t run = incl - s;
    for (int i = b; i < end; ++i) {
      const int32_t v = off[i];
      off[i] = run;
      run += v;
    }
    if (lane == kWave - 1) off[E] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = lane; e < E; e += kWave) {
      h.expert_counts[e] = off[e + 1] - off[e];
      h.expert_offsets[e] = off[e];
    }
    for (int r = lane; r < R; r += kWave) {
      h.rank_offsets[r] = off[r * El];
      h.rank_counts[r] = off[(r + 1) * El] - off[r * El];
    }
    if (lane == 0) {
      h.expert_offsets[E] = off[E];
      h.rank_offsets[R] = off[E];
      h.error_flag[0] = bad ? (int32_t)EP_DEVERR_INDEX : 0;
    }
  }
  if (bad) return;  // uniform: nothing is dispatched for a bad index array

  for (; u < units; u += gridDim.x) {
    const int64_t t = u / nseg;
    const int seg = (int)(u % nseg);
    if (u != (int64_t)blockIdx.x) load_payload<FP8>(x, t, seg, H, lane, pv0, pv1);
    // lane j < k: the expert e of pair (t, j) and its slot = offset of e +
    // the earlier pairs with e: those before the token's first pair t*k,
    // counted for 8 of the token's experts at a time over every lane's
    // indices (two counts per 32-bit word, each < P <= 2048, reduced by DPP
    // row sums), plus the token's own earlier pairs with e
    const int32_t tk = (int32_t)(t * k);
    const int32_t my_e = (u == (int64_t)blockIdx.x) ? e_first : ((lane < k) ? idx[tk + lane] : 0);
    int32_t my_slot = 0;
    for (int j0 = 0; j0 < k; j0 += 8) {
      int32_t ej[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) ej[jj] = (j0 + jj < k) ? (int32_t)rdl((uint32_t)my_e, j0 + jj) : -1;
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kPL; ++i) {
        if (i < nv && i * kWave + lane < tk) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) c[jj / 2] += (ev[i] == ej[jj]) ? (1u << (16 * (jj & 1))) : 0u;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = wave_sum_u32(c[q]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)  // pairs j0 + jj >= k have no expert (ej = -1)
        if (j0 + jj < k && lane == j0 + jj)
          my_slot = off[ej[jj]] + (int32_t)((c[jj / 2] >> (16 * (jj & 1))) & 0xFFFFu);
    }
    for (int j = 0; j < k; ++j) my_slot += (j < lane && (int32_t)rdl((uint32_t)my_e, j) == my_e) ? 1 : 0;
    uint64_t dst = 0, sdst = 0;
    const int32_t r = (lane < k) ? my_e / El : 0;
    const uint64_t qbase = shfl64(my_q, r);
    const uint64_t sbase = FP8 ? shfl64(my_s, r) : 0;
    if (lane < k) {
      const int64_t row = (int64_t)my_slot - off[r * El];
      if (row >= 0 && row < cap) {  // always holds: slots are < T*k <= cap
        dst = qbase + (uint64_t)(row * (FP8 ? (int64_t)H : (int64_t)H * 2));
        if (FP8) sdst = sbase + (uint64_t)(row * nb * 4);
      }
      if (seg == 0) {
        const int64_t p = t * k + lane;
        h.slot_of[p] = my_slot;
        if ((uint64_t)(uint32_t)my_slot < (uint64_t)P) h.src_of[my_slot] = (int32_t)p;
      }
    }
    if (__ballot(lane < k && dst == 0) != 0) continue;
    if (FP8) {
      const int blk = seg * kFp8SegBlocks + lane / 8;
      const bool valid = blk < nb;
      const int ch = blk * 128 + (lane % 8) * 16;
      float s;
      const u32x4 q = quant_block16(pv0, pv1, s);
      for (int j = 0; j < k; ++j) {
        uint8_t *d = reinterpret_cast<uint8_t *>(readlane64(dst, j));
        float *sd = reinterpret_cast<float *>(readlane64(sdst, j));
        if (valid) {
          __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(d + ch));
          if ((lane % 8) == 0) sd[blk] = s;
        }
      }
    } else {
      const int c = seg * kWave + lane;
      const bool ok = c < nch;
      for (int j = 0; j < k; ++j) {
        u32x4 *d = reinterpret_cast<u32x4 *>(readlane64(dst, j));
        if (ok) __builtin_nontemporal_store(pv0, d + c);
      }
    }
  }
}

}  // namespace

bool fused_layout_dispatch_ok(const ep_config &c) {
  return (int64_t)c.num_tokens * c.num_topk <= kFusedMaxPairs;
}

hipError_t launch_layout_dispatch_small(const ep_config &c, const int32_t *topk_idx,
                                        const ep_layout_t &h, const void *x, const RankPtrs &rx,
                                        const ScalePtrs &rs, int64_t capacity_rows,
                                        hipStream_t s) {
  const bool fp8 = c.dispatch_dtype == EP_DTYPE_FP8_E4M3;
  const int64_t nseg = fp8 ? (c.hidden / 128 + kFp8SegBlocks - 1) / kFp8SegBlocks
                           : (c.hidden / 8 + kWave - 1) / kWave;
  const int grid = row_grid(c, (int64_t)c.num_tokens * nseg);
  const size_t lds = (size_t)(c.num_experts + 1) * sizeof(int32_t);
  if (fp8) {
    hipLaunchKernelGGL(layout_dispatch_small_kernel<true>, dim3(grid), dim3(kWave), lds, s,
                       topk_idx, static_cast<const uint16_t *>(x), c.num_tokens, c.hidden,
                       c.num_topk, c.num_experts, c.num_ranks, capacity_rows, rx, rs, h);
  } else {
    hipLaunchKernelGGL(layout_dispatch_small_kernel<false>, dim3(grid), dim3(kWave), lds, s,
                       topk_idx, static_cast<const uint16_t *>(x), c.num_tokens, c.hidden,
                       c.num_topk, c.num_experts, c.num_ranks, capacity_rows, rx, rs, h);
  }
  return hipGetLastError();
}

}  // namespace ep
