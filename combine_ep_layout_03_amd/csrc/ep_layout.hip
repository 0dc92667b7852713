// ep_layout.hip -- routing layout on gfx950: per-expert counts, prefix sums,
// per-rank ranges and the stable expert-contiguous slot assignment.
//
// Pages: [Perplexity blog] "Lower latency and higher throughput with
// multi-node DeepSeek deployment", "MoE-beirari" (dense dispatch/combine need
// the routing summed per expert, not per token); [DeepEP overview] "DeepSeek
// merilis library open source DeepEP ...", "Perubahan utama pada rilis V2"
// (a GEMM layout: experts contiguous) and "Pola penggunaan ..." (the handle
// carries per-expert token counts for the GEMM).
//
// Design (two launches, no global atomics, bit-identical on every run):
//   count   -- the T*k pairs are cut into C chunks of S pairs; one wavefront
//              builds its chunk's expert histogram in LDS and stores it as
//              row c of a [C][E+1] table (column E counts bad indices).
//   scatter -- every workgroup reads the whole table (C*(E+1) ints, L2
//              resident), so each has the expert totals, their exclusive
//              scan and, for its own chunks, the counts of all earlier chunks;
//              workgroup 0 writes the handle's counts / offsets / error word.
//              Each wavefront then walks its chunk 64 pairs at a time in
//              ascending order: lanes naming the same expert are found with
//              ceil(log2 E) ballots, a lane's rank among them is
//              popcount(match & lanes-below), and the group's highest lane
//              advances the expert's running base in LDS.  This reproduces
//              "slot = offset[e] + #earlier pairs of e" without any
//              order-dependent atomic.
#include "ep_internal.h"

namespace ep {

LayoutPlan plan_layout(int64_t P, int E) {
  LayoutPlan p{};
  p.P = P;
  // Bound the table every scatter workgroup reads to ~64K entries.
  int64_t cmax = 65536 / (E + 1);
  if (cmax < 4) cmax = 4;
  if (cmax > 256) cmax = 256;
  int64_t S = 1024;
  int64_t C = (P + S - 1) / S;
  if (C > cmax) {
    S = ((P + cmax - 1) / cmax + kWave - 1) / kWave * kWave;
    C = (P + S - 1) / S;
  }
  if (C < 1) C = 1;
  p.S = (int32_t)S;
  p.C = (int32_t)C;
  p.workgroups = (int32_t)((C + kLayoutWaves - 1) / kLayoutWaves);
  p.workspace_bytes = (size_t)C * (size_t)(E + 1) * sizeof(int32_t);
  return p;
}

namespace {

constexpr int kThreads = kLayoutWaves * kWave;

__global__ __launch_bounds__(kThreads) void layout_count_kernel(const int32_t *__restrict__ idx,
                                                                 int64_t P, int32_t E, int32_t S,
                                                                 int32_t C,
                                                                 int32_t *__restrict__ hist) {
  extern __shared__ int32_t lds[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int E1 = E + 1;
  int32_t *h = lds + wave * E1;
  for (int e = lane; e < E1; e += kWave) h[e] = 0;
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kLayoutWaves + wave;
  if (c < C) {
    const int64_t p0 = c * S;
    const int64_t p1 = (p0 + S < P) ? p0 + S : P;
    for (int64_t p = p0 + lane; p < p1; p += kWave) {
      const int32_t e = idx[p];
      atomicAdd(&h[((uint32_t)e < (uint32_t)E) ? e : E], 1);
    }
  }
  __syncthreads();
  if (c < C)
    for (int e = lane; e < E1; e += kWave) hist[c * E1 + e] = h[e];
}

__device__ inline int32_t wave_inclusive_scan(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t n = __shfl_up(v, d, kWave);
    if (lane >= d) v += n;
  }
  return v;
}

// Exclusive scan of a[0..n) in place, a[n] = total.  All kThreads threads
// call it; `wsum` holds kLayoutWaves ints of LDS.
__device__ void block_exclusive_scan(int32_t *a, int n, int32_t *wsum) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int per = (n + kThreads - 1) / kThreads;
  const int b = (tid * per < n) ? tid * per : n;
  const int end = (b + per < n) ? b + per : n;
  int32_t s = 0;
  for (int i = b; i < end; ++i) s += a[i];
  const int32_t incl = wave_inclusive_scan(s, lane);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  int32_t run = pre + incl - s;
  for (int i = b; i < end; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
  if (tid == kThreads - 1) a[n] = pre + incl;
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void layout_scatter_kernel(
    const int32_t *__restrict__ idx, int64_t P, int32_t E, int32_t R, int32_t S, int32_t C,
    const int32_t *__restrict__ hist, ep_layout_t h) {
  extern __shared__ int32_t lds[];
  int32_t *off = lds;                        // [E+1]
  int32_t *base = lds + (E + 1);             // [kLayoutWaves][E]
  int32_t *misc = base + kLayoutWaves * E;   // [kLayoutWaves] scan scratch, [4] bad count
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int E1 = E + 1;
  const int32_t El = E / R;
  const int64_t c0 = (int64_t)blockIdx.x * kLayoutWaves;

  // Totals over all chunks and, for this workgroup's chunks, the sums over
  // the chunks before each of them.
  for (int e = tid; e < E1; e += kThreads) {
    int32_t run = 0;
    const int64_t cpre = (c0 < C) ? c0 : C;
#pragma unroll 8
    for (int64_t c = 0; c < cpre; ++c) run += hist[c * E1 + e];
    int32_t pre[kLayoutWaves];
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      pre[w] = run;
      if (c0 + w < C) run += hist[(c0 + w) * E1 + e];
    }
#pragma unroll 8
    for (int64_t c = c0 + kLayoutWaves; c < C; ++c) run += hist[c * E1 + e];
    if (e < E) {
      off[e] = run;
#pragma unroll
      for (int w = 0; w < kLayoutWaves; ++w) base[w * E + e] = pre[w];
    } else {
      misc[kLayoutWaves] = run;
    }
  }
  __syncthreads();
  const int32_t nbad = misc[kLayoutWaves];
  block_exclusive_scan(off, E, misc);

  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kThreads) {
      h.expert_counts[e] = off[e + 1] - off[e];
      h.expert_offsets[e] = off[e];
    }
    for (int r = tid; r < R; r += kThreads) {
      h.rank_offsets[r] = off[r * El];
      h.rank_counts[r] = off[(r + 1) * El] - off[r * El];
    }
    if (tid == 0) {
      h.expert_offsets[E] = off[E];
      h.rank_offsets[R] = off[E];
      h.error_flag[0] = nbad ? (int32_t)EP_DEVERR_INDEX : 0;
    }
  }
  if (nbad) return;  // uniform: the handle's slots are unspecified on error

  for (int i = tid; i < kLayoutWaves * E; i += kThreads) base[i] += off[i % E];
  __syncthreads();

  const int64_t c = c0 + wave;
  if (c >= C) return;
  int32_t *bw = base + wave * E;
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int64_t p0 = c * S;
  const int64_t p1 = (p0 + S < P) ? p0 + S : P;
  for (int64_t q = p0; q < p1; q += kWave) {
    const int64_t p = q + lane;
    const bool valid = p < p1;
    const int32_t e = valid ? idx[p] : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    if (valid) {
      const int32_t slot = bw[e] + __popcll(m & below);
      h.slot_of[p] = slot;
      if ((uint64_t)(uint32_t)slot < (uint64_t)P) h.src_of[slot] = (int32_t)p;
      else atomicOr(h.error_flag, (int32_t)EP_DEVERR_INTERNAL);  // cannot happen; never write out of range
      if ((m >> lane) == 1ull) bw[e] += __popcll(m);  // the group's highest lane
    }
  }
}

}  // namespace

hipError_t launch_layout(const ep_config &c, const LayoutPlan &plan, const int32_t *topk_idx,
                         const ep_layout_t &h, void *workspace, hipStream_t s) {
  const int E = c.num_experts;
  int32_t *hist = static_cast<int32_t *>(workspace);
  const size_t lds_count = (size_t)kLayoutWaves * (E + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(layout_count_kernel, dim3(plan.workgroups), dim3(kThreads), lds_count, s,
                     topk_idx, plan.P, E, plan.S, plan.C, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds_scatter = ((size_t)(E + 1) + (size_t)kLayoutWaves * E + 8) * sizeof(int32_t);
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(plan.workgroups), dim3(kThreads), lds_scatter, s,
                     topk_idx, plan.P, E, c.num_ranks, plan.S, plan.C, (const int32_t *)hist, h);
  return hipGetLastError();
}

}  // namespace ep
