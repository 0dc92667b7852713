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
// Design (deterministic: no order-dependent atomics, identical bytes on every
// run).  The T*k pairs are cut into chunks, one chunk per wavefront:
//   count   -- each wavefront builds its chunk's expert histogram in LDS;
//   scan    -- expert totals, their exclusive scan (expert_offsets), rank
//              ranges, and for every chunk the counts of all earlier chunks;
//   walk    -- each wavefront walks its chunk 64 pairs at a time in
//              ascending order: lanes naming the same expert are found with
//              ceil(log2 E) ballots, a lane's rank among them is
//              popcount(match & lanes-below), and the group's highest lane
//              advances the expert's running base in LDS.  This reproduces
//              "slot = offset[e] + #earlier pairs of e" exactly.
// Decode-sized problems (P <= kFusedMaxPairs) run in ONE launch of one
// single-wave workgroup per 64 pairs, each counting every pair itself.  Small
// problems (P <= kSmallMaxPairs, E <= kSmallMaxExperts) run all three phases
// in ONE launch of one or two 16-wave workgroups of ~4096 pairs (their waves
// are the chunks), each again counting every pair itself.  Larger ones use
// two launches: a count kernel writes
// a [C/4][E+1][4] table of chunk histograms (a workgroup's 4 chunks are one
// 16-byte group per expert; entry E counts bad indices) to the workspace,
// and a scatter kernel in which every workgroup reads the whole table --
// thread e takes expert e's groups, consecutive threads on consecutive 16
// bytes, all loads in flight -- to get the totals and its own chunks'
// prefixes before walking.  (Measured at T*k = 65536: reading expert-major
// rows, each instruction touching 64 lines, cost 5.8 us of a 15 us scatter
// kernel; making every workgroup of one launch count all pairs itself costs
// more in LDS atomics than the second launch.)  In ep_route_layout the router
// writes that table itself (plan_route_count: one router workgroup per
// chunk), and only the scatter kernel runs here.
#include <mutex>

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

LayoutPlan plan_layout(int64_t P, int E) {
  LayoutPlan p{};
  p.P = P;
  if (P <= kFusedMaxPairs) {
    // single launch: one single-wave workgroup per 64 pairs
    p.tiny = true;
    p.S = kWave;
    p.C = (int32_t)((P + kWave - 1) / kWave);
    p.workgroups = p.C;
    p.workspace_bytes = 256;  // unused; a minimal buffer keeps the contract uniform
    return p;
  }
  if (P <= kSmallMaxPairs && E <= kSmallMaxExperts) {
    // single launch: G workgroups of kSmallWaves waves, ~4096 pairs each
    int64_t G = (P + 4095) / 4096;
    if (G < 1) G = 1;
    if (G > 64) G = 64;
    const int64_t unit = (int64_t)kSmallWaves * kWave;
    const int64_t S = ((P + G - 1) / G + unit - 1) / unit * unit;
    p.small = true;
    p.S = (int32_t)S;
    p.C = (int32_t)((P + S - 1) / S);
    p.workgroups = p.C;
    p.workspace_bytes = 256;  // unused; a minimal buffer keeps the contract uniform
    return p;
  }
  // Bound the table every scatter workgroup reads to ~64K entries.
  int64_t cmax = 65536 / (E + 1);
  if (cmax < 4) cmax = 4;
  if (cmax > kLayoutMaxChunks) cmax = kLayoutMaxChunks;
  int64_t S = kLayoutChunk;
  int64_t C = (P + S - 1) / S;
  if (C > cmax) {
    S = ((P + cmax - 1) / cmax + kWave - 1) / kWave * kWave;
    C = (P + S - 1) / S;
  }
  if (C < 1) C = 1;
  p.S = (int32_t)S;
  p.C = (int32_t)C;
  p.workgroups = (int32_t)((C + kLayoutWaves - 1) / kLayoutWaves);
  // one 16-byte group of kLayoutWaves chunk counts per (workgroup, expert)
  p.workspace_bytes = (size_t)p.workgroups * kLayoutWaves * (size_t)(E + 1) * sizeof(int32_t);
  return p;
}

LayoutPlan plan_route_count(int64_t T, int k, int E) {
  const LayoutPlan lp = plan_layout(T * k, E);
  LayoutPlan p{};
  if (lp.tiny || lp.small || E > kRouteCountMaxExperts) return p;
  // the fewest steps per workgroup that keep C <= kLayoutMaxChunks
  const int64_t per = (T + kRouteCountStep - 1) / kRouteCountStep;
  const int64_t steps = (per + kLayoutMaxChunks - 1) / kLayoutMaxChunks;
  const int64_t tpc = steps * kRouteCountStep;
  p.P = T * k;
  p.tpc = (int32_t)tpc;
  p.S = (int32_t)(tpc * k);
  p.C = (int32_t)((T + tpc - 1) / tpc);
  p.workgroups = (p.C + kLayoutWaves - 1) / kLayoutWaves;
  p.workspace_bytes = (size_t)p.workgroups * kLayoutWaves * (size_t)(E + 1) * sizeof(int32_t);
  return p;
}

namespace {

constexpr int kThreads = kLayoutWaves * kWave;

using dev::i32x4;
using dev::wave_inclusive_scan;

// Chunk histograms: wave c counts the pairs [c*S, c*S+S) in LDS and writes
// them to the table hist[C/4][E+1][4]: workgroup g's kLayoutWaves chunks form
// one 16-byte group per expert (entry E counts indices outside [0,E)).
// The first of two launches, so it also clears the handle's error word: the
// scatter kernel after it only ORs bits in.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(const int32_t *__restrict__ idx,
                                                                 int64_t P, int32_t E, int32_t S,
                                                                 int32_t C,
                                                                 int32_t *__restrict__ hist,
                                                                 int32_t *__restrict__ err) {
  extern __shared__ int32_t lds[];
  const int wave = dev::wave_id(), lane = threadIdx.x % kWave;
  if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
  const int E1 = E + 1;
  int32_t *h = lds + wave * E1;
  for (int e = lane; e < E1; e += kWave) h[e] = 0;
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * kLayoutWaves + wave;
  if (c < C) {
    const int64_t p0 = c * S;
    const int64_t p1 = (p0 + S < P) ? p0 + S : P;
    const bool vec = (((uintptr_t)(idx + p0)) & 15u) == 0;
    // 16 pairs per lane per batch (4 x 16-byte loads in flight)
    for (int64_t q = p0; q < p1; q += 16 * kWave) {
      i32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t p = q + ((int64_t)u * kWave + lane) * 4;
        if (vec && p + 4 <= p1) {
          v[u] = *reinterpret_cast<const i32x4 *>(idx + p);
        } else {
          i32x4 t = {0, 0, 0, 0};
          for (int i = 0; i < 4; ++i) t[i] = (p + i < p1) ? idx[p + i] : 0;
          v[u] = t;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t p = q + ((int64_t)u * kWave + lane) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (p + i < p1) atomicAdd(&h[((uint32_t)v[u][i] < (uint32_t)E) ? v[u][i] : E], 1);
      }
    }
  }
  __syncthreads();
  // every wave of the last workgroup writes, so chunks past C read as 0
  int32_t *grp = hist + (int64_t)blockIdx.x * E1 * kLayoutWaves + wave;
  for (int e = lane; e < E1; e += kWave) grp[(int64_t)e * kLayoutWaves] = h[e];
}

// Exclusive scan of a[0..n) in place, a[n] = total.  All NT threads of the
// workgroup call it; `wsum` holds NT/64 ints of LDS.
template <int NT>
__device__ void block_exclusive_scan(int32_t *a, int n, int32_t *wsum) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int per = (n + NT - 1) / NT;
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
  if (tid == NT - 1) a[n] = pre + incl;
  __syncthreads();
}

// Counts, offsets, rank ranges and error word from the scanned offsets
// off[0..E] (every thread of the workgroup takes part).  RESET: a one-launch
// layout stores the word (0 or EP_DEVERR_INDEX) from its workgroup 0, the one
// workgroup that ever writes it in that launch; the second launch of a
// two-launch layout, whose first launch cleared it, only ORs the bit in.
template <int NT, bool RESET>
__device__ void write_handle(const int32_t *off, int32_t E, int32_t R, int32_t nbad,
                             const ep_layout_t &h) {
  const int tid = threadIdx.x;
  const int32_t El = E / R;
  for (int e = tid; e < E; e += NT) {
    h.expert_counts[e] = off[e + 1] - off[e];
    h.expert_offsets[e] = off[e];
  }
  for (int r = tid; r < R; r += NT) {
    h.rank_offsets[r] = off[r * El];
    h.rank_counts[r] = off[(r + 1) * El] - off[r * El];
  }
  if (tid == 0) {
    h.expert_offsets[E] = off[E];
    h.rank_offsets[R] = off[E];
    if (RESET) {
      h.error_flag[0] = nbad ? (int32_t)EP_DEVERR_INDEX : 0;
      __threadfence();  // ordered before this workgroup's own walk
    } else if (nbad) {
      atomicOr(h.error_flag, (int32_t)EP_DEVERR_INDEX);
    }
  }
}

constexpr int kTableBatch = 32;          // 16-byte table loads a scatter thread keeps in flight
constexpr int kIlp = 4;                  // 64-pair steps whose ballot matches run interleaved
constexpr int kStage = 16 * kWave;       // pairs a scatter-kernel wave stages in LDS at a time
constexpr int kSmallStage = 8 * kWave;   // pairs a small-kernel wave stages (P <= 8192 -> <= 512)

// One wavefront assigns the slots of pairs [p0, p1) in ascending order; bw[e]
// holds the next free slot of expert e for this chunk and is advanced.  The
// wave first copies 64*PL indices into its LDS stage (PL per lane, 16-byte
// loads, one round trip), then ranks them 64 at a time in a rolled loop: the
// layout runs few waves, each executing its code once, so compact loops
// (warm instruction cache) beat unrolled straight-line code here.
// Lane l's PL indices of the stage starting at pair qb (n pairs valid):
// pairs qb + l*PL .. qb + l*PL + PL - 1, 16-byte loads where aligned.
template <int PL>
__device__ inline void load_stage(const int32_t *__restrict__ idx, int64_t qb, int64_t n, int lane,
                                  i32x4 (&v)[PL / 4]) {
  const int64_t pl = qb + (int64_t)lane * PL;
  const bool vec = ((((uintptr_t)(idx + qb)) & 15u) == 0) && pl + PL <= qb + n;
#pragma unroll
  for (int u = 0; u < PL / 4; ++u) {
    if (vec) {
      v[u] = *reinterpret_cast<const i32x4 *>(idx + pl + 4 * u);
    } else {
      i32x4 t = {0, 0, 0, 0};
      for (int i = 0; i < 4; ++i) t[i] = (pl + 4 * u + i < qb + n) ? idx[pl + 4 * u + i] : 0;
      v[u] = t;
    }
  }
}

// `first`, if given, holds this lane's load_stage of the first stage (p0),
// issued earlier by the caller so that its latency overlaps other work.  A
// slot outside [0,P) cannot happen; should it, the pair's slot_of is -1, so
// every later call on the handle reports EP_DEVERR_ROW for its token, and
// EP_DEVERR_INTERNAL is ORed into the error word where that cannot race with
// the word's reset (`flag`: the second launch of a two-launch layout, or
// workgroup 0 of a one-launch layout after its own store).
template <int PL>
__device__ void wave_walk(const int32_t *__restrict__ idx, int64_t p0, int64_t p1, int64_t P,
                          int32_t E, int32_t *bw, int32_t *stage, const ep_layout_t &h, bool flag,
                          const i32x4 *first = nullptr) {
  static_assert(PL % 4 == 0, "whole 16-byte groups per lane");
  constexpr int kSt = PL * kWave;
  const int lane = threadIdx.x % kWave;
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t qb = p0; qb < p1; qb += kSt) {
    const int64_t n = (p1 - qb < kSt) ? p1 - qb : kSt;
    i32x4 v[PL / 4];
    if (first && qb == p0) {
#pragma unroll
      for (int u = 0; u < PL / 4; ++u) v[u] = first[u];
    } else {
      load_stage<PL>(idx, qb, n, lane, v);
    }
#pragma unroll
    for (int u = 0; u < PL / 4; ++u) *reinterpret_cast<i32x4 *>(stage + lane * PL + 4 * u) = v[u];
    // kIlp steps of 64 pairs at a time: their match masks are independent
    // (only the running bases carry from step to step), so their ballot
    // chains are interleaved to hide each other's latency; the base updates
    // then run in step order.
#pragma unroll 1
    for (int i0 = 0; i0 * kWave < n; i0 += kIlp) {
      int32_t e[kIlp];
      bool valid[kIlp];
      uint64_t m[kIlp];
#pragma unroll
      for (int s = 0; s < kIlp; ++s) {
        const int i = (i0 + s) * kWave + lane;
        valid[s] = i < n;
        e[s] = valid[s] ? stage[i] : 0;
        m[s] = __ballot(valid[s]);
      }
      // lanes whose expert matches this lane's in every bit: m &= (bit ? B : ~B)
      for (int b = 0; b < nbits; ++b) {
#pragma unroll
        for (int s = 0; s < kIlp; ++s) {
          const uint32_t bit = ((uint32_t)e[s] >> b) & 1u;
          const uint64_t bb = __ballot(bit != 0u);
          const uint32_t flip = bit - 1u;  // 0 if the bit is set, all ones if not
          m[s] &= bb ^ (((uint64_t)flip << 32) | flip);
        }
      }
#pragma unroll
      for (int s = 0; s < kIlp; ++s) {
        if (valid[s]) {
          const int64_t p = qb + (int64_t)(i0 + s) * kWave + lane;
          const int32_t slot = bw[e[s]] + __popcll(m[s] & below);
          if ((uint64_t)(uint32_t)slot < (uint64_t)P) {
            h.slot_of[p] = slot;
            h.src_of[slot] = (int32_t)p;
          } else {  // cannot happen; never write out of range
            h.slot_of[p] = -1;
            if (flag) atomicOr(h.error_flag, (int32_t)EP_DEVERR_INTERNAL);
          }
          if ((m[s] >> lane) == 1ull) bw[e[s]] += __popcll(m[s]);  // the group's highest lane
        }
      }
    }
  }
}

// Single-launch layout for P <= kFusedMaxPairs (decode batches): workgroup g
// (one wave) owns pairs [64g, 64g + 64).  Every workgroup holds all P indices
// in registers (coalesced loads, at most kTinyPL per lane) and counts in LDS
// the expert totals and the pairs before its own 64, scans the totals, and
// ranks its own pairs with the ballot match; no workgroup waits for another.
// (The one-workgroup small path took 8 us at 1024 pairs, a chain of
// barriers and per-wave prefix loops.)
constexpr int kTinyPL = (int)(kFusedMaxPairs / kWave);
static_assert(kFusedMaxPairs < (1 << 16), "the decode layout packs two 16-bit counts per expert");

__global__ __launch_bounds__(kWave) void layout_tiny_kernel(const int32_t *__restrict__ idx,
                                                            int64_t P, int32_t E, int32_t R,
                                                            ep_layout_t h) {
  extern __shared__ int32_t lds[];
  // [E] an expert's two counts in one word, so a pair costs one LDS atomic:
  // low 16 bits all its pairs, high 16 bits those before this workgroup's 64
  // (each < 2^16: P <= kFusedMaxPairs)
  uint32_t *cnt = reinterpret_cast<uint32_t *>(lds);
  int32_t *tot = lds + E;  // [E+1] exclusive offsets
  const int lane = threadIdx.x;
  const int nv = (int)((P + kWave - 1) / kWave);
  const int64_t p = (int64_t)blockIdx.x * kWave + lane;  // this lane's own pair
  const bool own = p < P;
  const int32_t pe = own ? idx[p] : 0;
  int32_t ev[kTinyPL];
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < kTinyPL; ++i) {
    const int64_t q = (int64_t)i * kWave + lane;
    ev[i] = (i < nv && q < P) ? idx[q] : 0;
    if (i < nv && q < P && (uint32_t)ev[i] >= (uint32_t)E) ++bad;
  }
  for (int e = lane; e < E; e += kWave) cnt[e] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTinyPL; ++i) {
    const int64_t q = (int64_t)i * kWave + lane;
    if (i < nv && q < P && (uint32_t)ev[i] < (uint32_t)E)  // pair q = 64i + lane precedes 64g if i < g
      atomicAdd(&cnt[ev[i]], (i < (int)blockIdx.x) ? 0x10001u : 1u);
  }
  bad = dev::wave_sum_u32(bad);
  __syncthreads();
  {  // exclusive scan of tot[0..E), tot[E] = total
    const int per = (E + kWave - 1) / kWave;
    const int b = (lane * per < E) ? lane * per : E;
    const int end = (b + per < E) ? b + per : E;
    int32_t s = 0;
    for (int i = b; i < end; ++i) s += (int32_t)(cnt[i] & 0xFFFFu);
    const int32_t incl = wave_inclusive_scan(s, lane);
    int32_t run = incl - s;
    for (int i = b; i < end; ++i) {
      const int32_t v = (int32_t)(cnt[i] & 0xFFFFu);
      tot[i] = run;
      run += v;
    }
    if (lane == kWave - 1) tot[E] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    const int32_t El = E / R;
    for (int e = lane; e < E; e += kWave) {
      h.expert_counts[e] = tot[e + 1] - tot[e];
      h.expert_offsets[e] = tot[e];
    }
    for (int r = lane; r < R; r += kWave) {
      h.rank_offsets[r] = tot[r * El];
      h.rank_counts[r] = tot[(r + 1) * El] - tot[r * El];
    }
    if (lane == 0) {  // the only writer of the error word in this launch but for
                      // workgroup 0's own internal check below
      h.expert_offsets[E] = tot[E];
      h.rank_offsets[R] = tot[E];
      h.error_flag[0] = bad ? (int32_t)EP_DEVERR_INDEX : 0;
      __threadfence();
    }
  }
  if (bad) return;  // uniform: the handle's slots are unspecified on error
  // lanes whose expert matches this lane's in every bit: m &= (bit ? B : ~B)
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  uint64_t m = __ballot(own);
  for (int b = 0; b < nbits; ++b) {
    const uint32_t bit = ((uint32_t)pe >> b) & 1u;
    const uint64_t bb = __ballot(bit != 0u);
    const uint32_t flip = bit - 1u;
    m &= bb ^ (((uint64_t)flip << 32) | flip);
  }
  if (own) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int32_t slot = tot[pe] + (int32_t)(cnt[pe] >> 16) + __popcll(m & below);
    if ((uint64_t)(uint32_t)slot < (uint64_t)P) {
      h.slot_of[p] = slot;
      h.src_of[slot] = (int32_t)p;
    } else {  // cannot happen; never write out of range (see wave_walk)
      h.slot_of[p] = -1;
      if (blockIdx.x == 0) atomicOr(h.error_flag, (int32_t)EP_DEVERR_INTERNAL);
    }
  }
}

constexpr int kSmallThreads = kSmallWaves * kWave;
constexpr int kSmallRounds = 2;  // int4 loads per thread per batch (2 x 4096 pairs: P <= 8192 is one batch)

// Single-launch layout: workgroup g owns pairs [g*S, g*S+S) (S a multiple of
// kSmallWaves*64) and, inside it, wave w owns S/kSmallWaves pairs.  Every
// workgroup streams ALL P indices (int4 loads, a batch of 16 per thread in
// flight) and counts in LDS the expert totals, the pairs before its own
// chunk, and its own waves' pairs, so no workgroup needs another's results.
__global__ __launch_bounds__(kSmallThreads) void layout_small_kernel(
    const int32_t *__restrict__ idx, int64_t P, int32_t E, int32_t R, int32_t S, ep_layout_t h) {
  extern __shared__ int32_t lds[];
  int32_t *tot = lds;                      // [E+1] totals, then exclusive offsets
  int32_t *pre = tot + E + 1;              // [E]   pairs of e before this chunk
  int32_t *cnt = pre + E;                  // [kSmallWaves][E]: own counts, then bases
  int32_t *misc = cnt + kSmallWaves * E;   // [kSmallWaves] scan scratch, [kSmallWaves] bad
  int32_t *stage = lds + (((kSmallWaves + 2) * E + 1 + 2 * kSmallWaves + 3) / 4 * 4);  // [kSmallWaves][kSmallStage]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < (kSmallWaves + 2) * E + 1; i += kSmallThreads) lds[i] = 0;
  __syncthreads();

  const int64_t c0 = (int64_t)blockIdx.x * S;
  const int64_t c1 = (c0 + S < P) ? c0 + S : P;
  const int32_t Sw = S / kSmallWaves;
  int32_t bad = 0;
  // pairs covered by whole 16-byte loads (none if the caller's array is not 16-byte aligned)
  const int64_t P4 = ((uintptr_t)idx & 15u) ? 0 : (P & ~(int64_t)3);
  for (int64_t base = 0; base < P; base += (int64_t)kSmallRounds * kSmallThreads * 4) {
    i32x4 v[kSmallRounds];
#pragma unroll
    for (int u = 0; u < kSmallRounds; ++u) {
      const int64_t p = base + ((int64_t)u * kSmallThreads + tid) * 4;
      if (p + 4 <= P4) {
        v[u] = *reinterpret_cast<const i32x4 *>(idx + p);
      } else {
        i32x4 t = {-1, -1, -1, -1};
        for (int i = 0; i < 4; ++i)
          if (p + i < P) t[i] = idx[p + i];
        v[u] = t;
      }
    }
#pragma unroll
    for (int u = 0; u < kSmallRounds; ++u) {
      const int64_t p = base + ((int64_t)u * kSmallThreads + tid) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t q = p + i;
        if (q < P) {
          const int32_t e = v[u][i];
          if ((uint32_t)e >= (uint32_t)E) {
            ++bad;
          } else {
            atomicAdd(&tot[e], 1);
            if (q < c0) atomicAdd(&pre[e], 1);
            else if (q < c1) atomicAdd(&cnt[(int)((q - c0) / Sw) * E + e], 1);
          }
        }
      }
    }
  }
  bad = wave_inclusive_scan(bad, lane);
  if (lane == kWave - 1) misc[kSmallWaves + wave] = bad;
  __syncthreads();

  // cnt[w][e] becomes pre[e] + the counts of this chunk's earlier waves
  for (int e = tid; e < E; e += kSmallThreads) {
    int32_t run = pre[e];
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      const int32_t c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  int32_t nbad = 0;
  for (int w = 0; w < kSmallWaves; ++w) nbad += misc[kSmallWaves + w];
  block_exclusive_scan<kSmallThreads>(tot, E, misc);  // synchronizes
  if (blockIdx.x == 0) write_handle<kSmallThreads, true>(tot, E, R, nbad, h);
  if (nbad) return;  // uniform: the handle's slots are unspecified on error
  for (int i = tid; i < kSmallWaves * E; i += kSmallThreads) cnt[i] += tot[i % E];
  __syncthreads();
  const int64_t p0 = c0 + (int64_t)wave * Sw;
  const int64_t p1 = (p0 + Sw < c1) ? p0 + Sw : c1;
  wave_walk<kSmallStage / kWave>(idx, p0, p1, P, E, cnt + wave * E, stage + wave * kSmallStage, h,
                                 blockIdx.x == 0);
}

__global__ __launch_bounds__(kThreads) void layout_scatter_kernel(
    const int32_t *__restrict__ idx, int64_t P, int32_t E, int32_t R, int32_t S, int32_t C,
    const int32_t *__restrict__ hist, ep_layout_t h) {
  extern __shared__ int32_t lds[];
  int32_t *off = lds;                        // [E+1]
  int32_t *base = lds + (E + 1);             // [kLayoutWaves][E]
  int32_t *misc = base + kLayoutWaves * E;   // [kLayoutWaves] scan scratch, [kLayoutWaves] bad counts
  int32_t *stage = lds + ((E + 1) + kLayoutWaves * E + 8 + 3) / 4 * 4;  // [kLayoutWaves][kStage], 16-byte aligned
  const int tid = threadIdx.x, wave = tid / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * kLayoutWaves;
  // this wave's chunk, and its first stage of indices loaded now: the
  // loads overlap the table reads below
  const int64_t wc = c0 + wave;
  const int64_t wp0 = wc * S;
  const int64_t wp1 = (wp0 + S < P) ? wp0 + S : P;
  i32x4 first[kStage / kWave / 4];
  if (wc < C) {
    const int64_t n0 = (wp1 - wp0 < kStage) ? wp1 - wp0 : kStage;
    load_stage<kStage / kWave>(idx, wp0, n0, tid % kWave, first);
  }

  // Group q of the table holds the counts of chunks [4q, 4q+4) for every
  // expert (and, at E, of bad indices).  Thread e reads the 16-byte groups of
  // expert e: consecutive threads read consecutive groups, a batch of
  // kTableBatch loads is in flight (one round trip for up to 4*kTableBatch
  // chunks), the groups before this workgroup's give its prefix and its own
  // group its chunks' counts.
  const int64_t E1 = (int64_t)E + 1;
  const int Q = (int)gridDim.x;  // groups = workgroups
  const i32x4 *tab = reinterpret_cast<const i32x4 *>(hist);
  int32_t badpart = 0;
  if (tid < Q) {
    const i32x4 b = tab[(int64_t)tid * E1 + E];
    badpart = b[0] + b[1] + b[2] + b[3];
  }
  for (int e = tid; e < E; e += kThreads) {
    int32_t run = 0, before = 0;
    const i32x4 mine = tab[(int64_t)blockIdx.x * E1 + e];
#pragma unroll 1
    for (int qb = 0; qb < Q; qb += kTableBatch) {
      i32x4 v[kTableBatch];
#pragma unroll
      for (int u = 0; u < kTableBatch; ++u) {
        const i32x4 z = {0, 0, 0, 0};
        v[u] = (qb + u < Q) ? tab[(int64_t)(qb + u) * E1 + e] : z;
      }
#pragma unroll
      for (int u = 0; u < kTableBatch; ++u) {
        const int32_t s4 = v[u][0] + v[u][1] + v[u][2] + v[u][3];
        run += s4;
        before += (qb + u < (int)blockIdx.x) ? s4 : 0;
      }
    }
    int32_t pre[kLayoutWaves];
    pre[0] = before;
#pragma unroll
    for (int w = 1; w < kLayoutWaves; ++w) pre[w] = pre[w - 1] + mine[w - 1];
    off[e] = run;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) base[w * E + e] = pre[w];
  }
  badpart = wave_inclusive_scan(badpart, tid % kWave);
  if (tid % kWave == kWave - 1) misc[kLayoutWaves + tid / kWave] = badpart;
  __syncthreads();
  int32_t nbad = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) nbad += misc[kLayoutWaves + w];
  block_exclusive_scan<kThreads>(off, E, misc);
  if (blockIdx.x == 0) write_handle<kThreads, false>(off, E, R, nbad, h);
  if (nbad) return;  // uniform: the handle's slots are unspecified on error

  for (int i = tid; i < kLayoutWaves * E; i += kThreads) base[i] += off[i % E];
  __syncthreads();

  if (wc >= C) return;
  wave_walk<kStage / kWave>(idx, wp0, wp1, P, E, base + wave * E, stage + wave * kStage, h, true,
                            first);
}

}  // namespace

hipError_t launch_layout(const ep_config &c, const LayoutPlan &plan, const int32_t *topk_idx,
                         const ep_layout_t &h, void *workspace, hipStream_t s) {
  const int E = c.num_experts;
  if (plan.tiny) {
    hipLaunchKernelGGL(layout_tiny_kernel, dim3(plan.workgroups), dim3(kWave),
                       (size_t)(2 * E + 1) * sizeof(int32_t), s, topk_idx, plan.P, E, c.num_ranks,
                       h);
    return hipGetLastError();
  }
  if (plan.small) {
    const size_t lds_bytes = (((size_t)(kSmallWaves + 2) * E + 1 + 2 * kSmallWaves + 3) / 4 * 4 +
                              (size_t)kSmallWaves * kSmallStage) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_small_kernel, dim3(plan.workgroups), dim3(kSmallThreads), lds_bytes, s,
                       topk_idx, plan.P, E, c.num_ranks, plan.S, h);
    return hipGetLastError();
  }
  int32_t *hist = static_cast<int32_t *>(workspace);
  const size_t lds_count = (size_t)kLayoutWaves * (E + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(layout_count_kernel, dim3(plan.workgroups), dim3(kThreads), lds_count, s,
                     topk_idx, plan.P, E, plan.S, plan.C, hist, h.error_flag);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_layout_scatter(c, plan, topk_idx, h, workspace, s);
}

// ---- the layout without a caller workspace ------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the chunk table lives in a file-scope device array instead of a
// workspace argument.  Every GPU the library runs on holds its own copy until
// the process ends; its address on the current device is resolved once per
// device with hipGetSymbolAddress, and only that address is handed to the
// kernels (the array's name is a host-side stand-in).  kLayoutScratchBytes
// covers plan_layout's table for every valid config (its largest is 285 840
// bytes, at E = 1984).  The count kernel writes every entry the scatter
// kernel reads, so the array needs no clearing; calls that overlap on one
// GPU share it and race.
static __device__ __align__(256) int32_t scratch[kLayoutScratchBytes / sizeof(int32_t)];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t layout_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_layout_scatter(const ep_config &c, const LayoutPlan &plan,
                                 const int32_t *topk_idx, const ep_layout_t &h, void *workspace,
                                 hipStream_t s) {
  const int E = c.num_experts;
  const size_t lds_scatter =
      (((size_t)(E + 1) + (size_t)kLayoutWaves * E + 8 + 3) / 4 * 4 + (size_t)kLayoutWaves * kStage) *
      sizeof(int32_t);
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(plan.workgroups), dim3(kThreads), lds_scatter, s,
                     topk_idx, plan.P, E, c.num_ranks, plan.S, plan.C,
                     (const int32_t *)workspace, h);
  return hipGetLastError();
}

}  // namespace ep
