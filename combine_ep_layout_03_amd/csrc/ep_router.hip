// ep_router.hip -- the MoE router on gfx950: gate scores, group-limited
// top-k, weights and the redundant-expert mapping; one wave per token, or
// four tokens per wave for large batches.
//
// Pages: [Perplexity blog] "Lower latency and higher throughput with multi-
// node DeepSeek deployment", "MoE-beirari" (one router for every MoE model:
// DeepSeek's group-limited top-k, Mixtral's being the case of one group with
// every expert; indices and scores per token); [EPLB page] "DeepSeek V3/R1 ...
// DualPipe, EPLB, Profile-Data" (group-limited expert routing, redundant
// experts); [torchtitan PR] "Integrate DeepEP to experimental torchtitan"
// (node-limited routing).
//
// Design.  A single-wave workgroup takes one token at a time (grid-stride).
// Lane l holds the NPER consecutive experts [l*NPER, (l+1)*NPER) in
// registers (NPER a power of two, 64*NPER >= El).  The gate is evaluated in
// binary64 and rounded once to binary32, so the scores -- and with them every
// selection, which compares binary32 values only -- barely depend on how a
// device or host libm rounds its exp; the softmax denominator is the binary64
// sum of the numerators in ascending expert order (a serial fold over the
// lanes), the order a plain loop over the experts takes.  Scores are non-negative, so their bit
// patterns order like the values; a wave maximum of 32-bit patterns is four
// DPP steps inside each row of 16 lanes, four readlanes and a scalar max, and
// a ballot of the lanes holding that maximum names the winner: the lowest such
// lane holds the lowest expert id, which is the tie rule.  Groups whose
// experts cover whole, power-of-two runs of lanes are scored by a top-2 merge
// across those lanes; other shapes stage the scores in LDS and let lane c
// score group c.  Renormalization sums the k picks in order with readlane, so
// the weights are the same binary32 operations as a sequential loop.  fp
// contraction is off: the scores are exact compositions of correctly rounded
// operations.  Large batches take a second kernel that routes four tokens
// per wave (same results); in ep_route_layout it also counts the layout's
// per-chunk expert histograms, one workgroup per chunk, so the layout's
// count launch is not needed.
#include <math.h>

#include "ep_device.h"
#include "ep_internal.h"

#pragma clang fp contract(off)

namespace ep {
namespace {

using namespace dev;

__device__ inline uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ inline uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Maximum over the wave (unsigned), uniform result.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<kDppXor1>(v));
  v = umax(v, dpp<kDppXor2>(v));
  v = umax(v, dpp<kDppHalfMirror>(v));
  v = umax(v, dpp<kDppMirror>(v));
  return umax(umax(rdl(v, 0), rdl(v, 16)), umax(rdl(v, 32), rdl(v, 48)));
}

__device__ inline float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppMirror>(__float_as_uint(v))));
  const float a = fmaxf(__uint_as_float(rdl(__float_as_uint(v), 0)),
                        __uint_as_float(rdl(__float_as_uint(v), 16)));
  const float b = fmaxf(__uint_as_float(rdl(__float_as_uint(v), 32)),
                        __uint_as_float(rdl(__float_as_uint(v), 48)));
  return fmaxf(a, b);
}

__device__ inline double rdl_f64(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return __longlong_as_double(
      (long long)(((uint64_t)rdl((uint32_t)(u >> 32), lane) << 32) | rdl((uint32_t)u, lane)));
}

// Value of `src`'s v in every lane (src may differ between lanes).
__device__ inline double shfl_f64(double v, int src) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)u, src, kWave);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(u >> 32), src, kWave);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Value of lane (lane ^ off) for off a power of two below 64.
__device__ inline uint32_t xor_lane(uint32_t v, int off) {
  switch (off) {
    case 1: return dpp<kDppXor1>(v);
    case 2: return dpp<kDppXor2>(v);
    default: return (uint32_t)__shfl_xor((int)v, off, kWave);
  }
}

// Winner among the lanes that offer `bits` (has == true): the largest bits,
// then the lowest lane.  Returns -1 when no lane offers.
__device__ inline int wave_pick(bool has, uint32_t bits, uint32_t &best_bits) {
  const uint32_t mx = wave_max_u32(has ? bits : 0u);
  const uint64_t b = __ballot(has && bits == mx);
  best_bits = mx;
  return b ? (int)__builtin_ctzll(b) : -1;
}

template <int NPER>
__global__ __launch_bounds__(kWave) void route_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias,
    const int32_t *__restrict__ rep_off, const int32_t *__restrict__ rep_slots, int32_t T,
    int32_t El, int32_t k, int32_t gate, int32_t G, int32_t TG, int32_t topn, int32_t renorm,
    int32_t *__restrict__ idx, float *__restrict__ wout) {
  extern __shared__ float lds_s[];  // [El], only for groups that split a lane's experts
  const int lane = threadIdx.x;
  const int e0 = lane * NPER;
  const int gs = El / G;
  const int lpg = gs / NPER;  // lanes per group on the register path
  const bool lane_groups = G > 1 && gs % NPER == 0 && (lpg & (lpg - 1)) == 0;
  const bool vec = NPER >= 4 && (El & 3) == 0 && (((uintptr_t)logits) & 15u) == 0 &&
                   (!bias || (((uintptr_t)bias) & 15u) == 0);
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) valid |= (e0 + i < El) ? 1u << i : 0u;

  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float *zr = logits + t * (int64_t)El;
    float z[NPER];
    if (vec) {
#pragma unroll
      for (int i = 0; i < NPER; i += 4) {
        float4 v = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (e0 + i < El) {
          v = *reinterpret_cast<const float4 *>(zr + e0 + i);
          if (bias) b = *reinterpret_cast<const float4 *>(bias + e0 + i);
        }
        z[i] = bias ? v.x + b.x : v.x;
        z[i + 1] = bias ? v.y + b.y : v.y;
        z[i + 2] = bias ? v.z + b.z : v.z;
        z[i + 3] = bias ? v.w + b.w : v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int e = e0 + i;
        z[i] = e < El ? (bias ? zr[e] + bias[e] : zr[e]) : 0.0f;
      }
    }

    // gate scores: binary64, rounded once
    float s[NPER];
    if (gate == EP_GATE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if ((valid >> i) & 1u) m = fmaxf(m, z[i]);
      m = wave_max_f32(m);
      double ex[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) ex[i] = ((valid >> i) & 1u) ? exp((double)z[i] - (double)m) : 0.0;
      // the denominator in ascending expert order, one binary64 addition at a
      // time (lane l holds experts l*NPER ..); the padding past El adds +0
      double sum = 0.0;
      const int nl = (El + NPER - 1) / NPER;
      for (int l = 0; l < nl; ++l) {
#pragma unroll
        for (int i = 0; i < NPER; ++i) sum += rdl_f64(ex[i], l);
      }
#pragma unroll
      for (int i = 0; i < NPER; ++i) s[i] = (float)(ex[i] / sum);
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) s[i] = (float)(1.0 / (1.0 + exp(-(double)z[i])));
    }

    // eligible experts (bit i of elig): every valid one, or those of the TG
    // best groups
    uint32_t elig = valid;
    if (lane_groups) {
      // this lane's two best, then a top-2 merge across the group's lanes
      uint32_t a1 = 0, a2 = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const uint32_t b = __float_as_uint(s[i]);
        if ((valid >> i) & 1u) {
          a2 = umax(a2, umin(a1, b));
          a1 = umax(a1, b);
        }
      }
      for (int off = 1; off < lpg; off <<= 1) {
        const uint32_t b1 = xor_lane(a1, off), b2 = xor_lane(a2, off);
        a2 = umax(umin(a1, b1), umax(a2, b2));
        a1 = umax(a1, b1);
      }
      const int grp = lane / lpg;
      const float g = (topn == 1 || gs == 1) ? __uint_as_float(a1)
                                             : __uint_as_float(a1) + __uint_as_float(a2);
      bool offer = (lane % lpg) == 0 && grp < G;
      uint64_t kept = 0;
      for (int r = 0; r < TG; ++r) {
        uint32_t bb;
        const int wl = wave_pick(offer, __float_as_uint(g), bb);
        if (wl < 0) break;
        kept |= 1ull << (wl / lpg);
        if (lane == wl) offer = false;
      }
      elig = ((kept >> grp) & 1ull) ? valid : 0u;
    } else if (G > 1) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if ((valid >> i) & 1u) lds_s[e0 + i] = s[i];
      __syncthreads();
      float g = 0.0f;
      if (lane < G) {
        uint32_t a1 = 0, a2 = 0;
        for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
          const uint32_t b = __float_as_uint(lds_s[e]);
          a2 = umax(a2, umin(a1, b));
          a1 = umax(a1, b);
        }
        g = (topn == 1 || gs == 1) ? __uint_as_float(a1) : __uint_as_float(a1) + __uint_as_float(a2);
      }
      bool offer = lane < G;
      uint64_t kept = 0;
      for (int r = 0; r < TG; ++r) {
        uint32_t bb;
        const int wl = wave_pick(offer, __float_as_uint(g), bb);
        if (wl < 0) break;
        kept |= 1ull << wl;
        if (lane == wl) offer = false;
      }
      elig = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if ((valid >> i) & 1u) elig |= (uint32_t)((kept >> ((e0 + i) / gs)) & 1ull) << i;
      __syncthreads();  // the next token rewrites lds_s
    }

    // top-k: each lane offers its best eligible expert; lane j keeps pick j
    int ci = -1;
    uint32_t cb = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint32_t b = __float_as_uint(s[i]);
      if (((elig >> i) & 1u) && (ci < 0 || b > cb)) {
        ci = i;
        cb = b;
      }
    }
    int32_t sel = -1;
    float ws = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint32_t bb;
      const int wl = wave_pick(ci >= 0, cb, bb);
      if (wl < 0) break;  // fewer eligible experts than k: excluded on the host
      const int e = wl * NPER + (int)rdl((uint32_t)ci, wl);
      if (lane == j) {
        sel = e;
        ws = __uint_as_float(bb);
      }
      if (lane == wl) {
        elig &= ~(1u << ci);
        ci = -1;
        cb = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
          const uint32_t b = __float_as_uint(s[i]);
          if (((elig >> i) & 1u) && (ci < 0 || b > cb)) {
            ci = i;
            cb = b;
          }
        }
      }
    }

    if (renorm) {
      float sum = 0.0f;
      for (int j = 0; j < k; ++j) sum += __uint_as_float(rdl(__float_as_uint(ws), j));
      if (sum > 0.0f) ws = ws / sum;
    }
    if (lane < k) {
      int32_t phys = sel;
      if (rep_off && sel >= 0) {
        const int32_t n = rep_off[sel + 1] - rep_off[sel];
        phys = n > 0 ? rep_slots[rep_off[sel] + (int32_t)(t % n)] : -1;
      }
      idx[t * k + lane] = phys;
      wout[t * k + lane] = ws;
    }
  }
}

// ---- four tokens per wave ------------------------------------------------
// For T >= kRowMinTokens, El <= 512, k <= 16 and groups covering power-of-two
// runs of at most 16 lanes, each 16-lane row of the wave routes its own token: the same four DPP
// steps then leave every lane of a row holding that row's maximum (no
// readlanes), one ballot serves the four tokens' picks, and the winner's
// local index comes over with one shuffle, so the serial pick chain is shared
// by four tokens.  Results are those of route_kernel bit for bit (same
// binary32 scores, same tie rule: the lowest lane of a row holds the lowest
// id; renormalization sums the picks in order).
constexpr int kRowLanes = 16;
constexpr int kRowTokens = kWave / kRowLanes;
// Below this many tokens the one-token kernel is faster: with four tokens a
// wave each lane evaluates four times the gates in sequence, and a small
// batch has too few waves to hide that (measured on MI355X: 128 tokens x 256
// experts 7.1 us one-token, 12.0 us four-token; 8192 tokens 16.1 / 14.4 us).
constexpr int32_t kRowMinTokens = 2048;

__device__ inline uint32_t row_max_u32(uint32_t v) {
  v = umax(v, dpp<kDppXor1>(v));
  v = umax(v, dpp<kDppXor2>(v));
  v = umax(v, dpp<kDppHalfMirror>(v));
  return umax(v, dpp<kDppMirror>(v));
}

__device__ inline float row_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp<kDppMirror>(__float_as_uint(v))));
}

// Winner of each row among its offering lanes: the largest bits, then the
// lowest lane; the winner's index within the row, or -1 if none offers.
__device__ inline int row_pick(bool has, uint32_t bits, int row, uint32_t &best_bits) {
  const uint32_t mx = row_max_u32(has ? bits : 0u);
  const uint64_t b = __ballot(has && bits == mx);
  const uint32_t m = (uint32_t)(b >> (row * kRowLanes)) & 0xFFFFu;
  best_bits = mx;
  return m ? (int)__builtin_ctz(m) : -1;
}

// COUNT: the layout's chunk histograms come from the router itself.
// Workgroup c (kRouteCountWaves waves) routes exactly the tokens
// [c*tpc, c*tpc + tpc) -- the layout's chunk c -- counts the physical experts
// it writes (entry E: indices outside [0,E), i.e. -1 for a logical expert
// without a replica) in LDS with integer atomics, whose order does not change
// the counts, and writes them as column c of the scatter kernel's table
// [C/4][E+1][4]; the workgroup of the last chunk also zeroes the columns past
// C in its group.  The routing itself is the same code, so indices and
// weights are identical to the grid-stride launch.
static_assert(kRouteCountStep == kRouteCountWaves * kRowTokens, "router step");

template <int NPER, bool COUNT>
__global__ __launch_bounds__(COUNT ? kWave * kRouteCountWaves : kWave) void route_rows_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias,
    const int32_t *__restrict__ rep_off, const int32_t *__restrict__ rep_slots, int32_t T,
    int32_t El, int32_t k, int32_t gate, int32_t G, int32_t TG, int32_t topn, int32_t renorm,
    int32_t *__restrict__ idx, float *__restrict__ wout, int32_t E, int32_t tpc, int32_t C,
    int32_t *__restrict__ hist, int32_t *__restrict__ err) {
  extern __shared__ int32_t cnt[];  // COUNT: [E+1] this chunk's expert histogram
  const int lane = threadIdx.x % kWave, row = lane / kRowLanes, lr = lane % kRowLanes;
  const int e0 = lr * NPER;
  const int gs = El / G;
  const int lpg = gs / NPER;  // lanes per group (G > 1: a power of two <= 16)
  const bool vec = NPER >= 4 && (El & 3) == 0 && (((uintptr_t)logits) & 15u) == 0 &&
                   (!bias || (((uintptr_t)bias) & 15u) == 0);
  uint32_t valid_e = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) valid_e |= (e0 + i < El) ? 1u << i : 0u;

  int64_t tb0 = (int64_t)blockIdx.x * kRowTokens, tend = T, tstep = (int64_t)gridDim.x * kRowTokens;
  if (COUNT) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
    for (int e = threadIdx.x; e <= E; e += kWave * kRouteCountWaves) cnt[e] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * tpc;
    tb0 = c0 + (int64_t)wave_id() * kRowTokens;
    tend = (c0 + tpc < T) ? c0 + tpc : T;
    tstep = kRouteCountStep;
  }
  for (int64_t tb = tb0; tb < tend; tb += tstep) {
    const int64_t t = tb + row;
    const bool live = t < tend;
    const uint32_t valid = live ? valid_e : 0u;
    const float *zr = logits + (live ? t : 0) * (int64_t)El;
    float z[NPER];
    if (vec) {
#pragma unroll
      for (int i = 0; i < NPER; i += 4) {
        float4 v = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if ((valid >> i) & 1u) {
          v = *reinterpret_cast<const float4 *>(zr + e0 + i);
          if (bias) b = *reinterpret_cast<const float4 *>(bias + e0 + i);
        }
        z[i] = bias ? v.x + b.x : v.x;
        z[i + 1] = bias ? v.y + b.y : v.y;
        z[i + 2] = bias ? v.z + b.z : v.z;
        z[i + 3] = bias ? v.w + b.w : v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int e = e0 + i;
        z[i] = ((valid >> i) & 1u) ? (bias ? zr[e] + bias[e] : zr[e]) : 0.0f;
      }
    }

    float s[NPER];
    if (gate == EP_GATE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if ((valid >> i) & 1u) m = fmaxf(m, z[i]);
      m = row_max_f32(m);
      double ex[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) ex[i] = ((valid >> i) & 1u) ? exp((double)z[i] - (double)m) : 0.0;
      // the denominator in ascending expert order, as in route_kernel: lane
      // l of the row holds experts l*NPER ..; every lane of the row folds the
      // row's values in that order
      double sum = 0.0;
      const int nl = (El + NPER - 1) / NPER;
      for (int l = 0; l < nl; ++l) {
#pragma unroll
        for (int i = 0; i < NPER; ++i) sum += shfl_f64(ex[i], row * kRowLanes + l);
      }
#pragma unroll
      for (int i = 0; i < NPER; ++i) s[i] = (float)(ex[i] / sum);
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) s[i] = (float)(1.0 / (1.0 + exp(-(double)z[i])));
    }

    uint32_t elig = valid;
    if (G > 1) {
      uint32_t a1 = 0, a2 = 0;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const uint32_t b = __float_as_uint(s[i]);
        if ((valid >> i) & 1u) {
          a2 = umax(a2, umin(a1, b));
          a1 = umax(a1, b);
        }
      }
      for (int off = 1; off < lpg; off <<= 1) {
        const uint32_t b1 = xor_lane(a1, off), b2 = xor_lane(a2, off);
        a2 = umax(umin(a1, b1), umax(a2, b2));
        a1 = umax(a1, b1);
      }
      const int grp = lr / lpg;
      const float g = (topn == 1 || gs == 1) ? __uint_as_float(a1)
                                             : __uint_as_float(a1) + __uint_as_float(a2);
      bool offer = live && (lr % lpg) == 0 && grp < G;
      uint32_t kept = 0;
      for (int r = 0; r < TG; ++r) {
        uint32_t bb;
        const int wl = row_pick(offer, __float_as_uint(g), row, bb);
        if (wl >= 0) {
          kept |= 1u << (wl / lpg);
          if (lr == wl) offer = false;
        }
      }
      elig = ((kept >> grp) & 1u) ? valid : 0u;
    }

    int ci = -1;
    uint32_t cb = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint32_t b = __float_as_uint(s[i]);
      if (((elig >> i) & 1u) && (ci < 0 || b > cb)) {
        ci = i;
        cb = b;
      }
    }
    int32_t sel = -1;
    float ws = 0.0f;
    for (int j = 0; j < k; ++j) {
      uint32_t bb;
      const int wl = row_pick(ci >= 0, cb, row, bb);
      const int ciw = __shfl(ci, row * kRowLanes + (wl < 0 ? 0 : wl), kWave);
      if (wl >= 0) {
        if (lr == j) {
          sel = wl * NPER + ciw;
          ws = __uint_as_float(bb);
        }
        if (lr == wl) {
          elig &= ~(1u << ci);
          ci = -1;
          cb = 0;
#pragma unroll
          for (int i = 0; i < NPER; ++i) {
            const uint32_t b = __float_as_uint(s[i]);
            if (((elig >> i) & 1u) && (ci < 0 || b > cb)) {
              ci = i;
              cb = b;
            }
          }
        }
      }
    }

    if (renorm) {
      float sum = 0.0f;
      for (int j = 0; j < k; ++j) sum += __shfl(ws, row * kRowLanes + j, kWave);
      if (sum > 0.0f) ws = ws / sum;
    }
    if (live && lr < k) {
      int32_t phys = sel;
      if (rep_off && sel >= 0) {
        const int32_t n = rep_off[sel + 1] - rep_off[sel];
        phys = n > 0 ? rep_slots[rep_off[sel] + (int32_t)(t % n)] : -1;
      }
      idx[t * k + lr] = phys;
      wout[t * k + lr] = ws;
      if (COUNT) atomicAdd(&cnt[((uint32_t)phys < (uint32_t)E) ? phys : E], 1);
    }
  }
  if (COUNT) {
    __syncthreads();
    const int64_t E1 = (int64_t)E + 1;
    const int c = (int)blockIdx.x;
    int32_t *col = hist + (int64_t)(c / kLayoutWaves) * E1 * kLayoutWaves + c % kLayoutWaves;
    for (int e = threadIdx.x; e < E1; e += kWave * kRouteCountWaves) col[e * kLayoutWaves] = cnt[e];
    if (c == C - 1) {
      for (int cc = C; cc % kLayoutWaves != 0; ++cc) {
        int32_t *z = hist + (int64_t)(cc / kLayoutWaves) * E1 * kLayoutWaves + cc % kLayoutWaves;
        for (int e = threadIdx.x; e < E1; e += kWave * kRouteCountWaves) z[e * kLayoutWaves] = 0;
      }
    }
  }
}

}  // namespace

namespace {

// Experts per lane of the four-tokens-per-wave kernel, or 0 where it does not
// apply: T >= kRowMinTokens, El <= 512, k <= 16, and groups covering
// power-of-two runs of at most 16 lanes.
int rows_nper(const ep_config &c, const ep_router_t &rt) {
  const int El = rt.num_logical;
  int nrow = 1;
  while (nrow * kRowLanes < El) nrow *= 2;
  const int gs = El / rt.num_groups, lpg = gs / nrow;
  const bool rows = c.num_tokens >= kRowMinTokens && El <= kRowLanes * 32 &&
                    c.num_topk <= kRowLanes &&
                    (rt.num_groups == 1 ||
                     (gs % nrow == 0 && lpg <= kRowLanes && (lpg & (lpg - 1)) == 0));
  return rows ? nrow : 0;
}

// COUNT = false: grid-stride over the tokens, nothing counted (the plan is
// unused); COUNT = true: one workgroup per chunk of `plan`.
template <bool COUNT>
hipError_t launch_rows(const ep_config &c, const ep_router_t &rt, int nrow, const float *logits,
                       const float *bias, const int32_t *rep_off, const int32_t *rep_slots,
                       int32_t *topk_idx, float *topk_w, const LayoutPlan &plan, int32_t *hist,
                       int32_t *err, hipStream_t s) {
  const int grid = COUNT ? plan.C : row_grid(c, (c.num_tokens + kRowTokens - 1) / kRowTokens);
  const int block = COUNT ? kWave * kRouteCountWaves : kWave;
  const size_t lds = COUNT ? (size_t)(c.num_experts + 1) * sizeof(int32_t) : 0;
#define EP_ROUTE_ROWS(N)                                                                         \
  hipLaunchKernelGGL((route_rows_kernel<N, COUNT>), dim3(grid), dim3(block), lds, s, logits,     \
                     bias, rep_off, rep_slots, c.num_tokens, rt.num_logical, c.num_topk, rt.gate, \
                     rt.num_groups, rt.topk_groups, rt.group_topn, rt.renormalize, topk_idx,    \
                     topk_w, c.num_experts, plan.tpc, plan.C, hist, err)
  switch (nrow) {
    case 1: EP_ROUTE_ROWS(1); break;
    case 2: EP_ROUTE_ROWS(2); break;
    case 4: EP_ROUTE_ROWS(4); break;
    case 8: EP_ROUTE_ROWS(8); break;
    case 16: EP_ROUTE_ROWS(16); break;
    default: EP_ROUTE_ROWS(32); break;
  }
#undef EP_ROUTE_ROWS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const ep_config &c, const ep_router_t &rt, const float *logits,
                        const float *bias, const int32_t *rep_off, const int32_t *rep_slots,
                        int32_t *topk_idx, float *topk_w, hipStream_t s) {
  const int El = rt.num_logical;
  // four tokens per wave where the shape allows it
  const int nrow = rows_nper(c, rt);
  if (nrow > 0)
    return launch_rows<false>(c, rt, nrow, logits, bias, rep_off, rep_slots, topk_idx, topk_w,
                              LayoutPlan{}, nullptr, nullptr, s);
  const int grid = row_grid(c, c.num_tokens);
  const size_t lds = (size_t)rt.num_logical * sizeof(float);  // scores, for the LDS group path
#define EP_ROUTE_LAUNCH(N)                                                                     \
  hipLaunchKernelGGL(route_kernel<N>, dim3(grid), dim3(kWave), lds, s, logits, bias, rep_off, \
                     rep_slots, c.num_tokens, rt.num_logical, c.num_topk, rt.gate,            \
                     rt.num_groups, rt.topk_groups, rt.group_topn, rt.renormalize, topk_idx,  \
                     topk_w)
  if (El <= 64) EP_ROUTE_LAUNCH(1);
  else if (El <= 128) EP_ROUTE_LAUNCH(2);
  else if (El <= 256) EP_ROUTE_LAUNCH(4);
  else if (El <= 512) EP_ROUTE_LAUNCH(8);
  else if (El <= 1024) EP_ROUTE_LAUNCH(16);
  else EP_ROUTE_LAUNCH(32);
#undef EP_ROUTE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_route_layout(const ep_config &c, const ep_router_t &rt, const float *logits,
                               const float *bias, const int32_t *rep_off,
                               const int32_t *rep_slots, int32_t *topk_idx, float *topk_w,
                               const ep_layout_t &h, void *workspace, hipStream_t s) {
  const int nrow = rows_nper(c, rt);
  const LayoutPlan fp = plan_route_count(c.num_tokens, c.num_topk, c.num_experts);
  if (nrow == 0 || fp.C == 0 || c.num_workgroups > 0) {
    const hipError_t err = launch_route(c, rt, logits, bias, rep_off, rep_slots, topk_idx, topk_w, s);
    if (err != hipSuccess) return err;
    return launch_layout(c, plan_layout((int64_t)c.num_tokens * c.num_topk, c.num_experts),
                         topk_idx, h, workspace, s);
  }
  const hipError_t err = launch_rows<true>(c, rt, nrow, logits, bias, rep_off, rep_slots, topk_idx,
                                           topk_w, fp, static_cast<int32_t *>(workspace),
                                           h.error_flag, s);
  if (err != hipSuccess) return err;
  return launch_layout_scatter(c, fp, topk_idx, h, workspace, s);
}

}  // namespace ep
