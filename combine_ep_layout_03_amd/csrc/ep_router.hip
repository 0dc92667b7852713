// ep_router.hip -- the MoE router on gfx950: gate scores, group-limited
// top-k, weights and the redundant-expert mapping, one wave per token.
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
// Lane l holds experts l, l+64, ... (coalesced loads of the logit row).  The
// gate is evaluated in binary64 and rounded once to binary32, so the scores
// -- and with them every selection, which compares binary32 values only --
// do not depend on how a device or host libm rounds its exp; the binary64
// softmax denominator is a wave butterfly sum.  The scores go to LDS.  Lanes
// below G score one group each (its best, or the sum of its two best); TG
// rounds of a wave-wide maximum over 64-bit keys (score bits above the
// complement of the id, so equal scores favour the lower id) pick the
// eligible groups, and k more rounds pick the experts, each lane keeping the
// best key of its own experts and rescanning only when its key was taken.
// Lane j ends with pick j; renormalization sums the k picks in order with
// readlane, so the weights are the same binary32 operations as a sequential
// loop.  fp contraction is off in this file: the scores are exact
// compositions of correctly rounded operations.
#include <math.h>

#include "ep_device.h"
#include "ep_internal.h"

#pragma clang fp contract(off)

namespace ep {
namespace {

using namespace dev;

__device__ inline uint64_t rank_key(float s, int id) {
  return ((uint64_t)__float_as_uint(s) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ inline int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ inline float key_score(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, kWave);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Best key among this lane's experts that are eligible and not yet taken.
__device__ inline uint64_t lane_best(const float *s, int lane, int El, int gs, uint64_t kept,
                                     uint32_t taken) {
  uint64_t best = 0;
  for (int i = 0, e = lane; e < El; ++i, e += kWave) {
    if ((taken >> i) & 1u) continue;
    if (!((kept >> (e / gs)) & 1ull)) continue;
    const uint64_t key = rank_key(s[e], e);
    best = key > best ? key : best;
  }
  return best;
}

__global__ __launch_bounds__(kWave) void route_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias,
    const int32_t *__restrict__ rep_off, const int32_t *__restrict__ rep_slots, int32_t T,
    int32_t El, int32_t k, int32_t gate, int32_t G, int32_t TG, int32_t topn, int32_t renorm,
    int32_t *__restrict__ idx, float *__restrict__ wout) {
  extern __shared__ double lds[];
  double *ex = lds;                                               // [El] softmax numerators
  float *s = reinterpret_cast<float *>(lds + (gate == EP_GATE_SOFTMAX ? El : 0));  // [El]
  const int lane = threadIdx.x;
  const int gs = El / G;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float *zr = logits + t * (int64_t)El;
    if (gate == EP_GATE_SOFTMAX) {
      float m = -INFINITY;
      for (int e = lane; e < El; e += kWave) {
        const float z = bias ? zr[e] + bias[e] : zr[e];
        s[e] = z;  // the logit, until the score replaces it
        m = fmaxf(m, z);
      }
      m = wave_max_f32(m);
      double sum = 0.0;
      for (int e = lane; e < El; e += kWave) {
        const double x = exp((double)s[e] - (double)m);
        ex[e] = x;
        sum += x;
      }
      sum = wave_sum_f64(sum);
      for (int e = lane; e < El; e += kWave) s[e] = (float)(ex[e] / sum);
    } else {
      for (int e = lane; e < El; e += kWave) {
        const float z = bias ? zr[e] + bias[e] : zr[e];
        s[e] = (float)(1.0 / (1.0 + exp(-(double)z)));
      }
    }
    __syncthreads();

    // eligible groups (bit c of kept); one group keeps every expert
    uint64_t kept = ~0ull;
    if (G > 1) {
      uint64_t gkey = 0;
      if (lane < G) {
        uint64_t k1 = 0, k2 = 0;
        for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
          const uint64_t key = rank_key(s[e], e);
          if (key > k1) {
            k2 = k1;
            k1 = key;
          } else if (key > k2) {
            k2 = key;
          }
        }
        const float g = (topn == 1 || gs == 1) ? key_score(k1) : key_score(k1) + key_score(k2);
        gkey = rank_key(g, lane);
      }
      kept = 0;
      for (int r = 0; r < TG; ++r) {
        const uint64_t best = wave_max_u64(gkey);
        const int c = key_id(best);
        kept |= 1ull << c;
        if (lane == c) gkey = 0;
      }
    }

    // top-k: lane j keeps pick j
    uint32_t taken = 0;
    uint64_t mine = lane_best(s, lane, El, gs, kept, taken);
    int32_t sel = -1;
    float ws = 0.0f;
    for (int j = 0; j < k; ++j) {
      const uint64_t best = wave_max_u64(mine);
      if (best == 0) break;  // fewer eligible experts than k: excluded on the host
      const int e = key_id(best);
      if (lane == j) {
        sel = e;
        ws = key_score(best);
      }
      if (lane == (e % kWave)) {
        taken |= 1u << (e / kWave);
        mine = lane_best(s, lane, El, gs, kept, taken);
      }
    }

    if (renorm) {
      float sum = 0.0f;
      for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws), j));
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
    __syncthreads();  // the next token reuses the LDS scores
  }
}

}  // namespace

size_t route_lds_bytes(int32_t El, int32_t gate) {
  return (size_t)El * (gate == EP_GATE_SOFTMAX ? sizeof(double) + sizeof(float) : sizeof(float));
}

hipError_t launch_route(const ep_config &c, const ep_router_t &rt, const float *logits,
                        const float *bias, const int32_t *rep_off, const int32_t *rep_slots,
                        int32_t *topk_idx, float *topk_w, hipStream_t s) {
  const int grid = row_grid(c, c.num_tokens);
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(kWave), route_lds_bytes(rt.num_logical, rt.gate),
                     s, logits, bias, rep_off, rep_slots, c.num_tokens, rt.num_logical, c.num_topk,
                     rt.gate, rt.num_groups, rt.topk_groups, rt.group_topn, rt.renormalize,
                     topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace ep
