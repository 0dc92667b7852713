// ep_expert.hip -- expert-side activation on the received rows: SiLU-and-
// multiply followed by per-128-channel FP8 re-quantization.
//
// Pages: [Perplexity blog] "Lower latency and higher throughput with
// multi-node DeepSeek deployment", "Magntölun": the SiLU kernel quantizes its
// output per 128-element block with scales computed on the fly, and, under
// graphs, reads the per-expert token counts on the device and splits the
// work dynamically instead of sizing it from the upper-bound buffers.
//
// Design.  The input rows are the expert GEMM's outputs in the receive
// layout (R rank buffers, rows in slot order); the number of valid rows is
// T*k in total, split over the ranks by the handle's rank_offsets, which the
// kernel reads on the device (a binary search per work unit), so the launch
// needs no host copy of the counts and can be captured in a graph.  A unit is
// (slot, segment of 8 blocks of 128 channels); a lane holds 16 channels of
// gate and up, computes a = g * rcp(1 + e^-g) * u in binary32 (exp_neg below
// and the 1-ulp hardware reciprocal: the activation is specified to a
// tolerance against a binary64 reference, and the kernel is bound by its
// VALU work as much as by memory), then the block amax and the correctly
// rounded scale as dispatch does, and codes of a * (1/s) with one divide per
// block (within 1.5 binary32 ulps of a/s, inside the same tolerance).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kSegBlocks = 8;

// e^-g for the activation.  With x = -g, e^x = 2^(x log2 e) is taken on the
// hardware base-2 exponential with the argument reduction of the
// split-constant method: log2(e) = C_hi + C_lo (C_hi its binary32 rounding),
// t = RN(x * C_hi), and d = x*C_hi - t + x*C_lo recovered with two fused
// multiply-adds (the product's rounding error is exact in an fma), so
// e^x = 2^t * 2^d ~ 2^t * (1 + d ln 2).  Wherever 2^t is finite (|t| < 128)
// |d| < 2^-16, so the neglected (d ln 2)^2 / 2 is below 2^-33.  x is clamped
// to [-200, 200] first, beyond which 2^t is already 0 or +inf in binary32, so
// every special input gives what e^x gives; a NaN gate stays a NaN in the
// activation through the factor g.  Measured over every bf16 gate
// value: the activation is within 2.34 binary32 ulps of binary64 (2.25 with
// the device expf), with the same NaN / inf outputs; it takes about 110
// fewer VALU instructions per wave than expf.
__device__ inline float exp_neg(float g) {
  const float x = __builtin_amdgcn_fmed3f(-g, -200.0f, 200.0f);
  const float c_hi = 1.44269502162933349609375f;    // binary32 nearest log2(e)
  const float c_lo = 1.925963033500011e-08f;        // log2(e) - c_hi
  const float ln2 = 0.693147182464599609375f;       // binary32 nearest ln 2
  const float t = x * c_hi;
  const float d = __builtin_fmaf(x, c_lo, __builtin_fmaf(x, c_hi, -t));
  return __builtin_amdgcn_exp2f(t) * __builtin_fmaf(d, ln2, 1.0f);
}

__global__ __launch_bounds__(kWave) void silu_mul_quant_kernel(
    const int32_t *__restrict__ rank_offsets, const int32_t *__restrict__ err, int64_t P,
    int32_t R, int32_t I, int64_t cap, RankCPtrs in, RankPtrs q_out, ScalePtrs s_out) {
  if (*err & kLayoutErrBits) return;
  const int lane = threadIdx.x;
  const int nb = I / 128;
  const int nseg = (nb + kSegBlocks - 1) / kSegBlocks;
  const int64_t units = P * nseg;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t slot = u / nseg;
    const int seg = (int)(u % nseg);
    // rank r with rank_offsets[r] <= slot < rank_offsets[r+1] (uniform)
    int lo = 0, hi = R;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (rank_offsets[mid] <= slot) lo = mid;
      else hi = mid;
    }
    const int64_t row = slot - rank_offsets[lo];
    if (row < 0 || row >= cap) continue;  // cannot happen for a valid handle
    const int blk = seg * kSegBlocks + lane / 8;
    const bool valid = blk < nb;
    const int ch = blk * 128 + (lane % 8) * 16;
    const uint16_t *src = static_cast<const uint16_t *>(in.p[lo]) + row * (int64_t)(2 * I);
    u32x4 g0 = {0u, 0u, 0u, 0u}, g1 = g0, u0 = g0, u1 = g0;
    if (valid) {
      g0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + ch));
      g1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + ch + 8));
      u0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + I + ch));
      u1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + I + ch + 8));
    }
    float a[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 gv = i < 4 ? g0 : g1, uv = i < 4 ? u0 : u1;
      const uint32_t gw = gv[i % 4], uw = uv[i % 4];
      const float ga = __uint_as_float(gw << 16), gb = __uint_as_float(gw & 0xFFFF0000u);
      const float ua = __uint_as_float(uw << 16), ub = __uint_as_float(uw & 0xFFFF0000u);
      a[2 * i] = ga * __builtin_amdgcn_rcpf(1.0f + exp_neg(ga)) * ua;
      a[2 * i + 1] = gb * __builtin_amdgcn_rcpf(1.0f + exp_neg(gb)) * ub;
    }
    float s;
    const u32x4 q = quant_block16_f32(a, s);
    if (valid) {
      uint8_t *qd = static_cast<uint8_t *>(q_out.p[lo]) + row * (int64_t)I;
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(qd + ch));
      if ((lane % 8) == 0) s_out.p[lo][row * nb + blk] = s;
    }
  }
}

}  // namespace

hipError_t launch_silu_mul_quant(const ep_config &c, const ep_layout_t &h, int32_t I,
                                 const RankCPtrs &in, const RankPtrs &q, const ScalePtrs &s,
                                 int64_t capacity_rows, hipStream_t st) {
  const int64_t P = (int64_t)c.num_tokens * c.num_topk;
  const int64_t nseg = (I / 128 + kSegBlocks - 1) / kSegBlocks;
  const int grid = row_grid(c, P * nseg);
  hipLaunchKernelGGL(silu_mul_quant_kernel, dim3(grid), dim3(kWave), 0, st, h.rank_offsets,
                     h.error_flag, P, c.num_ranks, I, capacity_rows, in, q, s);
  return hipGetLastError();
}

}  // namespace ep
