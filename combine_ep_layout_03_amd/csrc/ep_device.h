// ep_device.h -- device helpers shared by the HIP kernels of libep (codecs,
// wave primitives).  Kernel-side only.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "ep_internal.h"

namespace ep {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// This wave's index in its workgroup as a wave-uniform value.  threadIdx.x /
// kWave is the same on every lane of a wave, but the compiler treats it as a
// per-lane value, and so every work-unit index derived from it: 64-bit
// divisions and loop control then run as vector instructions on every lane.
__device__ inline int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

__device__ inline uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Address of a pair's row in its rank's buffer, from per-lane rank tables:
// lane r < R holds rank r's first global slot (my_roff) and buffer base
// (my_base), loaded once per wave beside its first data loads, so a pair's
// row costs two shuffles instead of a chain of dependent loads (index, then
// the rank's offset, then its base pointer).  e and sl are the pair's expert
// and global slot (lanes without a pair pass e = -1).  Returns 0 when e is
// outside [0,E) or the row outside [0,cap); rank and row are set either way.
// Wave-wide: every lane must call it.
__device__ inline uint64_t row_addr(int32_t e, int32_t sl, int32_t E, int32_t El, int64_t cap,
                                    int32_t my_roff, uint64_t my_base, int64_t rowbytes,
                                    int &rank, int64_t &row) {
  const bool ein = (uint32_t)e < (uint32_t)E;
  rank = ein ? e / El : 0;
  const int32_t ro = __shfl(my_roff, rank, kWave);
  const uint64_t base = shfl64(my_base, rank);
  // slots and offsets lie in [-1, 2^31): their difference fits 32 bits, and
  // widening only the difference keeps the compiler from waiting on the slot
  // load to widen it before the unit's other loads are issued
  row = (int64_t)(sl - ro);
  return (ein && row >= 0 && row < cap) ? base + (uint64_t)(row * rowbytes) : 0;
}

__device__ inline int32_t wave_inclusive_scan(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t n = __shfl_up(v, d, kWave);
    if (lane >= d) v += n;
  }
  return v;
}

// DPP controls (gfx9): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror.  After these four steps of a commutative reduction every lane
// of a 16-lane row holds the row's result.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ inline uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ inline uint32_t rdl(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Sum over the wave (32-bit, wrapping), uniform result: four DPP steps in
// each row, then the four row sums.
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (rdl(v, 0) + rdl(v, 16)) + (rdl(v, 32) + rdl(v, 48));
}

// max over the low 15 bits (|x| of bf16, monotone for non-NaN) of 8 bf16.
__device__ inline uint32_t bf16_absbits_max(u32x4 v, uint32_t m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = v[i] & 0x7FFFu, hi = (v[i] >> 16) & 0x7FFFu;
    m = lo > m ? lo : m;
    m = hi > m ? hi : m;
  }
  return m;
}

// Four binary32 values (each |v| <= 448 * (1 + 2^-23)) -> four OCP E4M3
// ("fn": bias 7, max 448, no infinity) codes in one dword, byte i = code of
// a_i, by gfx950's v_cvt_pk_fp8_f32: nearest with ties to even, saturating at
// 448, signed zeros kept.  tests/test_gpu_cvt.py compares it code for code
// with the oracle's encoder on every binary32 value within 2^12 ulps of each
// E4M3 value and rounding midpoint and on every 257th pattern up to |v| = 450,
// both signs.  A block quotient x/s never exceeds 448 * (1 + 2^-23).
__device__ inline uint32_t e4m3_pack4(float a0, float a1, float a2, float a3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, w, true);
  return (uint32_t)w;
}

// 4 bf16 pairs -> 8 E4M3 codes of (x / s) in 2 dwords, channel order kept;
// zero (an all-zero block) gives 0x00 codes.
__device__ inline void quant8(u32x4 v, float s, bool zero, uint32_t &w0, uint32_t &w1) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __uint_as_float(v[i] << 16) / s;
    r[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u) / s;
  }
  w0 = zero ? 0u : e4m3_pack4(r[0], r[1], r[2], r[3]);
  w1 = zero ? 0u : e4m3_pack4(r[4], r[5], r[6], r[7]);
}

// One lane's share of a 128-channel block (16 channels as two 16-byte bf16
// vectors) -> 16 E4M3 codes and the block scale.  The 8 lanes of a block are
// the aligned groups of 8 lanes; lanes outside the row pass zeros as whole
// groups.  s = a/448 (correctly rounded), codes of the correctly rounded x/s.
__device__ inline u32x4 quant_block16(u32x4 v0, u32x4 v1, float &s_out) {
  uint32_t m = bf16_absbits_max(v1, bf16_absbits_max(v0, 0u));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4, kWave));
  const bool zero = (m == 0u);
  const float s = zero ? 0.0f : __uint_as_float(m << 16) / 448.0f;
  uint32_t q0, q1, q2, q3;
  quant8(v0, s, zero, q0, q1);
  quant8(v1, s, zero, q2, q3);
  s_out = s;
  return u32x4{q0, q1, q2, q3};
}

// Block quantization of 16 binary32 activations per lane (8 lanes per
// 128-element block) for the expert-side re-quantization, where the
// activation itself is only specified to a tolerance: amax on |a| bit
// patterns, s = a/448 (correctly rounded), codes of a * (1/s) -- one divide
// per block instead of one per element, within 1.5 binary32 ulps of a/s, so a
// code can differ from E4M3(a/s) only where a/s lies that close to an E4M3
// rounding boundary.  Blocks so small that 1/s overflows divide exactly.
__device__ inline u32x4 quant_block16_f32(const float *a, float &s_out) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = __float_as_uint(a[i]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4, kWave));
  const bool zero = (m == 0u);
  const float s = zero ? 0.0f : __uint_as_float(m) / 448.0f;
  uint32_t w[4];
  if (zero) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = 0u;
  } else {
    const float inv = 1.0f / s;
    if (inv <= 3.0e38f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = e4m3_pack4(a[4 * i] * inv, a[4 * i + 1] * inv, a[4 * i + 2] * inv, a[4 * i + 3] * inv);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = e4m3_pack4(a[4 * i] / s, a[4 * i + 1] / s, a[4 * i + 2] / s, a[4 * i + 3] / s);
    }
  }
  s_out = s;
  return u32x4{w[0], w[1], w[2], w[3]};
}

// binary32 -> bf16 bits, nearest with ties to even; NaN stays a quiet NaN.
__device__ inline uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 binary32 -> 8 bf16 (bf16_bits each), two per dword, channel order kept.
__device__ inline u32x4 pack8(const float *acc) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16_bits(acc[2 * i]) | (bf16_bits(acc[2 * i + 1]) << 16);
  return o;
}

}  // namespace dev
}  // namespace ep
