// ep_combine.hip -- combine and un-permute on gfx950.
//
// Pages: [Perplexity blog] "Lower latency and higher throughput with
// multi-node DeepSeek deployment", "Sérfræðinga-samsíðun" (each token's 8
// routed results are weighted and summed) and "Skörun" (combine was the
// largest communication item: 1012 us before micro-batching);
// [DeepEP overview] "DeepSeek merilis library open source DeepEP ...",
// "Pola penggunaan ..." (combine reduces expert outputs back to the source
// rank; the backward of dispatch is a combine) and "Hasil pengukuran
// performa" (BF16 combine); [torchtitan PR] "Integrate DeepEP to experimental
// torchtitan" (the token unpermute after the experts).
//
// Design.  The work unit is one (token, segment) pair, where a segment is
// 128 16-byte chunks (1024 channels) of the output row; one single-wave
// workgroup takes one unit at a time (grid-stride), so a token's row is spread
// over several short-lived waves.  Lanes 0..k-1 resolve the token's k
// received rows (up to 16384 units from the per-lane rank tables, all of a
// unit's small loads in one round trip; above, by a chain of dependent loads,
// which the memory queues hide there) and weights; each lane then owns two
// chunks (c and c+64) and issues the 2*k gathered 16-byte non-temporal loads
// of its chunks (up to 16 in flight) before any arithmetic, folds them in
// ascending j with fp32 fused multiply-adds from +0, rounds to bf16
// nearest-even and writes each output
// chunk once with a non-temporal store.  No atomics; the un-permute is fused
// into the loads.  (Measured on MI355X at T=8192, H=7168, k=8: one-wave
// workgroups and two chunks per lane beat four-wave workgroups, one chunk and
// four chunks per lane; plain stores are slower than non-temporal ones.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dev;

constexpr int kThreads = kRowWaves * kWave;
constexpr int kJB = 8;                 // rows whose loads are issued together
constexpr int kSegChunks = 2 * kWave;  // 16-byte chunks per work unit

// acc[0..7] += w * (8 bf16 of v), element by element, one fma each.
__device__ inline void fma8(float *acc, float w, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = __builtin_fmaf(w, __uint_as_float(v[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(w, __uint_as_float(v[i] & 0xFFFF0000u), acc[2 * i + 1]);
  }
}

// acc[0..7] += (8 bf16 of v), one binary32 addition each.
__device__ inline void add8(float *acc, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = acc[2 * i] + __uint_as_float(v[i] << 16);
    acc[2 * i + 1] = acc[2 * i + 1] + __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// Lane j < k: byte address of pair (t, j)'s received row (0 if unusable,
// which raises EP_DEVERR_ROW).
__device__ inline uint64_t src_row(const int32_t *__restrict__ idx,
                                   const int32_t *__restrict__ slot_of,
                                   const int32_t *__restrict__ rank_offsets,
                                   int32_t *__restrict__ err, int64_t p, int32_t E, int32_t El,
                                   int64_t cap, const RankCPtrs &ry, int64_t rowbytes) {
  const int32_t e = idx[p];
  if ((uint32_t)e < (uint32_t)E) {
    const int32_t r = e / El;
    const int64_t rr = (int64_t)slot_of[p] - rank_offsets[r];
    if (rr >= 0 && rr < cap) return (uint64_t)ry.p[r] + (uint64_t)(rr * rowbytes);
  }
  atomicOr(err, (int32_t)EP_DEVERR_ROW);
  return 0;
}

// HasShared: the shared expert's row is added after the routed fold
// ([Perplexity blog], "Sérfræðinga-samsíðun": every token also runs through
// the shared expert, whose result is added to the routed experts' result).
template <bool HasShared>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ rank_offsets, int32_t *__restrict__ err,
    const float *__restrict__ w, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El,
    int32_t R, int64_t cap, RankCPtrs ry, const uint16_t *__restrict__ shared,
    uint16_t *__restrict__ out) {
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nch = H / 8;
  const int nseg = (nch + kSegChunks - 1) / kSegChunks;
  const int64_t units = (int64_t)T * nseg;
  const int64_t u0 = (int64_t)blockIdx.x * kRowWaves + wave;
  if (u0 >= units) return;
  int32_t err0 = 0;
  // One unit; false once the error word is found set (nothing is written).
  // The token's indices, slots and weights, the per-lane rank tables and the
  // shared row are loaded together (the error word, read once by the first
  // unit, after them); the k source rows then come from row_addr's shuffles.
  auto unit = [&](int64_t u, bool first) -> bool {
    const int64_t t = u / nseg;
    const int c0 = (int)(u % nseg) * kSegChunks + lane;
    const int c1 = c0 + kWave;
    const bool ok0 = c0 < nch, ok1 = c1 < nch;
    int32_t e = -1, sl = 0;
    float wj = 0.0f;
    if (lane < k) {
      e = idx[t * k + lane];
      sl = slot_of[t * k + lane];
      wj = w ? w[t * k + lane] : 1.0f;
    }
    int32_t my_roff = 0;
    uint64_t my_base = 0;
    if (lane < R) {
      my_roff = rank_offsets[lane];
      my_base = (uint64_t)ry.p[lane];
    }
    u32x4 sh0 = {0u, 0u, 0u, 0u}, sh1 = {0u, 0u, 0u, 0u};
    if (HasShared) {
      const u32x4 *srow = reinterpret_cast<const u32x4 *>(shared + t * H);
      if (ok0) sh0 = __builtin_nontemporal_load(srow + c0);
      if (ok1) sh1 = __builtin_nontemporal_load(srow + c1);
    }
    if (first) err0 = *err;
    if (err0 & kLayoutErrBits) return false;
    int rank;
    int64_t row;
    uint64_t src = row_addr(e, sl, E, El, cap, my_roff, my_base, (int64_t)H * 2, rank, row);
    if (lane >= k) src = 0;
    else if (src == 0) atomicOr(err, (int32_t)EP_DEVERR_ROW);
    if (__ballot(lane < k && src == 0) != 0) return true;  // a bad row: write nothing for t
    float acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc0[i] = acc1[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kJB) {
      u32x4 v0[kJB], v1[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < k) {
          const u32x4 *yrow = reinterpret_cast<const u32x4 *>(readlane64(src, j0 + jj));
          if (ok0) v0[jj] = __builtin_nontemporal_load(yrow + c0);
          if (ok1) v1[jj] = __builtin_nontemporal_load(yrow + c1);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < k) {
          const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j0 + jj));
          fma8(acc0, wv, v0[jj]);
          fma8(acc1, wv, v1[jj]);
        }
      }
    }
    if (HasShared) {
      add8(acc0, sh0);
      add8(acc1, sh1);
    }
    u32x4 *orow = reinterpret_cast<u32x4 *>(out + t * H);
    if (ok0) __builtin_nontemporal_store(pack8(acc0), orow + c0);
    if (ok1) __builtin_nontemporal_store(pack8(acc1), orow + c1);
    return true;
  };
  // the first unit outside the loop, so that its loads and the error word's
  // are in flight together (one unit per wave by default)
  if (!unit(u0, true)) return;
  for (int64_t u = u0 + (int64_t)gridDim.x * kRowWaves; u < units;
       u += (int64_t)gridDim.x * kRowWaves)
    unit(u, false);
}

// The same combine with each pair's row resolved by a chain of dependent
// loads (index, then the rank's offset, then its base pointer) and the error
// word read at the start: for large batches, where the memory queues hide that
// chain, this form measured 0.3 % (8192 tokens, uniform routing) to 1 %
// (Zipf-skewed) faster than combine_kernel's one round trip of loads, which
// wins at decode and mid-size batches (up to 13 %).  Both write the same bytes.
template <bool HasShared>
__global__ __launch_bounds__(kThreads) void combine_chain_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ rank_offsets, int32_t *__restrict__ err,
    const float *__restrict__ w, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El,
    int64_t cap, RankCPtrs ry, const uint16_t *__restrict__ shared, uint16_t *__restrict__ out) {
  if (*err & kLayoutErrBits) return;
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nch = H / 8;
  const int nseg = (nch + kSegChunks - 1) / kSegChunks;
  const int64_t units = (int64_t)T * nseg;
  for (int64_t u = (int64_t)blockIdx.x * kRowWaves + wave; u < units;
       u += (int64_t)gridDim.x * kRowWaves) {
    const int64_t t = u / nseg;
    const int c0 = (int)(u % nseg) * kSegChunks + lane;
    const int c1 = c0 + kWave;
    const bool ok0 = c0 < nch, ok1 = c1 < nch;
    uint64_t src = 0;
    float wj = 0.0f;
    if (lane < k) {
      src = src_row(idx, slot_of, rank_offsets, err, t * k + lane, E, El, cap, ry, (int64_t)H * 2);
      wj = w ? w[t * k + lane] : 1.0f;
    }
    if (__ballot(lane < k && src == 0) != 0) continue;  // a bad row: write nothing for t
    float acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc0[i] = acc1[i] = 0.0f;
    u32x4 sh0 = {0u, 0u, 0u, 0u}, sh1 = {0u, 0u, 0u, 0u};
    if (HasShared) {
      const u32x4 *srow = reinterpret_cast<const u32x4 *>(shared + t * H);
      if (ok0) sh0 = __builtin_nontemporal_load(srow + c0);
      if (ok1) sh1 = __builtin_nontemporal_load(srow + c1);
    }
    for (int j0 = 0; j0 < k; j0 += kJB) {
      u32x4 v0[kJB], v1[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < k) {
          const u32x4 *yrow = reinterpret_cast<const u32x4 *>(readlane64(src, j0 + jj));
          if (ok0) v0[jj] = __builtin_nontemporal_load(yrow + c0);
          if (ok1) v1[jj] = __builtin_nontemporal_load(yrow + c1);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < k) {
          const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j0 + jj));
          fma8(acc0, wv, v0[jj]);
          fma8(acc1, wv, v1[jj]);
        }
      }
    }
    if (HasShared) {
      add8(acc0, sh0);
      add8(acc1, sh1);
    }
    u32x4 *orow = reinterpret_cast<u32x4 *>(out + t * H);
    if (ok0) __builtin_nontemporal_store(pack8(acc0), orow + c0);
    if (ok1) __builtin_nontemporal_store(pack8(acc1), orow + c1);
  }
}

// Backward of combine ([DeepEP overview], "Pola penggunaan ...": the backward
// of combine is a dispatch), for large batches, in two launches.  The
// gradient rows bf16(RN32(w_j * g)) are a BF16 dispatch of grad_out with one
// multiply per copy (combine_backward_rows_kernel, ep_dispatch.hip, capped
// like dispatch at 12 resident workgroups per CU); this kernel then computes
// grad_w alone: one wave per token (grid-stride), the k pairs in blocks of 8,
// for each block the token's grad_out row streamed once beside the block's
// received rows, each pair's dot product <g, y_j> accumulated per lane (fp32
// fma over the lane's channels in order) and reduced across the wave with a
// fixed xor-butterfly, so the result is deterministic.  A token with an
// unusable row gets no grad_w (the rows kernel raises EP_DEVERR_ROW for it).
// (Measured on MI355X at T=8192, H=7168, k=8: 212 + 157 us against 387 us
// for one wave per token writing the rows and the dots together, whose
// scattered row stores and gathered row loads shared each wave; 329 against
// 382 us with Zipf-skewed routing; equal at T=4096, H=2048, k=6.)
__global__ __launch_bounds__(kThreads) void combine_backward_dots_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ rank_offsets, const int32_t *__restrict__ err,
    const uint16_t *__restrict__ gout, int32_t T, int32_t H, int32_t k, int32_t E, int32_t El,
    int64_t cap, RankCPtrs ry, float *__restrict__ gw) {
  if (*err & kLayoutErrBits) return;
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nch = H / 8;
  for (int64_t t = (int64_t)blockIdx.x * kRowWaves + wave; t < T;
       t += (int64_t)gridDim.x * kRowWaves) {
    uint64_t src = 0;
    if (lane < k) {
      const int64_t p = t * k + lane;
      const int32_t e = idx[p];
      if ((uint32_t)e < (uint32_t)E) {
        const int32_t r = e / El;
        const int64_t rr = (int64_t)slot_of[p] - rank_offsets[r];
        if (rr >= 0 && rr < cap) src = (uint64_t)ry.p[r] + (uint64_t)(rr * (int64_t)H * 2);
      }
    }
    if (__ballot(lane < k && src == 0) != 0) continue;  // a bad row: no grad_w for t
    const u32x4 *grow = reinterpret_cast<const u32x4 *>(gout + t * H);
    for (int j0 = 0; j0 < k; j0 += kJB) {
      float acc[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) acc[jj] = 0.0f;
      for (int c = lane; c < nch; c += kWave) {
        const u32x4 g = grow[c];
        u32x4 v[kJB];
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj)
          if (j0 + jj < k)
            v[jj] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(readlane64(src, j0 + jj)) + c);
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj) {
          if (j0 + jj < k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[jj] = __builtin_fmaf(__uint_as_float(g[i] << 16),
                                       __uint_as_float(v[jj][i] << 16), acc[jj]);
              acc[jj] = __builtin_fmaf(__uint_as_float(g[i] & 0xFFFF0000u),
                                       __uint_as_float(v[jj][i] & 0xFFFF0000u), acc[jj]);
            }
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        float a = acc[jj];
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
        if (lane == 0 && j0 + jj < k) gw[t * k + j0 + jj] = a;
      }
    }
  }
}

// The backward for small batches (T < kBwdWgMaxTokens, e.g. decode), in one
// launch, since there a second launch costs more than it saves and one wave
// per token leaves the GPU nearly idle.  One workgroup of kBwdWaves waves per
// token (grid-stride), its threads splitting the row's 16-byte chunks; the k pairs
// are taken in blocks of 8: for each block the workgroup streams the token's
// grad_out row once, writes bf16(RN32(w_j * g)) into each pair's gradient row
// and, when y is given, accumulates each pair's dot product <g, y_j> per
// thread (fp32 fma over its channels in order), reduces it across each wave
// with a fixed xor-butterfly and then over the waves in ascending order, so
// the result is deterministic and needs no scratch memory.  (Measured on
// MI355X: at 128 tokens 16 us against 50 us for one wave per token writing
// the rows and the dots together; at 8192 tokens 411 us against 387 us for
// that kernel, and the two launches above take 351 us.)
constexpr int kBwdWaves = 8;
constexpr int32_t kBwdWgMaxTokens = 2048;
constexpr int kBwdThreads = kBwdWaves * kWave;

__global__ __launch_bounds__(kBwdThreads) void combine_backward_wg_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ rank_offsets, int32_t *__restrict__ err,
    const uint16_t *__restrict__ gout, const float *__restrict__ w, int32_t T, int32_t H,
    int32_t k, int32_t E, int32_t El, int32_t R, int64_t cap, RankCPtrs ry, RankPtrs rg,
    float *__restrict__ gw) {
  __shared__ float part[kBwdWaves][EP_MAX_TOPK];  // per-wave dot products
  if (*err & kLayoutErrBits) return;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nch = H / 8;
  const bool want_w = gw != nullptr;
  // per-lane rank tables (row_addr): the token's rows cost one round trip of
  // loads instead of a dependent chain, which matters at decode sizes; the
  // grad_w kernel for large batches keeps the chain (its long rows hide it)
  int32_t my_roff = 0;
  uint64_t my_g = 0, my_y = 0;
  if (lane < R) {
    my_roff = rank_offsets[lane];
    my_g = (uint64_t)rg.p[lane];
    if (want_w) my_y = (uint64_t)ry.p[lane];
  }
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    // every wave resolves the token's rows itself (L2 hits), so all waves
    // agree on skipping a bad token without a barrier
    int32_t e = -1, sl = 0;
    float wj = 0.0f;
    if (lane < k) {
      e = idx[t * k + lane];
      sl = slot_of[t * k + lane];
      wj = w ? w[t * k + lane] : 1.0f;
    }
    int rank;
    int64_t row;
    uint64_t dst = row_addr(e, sl, E, El, cap, my_roff, my_g, (int64_t)H * 2, rank, row);
    const uint64_t ybase = shfl64(my_y, rank);
    uint64_t src = 0;
    if (lane >= k) dst = 0;
    else if (dst == 0 && wave == 0) atomicOr(err, (int32_t)EP_DEVERR_ROW);
    else if (dst != 0 && want_w) src = ybase + (uint64_t)(row * (int64_t)H * 2);
    if (__ballot(lane < k && dst == 0) != 0) continue;  // a bad row: write nothing for t
    const u32x4 *grow = reinterpret_cast<const u32x4 *>(gout + t * H);
    for (int j0 = 0; j0 < k; j0 += kJB) {
      float acc[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) acc[jj] = 0.0f;
      for (int c = tid; c < nch; c += kBwdThreads) {
        const u32x4 g = __builtin_nontemporal_load(grow + c);
        u32x4 v[kJB];
        if (want_w) {
#pragma unroll
          for (int jj = 0; jj < kJB; ++jj)
            if (j0 + jj < k)
              v[jj] = __builtin_nontemporal_load(
                  reinterpret_cast<const u32x4 *>(readlane64(src, j0 + jj)) + c);
        }
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj) {
          if (j0 + jj < k) {
            const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j0 + jj));
            float prod[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              prod[2 * i] = wv * __uint_as_float(g[i] << 16);
              prod[2 * i + 1] = wv * __uint_as_float(g[i] & 0xFFFF0000u);
            }
            u32x4 *drow = reinterpret_cast<u32x4 *>(readlane64(dst, j0 + jj));
            __builtin_nontemporal_store(pack8(prod), drow + c);
            if (want_w) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[jj] = __builtin_fmaf(__uint_as_float(g[i] << 16),
                                         __uint_as_float(v[jj][i] << 16), acc[jj]);
                acc[jj] = __builtin_fmaf(__uint_as_float(g[i] & 0xFFFF0000u),
                                         __uint_as_float(v[jj][i] & 0xFFFF0000u), acc[jj]);
              }
            }
          }
        }
      }
      if (want_w) {
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj) {
          float a = acc[jj];
#pragma unroll
          for (int o = kWave / 2; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
          if (lane == 0 && j0 + jj < k) part[wave][j0 + jj] = a;
        }
      }
    }
    if (want_w) {
      __syncthreads();
      if (tid < k) {
        float a = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kBwdWaves; ++wv) a += part[wv][tid];
        gw[t * k + tid] = a;
      }
      __syncthreads();  // part is reused for the next token
    }
  }
}

__global__ __launch_bounds__(kThreads) void unpermute_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ rank_offsets, int32_t *__restrict__ err, int64_t P, int32_t H,
    int32_t E, int32_t El, int64_t cap, RankCPtrs ry, uint16_t *__restrict__ out) {
  if (*err & kLayoutErrBits) return;
  const int wave = wave_id(), lane = threadIdx.x % kWave;
  const int nch = H / 8;
  for (int64_t p = (int64_t)blockIdx.x * kRowWaves + wave; p < P;
       p += (int64_t)gridDim.x * kRowWaves) {
    uint64_t src = 0;
    if (lane == 0) src = src_row(idx, slot_of, rank_offsets, err, p, E, El, cap, ry, (int64_t)H * 2);
    src = readlane64(src, 0);
    if (src == 0) continue;
    const u32x4 *yrow = reinterpret_cast<const u32x4 *>(src);
    u32x4 *orow = reinterpret_cast<u32x4 *>(out + p * H);
    for (int c = lane; c < nch; c += kWave) orow[c] = yrow[c];
  }
}

}  // namespace

// Units (token, segment) up to which combine takes the one-round-trip form;
// above, the chain form (see combine_chain_kernel).  About twice the waves
// the GPU holds at once.
constexpr int64_t kCombineTablesMaxUnits = 16384;
// Large combines keep at most 12 workgroups per CU resident
// (resident_cap_lds; the plain combine's registers allow 20, the
// shared-expert form's 16): at T=8192, H=7168, k=8 179.9 against 181.6 us,
// with Zipf-skewed routing 172.0 against 176.7 us (same process,
// interleaved; 16 per CU 179.8 and 174.7, 10 per CU 183.0 and 175.3); the
// shared-expert form took 196-197 us with and without the cap.
constexpr int kCombineWgPerCu = 12;

hipError_t launch_combine(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                          const RankCPtrs &ry, const float *w, const void *shared, void *out,
                          int64_t capacity_rows, hipStream_t s) {
  const int64_t nseg = (c.hidden / 8 + kSegChunks - 1) / kSegChunks;
  const int64_t units = (int64_t)c.num_tokens * nseg;
  const int grid = row_grid(c, units);
  const int32_t El = c.num_experts / c.num_ranks;
  const uint16_t *sh = static_cast<const uint16_t *>(shared);
  uint16_t *o = static_cast<uint16_t *>(out);
  const size_t lds = resident_cap_lds(units, kCombineWgPerCu);
  if (units <= kCombineTablesMaxUnits) {
    if (shared)
      hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(kThreads), lds, s, topk_idx,
                         h.slot_of, h.rank_offsets, h.error_flag, w, c.num_tokens, c.hidden,
                         c.num_topk, c.num_experts, El, c.num_ranks, capacity_rows, ry, sh, o);
    else
      hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(kThreads), lds, s, topk_idx,
                         h.slot_of, h.rank_offsets, h.error_flag, w, c.num_tokens, c.hidden,
                         c.num_topk, c.num_experts, El, c.num_ranks, capacity_rows, ry, nullptr, o);
  } else {
    if (shared)
      hipLaunchKernelGGL(combine_chain_kernel<true>, dim3(grid), dim3(kThreads), lds, s, topk_idx,
                         h.slot_of, h.rank_offsets, h.error_flag, w, c.num_tokens, c.hidden,
                         c.num_topk, c.num_experts, El, capacity_rows, ry, sh, o);
    else
      hipLaunchKernelGGL(combine_chain_kernel<false>, dim3(grid), dim3(kThreads), lds, s, topk_idx,
                         h.slot_of, h.rank_offsets, h.error_flag, w, c.num_tokens, c.hidden,
                         c.num_topk, c.num_experts, El, capacity_rows, ry, nullptr, o);
  }
  return hipGetLastError();
}

hipError_t launch_combine_backward(const ep_config &c, const ep_layout_t &h,
                                   const int32_t *topk_idx, const void *grad_out, const float *w,
                                   const RankCPtrs &ry, const RankPtrs &rg, float *grad_w,
                                   int64_t capacity_rows, hipStream_t s) {
  // the path depends on T only, so results never depend on num_workgroups
  if (c.num_tokens < kBwdWgMaxTokens) {
    const int grid = c.num_workgroups > 0 ? c.num_workgroups : c.num_tokens;
    hipLaunchKernelGGL(combine_backward_wg_kernel, dim3(grid), dim3(kBwdThreads), 0, s, topk_idx,
                       h.slot_of, h.rank_offsets, h.error_flag,
                       static_cast<const uint16_t *>(grad_out), w, c.num_tokens, c.hidden,
                       c.num_topk, c.num_experts, c.num_experts / c.num_ranks, c.num_ranks,
                       capacity_rows, ry, rg, grad_w);
  } else {
    const hipError_t e =
        launch_combine_backward_rows(c, h, topk_idx, grad_out, w, rg, capacity_rows, s);
    if (e != hipSuccess || !grad_w) return e;
    hipLaunchKernelGGL(combine_backward_dots_kernel, dim3(row_grid(c, c.num_tokens)),
                       dim3(kThreads), 0, s, topk_idx,
                       h.slot_of, h.rank_offsets, h.error_flag,
                       static_cast<const uint16_t *>(grad_out), c.num_tokens, c.hidden,
                       c.num_topk, c.num_experts, c.num_experts / c.num_ranks, capacity_rows, ry,
                       grad_w);
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(const ep_config &c, const ep_layout_t &h, const int32_t *topk_idx,
                            const RankCPtrs &ry, void *out, int64_t capacity_rows, hipStream_t s) {
  const int64_t P = (int64_t)c.num_tokens * c.num_topk;
  const int grid = row_grid(c, P);
  hipLaunchKernelGGL(unpermute_kernel, dim3(grid), dim3(kThreads), 0, s, topk_idx, h.slot_of,
                     h.rank_offsets, h.error_flag, P, c.hidden, c.num_experts,
                     c.num_experts / c.num_ranks, capacity_rows, ry,
                     static_cast<uint16_t *>(out));
  return hipGetLastError();
}

}  // namespace ep
