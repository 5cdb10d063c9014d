// Row sweeps: the one pass over every logit that the verify step needs.
//
// Sampling mode: each workgroup reduces one chunk of one row to a pair
// (m, s) with m the chunk's largest logit and s = sum 2^((x - m) * c),
// c = log2(e) / T.  The normalisers log Z = m/T + ln(s) of the target and
// draft distributions p and q are combined from these pairs afterwards.
// Greedy mode: each workgroup reduces a chunk to (largest logit, lowest
// index holding it).
//
// Memory: rows are read once, 16 bytes per lane per load when every row is
// 16-byte aligned (4 fp32 or 8 bf16 values), coalesced across the wave; a
// lane issues all its loads before it computes.  HBM-bound by design: about
// six VALU operations and one v_exp_f32 per element against 2 or 4 bytes.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int kVecIters = 4;      // 16-byte loads per lane per chunk
constexpr int kScalarIters = 16;  // scalar loads per lane per chunk

// Zero the per-call arrival counters that the draw and refine kernels use.
// Runs in the first kernel of a call, so stream order makes the zeros visible.
__device__ inline void zero_counters(const Params& p) {
  const long z = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x;
  if (z < p.B) {
    p.cnt_draw[z] = 0u;
    p.cnt_ref[z] = 0u;
  }
  if (z == 0) p.list_count[0] = 0u;
}

// Row `row` of the sampling sweep: K+1 target rows then K draft rows per sequence.
template <int DT>
__device__ inline const void* sweep_row(const Params& p, long row) {
  const int per_seq = 2 * p.K + 1;
  const long s = row / per_seq;
  const int j = static_cast<int>(row % per_seq);
  return j <= p.K ? row_ptr<DT>(p.lp, s * (p.K + 1) + j, p.V)
                  : row_ptr<DT>(p.lq, s * p.K + (j - p.K - 1), p.V);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_sweep_lse(Params p) {
  zero_counters(p);
  const long row = blockIdx.x / p.nch1;
  const int chunk = blockIdx.x % p.nch1;
  const void* r = sweep_row<DT>(p, row);
  const float c = p.c;
  float m = -INFINITY, s = 0.f;

  if constexpr (VEC) {
    constexpr int PV = Elt<DT>::kPerVec;
    const long nvec = p.V / PV;
    const long v0 = static_cast<long>(chunk) * (kBlock * kVecIters) + threadIdx.x;
    float e[kVecIters][PV];
#pragma unroll
    for (int i = 0; i < kVecIters; ++i) {
      const long vi = v0 + static_cast<long>(i) * kBlock;
      if (vi < nvec) {
        Elt<DT>::unpack(load16(r, vi), e[i]);
      } else {
#pragma unroll
        for (int k = 0; k < PV; ++k) e[i][k] = -INFINITY;
      }
    }
#pragma unroll
    for (int i = 0; i < kVecIters; ++i)
#pragma unroll
      for (int k = 0; k < PV; ++k) m = fmaxf(m, e[i][k]);
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kVecIters; ++i) {
        float t[PV];
#pragma unroll
        for (int k = 0; k < PV; ++k) t[k] = ex2((e[i][k] - m) * c);
        // pairwise within the vector, then one add into the running sum
#pragma unroll
        for (int w = PV / 2; w > 0; w >>= 1)
#pragma unroll
          for (int k = 0; k < w; ++k) t[k] += t[k + w];
        s += t[0];
      }
    }
  } else {
    const long e0 = static_cast<long>(chunk) * (kBlock * kScalarIters) + threadIdx.x;
    float e[kScalarIters];
#pragma unroll
    for (int i = 0; i < kScalarIters; ++i) {
      const long idx = e0 + static_cast<long>(i) * kBlock;
      e[i] = idx < p.V ? Elt<DT>::at(r, idx) : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kScalarIters; ++i) m = fmaxf(m, e[i]);
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kScalarIters; i += 4)
        s += (ex2((e[i] - m) * c) + ex2((e[i + 1] - m) * c)) + (ex2((e[i + 2] - m) * c) + ex2((e[i + 3] - m) * c));
    }
  }

  wave_lse(m, s, c);
  __shared__ float lm[kWaves], ls[kWaves];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (lane == 0) { lm[w] = m; ls[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = lm[0], S = ls[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) lse_merge(M, S, lm[i], ls[i], c);
    p.part[row * p.nch1 + chunk] = make_float2(M, S);
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_sweep_argmax(Params p) {
  const long row = blockIdx.x / p.nch1;  // target rows only: row = s * (K+1) + k
  const int chunk = blockIdx.x % p.nch1;
  const void* r = row_ptr<DT>(p.lp, row, p.V);
  float bv = -INFINITY;
  int bi = 0x7fffffff;

  if constexpr (VEC) {
    constexpr int PV = Elt<DT>::kPerVec;
    const long nvec = p.V / PV;
    const long v0 = static_cast<long>(chunk) * (kBlock * kVecIters) + threadIdx.x;
    uint4 raw[kVecIters];
#pragma unroll
    for (int i = 0; i < kVecIters; ++i) {
      const long vi = v0 + static_cast<long>(i) * kBlock;
      if (vi < nvec) raw[i] = load16(r, vi);
    }
    // a lane visits its elements in increasing index order, so a strict
    // comparison keeps the lowest index among equal values
#pragma unroll
    for (int i = 0; i < kVecIters; ++i) {
      const long vi = v0 + static_cast<long>(i) * kBlock;
      if (vi < nvec) {
        float e[PV];
        Elt<DT>::unpack(raw[i], e);
#pragma unroll
        for (int k = 0; k < PV; ++k) argmax_merge(bv, bi, e[k], static_cast<int>(vi * PV + k));
      }
    }
  } else {
    const long e0 = static_cast<long>(chunk) * (kBlock * kScalarIters) + threadIdx.x;
#pragma unroll
    for (int i = 0; i < kScalarIters; ++i) {
      const long idx = e0 + static_cast<long>(i) * kBlock;
      if (idx < p.V) argmax_merge(bv, bi, Elt<DT>::at(r, idx), static_cast<int>(idx));
    }
  }

  wave_argmax(bv, bi);
  __shared__ float lv[kWaves];
  __shared__ int li[kWaves];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (lane == 0) { lv[w] = bv; li[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float V0 = lv[0];
    int I0 = li[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) argmax_merge(V0, I0, lv[i], li[i]);
    p.part[row * p.nch1 + chunk] = make_float2(V0, __int_as_float(I0));
  }
}

}  // namespace

hipError_t launch_sweep_lse(const Params& p, int dtype, hipStream_t st) {
  const long rows = static_cast<long>(p.B) * (2 * p.K + 1);
  const dim3 grid(static_cast<unsigned>(rows * p.nch1)), block(kBlock);
  if (dtype == 1) {
    if (p.vec) hipLaunchKernelGGL((k_sweep_lse<1, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_sweep_lse<1, false>), grid, block, 0, st, p);
  } else {
    if (p.vec) hipLaunchKernelGGL((k_sweep_lse<0, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_sweep_lse<0, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_sweep_argmax(const Params& p, int dtype, hipStream_t st) {
  const long rows = static_cast<long>(p.B) * (p.K + 1);
  const dim3 grid(static_cast<unsigned>(rows * p.nch1)), block(kBlock);
  if (dtype == 1) {
    if (p.vec) hipLaunchKernelGGL((k_sweep_argmax<1, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_sweep_argmax<1, false>), grid, block, 0, st, p);
  } else {
    if (p.vec) hipLaunchKernelGGL((k_sweep_argmax<0, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_sweep_argmax<0, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sv
