// The fp64 draw's weights and per-chunk sums (the method is described in
// k_exact.hip), shared by the fp64 draw's kernels and by k_verify, whose
// otherwise idle workgroups compute the chunk sums of every sequence of a
// small batch while the fast draw runs.
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kXWaves = kXBlock / kWave;
constexpr int kXGroupsMax = kVerifyBlock / kXBlock;  // groups of kXBlock threads in the largest workgroup
constexpr int kRun = 8;                          // elements per lane per rescan round (a whole bf16 vector)
constexpr int kRound = kXBlock * kRun;           // 1024 elements per round (the smallest chunk)
constexpr double kKappa = 1e-4;                  // near-flip window, relative to Q

// fp64 weight exp(x / T - L'), L' the natural-log reference.
struct ExactWeight {
  double inv_t, ap, aq;
  ExpConsts ec;
  __device__ double P(float x) const { return exp_f64(static_cast<double>(x) * inv_t - ap, ec); }
  __device__ double Q(float x) const { return exp_f64(static_cast<double>(x) * inv_t - aq, ec); }
};

__device__ inline ExactWeight exact_weight(const Params& p, const SeqRec& rec) {
  ExactWeight e;
  e.inv_t = p.inv_t;
  e.ec = p.ec;
  e.ap = rec.lzp * M_LN2;
  e.aq = rec.lzq * M_LN2;
  return e;
}

template <int DT>
struct Rows {
  const void* rp;
  const void* rq;  // null for a bonus draw
};

template <int DT>
__device__ inline Rows<DT> decisive_rows(const Params& p, long s, const SeqRec& rec) {
  Rows<DT> r;
  r.rp = row_ptr<DT>(p.lp, s * (p.K + 1) + rec.n, p.V);
  r.rq = rec.n == rec.kb ? nullptr : row_ptr<DT>(p.lq, s * p.K + rec.n, p.V);
  return r;
}

// ------------------------------------------------------------ chunk sums --
// Chunk r of the decisive row(s) -> out[0..4] = sum P, sum Q, A, G, H (only
// out[0] for a bonus draw), computed by one group of kXBlock threads: a
// whole workgroup of the fp64 kernels, or group threadIdx.x / kXBlock of a
// larger workgroup whose groups all call this together (it holds
// workgroup-wide barriers).  A group whose r lies past the row's last chunk
// loads nothing and writes nothing (out may then be null).  Loads go out
// branch-free, U units per lane, and are widened one unit at a time; the
// five sums are reduced over the group together.  Element mapping and
// reduction order depend only on the thread's index within its group, so
// every caller gets the same sums bit for bit.
template <int DT, bool VEC>
__device__ inline void exact_chunk_sums(const Params& p, const Rows<DT>& rows, const ExactWeight& wt, bool bonus,
                                        int r, double* out) {
  const int tid = static_cast<int>(threadIdx.x % kXBlock), grp = static_cast<int>(threadIdx.x / kXBlock);
  const long lo = static_cast<long>(r) * p.ch3;
  const long hi = min(static_cast<long>(p.V), lo + p.ch3);
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  constexpr int U = 8 / PV;  // eight elements per lane per iteration
  const long ulo = lo / PV, uhi = hi / PV;  // VEC: lo and hi are multiples of PV
  double acc[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (long r0 = ulo; r0 < uhi; r0 += static_cast<long>(kXBlock) * U) {
    uint4 rp[VEC ? U : 1], rq[VEC ? U : 1];
    float sp_[VEC ? 1 : U], sq_[VEC ? 1 : U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const long u = r0 + tid + static_cast<long>(i) * kXBlock;
      if constexpr (VEC) {
        const long uu = u < uhi ? u : uhi - 1;
        rp[i] = load16(rows.rp, uu);
        if (!bonus) rq[i] = load16(rows.rq, uu);
      } else {
        sp_[i] = load_masked<DT>(rows.rp, u, uhi);
        sq_[i] = bonus ? -INFINITY : load_masked<DT>(rows.rq, u, uhi);
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float ep[PV], eq[PV];
      if constexpr (VEC) {
        Elt<DT>::unpack(rp[i], ep);
        if (!bonus) Elt<DT>::unpack(rq[i], eq);
        if (bonus || r0 + tid + static_cast<long>(i) * kXBlock >= uhi) {
#pragma unroll
          for (int k = 0; k < PV; ++k) eq[k] = -INFINITY;
        }
        if (r0 + tid + static_cast<long>(i) * kXBlock >= uhi) {
#pragma unroll
          for (int k = 0; k < PV; ++k) ep[k] = -INFINITY;
        }
      } else {
        ep[0] = sp_[i];
        eq[0] = sq_[i];
      }
      double sp = 0.0, sq = 0.0, a = 0.0, g = 0.0, h = 0.0;
#pragma unroll
      for (int k = 0; k < PV; ++k) {
        const double P = wt.P(ep[k]);
        const double Q = wt.Q(eq[k]);  // 0 for -inf
        const double d = P - Q;
        sp += P;
        sq += Q;
        a += d > 0.0 ? d : 0.0;
        g += d > 0.0 ? Q : 0.0;
        h += (d <= kKappa * Q && -d <= kKappa * Q) ? Q : 0.0;
      }
      acc[0] += sp;
      acc[1] += sq;
      acc[2] += a;
      acc[3] += g;
      acc[4] += h;
    }
  }
  __shared__ double lds[kXGroupsMax][kXWaves][5];
  const int lane = tid % kWave, w = tid / kWave;
#pragma unroll
  for (int k = 0; k < 5; ++k) acc[k] = wave_sum(acc[k]);
  __syncthreads();  // the previous item's reads of lds are done
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 5; ++k) lds[grp][w][k] = acc[k];
  }
  __syncthreads();
  if (tid < 5 && out) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kXWaves; ++i) t += lds[grp][i][tid];
    if (!bonus || tid == 0) out[tid] = t;
  }
}

}  // namespace sv
