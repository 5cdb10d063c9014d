// fp64 refine of the draw for the sequences the fast path could not certify.
//
// Recomputes the decisive row(s) from the logits in fp64, with y = x / T:
//   refine_lse:  chunk partials (max y, sum exp(y - max)) of p_n and q_n;
//   refine_draw: log Z from the partials, w = max(0, p_n - q_n) (or p_K) per
//                chunk, chunk sums; the last workgroup of a sequence scans the
//                chunk sums, rescans the chunk holding t = u * Z and writes the
//                smallest token whose running sum exceeds t.
// If the residual mass is zero after rounding the draw falls back to p_n; if
// rounding leaves t at or past the last running sum it takes the last token
// with positive weight.  Both kernels walk the queue with a grid-stride loop,
// so their grids are sized on the host without knowing the queue length.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

template <int DT>
__device__ inline const void* decisive_row(const Params& p, long s, int n, int which) {
  return which == 0 ? row_ptr<DT>(p.lp, s * (p.K + 1) + n, p.V) : row_ptr<DT>(p.lq, s * p.K + n, p.V);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_refine_lse(Params p) {
  const long count = static_cast<long>(*p.list_count);
  const int R4 = p.R4;
  __shared__ double ld[kWaves];
  __shared__ float lf[kWaves];
  for (long item = blockIdx.x; item < count * R4 * 2; item += gridDim.x) {
    const long e = item / (2 * R4);
    const int which = static_cast<int>((item / R4) % 2);
    const int r = static_cast<int>(item % R4);
    const long s = p.list[e];
    const int n = p.rec[s].n;
    if (which == 1 && n == p.K) continue;  // bonus draw: no draft row (uniform over the workgroup)
    const void* row = decisive_row<DT>(p, s, n, which);
    const long lo = static_cast<long>(r) * p.ch4;
    const long hi = min(static_cast<long>(p.V), lo + p.ch4);
    float mx = -INFINITY;
    for (long v = lo + threadIdx.x; v < hi; v += kBlock) mx = fmaxf(mx, Elt<DT>::at(row, v));
    mx = block_max(mx, lf);
    const double M = static_cast<double>(mx) * p.inv_t;
    double S = 0.0;
    if (mx != -INFINITY)
      for (long v = lo + threadIdx.x; v < hi; v += kBlock) S += exp(static_cast<double>(Elt<DT>::at(row, v)) * p.inv_t - M);
    S = block_sum(S, ld);
    if (threadIdx.x == 0) p.rpart[(e * 2 + which) * R4 + r] = make_double2(M, S);
  }
}

// log Z of one row from its R4 chunk partials.
__device__ inline double combine_logz(const double2* part, int R4) {
  double M = -INFINITY;
  for (int r = 0; r < R4; ++r) M = fmax(M, part[r].x);
  double S = 0.0;
  for (int r = 0; r < R4; ++r)
    if (part[r].x != -INFINITY) S += part[r].y * exp(part[r].x - M);
  return M + log(S);
}

template <int DT>
struct RefRow {
  const void* rp;
  const void* rq;  // null for a bonus draw
  double lzp, lzq, inv_t;
  __device__ double p(long v) const { return exp(static_cast<double>(Elt<DT>::at(rp, v)) * inv_t - lzp); }
  // residual weight, or p itself for a bonus draw or the zero-mass fallback
  __device__ double w(long v, bool use_p) const {
    const double pv = p(v);
    if (!rq || use_p) return pv;
    return fmax(pv - exp(static_cast<double>(Elt<DT>::at(rq, v)) * inv_t - lzq), 0.0);
  }
};

template <int DT>
__global__ __launch_bounds__(kBlock) void k_refine_draw(Params p) {
  const long count = static_cast<long>(*p.list_count);
  const int R4 = p.R4, K = p.K;
  __shared__ double ld[kWaves];
  __shared__ double s_lzp, s_lzq, s_t, s_base;
  __shared__ int s_last, s_chunk, s_usep, s_j, s_jlast;
  for (long item = blockIdx.x; item < count * R4; item += gridDim.x) {
    const long e = item / R4;
    const int r = static_cast<int>(item % R4);
    const long s = p.list[e];
    const int n = p.rec[s].n;
    const bool bonus = n == K;
    __syncthreads();  // shared scalars of the previous item are no longer read
    if (threadIdx.x == 0) {
      s_lzp = combine_logz(p.rpart + (e * 2 + 0) * R4, R4);
      s_lzq = bonus ? 0.0 : combine_logz(p.rpart + (e * 2 + 1) * R4, R4);
    }
    __syncthreads();
    RefRow<DT> row;
    row.rp = decisive_row<DT>(p, s, n, 0);
    row.rq = bonus ? nullptr : decisive_row<DT>(p, s, n, 1);
    row.lzp = s_lzp;
    row.lzq = s_lzq;
    row.inv_t = p.inv_t;

    // chunk sums of the residual and of p (p is needed only for the zero-mass fallback)
    const long lo = static_cast<long>(r) * p.ch4;
    const long hi = min(static_cast<long>(p.V), lo + p.ch4);
    double W = 0.0, P = 0.0;
    for (long v = lo + threadIdx.x; v < hi; v += kBlock) {
      const double pv = row.p(v);
      P += pv;
      W += bonus ? pv : fmax(pv - exp(static_cast<double>(Elt<DT>::at(row.rq, v)) * p.inv_t - row.lzq), 0.0);
    }
    W = block_sum(W, ld);
    P = block_sum(P, ld);
    if (threadIdx.x == 0) {
      p.rsum[e * R4 + r] = make_double2(W, P);
      __threadfence();
      s_last = atomicAdd(&p.cnt_ref[e], 1u) == static_cast<uint32_t>(R4 - 1);
    }
    __syncthreads();
    if (!s_last) continue;
    __threadfence();

    // ---- finalise: total, chunk holding t (or the last positive chunk)
    const int lane = threadIdx.x % kWave;
    if (threadIdx.x < kWave) {
      const double2 cs = lane < R4 ? p.rsum[e * R4 + lane] : make_double2(0.0, 0.0);
      const double zw = wave_sum(cs.x);
      const int usep = !(zw > 0.0) && !bonus;  // zero residual mass: draw from p_n
      const double v = usep ? cs.y : cs.x;
      const double inc = wave_inclusive_scan(v);
      double excl = __shfl_up(inc, 1, kWave);
      if (lane == 0) excl = 0.0;
      const double z = __shfl(inc, kWave - 1, kWave);
      const double t = static_cast<double>(p.ur[s]) * z;
      const uint64_t hit = __ballot(lane < R4 && inc > t);
      const uint64_t pos = __ballot(lane < R4 && v > 0.0);
      int rc;
      if (hit) rc = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      else rc = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;  // last chunk with mass
      const double base = __shfl(excl, rc, kWave);
      if (lane == 0) {
        s_t = hit ? t : INFINITY;  // past the end: take the last positive token of chunk rc
        s_base = base;
        s_chunk = rc;
        s_usep = usep;
      }
    }
    if (threadIdx.x == 0) {
      s_j = 0x7fffffff;
      s_jlast = -1;
    }
    __syncthreads();

    // ---- rescan chunk s_chunk in fp64, lane-contiguous runs
    const bool usep = s_usep;
    const long clo = static_cast<long>(s_chunk) * p.ch4;
    const long chi = min(static_cast<long>(p.V), clo + p.ch4);
    const int ept = p.ch4 / kBlock;
    const long mylo = min(chi, clo + static_cast<long>(threadIdx.x) * ept);
    const long myhi = min(chi, mylo + ept);
    double mine = 0.0;
    for (long v = mylo; v < myhi; ++v) mine += row.w(v, usep);
    double total;
    double run = s_base + block_exclusive_scan(mine, ld, &total);
    const double t = s_t;
    long found = -1, lastpos = -1;
    for (long v = mylo; v < myhi; ++v) {
      const double wv = row.w(v, usep);
      if (wv > 0.0) lastpos = v;
      run += wv;
      if (found < 0 && wv > 0.0 && run > t) found = v;
    }
    if (found >= 0) atomicMin(&s_j, static_cast<int>(found));
    if (lastpos >= 0) atomicMax(&s_jlast, static_cast<int>(lastpos));
    __syncthreads();
    if (threadIdx.x == 0) {
      const int j = s_j != 0x7fffffff ? s_j : s_jlast;
      p.out_tokens[s * (K + 1) + n] = j;
      if (p.out_flags) p.out_flags[s] |= SPECV_FLAG_REFINED | (usep ? SPECV_FLAG_ZW_ZERO : 0);
    }
  }
}

}  // namespace

hipError_t launch_refine(const Params& p, int dtype, hipStream_t st) {
  const dim3 block(kBlock);
  const dim3 g1(static_cast<unsigned>(p.refine_grid * 2)), g2(static_cast<unsigned>(p.refine_grid));
  if (dtype == 1) {
    hipLaunchKernelGGL((k_refine_lse<1>), g1, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_draw<1>), g2, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((k_refine_lse<0>), g1, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_draw<0>), g2, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sv
