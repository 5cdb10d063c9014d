// fp64 refine of the draw for the sequences the fast path could not certify.
//
// Recomputes the decisive row(s) from the logits in fp64, with y = x / T:
//   refine_lse:    chunk partials (max y, sum exp(y - max)) of p_n and q_n;
//   refine_chunks: log Z of each row from its partials, then per chunk the sums
//                  of w = max(0, p_n - q_n) (or p_K) and of p;
//   refine_select: one workgroup per queued sequence scans the chunk sums,
//                  rescans the chunk holding t = u * Z and writes the smallest
//                  token whose running sum exceeds t.
// If the residual mass is zero after rounding the draw falls back to p_n; if
// rounding leaves t at or past the last running sum it takes the last token
// with positive weight.  All three walk the queue with grid-stride loops, so
// their grids are sized on the host without knowing the queue length.  Kernel
// boundaries order the phases; no workgroup waits for another.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRun = 8;
constexpr int kRound = kBlock * kRun;
constexpr int kPer = 16;                 // elements per lane per strided round
constexpr int kStride = kBlock * kPer;   // 4096 elements per strided round

// Elements base + lane + 256 k (k < kPer) of a row, -inf past hi; all loads
// are issued before any is used.
template <int DT>
__device__ inline void load_round(const void* row, long base, long hi, float (&e)[kPer]) {
#pragma unroll
  for (int k = 0; k < kPer; ++k) e[k] = load_masked<DT>(row, base + threadIdx.x + static_cast<long>(k) * kBlock, hi);
}

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
    // lane-local (max, sum) over strided rounds, rescaled when the max grows
    float mx = -INFINITY;
    double sl = 0.0;
    for (long r0 = lo; r0 < hi; r0 += kStride) {
      float ev[kPer];
      load_round<DT>(row, r0, hi, ev);
      float m2 = mx;
#pragma unroll
      for (int k = 0; k < kPer; ++k) m2 = fmaxf(m2, ev[k]);
      if (m2 == -INFINITY) continue;
      if (m2 > mx) {
        sl = mx == -INFINITY ? 0.0 : sl * exp_f64(static_cast<double>(mx - m2) * p.inv_t);
        mx = m2;
      }
      const double ym = static_cast<double>(mx) * p.inv_t;
#pragma unroll
      for (int k = 0; k < kPer; ++k) sl += exp_f64(static_cast<double>(ev[k]) * p.inv_t - ym);
    }
    const float bm = block_max(mx, lf);
    const double M = static_cast<double>(bm) * p.inv_t;
    double S = (mx == -INFINITY) ? 0.0 : sl * exp_f64(static_cast<double>(mx - bm) * p.inv_t);
    S = block_sum(S, ld);
    if (threadIdx.x == 0) p.rpart[(e * 2 + which) * R4 + r] = make_double2(M, S);
  }
}

// log Z of row `which` of queue entry e from its R4 partials; call from one
// whole wave (lane r holds partial r), every lane gets the result.
__device__ inline double wave_logz(const Params& p, long e, int which) {
  const int lane = threadIdx.x % kWave;
  const double2 pr = lane < p.R4 ? p.rpart[(e * 2 + which) * p.R4 + lane] : make_double2(-INFINITY, 0.0);
  double M = pr.x;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, kWave));
  const double S = wave_sum(pr.x == -INFINITY ? 0.0 : pr.y * exp_f64(pr.x - M));
  return M + log(S);
}

template <int DT>
struct RefRow {
  const void* rp;
  const void* rq;  // null for a bonus draw
  double lzp, lzq, inv_t;
  __device__ double p_of(float x) const { return exp_f64(static_cast<double>(x) * inv_t - lzp); }
  // residual weight, or p itself for a bonus draw or the zero-mass fallback
  __device__ double w_of(float xp, float xq, bool use_p) const {
    const double pv = p_of(xp);
    if (!rq || use_p) return pv;
    return fmax(pv - exp_f64(static_cast<double>(xq) * inv_t - lzq), 0.0);
  }
};

template <int DT>
__device__ inline RefRow<DT> refine_row(const Params& p, long s, int n, double lzp, double lzq) {
  RefRow<DT> row;
  row.rp = decisive_row<DT>(p, s, n, 0);
  row.rq = n == p.K ? nullptr : decisive_row<DT>(p, s, n, 1);
  row.lzp = lzp;
  row.lzq = lzq;
  row.inv_t = p.inv_t;
  return row;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_refine_chunks(Params p) {
  const long count = static_cast<long>(*p.list_count);
  const int R4 = p.R4;
  __shared__ double ld[kWaves];
  __shared__ double s_lz[2];
  for (long item = blockIdx.x; item < count * R4; item += gridDim.x) {
    const long e = item / R4;
    const int r = static_cast<int>(item % R4);
    const long s = p.list[e];
    const int n = p.rec[s].n;
    const bool bonus = n == p.K;
    __syncthreads();  // s_lz of the previous item is no longer read
    if (threadIdx.x < kWave) {
      const double lzp = wave_logz(p, e, 0);
      const double lzq = bonus ? 0.0 : wave_logz(p, e, 1);
      if (threadIdx.x == 0) {
        s_lz[0] = lzp;
        s_lz[1] = lzq;
      }
    }
    __syncthreads();
    const RefRow<DT> row = refine_row<DT>(p, s, n, s_lz[0], s_lz[1]);
    const long lo = static_cast<long>(r) * p.ch4;
    const long hi = min(static_cast<long>(p.V), lo + p.ch4);
    double W = 0.0, P = 0.0;
    for (long r0 = lo; r0 < hi; r0 += kStride) {
      float ep[kPer], eq[kPer];
      load_round<DT>(row.rp, r0, hi, ep);
      if (!bonus) load_round<DT>(row.rq, r0, hi, eq);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const double pv = row.p_of(ep[k]);
        P += pv;
        W += bonus ? pv : fmax(pv - exp_f64(static_cast<double>(eq[k]) * p.inv_t - row.lzq), 0.0);
      }
    }
    W = block_sum(W, ld);
    P = block_sum(P, ld);
    if (threadIdx.x == 0) p.rsum[e * R4 + r] = make_double2(W, P);
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_refine_select(Params p) {
  const long count = static_cast<long>(*p.list_count);
  const int R4 = p.R4, K = p.K;
  __shared__ double ld[kWaves];
  __shared__ double s_lz[2], s_t, s_base;
  __shared__ int s_chunk, s_usep, s_j, s_jlast;
  for (long e = blockIdx.x; e < count; e += gridDim.x) {
    const long s = p.list[e];
    const int n = p.rec[s].n;
    const bool bonus = n == K;
    __syncthreads();  // shared scalars of the previous entry are no longer read
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const double lzp = wave_logz(p, e, 0);
      const double lzq = bonus ? 0.0 : wave_logz(p, e, 1);
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
        s_lz[0] = lzp;
        s_lz[1] = lzq;
        s_t = hit ? t : INFINITY;  // past the end: take the last positive token of chunk rc
        s_base = base;
        s_chunk = rc;
        s_usep = usep;
        s_j = 0x7fffffff;
        s_jlast = -1;
      }
    }
    __syncthreads();
    const RefRow<DT> row = refine_row<DT>(p, s, n, s_lz[0], s_lz[1]);
    const bool usep = s_usep;
    const long clo = static_cast<long>(s_chunk) * p.ch4;
    const long chi = min(static_cast<long>(p.V), clo + p.ch4);
    const double t = s_t;
    double base = s_base;
    for (long r0 = clo; r0 < chi; r0 += kRound) {
      const long v0 = r0 + static_cast<long>(threadIdx.x) * kRun;
      double wv[kRun];
      float ep[kRun], eq[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) {
        ep[k] = load_masked<DT>(row.rp, v0 + k, chi);
        eq[k] = row.rq ? load_masked<DT>(row.rq, v0 + k, chi) : -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < kRun; ++k) wv[k] = v0 + k < chi ? row.w_of(ep[k], eq[k], usep) : 0.0;
      double mine = 0.0;
#pragma unroll
      for (int k = 0; k < kRun; ++k) mine += wv[k];
      double total;
      double run = base + block_exclusive_scan(mine, ld, &total);
      long found = -1, lastpos = -1;
#pragma unroll
      for (int k = 0; k < kRun; ++k) {
        if (wv[k] > 0.0) lastpos = v0 + k;
        run += wv[k];
        if (found < 0 && wv[k] > 0.0 && run > t) found = v0 + k;
      }
      if (found >= 0) atomicMin(&s_j, static_cast<int>(found));
      if (lastpos >= 0) atomicMax(&s_jlast, static_cast<int>(lastpos));
      __syncthreads();
      if (s_j != 0x7fffffff) break;  // uniform: every lane reads the same LDS value
      base += total;
    }
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
  const dim3 g3(static_cast<unsigned>(p.B < 256 ? p.B : 256));
  if (dtype == 1) {
    hipLaunchKernelGGL((k_refine_lse<1>), g1, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_chunks<1>), g2, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_select<1>), g3, block, 0, st, p);
  } else {
    hipLaunchKernelGGL((k_refine_lse<0>), g1, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_chunks<0>), g2, block, 0, st, p);
    hipLaunchKernelGGL((k_refine_select<0>), g3, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sv
