// The left-to-right acceptance scan.
//
// Sampling mode (one workgroup per sequence): its waves first combine the
// sweep's partials into the normalisers of the 2K+1 rows of the sequence,
// each row's partials folded in one pass per lane.  Lane k of wave 0 evaluates draft
// k's test u_k < min(1, p_k(x_k) / q_k(x_k)) as a log2-domain ratio in fp64,
// and a ballot turns the K answers into n, the index of the first rejection
// (K if none).  Scanning "in parallel" is exact: the outcome is the first
// failing test, which is what stopping at the first rejection yields.
// Greedy mode (one wave per sequence): lane k compares x_k with the arg-max
// of target row k.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRowsMax = 2 * SPECV_MAX_K + 1;

// log2 sum 2^(x c) of one row from its sweep partials (R whole, s scaled):
// one pass per lane with exact power-of-two rescales, then a wave merge.
// Call from a whole wave; every lane gets the result.
__device__ inline double wave_row_log2z(const float2* pr, int np) {
  const int lane = threadIdx.x % kWave;
  float ml = -INFINITY;
  double sl = 0.0;
  for (int j = lane; j < np; j += kWave) {
    const float2 q = pr[j];
    if (q.x == -INFINITY) continue;
    if (q.x > ml) {
      sl = ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - q.x, -1000.f)));
      ml = q.x;
    }
    sl += ldexp(static_cast<double>(q.y), static_cast<int>(fmaxf(q.x - ml, -1000.f)));
  }
  const float M = wave_max(ml);
  const double S = wave_sum(ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - M, -1000.f))));
  return static_cast<double>(M) + log2(S);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_accept_scan(Params p) {
  const long s = blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, nrows = 2 * K + 1, np = p.nch1 * kWaves;
  __shared__ float sW[kRowsMax];   // whole part of each row's log2 normaliser
  __shared__ double sF[kRowsMax];  // fractional part, in [-1/2, 1/2]
  for (int i = w; i < nrows; i += kWaves) {
    const double lz2 = wave_row_log2z(p.part + (s * nrows + i) * np, np);
    if (lane == 0) {
      const double whole = rint(lz2);
      sW[i] = static_cast<float>(whole);
      sF[i] = lz2 - whole;
      if (p.out_logz) p.out_logz[s * nrows + i] = static_cast<float>(lz2 * M_LN2);
    }
  }
  __syncthreads();
  if (w != 0) return;

  bool accept = false, valid = true;
  int xk = 0;
  if (lane < K) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
    if (valid) {
      const double xp = Elt<DT>::at(row_ptr<DT>(p.lp, s * (K + 1) + lane, p.V), xk);
      const double xq = Elt<DT>::at(row_ptr<DT>(p.lq, s * K + lane, p.V), xk);
      const double c = p.c;
      // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
      const double lr = ((xp * c - sW[lane]) - sF[lane]) - ((xq * c - sW[K + 1 + lane]) - sF[K + 1 + lane]);
      const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
      accept = static_cast<double>(p.ua[s * K + lane]) < thr;
    }
  }
  const uint64_t lim = (K >= 64) ? ~0ull : ((1ull << K) - 1ull);
  const uint64_t rejected = ~static_cast<uint64_t>(__ballot(accept)) & lim;
  const int n = rejected ? __ffsll(static_cast<unsigned long long>(rejected)) - 1 : K;
  const bool bad = __shfl(valid ? 1 : 0, n < K ? n : 0, kWave) == 0 && n < K;

  if (lane <= K) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : -1;  // slot n is filled by the draw
  if (lane == 0) {
    p.out_n[s] = n;
    SeqRec r;
    r.n = n;
    r.flags = bad ? SPECV_FLAG_BAD_DRAFT : 0;
    r.mp = sW[n];
    r.lp2 = sF[n];
    r.mq = n < K ? sW[K + 1 + n] : 0.f;
    r.lq2 = n < K ? sF[K + 1 + n] : 0.0;
    p.rec[s] = r;
  }
}

__global__ __launch_bounds__(kBlock) void k_greedy_scan(Params p) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long s = static_cast<long>(blockIdx.x) * kWaves + w;
  if (s >= p.B) return;  // no workgroup barrier below
  const int K = p.K;
  int a = 0;
  if (lane <= K) {
    const int np = p.nch1 * kWaves;
    const float2* pr = p.part + (s * (K + 1) + lane) * np;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < np; ++c) argmax_merge(bv, bi, pr[c].x, __float_as_int(pr[c].y));
    a = bi;
  }
  int xk = 0;
  bool match = false, valid = true;
  if (lane < K) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
    match = xk == a;
  }
  const uint64_t lim = (1ull << K) - 1ull;
  const uint64_t miss = ~static_cast<uint64_t>(__ballot(match)) & lim;
  const int n = miss ? __ffsll(static_cast<unsigned long long>(miss)) - 1 : K;
  const int an = __shfl(a, n, kWave);
  const bool bad = n < K && __shfl(valid ? 1 : 0, n, kWave) == 0;
  if (lane <= K) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : (lane == n ? an : -1);
  if (lane == 0) {
    p.out_n[s] = n;
    if (p.out_flags) p.out_flags[s] = bad ? SPECV_FLAG_BAD_DRAFT : 0;
  }
}

}  // namespace

hipError_t launch_accept_scan(const Params& p, int dtype, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.B)), block(kBlock);
  if (dtype == 1) hipLaunchKernelGGL((k_accept_scan<1>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_accept_scan<0>), grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_greedy_scan(const Params& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((p.B + kWaves - 1) / kWaves)), block(kBlock);
  hipLaunchKernelGGL(k_greedy_scan, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
