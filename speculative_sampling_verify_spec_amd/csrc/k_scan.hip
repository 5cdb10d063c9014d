// The left-to-right acceptance scan, one 64-lane wave per sequence.
//
// Sampling mode: the wave first combines the sweep's chunk pairs into the
// normalisers of the 2K+1 rows of its sequence.  Lane k then evaluates draft
// k's test u_k < min(1, p_k(x_k) / q_k(x_k)) as a log2-domain ratio in fp64,
// and a ballot turns the K answers into n, the index of the first rejection
// (K if none).  Scanning "in parallel" is exact: the outcome is the first
// failing test, which is what stopping at the first rejection yields.
// Greedy mode: lane k compares x_k with the arg-max of target row k.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRowsMax = 2 * SPECV_MAX_K + 1;

template <int DT>
__global__ __launch_bounds__(kBlock) void k_accept_scan(Params p) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long s = static_cast<long>(blockIdx.x) * kWaves + w;
  const bool active = s < p.B;
  const int K = p.K, nrows = 2 * K + 1;
  __shared__ float sM[kWaves][kRowsMax];
  __shared__ double sL[kWaves][kRowsMax];

  if (active) {
    for (int i = lane; i < nrows; i += kWave) {
      const float2* pr = p.part + (s * nrows + i) * p.nch1;
      float M = -INFINITY;
      for (int c = 0; c < p.nch1; ++c) M = fmaxf(M, pr[c].x);
      double S = 0.0;
      for (int c = 0; c < p.nch1; ++c)
        if (pr[c].x != -INFINITY) S += static_cast<double>(pr[c].y) * exp2(static_cast<double>(pr[c].x - M) * p.c);
      const double L2 = log2(S);  // log2 sum_v 2^((x_v - M) c)
      sM[w][i] = M;
      sL[w][i] = L2;
      if (p.out_logz) p.out_logz[s * nrows + i] = static_cast<float>(static_cast<double>(M) * p.inv_t + L2 * M_LN2);
    }
  }
  __syncthreads();
  if (!active) return;

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
      const double lr = ((xp - sM[w][lane]) * c - sL[w][lane]) - ((xq - sM[w][K + 1 + lane]) * c - sL[w][K + 1 + lane]);
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
    r.mp = sM[w][n];
    r.lp2 = sL[w][n];
    r.mq = n < K ? sM[w][K + 1 + n] : 0.f;
    r.lq2 = n < K ? sL[w][K + 1 + n] : 0.0;
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
    const float2* pr = p.part + (s * (K + 1) + lane) * p.nch1;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < p.nch1; ++c) argmax_merge(bv, bi, pr[c].x, __float_as_int(pr[c].y));
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
  const dim3 grid(static_cast<unsigned>((p.B + kWaves - 1) / kWaves)), block(kBlock);
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
