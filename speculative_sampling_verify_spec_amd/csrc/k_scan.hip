// The left-to-right acceptance scan.
//
// Sampling mode (one workgroup per sequence): its waves first combine the
// sweep's partials into the normalisers of the 2K+1 rows of the sequence,
// each row's partials folded in one pass per lane.  Lane k of wave 0 evaluates draft
// k's test u_k < min(1, p_k(x_k) / q_k(x_k)) as a log2-domain ratio in fp64,
// and a ballot turns the K answers into n, the index of the first rejection
// (K if none).  Scanning "in parallel" is exact: the outcome is the first
// failing test, which is what stopping at the first rejection yields.
// Greedy mode (one workgroup per sequence): the waves reduce the target rows'
// arg-max partials, then lane k compares x_k with the arg-max of row k.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRowsMax = 2 * SPECV_MAX_K + 1;

constexpr int kScanBlock = 1024;                      // acceptance scan: 16 waves per sequence
constexpr int kScanWaves = kScanBlock / kWave;
constexpr int kRowsPerWave = (kRowsMax + kScanWaves - 1) / kScanWaves;  // 5 rows per wave at most

// Fold one lane's (R, s) sweep partial into its running pair (ml, sl):
// exact power-of-two rescales, fp64 sums.
__device__ inline void fold_partial(float& ml, double& sl, float2 q) {
  if (q.x == -INFINITY) return;
  if (q.x > ml) {
    sl = ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - q.x, -1000.f)));
    ml = q.x;
  }
  sl += ldexp(static_cast<double>(q.y), static_cast<int>(fmaxf(q.x - ml, -1000.f)));
}

// log2 sum 2^(x c) of a row from the lanes' running pairs (whole wave).  The
// exponent of the sum is exact (frexp); its mantissa's log2 comes from
// v_log_f32, good to ~1e-7 absolute, which is all the uses of the normaliser
// need (the acceptance test's near-tie window is 1e-5 and the draw normalises
// by its own sums).
__device__ inline double wave_log2z(float ml, double sl) {
  const float M = wave_max(ml);
  const double S = wave_sum(ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - M, -1000.f))));
  int e;
  const double m = frexp(S, &e);  // S = m 2^e, m in [1/2, 1)
  return static_cast<double>(M) + e + __builtin_amdgcn_logf(static_cast<float>(m));
}

template <int DT>
__global__ __launch_bounds__(kScanBlock) void k_accept_scan(Params p) {
  const long s = p.seq0 + blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, nrows = 2 * K + 1, np = p.nch1 * kWaves;
  __shared__ double sL[kRowsMax];  // log2 sum_v 2^(x_v c) of each row
  if (blockIdx.x == 0 && threadIdx.x == 0) p.qcount[0] = 0u;  // the exact-draw queue

  // wave 0 starts the draft-token gathers at once: they do not need the normalisers
  int xk = 0;
  bool valid = true;
  float xp = 0.f, xq = 0.f;
  if (w == 0 && lane < K) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
    const int xs = valid ? xk : 0;
    xp = Elt<DT>::at(row_ptr<DT>(p.lp, s * (K + 1) + lane, p.V), xs);
    xq = Elt<DT>::at(row_ptr<DT>(p.lq, s * K + lane, p.V), xs);
  }

  // each wave folds its rows; all partial loads of the first 64 per row go out together
  float ml[kRowsPerWave];
  double sl[kRowsPerWave];
  {
    float2 q[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int i = w + r * kScanWaves;
      q[r] = (i < nrows && lane < np) ? p.part[(s * nrows + i) * np + lane] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      ml[r] = -INFINITY;
      sl[r] = 0.0;
      fold_partial(ml[r], sl[r], q[r]);
    }
  }
  for (int j = lane + kWave; j < np; j += kWave)  // long rows: the rest of the partials
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int i = w + r * kScanWaves;
      if (i < nrows) fold_partial(ml[r], sl[r], p.part[(s * nrows + i) * np + j]);
    }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = w + r * kScanWaves;
    if (i >= nrows) break;  // uniform over the wave
    const double lz2 = wave_log2z(ml[r], sl[r]);
    if (lane == 0) {
      sL[i] = lz2;
      if (p.out_logz) p.out_logz[s * nrows + i] = static_cast<float>(lz2 * M_LN2);
    }
  }
  __syncthreads();
  if (w != 0) return;

  bool accept = false;
  if (lane < K && valid) {
    const double c = p.c;
    // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
    const double lr = (static_cast<double>(xp) * c - sL[lane]) - (static_cast<double>(xq) * c - sL[K + 1 + lane]);
    const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
    accept = static_cast<double>(p.ua[s * K + lane]) < thr;
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
    r.lzp = sL[n];
    r.lzq = n < K ? sL[K + 1 + n] : 0.0;
    p.rec[s] = r;
  }
}

// Greedy: one workgroup per sequence; wave w finds the arg-max of target rows
// w, w + 4, ...; then wave 0 compares with the drafts.
__global__ __launch_bounds__(kBlock) void k_greedy_scan(Params p) {
  const long s = p.seq0 + blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, np = p.nch1 * kWaves;
  __shared__ int sA[SPECV_MAX_K + 1];
  int xk = 0;
  bool valid = true;
  if (w == 0 && lane < K) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
  }
  for (int i = w; i <= K; i += kWaves) {
    const float2* pr = p.part + (s * (K + 1) + i) * np;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < np; j += kWave) argmax_merge(bv, bi, pr[j].x, __float_as_int(pr[j].y));
    wave_argmax(bv, bi);
    if (lane == 0) sA[i] = bi;
  }
  __syncthreads();
  if (w != 0) return;
  const int a = lane <= K ? sA[lane] : 0;
  const bool match = lane < K && xk == a;
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
  const dim3 grid(static_cast<unsigned>(p.nseq)), block(kScanBlock);
  if (dtype == 1) hipLaunchKernelGGL((k_accept_scan<1>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_accept_scan<0>), grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_greedy_scan(const Params& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.nseq)), block(kBlock);
  hipLaunchKernelGGL(k_greedy_scan, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
