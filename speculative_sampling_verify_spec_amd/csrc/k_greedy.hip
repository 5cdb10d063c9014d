// Greedy acceptance (T = 0), one workgroup per sequence: the waves reduce the
// target rows' arg-max partials from the sweep (largest logit, lowest index
// holding it), then lane k of wave 0 compares draft x_k with the arg-max of
// row k; a ballot gives n, the first mismatch (K if none), and the emitted
// token is the arg-max of row n.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

// Greedy: one workgroup per sequence; wave w finds the arg-max of target rows
// w, w + 4, ...; then wave 0 compares with the drafts.
__global__ __launch_bounds__(kBlock) void k_greedy_scan(Params p) {
  const long s = p.seq0 + blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, np = p.nch1 * kWaves;
  const int kb = seq_kb(p, s);  // the sequence's own draft count; rows past it are not read
  __shared__ int sA[SPECV_MAX_K + 1];
  int xk = 0;
  bool valid = true;
  if (w == 0 && lane < kb) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
  }
  for (int i = w; i <= kb; i += kWaves) {
    const float2* pr = p.part + (s * (K + 1) + i) * np;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < np; j += kWave) argmax_merge(bv, bi, pr[j].x, __float_as_int(pr[j].y));
    wave_argmax(bv, bi);
    if (lane == 0) sA[i] = bi;
  }
  __syncthreads();
  if (w != 0) return;
  const int a = lane <= kb ? sA[lane] : 0;
  const bool match = lane < kb && xk == a;
  const uint64_t lim = (1ull << kb) - 1ull;
  const uint64_t miss = ~static_cast<uint64_t>(__ballot(match)) & lim;
  const int n = miss ? __ffsll(static_cast<unsigned long long>(miss)) - 1 : kb;
  const int an = __builtin_amdgcn_readlane(a, n);  // n is uniform (from a ballot)
  const bool bad = n < kb && __builtin_amdgcn_readlane(valid ? 1 : 0, n) == 0;
  if (lane <= K) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : (lane == n ? an : -1);
  if (lane == 0) {
    p.out_n[s] = n;
    if (p.out_flags) p.out_flags[s] = bad ? SPECV_FLAG_BAD_DRAFT : 0;
  }
}

}  // namespace

hipError_t launch_greedy_scan(const Params& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.nseq)), block(kBlock);
  hipLaunchKernelGGL(k_greedy_scan, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
