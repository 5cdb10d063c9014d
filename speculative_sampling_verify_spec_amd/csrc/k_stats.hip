// Per-position acceptance counters ([D] "Когда процент принятия падает":
// acceptance changes with the position in the draft; [D] "Мониторинг в
// производстве": the rate to watch).  For every sequence, draft k was tested
// when k <= n and k < K_b, and accepted when k < n.  Each wave counts 64
// sequences per position with a ballot, the workgroup gathers the counts in
// LDS, and one atomic per position and workgroup adds them to the caller's
// counters; a few workgroups at most, so those atomics hardly contend.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kStatsBlock = 1024;
constexpr int kStatsMaxBlocks = 8;

__global__ __launch_bounds__(kStatsBlock) void k_position_stats(Params p) {
  __shared__ unsigned int cnt[2 * SPECV_MAX_K];
  const int lane = threadIdx.x % kWave;
  const int K = p.K;
  if (static_cast<int>(threadIdx.x) < 2 * K) cnt[threadIdx.x] = 0u;
  __syncthreads();
  const long stride = static_cast<long>(gridDim.x) * kStatsBlock;
  const long base0 = static_cast<long>(blockIdx.x) * kStatsBlock + (threadIdx.x - lane);
  for (long base = base0; base < p.nseq; base += stride) {  // uniform over the wave
    const long s = base + lane;
    const bool in = s < p.nseq;
    const int n = in ? p.out_n[p.seq0 + s] : 0;
    const int kb = in ? seq_kb(p, p.seq0 + s) : 0;
    for (int k = 0; k < K; ++k) {
      const unsigned tested = __popcll(__ballot(in && k <= n && k < kb));
      const unsigned accepted = __popcll(__ballot(in && k < n));
      if (lane == 0) {
        if (tested) atomicAdd(&cnt[k], tested);
        if (accepted) atomicAdd(&cnt[K + k], accepted);
      }
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < 2 * K && cnt[threadIdx.x]) atomicAdd(&p.stats[threadIdx.x], static_cast<unsigned long long>(cnt[threadIdx.x]));
}

}  // namespace

hipError_t launch_position_stats(const Params& p, hipStream_t st) {
  const long blocks = (static_cast<long>(p.nseq) + kStatsBlock - 1) / kStatsBlock;
  const dim3 grid(static_cast<unsigned>(blocks < kStatsMaxBlocks ? blocks : kStatsMaxBlocks));
  hipLaunchKernelGGL(k_position_stats, grid, dim3(kStatsBlock), 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
