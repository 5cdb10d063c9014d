// Device-side input validation, a debugging aid (SPECV_DEBUG=1 in the
// environment, or spec_debug_enable): before a verify call's sweep, one pass
// over the inputs the call uses counts what breaks the input contract into
// per-device counters (SPECV_DBG_* in specverify.h):
//  - draft ids outside [0, V) among positions 0 .. K_b - 1;
//  - accept uniforms (positions 0 .. K_b - 1) and resample uniforms outside
//    the open interval (0, 1), NaN included (sampling mode only);
//  - NaN and +inf logits, and rows without a finite logit, among the rows
//    the call reads (target rows 0 .. K_b, draft rows 0 .. K_b - 1).
// The verify kernels still run on such inputs; they index memory only by
// clamped or ballot-derived values, so these give unspecified tokens, never
// an out-of-bounds access.  The pass reads every used logit once more: it is
// for debugging, not for timing.
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "sv_device.h"
#include "specverify.h"

namespace sv {

// The counters of this device (a file-scope device array: each GPU holds its
// own copy, at its own address).
__device__ __align__(16) unsigned long long debug_counters[SPECV_DEBUG_COUNTERS];

namespace {

// One workgroup per row (a grid-stride loop over the launch's rows: target
// rows seq0 .. seq0 + nseq - 1 times K + 1, then their draft rows).  The
// workgroup of a sequence's target row 0 also checks its draft ids and
// uniforms.  Counters are bumped only for what is found (plus one per call),
// so a clean call costs one atomic.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_validate(Params p, unsigned long long* dbg, int greedy) {
  const int K = p.K, V = p.V;
  const long nt = static_cast<long>(p.nseq) * (K + 1);
  const long nd = greedy ? 0 : static_cast<long>(p.nseq) * K;
  __shared__ unsigned int s_cnt[3][kWaves];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  for (long row = blockIdx.x; row < nt + nd; row += gridDim.x) {
    const bool draft = row >= nt;
    const long local = draft ? (row - nt) / K : row / (K + 1);
    const int j = static_cast<int>(draft ? (row - nt) - local * K : row - local * (K + 1));
    const long s = p.seq0 + local;
    const int kb = seq_kb(p, s);
    if (draft ? j >= kb : j > kb) continue;  // a row the call does not read (uniform)
    const void* r = draft ? row_ptr<DT>(p.lq, s * K + j, V) : row_ptr<DT>(p.lp, s * (K + 1) + j, V);
    unsigned int nan = 0, pinf = 0, fin = 0;
    for (long v = threadIdx.x; v < V; v += kBlock) {
      const float x = Elt<DT>::at(r, v);
      nan += isnan(x) ? 1u : 0u;
      pinf += (x == INFINITY) ? 1u : 0u;
      fin += isfinite(x) ? 1u : 0u;
    }
    const int a = wave_reduce_i32(static_cast<int>(nan), [](int u, int x) { return u + x; });
    const int b = wave_reduce_i32(static_cast<int>(pinf), [](int u, int x) { return u + x; });
    const int c = wave_reduce_i32(static_cast<int>(fin), [](int u, int x) { return u + x; });
    __syncthreads();  // the previous row's reads of s_cnt are done
    if (lane == 0) {
      s_cnt[0][w] = a;
      s_cnt[1][w] = b;
      s_cnt[2][w] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long tn = 0, tp = 0, tf = 0;
      for (int i = 0; i < kWaves; ++i) {
        tn += s_cnt[0][i];
        tp += s_cnt[1][i];
        tf += s_cnt[2][i];
      }
      if (tn) atomicAdd(dbg + SPECV_DBG_NAN_LOGITS, tn);
      if (tp) atomicAdd(dbg + SPECV_DBG_INF_LOGITS, tp);
      if (!tf) atomicAdd(dbg + SPECV_DBG_ROWS_NO_FINITE, 1ull);
    }
    if (!draft && j == 0 && threadIdx.x < kWave) {  // the sequence's draft ids and uniforms (wave 0)
      bool bad_id = false, bad_ua = false;
      if (lane < kb) {
        const int x = p.x[s * K + lane];
        bad_id = x < 0 || x >= V;
        if (!greedy) {
          const float u = p.ua[s * K + lane];
          bad_ua = !(u > 0.f && u < 1.f);
        }
      }
      const int ni = __popcll(__ballot(bad_id)), nu = __popcll(__ballot(bad_ua));
      if (lane == 0) {
        if (ni) atomicAdd(dbg + SPECV_DBG_BAD_DRAFT_IDS, static_cast<unsigned long long>(ni));
        if (nu) atomicAdd(dbg + SPECV_DBG_BAD_U_ACCEPT, static_cast<unsigned long long>(nu));
        if (!greedy) {
          const float u = p.ur[s];
          if (!(u > 0.f && u < 1.f)) atomicAdd(dbg + SPECV_DBG_BAD_U_RESAMPLE, 1ull);
        }
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(dbg + SPECV_DBG_CALLS, 1ull);
}

constexpr int kMaxDevices = 64;
constexpr unsigned kValidateBlocks = 4096;

}  // namespace

bool debug_enabled_flag(int* set_to) {
  static std::atomic<int> on{-1};  // -1: not yet read from the environment
  static std::once_flag once;
  std::call_once(once, [] {
    const char* e = std::getenv("SPECV_DEBUG");
    int expected = -1;
    on.compare_exchange_strong(expected, (e && e[0] == '1') ? 1 : 0);
  });
  if (set_to) return on.exchange(*set_to ? 1 : 0) != 0;
  return on.load() != 0;
}

// Device address of debug_counters on the current device, looked up once per
// device with that device current; null if the lookup fails.
unsigned long long* debug_counters_ptr() {
  static std::once_flag once[kMaxDevices];
  static void* ptr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev] {
    void* q = nullptr;
    ptr[dev] = hipGetSymbolAddress(&q, HIP_SYMBOL(debug_counters)) == hipSuccess ? q : nullptr;
  });
  return static_cast<unsigned long long*>(ptr[dev]);
}

hipError_t launch_validate(const Params& p, int dtype, bool greedy, unsigned long long* dbg, hipStream_t st) {
  const long rows = static_cast<long>(p.nseq) * (greedy ? p.K + 1 : 2 * p.K + 1);
  const dim3 grid(static_cast<unsigned>(rows < kValidateBlocks ? rows : kValidateBlocks)), block(kBlock);
  if (dtype == 1) hipLaunchKernelGGL((k_validate<1>), grid, block, 0, st, p, dbg, greedy ? 1 : 0);
  else hipLaunchKernelGGL((k_validate<0>), grid, block, 0, st, p, dbg, greedy ? 1 : 0);
  return hipGetLastError();
}

}  // namespace sv
