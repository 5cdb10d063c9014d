// Host side of libspecverify: argument checks, workspace layout and the
// launch sequence of one verify step.  Nothing here allocates, and nothing
// synchronises but the debug counters' read and reset.  State kept between
// calls: per device, the CU count and the static scratch's address (each
// looked up once) and the debug counters; per process, the two path
// thresholds (spec_rounds_min_bytes, spec_short_max_seqs).
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <limits>
#include <mutex>

#include "specverify.h"
#include "sv_internal.h"

// Scratch of spec_verify_noalloc: the workspace of a call that cannot
// allocate, in device memory the library holds on every device it runs on
// until the process ends.  In host code `scratch` names a host-side stand-in;
// its device address comes from hipGetSymbolAddress (scratch_ptr below).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace sv {

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elt_bytes(int dtype) { return dtype == SPECV_BF16 ? 2 : 4; }

}  // namespace

Layout make_layout(int B, int K, int V, int dtype, bool vec, bool greedy, bool tree) {
  Layout L{};
  // sweep chunks: equal shares of a row, each at most one workgroup's worth
  const int per_vec = vec ? (dtype == SPECV_BF16 ? 8 : 4) : 1;
  const bool bf = dtype == SPECV_BF16;
  auto elems = [&](bool large) {
    if (!vec) return kSweepElems<0, false, false, false>();
    if (greedy) return large ? (bf ? kSweepElems<1, true, true, true>() : kSweepElems<0, true, true, true>())
                             : (bf ? kSweepElems<1, true, true, false>() : kSweepElems<0, true, true, false>());
    return large ? (bf ? kSweepElems<1, true, false, true>() : kSweepElems<0, true, false, true>())
                 : (bf ? kSweepElems<1, true, false, false>() : kSweepElems<0, true, false, false>());
  };
  const long rows = static_cast<long>(B) * (greedy ? K + 1 : 2 * K + 1);
  const long units = static_cast<long>(V) / per_vec;
  auto chunks = [&](int lane_elems) {  // at least one, also for a row shorter than one vector
    const long units_per_chunk = static_cast<long>(kBlock) * (lane_elems / per_vec);
    return units > 0 ? (units + units_per_chunk - 1) / units_per_chunk : 1L;
  };
  // the large shape when it still gives a launch enough workgroups, judged on
  // the whole sweep for token trees, else on the first round of the
  // early-exit sweep (position 0 of every sequence):
  // the better rule for rounds (headline: 138.6 against 143.1 us per step
  // with the small shape; the sharp fp32 workload, whose first round alone
  // has 36864 large-shape workgroups: 727 against 766 us with the large
  // one).  The one-sweep path takes the same shape, so that both compute
  // bit-identical partials and hence identical outputs.
  const long launch_rows = tree ? rows : static_cast<long>(B) * (greedy ? 1 : 2);
  L.sweep_large = vec && launch_rows * chunks(elems(true)) >= kSweepLargeMinGroups ? 1 : 0;
  const int lane_elems = elems(L.sweep_large != 0);
  L.ch1 = kBlock * lane_elems;  // elements per chunk, at most
  L.nch1 = static_cast<int>(chunks(lane_elems));
  L.cq = static_cast<int>(units / L.nch1);
  L.cr = static_cast<int>(units % L.nch1);
  size_t off = 0;
  L.part = off;
  off = align_up(off + static_cast<size_t>(rows) * L.nch1 * kWaves * sizeof(float2));
  L.kbs = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(int32_t));
  if (greedy) {
    if (tree) {  // token trees read in rounds: per node, whether the round reads its row
      L.tneed = off;
      off = align_up(off + static_cast<size_t>(B) * (K + 1));
    }
    L.total = off;
    return L;
  }
  // fp64 draw chunks: multiples of 1024 elements, at most kMaxDrawChunks per row
  long ch = 1024;
  const long need = (static_cast<long>(V) + kMaxDrawChunks - 1) / kMaxDrawChunks;
  if (need > ch) ch = (need + 1023) / 1024 * 1024;
  L.ch3 = static_cast<int>(ch);
  L.R3 = static_cast<int>((V + ch - 1) / ch);
  L.xsum = off;
  off = align_up(off + static_cast<size_t>(B) * L.R3 * 5 * sizeof(double));
  L.queue = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(SeqRec));
  L.qcount = off;
  off = align_up(off + sizeof(uint32_t));
  // the split fast draw (batches of at most kSplitMaxSeqs): segment masses,
  // per-workgroup sums and per-sequence counters
  const long nsplit = B <= kSplitMaxSeqs ? B : 0;
  const SegGeom sg = seg_geom(V, per_vec, vec);
  L.segm = off;
  off = align_up(off + static_cast<size_t>(nsplit) * sg.nseg * sizeof(float));
  L.spq = off;
  off = align_up(off + static_cast<size_t>(nsplit) * kMaxSplit * 2 * sizeof(double));
  L.vcount = off;
  off = align_up(off + static_cast<size_t>(nsplit) * sizeof(uint32_t));
  L.total = off;
  return L;
}

namespace {

constexpr int kMaxDevices = 64;  // devices the per-device lookups below cover

// Device address of `scratch` on the current device, looked up once per
// device with that device current; null if the lookup fails.
void* scratch_ptr() {
  static std::once_flag once[kMaxDevices];
  static void* ptr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev] {
    void* q = nullptr;
    ptr[dev] = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) == hipSuccess ? q : nullptr;
  });
  return ptr[dev];
}

// Compute units of the current device, queried once per device (0 when the
// device cannot be queried).
int device_cus() {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::call_once(once[dev], [dev] {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  });
  return cus[dev];
}

// Workgroups per sequence for the fast draw: one per idle CU, at most one per
// block of kVerifyWaves segments and at most kMaxSplit; 1 for larger batches,
// for rows of fewer than kSplitMinBlocks blocks, or if the device cannot be
// queried.
int verify_split(int B, int V, int dtype, bool vec) {
  if (B > kSplitMaxSeqs) return 1;
  const int cus = device_cus();
  if (cus < 1) return 1;
  const int per_vec = vec ? (dtype == SPECV_BF16 ? 8 : 4) : 1;
  const SegGeom sg = seg_geom(V, per_vec, vec);
  const int blocks = (sg.nseg + kVerifyWaves - 1) / kVerifyWaves;
  if (blocks < kSplitMinBlocks) return 1;
  return std::max(1, std::min(std::min(cus / B, blocks), kMaxSplit));
}

// Bytes of logit rows from which the sweep runs in rounds: kRoundsMinBytes,
// or SPECV_ROUNDS_MIN_BYTES from the environment (read at the first use), or
// what spec_rounds_min_bytes set.
std::atomic<double>& rounds_threshold() {
  static std::atomic<double> v{[] {
    double t = kRoundsMinBytes;
    const char* e = std::getenv("SPECV_ROUNDS_MIN_BYTES");
    if (e && *e) {
      char* end = nullptr;
      const double d = std::strtod(e, &end);
      if (end != e && d >= 0.0) t = d;
    }
    return t;
  }()};
  return v;
}

double rounds_min_bytes() { return rounds_threshold().load(std::memory_order_relaxed); }

// Largest batch that takes the one-launch path for short rows (k_short): no
// limit, or SPECV_SHORT_MAX_SEQS from the environment (read at the first
// use), or what spec_short_max_seqs set (0 turns the path off).
std::atomic<int>& short_limit() {
  static std::atomic<int> v{[] {
    int t = INT_MAX;
    const char* e = std::getenv("SPECV_SHORT_MAX_SEQS");
    if (e && *e) {
      char* end = nullptr;
      const long d = std::strtol(e, &end, 10);
      if (end != e && d >= 0) t = static_cast<int>(std::min(d, static_cast<long>(INT_MAX)));
    }
    return t;
  }()};
  return v;
}

int short_max_seqs() { return short_limit().load(std::memory_order_relaxed); }

// The first level of the last round for K drafts.
int last_round_begin(int K) {
  int b = 0;
  for (int r = 0; r < kMaxRounds && round_begin(r) <= K; ++r) b = round_begin(r);
  return b;
}

// Events recorded with each sweep launch (spec_verify_sweep_timed): launch r
// < n starts with begin[r] and ends with end[r]; `launches` receives the
// number of sweep launches of the call.
struct SweepTiming {
  const hipEvent_t* begin;
  const hipEvent_t* end;
  int n;
  int launches;
};

// The sweep's launches for one call: every row at once when `full`, else
// rounds of levels (see round_begin) with k_round_accept between them.  The
// events e0 and e1 go to the first and the last sweep launch; with `tm`,
// each launch gets its own pair instead.
hipError_t launch_sweeps(Params P, int dtype, bool greedy, bool full, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                         SweepTiming* tm = nullptr) {
  auto launch = [&](const Params& q, hipEvent_t a, hipEvent_t b) {
    return greedy ? launch_sweep_argmax(q, dtype, st, a, b) : launch_sweep_lse(q, dtype, st, a, b);
  };
  auto begin_ev = [&](int r) { return tm ? (r < tm->n ? tm->begin[r] : nullptr) : (r == 0 ? e0 : nullptr); };
  auto end_ev = [&](int r, int nr) { return tm ? (r < tm->n ? tm->end[r] : nullptr) : (r == nr - 1 ? e1 : nullptr); };
  if (full) {
    P.grid3 = P.kb ? 1 : 0;  // per-sequence counts need the 3-D grid
    P.lv0 = 0;
    P.lv1 = P.K + 1;
    if (tm) tm->launches = 1;
    return launch(P, begin_ev(0), end_ev(0, 1));
  }
  int bounds[kMaxRounds + 1], nr = 0;
  for (int r = 0; r < kMaxRounds && round_begin(r) <= P.K; ++r) bounds[nr++] = round_begin(r);
  bounds[nr] = P.K + 1;
  if (tm) tm->launches = nr;
  P.grid3 = 1;
  for (int r = 0; r < nr; ++r) {
    if (r > 0) {  // the tests of the round just swept
      Params A = P;
      A.lv0 = bounds[r - 1];
      A.lv1 = bounds[r];
      const hipError_t rc = launch_round_accept(A, dtype, greedy, st);
      if (rc != hipSuccess) return rc;
    }
    P.lv0 = bounds[r];
    P.lv1 = bounds[r + 1];
    const hipError_t rc = launch(P, begin_ev(r), end_ev(r, nr));
    if (rc != hipSuccess) return rc;
  }
  return hipSuccess;
}

bool valid_temperature(float T) {
  if (!std::isfinite(T) || T < 0.f) return false;
  if (T == 0.f) return true;
  return std::isfinite(static_cast<float>(M_LOG2E / static_cast<double>(T)));
}

bool valid_shape(int B, int K, int V, bool greedy) {
  if (B < 1 || K < 1 || K > SPECV_MAX_K || V < 1) return false;
  // every grid is one-dimensional; keep workgroup counts and element offsets in range
  const long rows = static_cast<long>(B) * (greedy ? K + 1 : 2 * K + 1);
  const long nch_max = (static_cast<long>(V) + kBlock * 16 - 1) / (kBlock * 16);
  if (rows * nch_max >= (1L << 31)) return false;
  if (static_cast<double>(rows) * V * 4.0 > 9.0e18) return false;
  if (!greedy && static_cast<long>(B) * kMaxDrawChunks >= (1L << 31)) return false;
  return true;
}

}  // namespace
}  // namespace sv

extern "C" {

size_t spec_verify_workspace_size(int B, int K, int V, int dtype, float T) {
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return 0;
  if (!sv::valid_temperature(T)) return 0;
  const bool greedy = T == 0.f;
  if (!sv::valid_shape(B, K, V, greedy)) return 0;
  const size_t a = sv::make_layout(B, K, V, dtype, false, greedy, false).total;
  const size_t b = sv::make_layout(B, K, V, dtype, true, greedy, false).total;
  return a > b ? a : b;
}

namespace sv {
namespace {

// Every entry point: host-side checks, then the launches on `stream`.
int verify_impl(const void* logits_p, const void* logits_q, const int32_t* draft_tokens, const int32_t* num_drafts,
                const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                int32_t* out_tokens, int32_t* out_n_accepted, unsigned long long* position_stats, int dtype,
                void* workspace, size_t workspace_bytes, void* stream, float* out_logz, int32_t* out_flags,
                void* ev_sweep_begin, void* ev_sweep_end, size_t* need = nullptr, SweepTiming* tm = nullptr) {
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_E_DTYPE;
  if (!valid_temperature(T)) return SPECV_E_TEMP;
  const bool greedy = T == 0.f;
  if (!logits_p || !draft_tokens || !out_tokens || !out_n_accepted) return SPECV_E_NULL;
  if (!greedy && (!logits_q || !u_accept || !u_resample)) return SPECV_E_NULL;
  if (!valid_shape(B, K, V, greedy)) return SPECV_E_SHAPE;
  const uintptr_t eb = static_cast<uintptr_t>(elt_bytes(dtype));
  const uintptr_t ap = reinterpret_cast<uintptr_t>(logits_p);
  const uintptr_t aq = greedy ? 0 : reinterpret_cast<uintptr_t>(logits_q);
  if (ap % eb || aq % eb) return SPECV_E_ALIGN;
  const bool vec = ap % 16 == 0 && aq % 16 == 0 && (static_cast<long>(V) * eb) % 16 == 0;
  // one sweep of every row when every row's normaliser is asked for or the
  // input is small; else rounds
  const long all_rows = static_cast<long>(B) * (greedy ? K + 1 : 2 * K + 1);
  const bool full = out_logz != nullptr || static_cast<double>(all_rows) * V * eb < rounds_min_bytes();
  const Layout L = make_layout(B, K, V, dtype, vec, greedy, false);
  if (need) *need = L.total;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign || workspace_bytes < L.total)
    return SPECV_E_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  Params P{};
  P.lp = logits_p;
  P.lq = greedy ? nullptr : logits_q;
  P.x = draft_tokens;
  P.ua = u_accept;
  P.ur = u_resample;
  P.kb = num_drafts;
  P.stats = position_stats;
  P.B = B;
  P.K = K;
  P.V = V;
  P.vec = vec ? 1 : 0;
  P.out_tokens = out_tokens;
  P.out_n = out_n_accepted;
  P.out_logz = out_logz;
  P.out_flags = out_flags;
  P.part = reinterpret_cast<float2*>(ws + L.part);
  P.seq0 = 0;
  P.nseq = B;
  P.nch1 = L.nch1;
  P.ch1 = L.ch1;
  P.cq = L.cq;
  P.cr = L.cr;
  P.sweep_large = L.sweep_large;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(ev_sweep_begin), e1 = static_cast<hipEvent_t>(ev_sweep_end);
  const bool timed = e0 && e1;

  P.kbs = reinterpret_cast<int32_t*>(ws + L.kbs);
  if (debug_enabled_flag(nullptr)) {  // input validation, a debugging aid (see k_validate.hip)
    unsigned long long* dbg = debug_counters_ptr();
    if (!dbg || launch_validate(P, dtype, greedy, dbg, st) != hipSuccess) return SPECV_E_HIP;
  }
  if (greedy) {
    if (launch_sweeps(P, dtype, true, full, st, timed ? e0 : nullptr, timed ? e1 : nullptr, tm) != hipSuccess)
      return SPECV_E_HIP;
    if (launch_greedy_scan(P, st) != hipSuccess) return SPECV_E_HIP;
    if (position_stats && launch_position_stats(P, st) != hipSuccess) return SPECV_E_HIP;
    return SPECV_OK;
  }

  const double T64 = static_cast<double>(T);
  const double c64 = M_LOG2E / T64;
  P.c = static_cast<float>(c64);
  P.inv_t = 1.0 / T64;
  P.ec = make_exp_consts();
  P.xsum = reinterpret_cast<double*>(ws + L.xsum);
  P.queue = reinterpret_cast<SeqRec*>(ws + L.queue);
  P.qcount = reinterpret_cast<uint32_t*>(ws + L.qcount);
  P.R3 = L.R3;
  P.ch3 = L.ch3;
  P.split = verify_split(B, V, dtype, vec);
  P.nseg = seg_geom(V, vec ? (dtype == SPECV_BF16 ? 8 : 4) : 1, vec).nseg;
  P.segm = reinterpret_cast<float*>(ws + L.segm);
  P.spq = reinterpret_cast<double*>(ws + L.spq);
  P.vcount = reinterpret_cast<uint32_t*>(ws + L.vcount);

  if (P.R3 <= kSoloMaxChunks && V <= kShortMaxV && B <= short_max_seqs()) {
    // short rows: the whole step in one launch, which carries the sweep's events
    hipEvent_t a = timed ? e0 : nullptr, b = timed ? e1 : nullptr;
    if (tm) {
      a = tm->n > 0 ? tm->begin[0] : nullptr;
      b = tm->n > 0 ? tm->end[0] : nullptr;
      tm->launches = 1;
    }
    if (launch_short(P, dtype, st, a, b) != hipSuccess) return SPECV_E_HIP;
    if (position_stats && launch_position_stats(P, st) != hipSuccess) return SPECV_E_HIP;
    return SPECV_OK;
  }
  if (launch_sweeps(P, dtype, false, full, st, timed ? e0 : nullptr, timed ? e1 : nullptr, tm) != hipSuccess)
    return SPECV_E_HIP;
  P.vpre = full ? 0 : last_round_begin(K);
  // more sequences than CUs: two smaller workgroups per CU (see launch_verify)
  const int cus = device_cus();
  P.vwaves = (P.split <= 1 && cus > 0 && B > cus) ? kVerifyWavesSmall : kVerifyWaves;
  // at most half the CUs busy with sequences: the rest compute every
  // sequence's fp64 chunk sums during the fast draw, at most kEagerMaxRounds
  // chunks per 128-thread group (see k_verify)
  P.xeager = 0;
  P.xper = 0;
  if (P.split <= 1 && P.vwaves == kVerifyWaves && cus > 0 && P.R3 > kSoloMaxChunks) {
    const int spare = cus / B - 1;  // workgroups per sequence besides its own
    const int groups = kVerifyBlock / kXBlock;
    if (spare >= 1) {
      const int xe = std::min(spare, (P.R3 + groups - 1) / groups);
      const int per = (P.R3 + xe - 1) / xe;
      if ((per + groups - 1) / groups <= kEagerMaxRounds) {
        P.xeager = xe;
        P.xper = per;
      }
    }
  }
  if (launch_verify(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  if (launch_exact(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  if (position_stats && launch_position_stats(P, st) != hipSuccess) return SPECV_E_HIP;
  return SPECV_OK;
}

}  // namespace
}  // namespace sv

int spec_verify_ex(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                   const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                   int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream,
                   float* out_logz, int32_t* out_flags, void* ev_sweep_begin, void* ev_sweep_end) {
  return sv::verify_impl(logits_p, logits_q, draft_tokens, nullptr, u_accept, u_resample, T, B, K, V, out_tokens,
                         out_n_accepted, nullptr, dtype, workspace, workspace_bytes, stream, out_logz, out_flags,
                         ev_sweep_begin, ev_sweep_end);
}

int spec_verify_sweep_timed(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                            const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                            int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream,
                            float* out_logz, int32_t* out_flags, void* const* ev_begin, void* const* ev_end,
                            int n_events, int* n_sweeps) {
  if (n_sweeps) *n_sweeps = 0;
  if (n_events < 0) return SPECV_E_SHAPE;
  if (n_events > 0 && (!ev_begin || !ev_end)) return SPECV_E_NULL;
  sv::SweepTiming tm{reinterpret_cast<const hipEvent_t*>(ev_begin), reinterpret_cast<const hipEvent_t*>(ev_end),
                     n_events, 0};
  const int rc = sv::verify_impl(logits_p, logits_q, draft_tokens, nullptr, u_accept, u_resample, T, B, K, V,
                                 out_tokens, out_n_accepted, nullptr, dtype, workspace, workspace_bytes, stream,
                                 out_logz, out_flags, nullptr, nullptr, nullptr, &tm);
  if (n_sweeps) *n_sweeps = tm.launches;
  return rc;
}

int spec_verify_noalloc(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                        const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                        int32_t* out_tokens, int32_t* out_n_accepted, int dtype, void* stream) {
  // every argument check of spec_verify first (no workspace: it stops there)
  size_t need = 0;
  const int rc = sv::verify_impl(logits_p, logits_q, draft_tokens, nullptr, u_accept, u_resample, T, B, K, V,
                                 out_tokens, out_n_accepted, nullptr, dtype, nullptr, 0, stream, nullptr, nullptr,
                                 nullptr, nullptr, &need);
  if (rc != SPECV_E_WORKSPACE) return rc;
  if (need > kScratchBytes) return SPECV_E_SCRATCH;
  void* ws = sv::scratch_ptr();
  if (!ws) return SPECV_E_HIP;
  return sv::verify_impl(logits_p, logits_q, draft_tokens, nullptr, u_accept, u_resample, T, B, K, V, out_tokens,
                         out_n_accepted, nullptr, dtype, ws, kScratchBytes, stream, nullptr, nullptr, nullptr,
                         nullptr);
}

int spec_verify_ragged_ex(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                          const int32_t* num_drafts, const float* u_accept, const float* u_resample, float T,
                          int B, int K, int V, int32_t* out_tokens, int32_t* out_n_accepted,
                          uint64_t* position_stats, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream, float* out_logz, int32_t* out_flags) {
  if (!num_drafts) return SPECV_E_NULL;
  return sv::verify_impl(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T, B, K, V, out_tokens,
                         out_n_accepted, reinterpret_cast<unsigned long long*>(position_stats), dtype, workspace,
                         workspace_bytes, stream, out_logz, out_flags, nullptr, nullptr);
}

int spec_verify_ragged(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                       const int32_t* num_drafts, const float* u_accept, const float* u_resample, float T,
                       int B, int K, int V, int32_t* out_tokens, int32_t* out_n_accepted,
                       uint64_t* position_stats, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return spec_verify_ragged_ex(logits_p, logits_q, draft_tokens, num_drafts, u_accept, u_resample, T, B, K, V,
                               out_tokens, out_n_accepted, position_stats, dtype, workspace, workspace_bytes, stream,
                               nullptr, nullptr);
}

int spec_verify(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  return spec_verify_ex(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, B, K, V, out_tokens,
                        out_n_accepted, dtype, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr,
                        nullptr);
}

namespace sv {
namespace {

bool valid_tree_shape(int B, int N, int V) {
  if (B < 1 || N < 1 || N > SPECV_MAX_TREE || V < 1) return false;
  const long nch_max = (static_cast<long>(V) + kBlock * 16 - 1) / (kBlock * 16);
  if (static_cast<long>(B) * N * nch_max >= (1L << 31)) return false;
  return static_cast<double>(B) * N * V * 4.0 <= 9.0e18;
}

size_t tree_workspace(int B, int N, int V, int dtype) {
  const size_t a = make_layout(B, N - 1, V, dtype, false, true, true).total;
  const size_t b = make_layout(B, N - 1, V, dtype, true, true, true).total;
  return a > b ? a : b;
}

}  // namespace
}  // namespace sv

size_t spec_verify_tree_workspace_size(int B, int N, int V, int dtype) {
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return 0;
  if (!sv::valid_tree_shape(B, N, V)) return 0;
  return sv::tree_workspace(B, N, V, dtype);
}

int spec_verify_tree_greedy(const void* logits, const int32_t* tree_tokens, const int32_t* parents, int B, int N,
                            int V, int32_t* out_tokens, int32_t* out_path, int32_t* out_n_accepted, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  using namespace sv;
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_E_DTYPE;
  if (!logits || !tree_tokens || !parents || !out_tokens || !out_n_accepted) return SPECV_E_NULL;
  if (!valid_tree_shape(B, N, V)) return SPECV_E_SHAPE;
  const uintptr_t eb = static_cast<uintptr_t>(elt_bytes(dtype));
  const uintptr_t ap = reinterpret_cast<uintptr_t>(logits);
  if (ap % eb) return SPECV_E_ALIGN;
  const bool vec = ap % 16 == 0 && (static_cast<long>(V) * eb) % 16 == 0;
  const Layout L = make_layout(B, N - 1, V, dtype, vec, true, true);
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign || workspace_bytes < L.total)
    return SPECV_E_WORKSPACE;
  Params P{};
  P.lp = logits;
  P.x = tree_tokens;
  P.parents = parents;
  P.out_path = out_path;
  P.B = B;
  P.K = N - 1;
  P.V = V;
  P.vec = vec ? 1 : 0;
  P.out_tokens = out_tokens;
  P.out_n = out_n_accepted;
  P.part = reinterpret_cast<float2*>(static_cast<char*>(workspace) + L.part);
  P.seq0 = 0;
  P.nseq = B;
  P.nch1 = L.nch1;
  P.ch1 = L.ch1;
  P.cq = L.cq;
  P.cr = L.cr;
  P.sweep_large = L.sweep_large;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // rounds by depth on large inputs, as for draft positions: the roots, then
  // depths 1-2, then the rest, each after k_tree_round has marked the rows
  // the round needs
  const bool rounds = N > 1 && static_cast<double>(B) * N * V * eb >= rounds_min_bytes();
  if (!rounds) {
    if (launch_sweep_argmax(P, dtype, st, nullptr, nullptr) != hipSuccess) return SPECV_E_HIP;
  } else {
    P.tneed = reinterpret_cast<uint8_t*>(static_cast<char*>(workspace) + L.tneed);
    P.grid3 = 1;
    P.lv0 = 0;
    P.lv1 = 1;
    if (launch_sweep_argmax(P, dtype, st, nullptr, nullptr) != hipSuccess) return SPECV_E_HIP;
    P.lv0 = 1;
    P.lv1 = N;
    const int d[3] = {1, 3, SPECV_MAX_TREE};  // depth bounds of the later rounds
    for (int r = 0; r < 2 && d[r] < N; ++r) {  // a tree of N nodes has depths below N
      if (launch_tree_round(P, d[r], d[r + 1], st) != hipSuccess) return SPECV_E_HIP;
      if (launch_sweep_argmax_tree(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
    }
  }
  if (launch_tree_scan(P, st) != hipSuccess) return SPECV_E_HIP;
  return SPECV_OK;
}

int spec_ngram_propose(const int32_t* history, const int32_t* lengths, int B, int L_max, int n_min, int n_max,
                       int min_hits, int K, int32_t* out_draft, int32_t* out_count, void* stream) {
  if (!history || !lengths || !out_draft || !out_count) return SPECV_E_NULL;
  if (B < 1 || L_max < 1 || n_min < 1 || n_max < n_min || n_max > SPECV_MAX_NGRAM || min_hits < 1 || K < 1 ||
      K > SPECV_MAX_K)
    return SPECV_E_SHAPE;
  if (sv::launch_ngram(history, lengths, B, L_max, n_min, n_max, min_hits, K, out_draft, out_count,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPECV_E_HIP;
  return SPECV_OK;
}

size_t spec_ngram_map_bytes(int B, int capacity) {
  if (B < 1 || capacity < SPECV_NGRAM_MAP_MIN_SLOTS || capacity > SPECV_NGRAM_MAP_MAX_SLOTS ||
      (capacity & (capacity - 1)) != 0)
    return 0;
  return static_cast<size_t>(B) * (16 + 16 * static_cast<size_t>(capacity));
}

int spec_ngram_map_update(void* tables, int capacity, const int32_t* history, const int32_t* len_old,
                          const int32_t* len_new, int B, int L_max, int n_min, int n_max, int min_hits, int K,
                          int32_t* out_draft, int32_t* out_count, int32_t* out_status, void* stream) {
  if (!tables || !history || !len_old || !len_new || !out_draft || !out_count) return SPECV_E_NULL;
  if (spec_ngram_map_bytes(B, capacity) == 0 || L_max < 1 || n_min < 1 || n_max < n_min ||
      n_max > SPECV_MAX_NGRAM || min_hits < 1 || K < 1 || K > SPECV_MAX_K)
    return SPECV_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(tables) % 16) return SPECV_E_ALIGN;
  if (sv::launch_ngram_map(tables, capacity, history, len_old, len_new, B, L_max, n_min, n_max, min_hits, K,
                           out_draft, out_count, out_status, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPECV_E_HIP;
  return SPECV_OK;
}

int spec_tree_mask(const int32_t* parents, int B, int N, uint8_t* out_mask, int32_t* out_depth, void* stream) {
  if (!parents || (!out_mask && !out_depth)) return SPECV_E_NULL;
  if (B < 1 || N < 1 || N > SPECV_MAX_TREE || static_cast<long>(B) * N * N >= (1L << 40)) return SPECV_E_SHAPE;
  if (sv::launch_tree_mask(parents, B, N, out_mask, out_depth, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPECV_E_HIP;
  return SPECV_OK;
}

double spec_rounds_min_bytes(double bytes) {
  std::atomic<double>& t = sv::rounds_threshold();
  return bytes >= 0.0 && std::isfinite(bytes) ? t.exchange(bytes) : t.load();
}

int spec_short_max_seqs(int n) {
  std::atomic<int>& t = sv::short_limit();
  return n >= 0 ? t.exchange(n) : t.load();
}

int spec_debug_enable(int on) { return sv::debug_enabled_flag(&on) ? 1 : 0; }

int spec_debug_counters(unsigned long long* out, int n) {
  if (!out) return SPECV_E_NULL;
  if (n < 1 || n > SPECV_DEBUG_COUNTERS) return SPECV_E_SHAPE;
  unsigned long long* d = sv::debug_counters_ptr();
  if (!d || hipDeviceSynchronize() != hipSuccess) return SPECV_E_HIP;
  return hipMemcpy(out, d, static_cast<size_t>(n) * sizeof(unsigned long long), hipMemcpyDeviceToHost) == hipSuccess
             ? SPECV_OK
             : SPECV_E_HIP;
}

int spec_debug_reset(void) {
  unsigned long long* d = sv::debug_counters_ptr();
  if (!d || hipDeviceSynchronize() != hipSuccess) return SPECV_E_HIP;
  const unsigned long long zero[SPECV_DEBUG_COUNTERS] = {};
  return hipMemcpy(d, zero, sizeof zero, hipMemcpyHostToDevice) == hipSuccess ? SPECV_OK : SPECV_E_HIP;
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SPECV_OK: return "ok";
    case SPECV_E_NULL: return "a required pointer is NULL";
    case SPECV_E_SHAPE: return "invalid shape or size (B >= 1, 1 <= K <= 32, 1 <= N <= 64 tree nodes, 1 <= n <= 16 n-gram sizes, V >= 1, sizes in range)";
    case SPECV_E_DTYPE: return "dtype must be SPECV_F32 or SPECV_BF16";
    case SPECV_E_TEMP: return "T must be 0 (greedy) or finite and > 0 with 1/T finite";
    case SPECV_E_WORKSPACE: return "workspace NULL, not 256-byte aligned, or too small";
    case SPECV_E_ALIGN: return "logits pointer not aligned to its element size";
    case SPECV_E_HIP: return "a HIP launch failed";
    case SPECV_E_SCRATCH: return "the shape needs more than the 32 MiB static scratch of spec_verify_noalloc";
    default: return "unknown error";
  }
}

const char* spec_verify_version(void) { return "libspecverify 0.1 gfx950"; }

}  // extern "C"
