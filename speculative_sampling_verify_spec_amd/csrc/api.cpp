// Host side of libspecverify: argument checks, workspace layout and the
// launch sequence of one verify step.  Nothing here allocates, synchronises
// or keeps state between calls.
#include <cmath>
#include <cstdint>
#include <limits>

#include "specverify.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elt_bytes(int dtype) { return dtype == SPECV_BF16 ? 2 : 4; }

// Error model of the fp32 draw, in units of u = 2^-24.  The sweep forms
// t = fma(x, c, -R) with R = rint(row-share max * c), so t <= 1/2 and its one
// rounding is at most u|t|; v_exp_f32 is taken as <= 2 ulp; lane sums add a
// tree of 8 and six adds; merges are exact power-of-two rescales in fp64.
// The draw forms log2 p = fma(x, c, -whole) - fraction (two roundings of
// size u |log2 p| + u/2) and a v_exp_f32.  c = log2(e)/T is itself rounded,
// which acts as a relative temperature change of at most u.  Weighted by p,
// |log2 p| averages at most log2 V, so each normalised row's prefix masses
// carry a relative error of at most u (7 ln V + 12) + 2 exp errors.
double row_error(int V) {
  const double u = std::ldexp(1.0, -24);
  return u * (7.0 * std::log(static_cast<double>(V)) + 12.0 + 8.0);
}

}  // namespace

Layout make_layout(int B, int K, int V, int dtype, bool vec, bool greedy) {
  Layout L{};
  // sweep chunks: equal shares of a row, each at most one workgroup's worth
  const int per_vec = vec ? (dtype == SPECV_BF16 ? 8 : 4) : 1;
  const int lane_elems = vec ? (dtype == SPECV_BF16 ? kSweepElems<1, true>() : kSweepElems<0, true>())
                             : kSweepElems<0, false>();
  L.ch1 = kBlock * lane_elems;  // elements per chunk, at most
  const long units = static_cast<long>(V) / per_vec;
  const long units_per_chunk = static_cast<long>(kBlock) * (lane_elems / per_vec);
  L.nch1 = static_cast<int>((units + units_per_chunk - 1) / units_per_chunk);
  L.cq = static_cast<int>(units / L.nch1);
  L.cr = static_cast<int>(units % L.nch1);
  const long rows = static_cast<long>(B) * (greedy ? K + 1 : 2 * K + 1);
  size_t off = 0;
  L.part = off;
  off = align_up(off + static_cast<size_t>(rows) * L.nch1 * kWaves * sizeof(float2));
  if (greedy) {
    L.total = off;
    return L;
  }
  // draw / refine chunks: multiples of 2048 elements, at most kMaxDrawChunks per row
  long ch = 4096;
  const long need = (static_cast<long>(V) + kMaxDrawChunks - 1) / kMaxDrawChunks;
  if (need > ch) ch = (need + 2047) / 2048 * 2048;
  L.ch3 = L.ch4 = static_cast<int>(ch);
  L.R3 = L.R4 = static_cast<int>((V + ch - 1) / ch);
  L.rec = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(SeqRec));
  L.cnt = off;
  off = align_up(off + sizeof(uint32_t));
  L.csum = off;
  off = align_up(off + static_cast<size_t>(B) * L.R3 * sizeof(double));
  L.list = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(int32_t));
  L.rpart = off;
  off = align_up(off + static_cast<size_t>(B) * 2 * L.R4 * sizeof(double2));
  L.rsum = off;
  off = align_up(off + static_cast<size_t>(B) * L.R4 * sizeof(double2));
  L.total = off;
  return L;
}

namespace {

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
  const size_t a = sv::make_layout(B, K, V, dtype, false, greedy).total;
  const size_t b = sv::make_layout(B, K, V, dtype, true, greedy).total;
  return a > b ? a : b;
}

int spec_verify_ex(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                   const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                   int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream,
                   float* out_logz, int32_t* out_flags, int draw_policy,
                   void* ev_sweep_begin, void* ev_sweep_end) {
  using namespace sv;
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_E_DTYPE;
  if (!valid_temperature(T)) return SPECV_E_TEMP;
  const bool greedy = T == 0.f;
  if (!logits_p || !draft_tokens || !out_tokens || !out_n_accepted) return SPECV_E_NULL;
  if (!greedy && (!logits_q || !u_accept || !u_resample)) return SPECV_E_NULL;
  if (!valid_shape(B, K, V, greedy)) return SPECV_E_SHAPE;
  if (draw_policy < SPECV_DRAW_CERTIFIED || draw_policy > SPECV_DRAW_FP32) return SPECV_E_ARG;
  const uintptr_t eb = static_cast<uintptr_t>(elt_bytes(dtype));
  const uintptr_t ap = reinterpret_cast<uintptr_t>(logits_p);
  const uintptr_t aq = greedy ? 0 : reinterpret_cast<uintptr_t>(logits_q);
  if (ap % eb || aq % eb) return SPECV_E_ALIGN;
  const bool vec = ap % 16 == 0 && aq % 16 == 0 && (static_cast<long>(V) * eb) % 16 == 0;
  const Layout L = make_layout(B, K, V, dtype, vec, greedy);
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign || workspace_bytes < L.total)
    return SPECV_E_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  Params P{};
  P.lp = logits_p;
  P.lq = greedy ? nullptr : logits_q;
  P.x = draft_tokens;
  P.ua = u_accept;
  P.ur = u_resample;
  P.B = B;
  P.K = K;
  P.V = V;
  P.vec = vec ? 1 : 0;
  P.out_tokens = out_tokens;
  P.out_n = out_n_accepted;
  P.out_logz = out_logz;
  P.out_flags = out_flags;
  P.policy = draw_policy;
  P.part = reinterpret_cast<float2*>(ws + L.part);
  P.nch1 = L.nch1;
  P.ch1 = L.ch1;
  P.cq = L.cq;
  P.cr = L.cr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(ev_sweep_begin), e1 = static_cast<hipEvent_t>(ev_sweep_end);
  const bool timed = e0 && e1;

  if (greedy) {
    if (timed && hipEventRecord(e0, st) != hipSuccess) return SPECV_E_HIP;
    if (launch_sweep_argmax(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
    if (timed && hipEventRecord(e1, st) != hipSuccess) return SPECV_E_HIP;
    if (launch_greedy_scan(P, st) != hipSuccess) return SPECV_E_HIP;
    return SPECV_OK;
  }

  const double T64 = static_cast<double>(T);
  P.c = static_cast<float>(M_LOG2E / T64);
  P.inv_t = 1.0 / T64;
  const double u = std::ldexp(1.0, -24);
  const double lnV = std::log(static_cast<double>(V));
  // residual draw: |C' - C| and |t' - t| each within 2 (row error + 17u), twice for safety
  P.e_abs_res = 2.0 * 4.0 * (row_error(V) + 17.0 * u);
  // bonus draw: only per-element rounding and the chunk sums remain (normaliser cancels)
  P.e_rel_bonus = 2.0 * 2.0 * u * (3.0 * lnV + 21.0);
  P.rec = reinterpret_cast<SeqRec*>(ws + L.rec);
  P.list_count = reinterpret_cast<uint32_t*>(ws + L.cnt);
  P.csum = reinterpret_cast<double*>(ws + L.csum);
  P.list = reinterpret_cast<int32_t*>(ws + L.list);
  P.rpart = reinterpret_cast<double2*>(ws + L.rpart);
  P.rsum = reinterpret_cast<double2*>(ws + L.rsum);
  P.R3 = L.R3;
  P.ch3 = L.ch3;
  P.R4 = L.R4;
  P.ch4 = L.ch4;
  P.refine_grid = (B < 64 ? B : 64) * L.R4;

  if (timed && hipEventRecord(e0, st) != hipSuccess) return SPECV_E_HIP;
  if (launch_sweep_lse(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  if (timed && hipEventRecord(e1, st) != hipSuccess) return SPECV_E_HIP;
  if (launch_accept_scan(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  if (launch_draw(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  if (launch_refine(P, dtype, st) != hipSuccess) return SPECV_E_HIP;
  return SPECV_OK;
}

int spec_verify(const void* logits_p, const void* logits_q, const int32_t* draft_tokens,
                const float* u_accept, const float* u_resample, float T, int B, int K, int V,
                int32_t* out_tokens, int32_t* out_n_accepted, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  return spec_verify_ex(logits_p, logits_q, draft_tokens, u_accept, u_resample, T, B, K, V, out_tokens,
                        out_n_accepted, dtype, workspace, workspace_bytes, stream, nullptr, nullptr,
                        SPECV_DRAW_CERTIFIED, nullptr, nullptr);
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SPECV_OK: return "ok";
    case SPECV_E_NULL: return "a required pointer is NULL";
    case SPECV_E_SHAPE: return "invalid shape (B >= 1, 1 <= K <= 32, V >= 1, sizes in range)";
    case SPECV_E_DTYPE: return "dtype must be SPECV_F32 or SPECV_BF16";
    case SPECV_E_TEMP: return "T must be 0 (greedy) or finite and > 0 with 1/T finite";
    case SPECV_E_WORKSPACE: return "workspace NULL, not 256-byte aligned, or too small";
    case SPECV_E_ALIGN: return "logits pointer not aligned to its element size";
    case SPECV_E_HIP: return "a HIP launch failed";
    case SPECV_E_ARG: return "argument out of range";
    default: return "unknown error";
  }
}

const char* spec_verify_version(void) { return "libspecverify 0.1 gfx950"; }

}  // extern "C"
