// Short rows, sampling mode: the whole verify step of one sequence in one
// workgroup, and of the batch in one launch.
//
// Rows of at most kShortMaxV tokens hold a few kilobytes, so on them a call
// of the general path is nothing but the fixed costs of its three dependent
// launches (row sweep, k_verify, fp64 draw) and of their memory round trips.
// Here workgroup s (512 threads) does every step for sequence s,
// with one round trip to memory for its inputs and one (to L2) for the
// decisive row(s):
//  - Loads.  Everything goes out first: the rows (wave w takes rows w, w + 8,
//    ... of target rows 0..K then draft rows 0..K-1, two per pass on the
//    vector path), the draft token each row is tested at, the acceptance
//    uniforms and the draw's uniform.
//  - Normalisers.  Per row: the largest logit m, R = rint(m c), lane sums of
//    2^(x c - R) in fp32 and their fp64 wave sum, whose log2 plus R is
//    log2 sum_v 2^(x c), the normaliser the sweep computes.  The lane that
//    holds the row's draft token picks its logit out of its registers, so the
//    acceptance test needs no gather.
//  - Acceptance.  Wave 0 tests u_k < min(1, p_k(x_k) / q_k(x_k)) as an fp64
//    log2 ratio per draft; a ballot gives n, the first rejection.
//  - Draw.  In fp64 over the whole workgroup, CAP / 512 tokens per thread in token
//    order.  P = exp(x / T - L'p) and Q = exp(y / T - L'q) from the decisive
//    row(s), normalised by their own sums: w = max(0, P - rho Q) with
//    rho = sum P / sum Q (w = P for a bonus draw, and when the residual sums
//    to zero after rounding).  One block scan gives the running sum C, and the
//    token is the smallest v with C(v) > u C(V-1) (past the end: the last
//    token of positive weight).  Each weight is good to about 1e-16, so the
//    token is the exact inverse CDF's unless u lies within about 1e-13 of an
//    interval edge; every draw carries SPECV_FLAG_FP64.
// Outputs are those of the general path: the accepted prefix, the draw at
// slot n, -1 after it, n, the flags and, when asked for, every used row's
// natural-log normaliser.
#include <hip/hip_ext.h>

#include <climits>

#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kSBlock = 512;  // threads per workgroup (8 waves: up to 256 registers each)
constexpr int kSWaves = kSBlock / kWave;
constexpr int kSRowsMax = 2 * SPECV_MAX_K + 1;
// Rows are held for a capacity CAP of tokens: kShortMaxV, or half of it for
// rows that fit (half the loads, exps and draw tokens per lane).
constexpr int kSCapSmall = kShortMaxV / 2;
static_assert(kSCapSmall % kSBlock == 0, "whole draw tokens per thread");

// One row's elements as a lane holds them: units lane, lane + 64, ...
// (16-byte vectors on the vector path, single elements otherwise), at most
// NU per lane for a row of CAP tokens.  Loads are branch-free: an index past
// the row reads the row's last unit again and is masked to -inf.
template <int DT, bool VEC, int CAP>
struct ShortRow {
  static constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  static constexpr int NU = CAP / PV / kWave;
  uint4 raw[VEC ? NU : 1];
  float el[VEC ? 1 : NU];

  __device__ void load(const void* row, long units) {
    const long lane = threadIdx.x % kWave;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const long u = lane + static_cast<long>(i) * kWave;
      if constexpr (VEC) raw[i] = load16(row, u < units ? u : units - 1);
      else el[i] = load_masked<DT>(row, u, units);
    }
  }
  // unit i's elements, -inf past the row's end
  __device__ void get(int i, long units, float (&e)[PV]) const {
    if constexpr (VEC) {
      Elt<DT>::unpack(raw[i], e);
      if (static_cast<long>(threadIdx.x % kWave) + static_cast<long>(i) * kWave >= units) {
#pragma unroll
        for (int k = 0; k < PV; ++k) e[k] = -INFINITY;
      }
    } else {
      e[0] = el[i];
    }
  }
  // Whole wave: log2 sum_v 2^(x_v c) over the row (-inf for a row of -inf),
  // and in *xv the logit at token xi (0 when xi is not a token of the row),
  // read from the registers of the lane that holds it (xi is the same in
  // every lane, so that lane is known to all).
  __device__ double log2z(long units, float c, int xi, int V, float* xv) const {
    const bool in = xi >= 0 && xi < V;
    const int owner = in ? (xi / PV) % kWave : 0;  // the lane whose units hold xi
    const int base = static_cast<int>(threadIdx.x % kWave) * PV;  // index of the lane's first element
    float m = -INFINITY, picked = 0.f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      float e[PV];
      get(i, units, e);
#pragma unroll
      for (int k = 0; k < PV; ++k) {
        m = fmaxf(m, e[k]);
        picked = base + i * kWave * PV + k == xi ? e[k] : picked;
      }
    }
    *xv = in ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(picked), owner)) : 0.f;
    m = wave_max(m);
    if (m == -INFINITY) return -INFINITY;  // uniform: wave_max returns a scalar
    const float R = rintf(m * c);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      float e[PV];
      get(i, units, e);
#pragma unroll
      for (int k = 0; k < PV; ++k) sum += ex2(fmaf(e[k], c, -R));
    }
    return wave_log2z(R, static_cast<double>(sum));
  }
};

template <int DT>
__device__ inline const void* short_row_ptr(const Params& p, long s, int i) {
  return i <= p.K ? row_ptr<DT>(p.lp, s * (p.K + 1) + i, p.V) : row_ptr<DT>(p.lq, s * p.K + (i - p.K - 1), p.V);
}

template <int DT, bool VEC, int CAP>
__global__ __launch_bounds__(kSBlock) void k_short(Params p) {
  using Row = ShortRow<DT, VEC, CAP>;
  constexpr int kSTok = CAP / kSBlock;  // draw tokens per thread
  const long s = p.seq0 + blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, nrows = 2 * K + 1;
  const int kb = seq_kb(p, s);
  const long units = VEC ? p.V / Row::PV : p.V;
  __shared__ double sL[kSRowsMax];  // log2 sum_v 2^(x_v c) of each used row
  __shared__ float sX[kSRowsMax];   // each used row's logit at its draft token
  __shared__ double s_sum[kSWaves][2], s_scan[kSWaves];
  __shared__ double s_lzp, s_lzq;
  __shared__ int s_n, s_flags, s_tok, s_last;
  // rows the sequence uses: target rows 0..kb, draft rows 0..kb-1
  auto used = [&](int i) { return i <= K ? i <= kb : i - K - 1 < kb; };
  // the draft token row i is tested at: x_k for target or draft row k < kb,
  // none (-1) for the bonus row; the load's index is clamped, not branched on
  auto row_x = [&](int i) {
    const int k = i <= K ? i : i - K - 1;
    const int xv = p.x[s * K + (k < K ? k : K - 1)];
    return k < kb ? xv : -1;
  };

  // wave 0's draft tokens and acceptance uniforms, and the draw's uniform, go
  // out with the rows
  const int kl = lane < K ? lane : K - 1;
  const int xk = p.x[s * K + kl];
  const float ua = p.ua[s * K + kl];
  const float ur = p.ur[s];

  auto keep = [&](int i, double lz, float xv) {
    if (lane == 0 && used(i)) {
      sL[i] = lz;
      sX[i] = xv;
      if (p.out_logz) p.out_logz[s * nrows + i] = static_cast<float>(lz * M_LN2);
    }
  };
  if constexpr (VEC) {
    // two rows per pass; a second row past the last is the first one again,
    // loaded and dropped
    for (int i0 = w; i0 < nrows; i0 += 2 * kSWaves) {
      const int i1 = i0 + kSWaves < nrows ? i0 + kSWaves : i0;
      const int x0 = row_x(i0), x1 = row_x(i1);
      Row a, b;
      a.load(short_row_ptr<DT>(p, s, i0), units);
      b.load(short_row_ptr<DT>(p, s, i1), units);
      float v0, v1;
      const double la = a.log2z(units, p.c, x0, p.V, &v0);
      const double lb = b.log2z(units, p.c, x1, p.V, &v1);
      keep(i0, la, v0);
      if (i1 != i0) keep(i1, lb, v1);
    }
  } else {  // lanes hold 32 elements per row: one row per pass
    for (int i0 = w; i0 < nrows; i0 += kSWaves) {
      const int x0 = row_x(i0);
      Row a;
      a.load(short_row_ptr<DT>(p, s, i0), units);
      float v0;
      const double la = a.log2z(units, p.c, x0, p.V, &v0);
      keep(i0, la, v0);
    }
  }
  __syncthreads();

  // acceptance: the first rejection n and the accepted prefix
  if (w == 0) {
    const bool valid = xk >= 0 && xk < p.V;
    bool accept = false;
    if (lane < kb && valid) {
      const double c = p.c;
      // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
      const double lr = (static_cast<double>(sX[lane]) * c - sL[lane]) -
                        (static_cast<double>(sX[K + 1 + lane]) * c - sL[K + 1 + lane]);
      const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
      accept = static_cast<double>(ua) < thr;
    }
    const uint64_t lim = (kb >= 64) ? ~0ull : ((1ull << kb) - 1ull);
    const uint64_t rejected = ~static_cast<uint64_t>(__ballot(accept)) & lim;
    const int n = rejected ? __ffsll(static_cast<unsigned long long>(rejected)) - 1 : kb;
    const bool bad = __builtin_amdgcn_readlane(valid ? 1 : 0, n < kb ? n : 0) == 0 && n < kb;
    if (lane <= K && lane != n) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : -1;
    if (lane == 0) {
      p.out_n[s] = n;
      s_n = n;
      s_flags = bad ? SPECV_FLAG_BAD_DRAFT : 0;
      s_lzp = sL[n];
      s_lzq = n < kb ? sL[K + 1 + n] : 0.0;
      s_tok = INT_MAX;
      s_last = -1;
    }
  }
  __syncthreads();

  // the draw: tokens v0 .. v0 + kSTok - 1 of this thread
  const int n = s_n;
  const bool bonus = n == kb;
  const void* rp = row_ptr<DT>(p.lp, s * (K + 1) + n, p.V);
  const void* rq = bonus ? rp : row_ptr<DT>(p.lq, s * K + n, p.V);  // a bonus draw loads, and drops, rp again
  const long v0 = static_cast<long>(kSTok) * threadIdx.x;
  float a[kSTok], b[kSTok];
#pragma unroll
  for (int j = 0; j < kSTok; ++j) {
    a[j] = load_masked<DT>(rp, v0 + j, p.V);
    b[j] = load_masked<DT>(rq, v0 + j, p.V);
  }
  const double ap = s_lzp * M_LN2, aq = s_lzq * M_LN2;
  double P[kSTok], Q[kSTok], sp = 0.0, sq = 0.0;
#pragma unroll
  for (int j = 0; j < kSTok; ++j) {
    P[j] = exp_f64(static_cast<double>(a[j]) * p.inv_t - ap, p.ec);
    Q[j] = bonus ? 0.0 : exp_f64(static_cast<double>(b[j]) * p.inv_t - aq, p.ec);
    sp += P[j];
    sq += Q[j];
  }
  double SP, SQ;
  {
    sp = wave_sum(sp);
    sq = wave_sum(sq);
    if (lane == 0) {
      s_sum[w][0] = sp;
      s_sum[w][1] = sq;
    }
    __syncthreads();
    SP = 0.0;
    SQ = 0.0;
#pragma unroll
    for (int i = 0; i < kSWaves; ++i) {
      SP += s_sum[i][0];
      SQ += s_sum[i][1];
    }
  }
  const double rho = bonus ? 1.0 : SP / SQ;
  double wv[kSTok], mine = 0.0;
#pragma unroll
  for (int j = 0; j < kSTok; ++j) {
    wv[j] = bonus ? P[j] : fmax(P[j] - rho * Q[j], 0.0);
    mine += wv[j];
  }
  double total;
  double run = block_exclusive_scan_n<kSWaves>(mine, s_scan, &total);
  const bool usep = !bonus && !(total > 0.0);  // uniform: the residual is zero after rounding
  if (usep) {
    mine = 0.0;
#pragma unroll
    for (int j = 0; j < kSTok; ++j) {
      wv[j] = P[j];
      mine += wv[j];
    }
    run = block_exclusive_scan_n<kSWaves>(mine, s_scan, &total);
  }
  const double t = static_cast<double>(ur) * total;
  // the running sum never decreases, so the smallest crossing over all
  // threads is the first one
  int cand = INT_MAX, last = -1;
#pragma unroll
  for (int j = 0; j < kSTok; ++j) {
    run += wv[j];
    if (cand == INT_MAX && run > t) cand = static_cast<int>(v0) + j;
    if (wv[j] > 0.0) last = static_cast<int>(v0) + j;
  }
  cand = wave_min_i32(cand);
  last = wave_max_i32(last);
  if (lane == 0) {
    if (cand != INT_MAX) atomicMin(&s_tok, cand);
    if (last >= 0) atomicMax(&s_last, last);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.out_tokens[s * (K + 1) + n] = s_tok != INT_MAX ? s_tok : s_last;
    if (p.out_flags) p.out_flags[s] = s_flags | SPECV_FLAG_FP64 | (usep ? SPECV_FLAG_ZW_ZERO : 0);
  }
}

template <int DT, bool VEC, int CAP>
void launch_short_cap(const Params& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(static_cast<unsigned>(p.nseq)), block(kSBlock);
  if (e0 || e1) hipExtLaunchKernelGGL((k_short<DT, VEC, CAP>), grid, block, 0, st, e0, e1, 0, p);
  else hipLaunchKernelGGL((k_short<DT, VEC, CAP>), grid, block, 0, st, p);
}

template <int DT, bool VEC>
void launch_short_t(const Params& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (p.V <= kSCapSmall) launch_short_cap<DT, VEC, kSCapSmall>(p, st, e0, e1);
  else launch_short_cap<DT, VEC, kShortMaxV>(p, st, e0, e1);
}

}  // namespace

hipError_t launch_short(const Params& p, int dtype, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (dtype == 1) {
    if (p.vec) launch_short_t<1, true>(p, st, e0, e1);
    else launch_short_t<1, false>(p, st, e0, e1);
  } else {
    if (p.vec) launch_short_t<0, true>(p, st, e0, e1);
    else launch_short_t<0, false>(p, st, e0, e1);
  }
  return hipGetLastError();
}

}  // namespace sv
