// The replacement / bonus draw.
//
// After n acceptances the emitted token is drawn from w = max(0, p_n - q_n)
// (n < K) or w = p_K (n == K) by inverse CDF: the smallest token v whose
// running sum C(v) exceeds t = u * Z, Z the total weight.  Only the decisive
// row (pair) of each sequence is reread.
//
// Self-normalisation.  The sweep gives each row's log2 normaliser L' to fp32
// accuracy.  With it as reference the draw forms P(v) = 2^(x c - Lp') and
// Q(v) = 2^(x c - Lq') (c = log2(e)/T), so p = P / sum P and q = Q / sum Q
// whatever the error of L', and
//   w(v) = max(0, p - q) = max(0, P - rho Q) / sum P,  rho = sum P / sum Q.
//
// Four kernels:
//   fast_chunks  (sequences x chunks): per chunk, in fp32, sum P, sum Q and
//                sum min(P, Q); the residual mass at rho = 1 is
//                sum P - sum min(P, Q).
//   fast_select  (one workgroup per sequence): the chunk sums give Z and the
//                chunk holding t; that chunk is rescanned (lane-contiguous
//                runs, fp64 block scan) for the smallest v whose running sum
//                exceeds t.  The fast path takes rho as 1; the answer stands
//                when t is further from both ends of v's interval than a
//                certified bound (fp32 rounding plus |sum P - sum Q| for
//                rho); otherwise the sequence joins the queue.
//   exact_chunks, exact_select: fp64 weights (P = exp(x/T - L')) for queued
//                sequences only.  Their chunk sums are taken at rho = 1 and
//                corrected to first order in rho - 1 with G = sum_{P > Q} Q,
//                exact up to the Q-mass of tokens whose sign flips, which is
//                bounded by H, the chunk's Q-mass within a relative kKappa of
//                P = Q.  Their error is ~1e-16 relative per weight, so they
//                match the exact inverse CDF unless t lies within ~1e-12 of a
//                bucket edge.
// The select rescans forward when rounding leaves the crossing past the
// located chunk; the exact path also restarts from the first chunk when t
// may lie before it, and recomputes the total when rho leaves the
// linearisation window.  Past the end it takes the last token with positive
// weight; a residual of zero mass (p == q to rounding) falls back to p_n and
// sets a flag.
#include <type_traits>

#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRun = 16;                // elements per lane per rescan round
constexpr int kRound = kBlock * kRun;   // 4096 elements per round (one draw chunk)
constexpr double kKappa = 1e-4;         // near-flip window, relative to Q
constexpr unsigned kExactSeqs = 32;     // queued sequences the exact kernels cover per pass

// ---------------------------------------------------------------- weights --
// fp32 weights scaled by the common factor 2^Fp: P' = 2^(x c - Wp) and
// Q' = 2^((y c - Wq) - D), with Wp, Wq = rint(L') whole, Fp, Fq the remaining
// fractions and D = Fq - Fp, so both references are kept to fp32 accuracy of
// the fractions, not of L'.  A common factor leaves the draw unchanged (it
// normalises by its own sums), and -inf logits give weights of exactly 0.
struct FastWeight {
  float c, Wp, Wq, D;
  __device__ float P(float x) const { return ex2(fmaf(x, c, -Wp)); }
  __device__ float Q(float x) const { return ex2(fmaf(x, c, -Wq) - D); }
  __device__ double resid(double P, double Q, double rho) const {
    return fmaxf(static_cast<float>(P) - static_cast<float>(rho) * static_cast<float>(Q), 0.f);
  }
};

// fp64 weight exp(x / T - L'), L' the natural-log reference.
struct ExactWeight {
  double inv_t, ap, aq;
  __device__ double P(float x) const { return exp_f64(static_cast<double>(x) * inv_t - ap); }
  __device__ double Q(float x) const { return exp_f64(static_cast<double>(x) * inv_t - aq); }
  __device__ double resid(double P, double Q, double rho) const { return fmax(P - rho * Q, 0.0); }
};

__device__ inline FastWeight fast_weight(const Params& p, const SeqRec& rec) {
  FastWeight f;
  f.c = p.c;
  const double wp = rint(rec.lzp), wq = rint(rec.lzq);
  f.Wp = static_cast<float>(wp);
  f.Wq = static_cast<float>(wq);
  f.D = static_cast<float>((rec.lzq - wq) - (rec.lzp - wp));
  return f;
}

__device__ inline ExactWeight exact_weight(const Params& p, const SeqRec& rec) {
  ExactWeight e;
  e.inv_t = p.inv_t;
  e.ap = rec.lzp * M_LN2;
  e.aq = rec.lzq * M_LN2;
  return e;
}

template <int DT>
struct Rows {
  const void* rp;
  const void* rq;  // null for a bonus draw
};

template <int DT>
__device__ inline Rows<DT> decisive_rows(const Params& p, long s, int n) {
  Rows<DT> r;
  r.rp = row_ptr<DT>(p.lp, s * (p.K + 1) + n, p.V);
  r.rq = n == p.K ? nullptr : row_ptr<DT>(p.lq, s * p.K + n, p.V);
  return r;
}

// ------------------------------------------------------------ chunk sums --
struct ChunkSums {
  double sp, sq, a, g, h;
};

// Exact chunk sums of chunk r of the decisive row(s): out[0..4] = sum P,
// sum Q, A = sum max(0, P - Q), G = sum_{P > Q} Q, H = sum_{near flip} Q
// (only out[0] for a bonus draw).  Loads go out branch-free, U units per lane.
template <int DT, bool VEC, class Wt>
__device__ inline void exact_chunk_sums(const Params& p, const Rows<DT>& rows, const Wt& wt, bool bonus, int r,
                                        double* out) {
  const long lo = static_cast<long>(r) * p.ch3;
  const long hi = min(static_cast<long>(p.V), lo + p.ch3);
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  constexpr int U = VEC ? 2 : 8;
  const long ulo = lo / PV, uhi = hi / PV;  // VEC: lo and hi are multiples of PV
  ChunkSums acc = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (long r0 = ulo; r0 < uhi; r0 += static_cast<long>(kBlock) * U) {
    float ep[U * PV], eq[U * PV];
    if constexpr (VEC) {
      uint4 rp[U], rq[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        const long uu = u < uhi ? u : uhi - 1;
        rp[i] = load16(rows.rp, uu);
        if (!bonus) rq[i] = load16(rows.rq, uu);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        Elt<DT>::unpack(rp[i], ep + i * PV);
        if (!bonus) Elt<DT>::unpack(rq[i], eq + i * PV);
        if (r0 + threadIdx.x + static_cast<long>(i) * kBlock >= uhi) {
#pragma unroll
          for (int k = 0; k < PV; ++k) ep[i * PV + k] = eq[i * PV + k] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        ep[i] = load_masked<DT>(rows.rp, u, uhi);
        eq[i] = bonus ? -INFINITY : load_masked<DT>(rows.rq, u, uhi);
      }
    }
    // pairwise within groups of eight in the weights' own precision, then
    // into the fp64 lane sums
#pragma unroll
    for (int g0 = 0; g0 < U * PV; g0 += 8) {
      using W = decltype(wt.P(0.f));
      W sp[8], sq[8], a[8], g[8], h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool in = g0 + k < U * PV;
        const W P = in ? wt.P(ep[g0 + k]) : W(0);
        const W Q = (in && !bonus) ? wt.Q(eq[g0 + k]) : W(0);
        const W d = P - Q;
        sp[k] = P;
        sq[k] = Q;
        a[k] = d > W(0) ? d : W(0);
        g[k] = d > W(0) ? Q : W(0);
        h[k] = (d <= W(kKappa) * Q && -d <= W(kKappa) * Q) ? Q : W(0);
      }
#pragma unroll
      for (int w = 4; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) {
          sp[k] += sp[k + w];
          sq[k] += sq[k + w];
          a[k] += a[k + w];
          g[k] += g[k + w];
          h[k] += h[k + w];
        }
      acc.sp += sp[0];
      acc.sq += sq[0];
      acc.a += a[0];
      acc.g += g[0];
      acc.h += h[0];
    }
  }
  __shared__ double lds[kWaves];
  const double sp = block_sum(acc.sp, lds);
  if (bonus) {
    if (threadIdx.x == 0) out[0] = sp;
    return;
  }
  const double sq = block_sum(acc.sq, lds);
  const double a = block_sum(acc.a, lds);
  const double g = block_sum(acc.g, lds);
  const double h = block_sum(acc.h, lds);
  if (threadIdx.x == 0) {
    out[0] = sp;
    out[1] = sq;
    out[2] = a;
    out[3] = g;
    out[4] = h;
  }
}

// Fast chunk sums of chunk r: sum P, sum Q and sum min(P, Q), pairwise over
// groups of eight in fp32, then fp64.  out[0..2] = sum P, sum Q and
// A = sum P - sum min(P, Q), the chunk's residual mass at rho = 1.  A bonus
// draw has only P.  Whole iterations (every one but a row's last) load and
// add without masks; the bonus case is its own loop, so neither pays for a
// select per element.
template <int DT, bool VEC, bool BONUS>
__device__ inline void fast_sums_loop(const Rows<DT>& rows, const FastWeight& wt, long ulo, long uhi,
                                      double& asp, double& asq, double& asm_) {
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  constexpr int U = VEC ? 2 : 8;
  constexpr long kStep = static_cast<long>(kBlock) * U;
  auto body = [&](long r0, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    float ep[U * PV], eq[U * PV];
    if constexpr (VEC) {
      uint4 rp[U], rq[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        const long uu = (!MASKED || u < uhi) ? u : uhi - 1;
        rp[i] = load16(rows.rp, uu);
        if constexpr (!BONUS) rq[i] = load16(rows.rq, uu);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        Elt<DT>::unpack(rp[i], ep + i * PV);
        if constexpr (!BONUS) Elt<DT>::unpack(rq[i], eq + i * PV);
        if (MASKED && r0 + threadIdx.x + static_cast<long>(i) * kBlock >= uhi) {
#pragma unroll
          for (int k = 0; k < PV; ++k) ep[i * PV + k] = eq[i * PV + k] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        ep[i] = load_masked<DT>(rows.rp, u, uhi);
        if constexpr (!BONUS) eq[i] = load_masked<DT>(rows.rq, u, uhi);
      }
    }
#pragma unroll
    for (int g0 = 0; g0 < U * PV; g0 += 8) {
      float sp[8], sq[8], sm[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float P = wt.P(ep[g0 + k]);
        sp[k] = P;
        if constexpr (!BONUS) {
          const float Q = wt.Q(eq[g0 + k]);
          sq[k] = Q;
          sm[k] = fminf(P, Q);
        }
      }
#pragma unroll
      for (int w = 4; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) {
          sp[k] += sp[k + w];
          if constexpr (!BONUS) {
            sq[k] += sq[k + w];
            sm[k] += sm[k + w];
          }
        }
      asp += sp[0];
      if constexpr (!BONUS) {
        asq += sq[0];
        asm_ += sm[0];
      }
    }
  };
  static_assert((U * PV) % 8 == 0, "groups of eight");
  long r0 = ulo;
  for (; r0 + kStep <= uhi; r0 += kStep) body(r0, std::false_type{});
  if (r0 < uhi) body(r0, std::true_type{});
}

template <int DT, bool VEC>
__device__ inline void fast_chunk_sums(const Params& p, const Rows<DT>& rows, const FastWeight& wt, bool bonus,
                                       int r, double* out) {
  const long lo = static_cast<long>(r) * p.ch3;
  const long hi = min(static_cast<long>(p.V), lo + p.ch3);
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  const long ulo = lo / PV, uhi = hi / PV;  // VEC: lo and hi are multiples of PV
  double asp = 0.0, asq = 0.0, asm_ = 0.0;
  if (bonus) fast_sums_loop<DT, VEC, true>(rows, wt, ulo, uhi, asp, asq, asm_);
  else fast_sums_loop<DT, VEC, false>(rows, wt, ulo, uhi, asp, asq, asm_);
  __shared__ double lds[kWaves];
  const double sp = block_sum(asp, lds);
  if (bonus) {
    if (threadIdx.x == 0) {
      out[0] = sp;
      out[1] = 0.0;
      out[2] = sp;
    }
    return;
  }
  const double sq = block_sum(asq, lds);
  const double sm = block_sum(asm_, lds);
  if (threadIdx.x == 0) {
    out[0] = sp;
    out[1] = sq;
    out[2] = fmax(sp - sm, 0.0);
  }
}

// Certified bound on how far the fast draw's t - C(v) can be from the exact
// one (C a running sum of the residual, t = u Z), in the units of P.
// Per weight, the exponent carries roundings that grow with its size |f|
// (c's own rounding, the fma, the subtraction of D; a common offset cancels
// when P is normalised by its own sum), at most u (3 |f| + 1), and v_exp_f32
// one ulp (measured <= 0.78), so the relative error is <= u (2.7 + 2.08 |f|),
// u = 2^-24.  Summed over a row, sum P |f| <= sum P (log2 V + 1) (an entropy
// bound), so a row's weights are off by at most u (2.7 + 2.08 (log2 V + 1))
// times its mass.  The fp32 pairwise sums, the residual's subtraction and the
// chunk differences add at most 7u sum P + 3u sum Q.  So one running sum is
// off by R <= u (10 + 2.1 (log2 V + 1)) (SP + SQ), and t by as much.  Taking
// rho as 1 moves each residual weight by at most |rho - 1| Q, so a running
// sum and Z by at most |SP - SQ|.  Both errors enter twice (t and C), and the
// whole carries a safety factor of 2.
__device__ inline double fast_bound(double SP, double SQ, int V, bool bonus) {
  const double u = 0x1p-24;
  const double R = u * (10.0 + 2.1 * (log2(static_cast<double>(V)) + 1.0)) * (SP + SQ);
  return 2.0 * (2.0 * R + (bonus ? 0.0 : 2.0 * fabs(SP - SQ)));
}

// A lane's run of kRun consecutive logits from v0, -inf at and past chi.
// VEC: v0 and chi are multiples of the vector width, so whole 16-byte units
// are loaded (index clamped below chi) and masked.
template <int DT, bool VEC>
__device__ inline void load_run(const void* row, long v0, long chi, float (&e)[kRun]) {
  if constexpr (VEC) {
    constexpr int PV = Elt<DT>::kPerVec;
    constexpr int NU = kRun / PV;
    static_assert(kRun % PV == 0, "whole units per run");
    const long u0 = v0 / PV, uend = chi / PV;
    uint4 raw[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) raw[i] = load16(row, u0 + i < uend ? u0 + i : uend - 1);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      Elt<DT>::unpack(raw[i], &e[i * PV]);
      if (u0 + i >= uend) {
#pragma unroll
        for (int k = 0; k < PV; ++k) e[i * PV + k] = -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRun; ++k) e[k] = load_masked<DT>(row, v0 + k, chi);
  }
}

// ---------------------------------------------------------------- select --
// Draw for one sequence from its chunk sums.  Thread 0 gets the token,
// whether the zero-mass fallback was used, and whether the answer is certain
// (always on the exact path; margin above the bound on the fast path).
template <int DT, bool VEC, bool EXACT, class Wt>
__device__ inline void select_token(const Params& p, const Rows<DT>& rows, const Wt& wt, bool bonus,
                                    const double* cs_base, double ur, int* token, bool* zw_zero, bool* certain) {
  const int lane = threadIdx.x % kWave;
  __shared__ double s_rho, s_t, s_base, s_bound;
  __shared__ int s_chunk, s_usep, s_exact_total;
  if (threadIdx.x < kWave) {
    const bool have = lane < p.R3;
    const double* cs = cs_base + (have ? lane : 0) * 5;
    const double sp = have ? cs[0] : 0.0;
    const double SP = wave_sum(sp);
    double v = sp, rho = 1.0, err = 0.0, SQ = 0.0;
    int usep = 1;
    if (!bonus) {
      const double sq = have ? cs[1] : 0.0, a = have ? cs[2] : 0.0;
      SQ = wave_sum(sq);
      rho = SP / SQ;
      double corrected = a;
      if (EXACT) {  // first-order correction to the exact rho, with its error bound
        const double g = have ? cs[3] : 0.0, h = have ? cs[4] : 0.0;
        corrected = fmax(a - (rho - 1.0) * g, 0.0);
        err = fabs(rho - 1.0) * h;
      }
      const double Z = wave_sum(corrected);
      usep = !(Z > 0.0);  // p == q to rounding: draw from p_n instead
      v = usep ? sp : corrected;
      if (usep) err = 0.0;
    }
    const double inc = wave_inclusive_scan(v);
    const double err_inc = wave_inclusive_scan(err);
    double excl = __shfl_up(inc, 1, kWave), err_excl = __shfl_up(err_inc, 1, kWave);
    if (lane == 0) excl = err_excl = 0.0;
    const double z = __shfl(inc, kWave - 1, kWave);
    const double err_all = __shfl(err_inc, kWave - 1, kWave);
    const double t = ur * z;
    const uint64_t hit = __ballot(have && inc > t);
    const uint64_t pos = __ballot(have && v > 0.0);
    int rc;
    if (hit) rc = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    else rc = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;  // past the end: last chunk with mass
    double base = __shfl(excl, rc, kWave);
    const double err_before = __shfl(err_excl, rc, kWave);
    // exact path: t may lie before the located chunk when it is within the
    // base's error, and the first-order correction needs rho near 1
    const bool bad_rho = EXACT && !bonus && !usep && !(fabs(rho - 1.0) <= kKappa);
    const bool near_edge = EXACT && hit && t - base <= err_before + 1e-14 * z;
    if (bad_rho || near_edge) {
      rc = 0;
      base = 0.0;
    }
    if (lane == 0) {
      s_rho = EXACT ? rho : 1.0;
      s_t = bad_rho ? ur : (hit || near_edge ? t : INFINITY);
      s_base = base;
      s_chunk = rc;
      s_usep = usep;
      s_exact_total = bad_rho;
      s_bound = EXACT ? 0.0 : fast_bound(SP, SQ, p.V, bonus);
    }
  }
  __shared__ double lds[kWaves];
  __shared__ int s_j, s_jlast;
  __shared__ double s_lo, s_hi;
  if (threadIdx.x == 0) {
    s_j = 0x7fffffff;
    s_jlast = -1;
  }
  __syncthreads();
  const bool usep = s_usep;
  const double rho = s_rho;
  double t = s_t;
  double base = s_base;

  // weights of this lane's kRun consecutive tokens from v0 (0 past chi)
  auto weights = [&](long v0, long chi, double* wv) {
    float ep[kRun], eq[kRun];
    load_run<DT, VEC>(rows.rp, v0, chi, ep);
    if (bonus || usep) {
#pragma unroll
      for (int k = 0; k < kRun; ++k) eq[k] = -INFINITY;
    } else {
      load_run<DT, VEC>(rows.rq, v0, chi, eq);
    }
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const double P = wt.P(ep[k]);
      wv[k] = (bonus || usep) ? P : wt.resid(P, wt.Q(eq[k]), rho);
    }
  };

  if (s_exact_total) {  // rare: exact total over every chunk, then t
    double z = 0.0;
    for (long r0 = 0; r0 < p.V; r0 += kRound) {
      double wv[kRun], mine = 0.0;
      weights(r0 + static_cast<long>(threadIdx.x) * kRun, p.V, wv);
#pragma unroll
      for (int k = 0; k < kRun; ++k) mine += wv[k];
      z += block_sum(mine, lds);
    }
    t = t * z;  // s_t held u in this case
  }

  // rescan from the chunk holding t until the crossing is found
  for (int c = s_chunk; c < p.R3; ++c) {
    const long clo = static_cast<long>(c) * p.ch3;
    const long chi = min(static_cast<long>(p.V), clo + p.ch3);
    for (long r0 = clo; r0 < chi; r0 += kRound) {
      const long v0 = r0 + static_cast<long>(threadIdx.x) * kRun;
      double wv[kRun], mine = 0.0;
      weights(v0, chi, wv);
#pragma unroll
      for (int k = 0; k < kRun; ++k) mine += wv[k];
      double total;
      double run = base + block_exclusive_scan(mine, lds, &total);
      long found = -1, lastpos = -1;
      double flo = 0.0, fhi = 0.0;
#pragma unroll
      for (int k = 0; k < kRun; ++k) {
        if (wv[k] > 0.0) lastpos = v0 + k;
        const double before = run;
        run += wv[k];
        if (found < 0 && wv[k] > 0.0 && run > t) {
          found = v0 + k;
          flo = before;
          fhi = run;
        }
      }
      if (found >= 0) atomicMin(&s_j, static_cast<int>(found));
      if (lastpos >= 0) atomicMax(&s_jlast, static_cast<int>(lastpos));
      __syncthreads();
      if (found >= 0 && found == s_j) {
        s_lo = flo;
        s_hi = fhi;
      }
      __syncthreads();
      if (s_j != 0x7fffffff) break;  // uniform: every lane reads the same LDS value
      base += total;
    }
    if (s_j != 0x7fffffff || t == INFINITY) break;  // found, or the past-the-end rule applies
  }
  if (threadIdx.x == 0) {
    const bool found = s_j != 0x7fffffff;
    *token = found ? s_j : s_jlast;
    *zw_zero = usep && !bonus;
    *certain = EXACT || (found && fmin(t - s_lo, s_hi - t) > s_bound);
  }
}

// ---------------------------------------------------------------- kernels --
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_fast_chunks(Params p) {
  const long s = p.seq0 + blockIdx.x / p.R3;
  const int r = blockIdx.x % p.R3;
  const SeqRec rec = p.rec[s];
  const bool bonus = rec.n == p.K;
  fast_chunk_sums<DT, VEC>(p, decisive_rows<DT>(p, s, rec.n), fast_weight(p, rec), bonus, r,
                           p.csum + (s * p.R3 + r) * 5);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_fast_select(Params p) {
  const long s = p.seq0 + blockIdx.x;
  const SeqRec rec = p.rec[s];
  const bool bonus = rec.n == p.K;
  int token;
  bool zw_zero, certain;
  select_token<DT, VEC, false>(p, decisive_rows<DT>(p, s, rec.n), fast_weight(p, rec), bonus,
                               p.csum + s * p.R3 * 5, static_cast<double>(p.ur[s]), &token, &zw_zero, &certain);
  if (threadIdx.x == 0) {
    if (p.out_flags) p.out_flags[s] = rec.flags;
    if (certain && !zw_zero) {
      p.out_tokens[s * (p.K + 1) + rec.n] = token;
    } else {
      const uint32_t slot = atomicAdd(&p.qcount[0], 1u);
      p.queue[p.seq0 + slot] = static_cast<int32_t>(s);
    }
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_exact_chunks(Params p) {
  const long count = static_cast<long>(p.qcount[0]);
  for (long item = blockIdx.x; item < count * p.R3; item += gridDim.x) {
    const long s = p.queue[p.seq0 + item / p.R3];
    const int r = static_cast<int>(item % p.R3);
    const SeqRec rec = p.rec[s];
    const bool bonus = rec.n == p.K;
    __syncthreads();  // the previous item's block sums are done with their scratch
    exact_chunk_sums<DT, VEC>(p, decisive_rows<DT>(p, s, rec.n), exact_weight(p, rec), bonus, r,
                              p.xsum + (s * p.R3 + r) * 5);
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_exact_select(Params p) {
  const long count = static_cast<long>(p.qcount[0]);
  for (long e = blockIdx.x; e < count; e += gridDim.x) {
    const long s = p.queue[p.seq0 + e];
    const SeqRec rec = p.rec[s];
    const bool bonus = rec.n == p.K;
    __syncthreads();  // shared scalars of the previous entry are no longer read
    int token;
    bool zw_zero, certain;
    select_token<DT, VEC, true>(p, decisive_rows<DT>(p, s, rec.n), exact_weight(p, rec), bonus,
                                p.xsum + s * p.R3 * 5, static_cast<double>(p.ur[s]), &token, &zw_zero, &certain);
    if (threadIdx.x == 0) {
      p.out_tokens[s * (p.K + 1) + rec.n] = token;
      if (p.out_flags && zw_zero) p.out_flags[s] |= SPECV_FLAG_ZW_ZERO;
    }
  }
}

template <int DT, bool VEC>
void launch_all(const Params& p, hipStream_t st) {
  const dim3 block(kBlock);
  const unsigned ns = static_cast<unsigned>(p.nseq);
  hipLaunchKernelGGL((k_fast_chunks<DT, VEC>), dim3(ns * p.R3), block, 0, st, p);
  hipLaunchKernelGGL((k_fast_select<DT, VEC>), dim3(ns), block, 0, st, p);
  // the exact kernels walk the queue; their grids cover up to kExactSeqs
  // queued sequences in one pass, and idle workgroups exit at once
  const unsigned nx = ns < kExactSeqs ? ns : kExactSeqs;
  hipLaunchKernelGGL((k_exact_chunks<DT, VEC>), dim3(nx * p.R3), block, 0, st, p);
  hipLaunchKernelGGL((k_exact_select<DT, VEC>), dim3(nx), block, 0, st, p);
}

}  // namespace

hipError_t launch_draw(const Params& p, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (p.vec) launch_all<1, true>(p, st);
    else launch_all<1, false>(p, st);
  } else {
    if (p.vec) launch_all<0, true>(p, st);
    else launch_all<0, false>(p, st);
  }
  return hipGetLastError();
}

}  // namespace sv
