// The verify step after the row sweep, sampling mode: one workgroup of 1024
// threads per sequence runs the acceptance scan and then the fast
// replacement / bonus draw, so no partial result has to cross workgroups.
// When the batch is small enough to leave CUs idle, a sequence gets `split`
// workgroups instead (see Split below); when it has more sequences than CUs,
// workgroups of 512 threads (see launch_verify_t).
//
// Acceptance.  The 16 waves fold the sweep's per-wave (R, s) partials of the
// sequence's 2K+1 rows into log2 normalisers (fp64 sums with exact
// power-of-two rescales; the exponent of the sum exact, its mantissa's log2
// from v_log_f32).  Lane k of wave 0 evaluates u_k < min(1, p_k(x_k) / q_k(x_k))
// as an fp64 log2 ratio, and a ballot turns the K answers into n, the index of
// the first rejection (K if none).  Testing all K at once is exact: the
// outcome is the first failing test, which is what stopping there yields.
//
// Draw.  After n acceptances the token is drawn from w = max(0, p_n - q_n)
// (n < K) or w = p_K (n == K) by inverse CDF: the smallest v whose running
// sum C(v) exceeds t = u Z, Z the total.  Only the decisive row (pair) is
// reread, once.
//  - Self-normalisation.  With the sweep's normalisers L' as references the
//    fp32 weights P'(v) = 2^(x c - Wp) and Q'(v) = 2^(y c - Wq - D) are p and
//    q up to one common factor, and w = max(0, P' - rho Q') / sum P' with
//    rho = sum P' / sum Q', which is 1 up to the normalisers' error.  The
//    fast draw takes rho as 1 and adds |sum P' - sum Q'| to its error bound.
//  - Streaming.  The row is cut into segments of one or more wave iterations
//    of 64 lanes x U units (16-byte vectors, or single elements on the scalar
//    path; U = 2 on the vector path: for this pattern, two rows per CU at
//    scattered addresses, fewer loads in flight per wave measured faster
//    than U = 4 or 8 or a prefetch of the next iteration); wave w takes
//    segments w, w + 16, ...  Each lane sums its weights in fp32 pairwise
//    groups, a DPP wave sum gives the segment's mass (kept in LDS), and
//    sum P', sum Q' go to fp64 lane totals.
//  - Split.  Every workgroup of a split sequence runs the acceptance scan
//    (cheap, and the same for all) and streams every split-th block of 16
//    segments.  Each publishes its segment masses and sums in the workspace
//    (device-scope stores, waited for) and counts itself done on the
//    sequence's counter; the one that completes the count reads them all and
//    makes the draw below.  Segment masses are the same values as unsplit.
//    Device-wide fences (an L2 write-back and an invalidate) measured about
//    as costly as the split's gain; instead the sweep leaves NaN in every
//    published slot, a NaN read back is read again a bounded number of times,
//    and one still NaN sends the sequence to the fp64 draw, so the result
//    never depends on when the stores become visible.
//  - Select.  Wave 0 scans the segment masses for the segment holding t,
//    recomputes that segment's weights and finds the token with wave scans in
//    token order.  The answer stands when t is further from both ends of the
//    token's interval than a certified bound (fast_bound); otherwise the
//    sequence joins the queue of the fp64 draw, which also takes the rare
//    cases of zero residual mass and of t at or past the end.
//  - Chunk sums ahead.  A batch of at most half as many sequences as CUs
//    leaves CUs idle: more workgroups of this kernel compute the fp64 draw's
//    chunk sums of every sequence meanwhile (see eager_chunks), so that the
//    fp64 draw of the few uncertain ones needs only its select.
#include "sv_device.h"
#include "sv_exact.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kVBlock = kVerifyBlock;         // threads per workgroup
constexpr int kVWaves = kVerifyWaves;         // 16
constexpr int kVWavesSmall = kVerifyWavesSmall;  // 8
constexpr int kRowsMax = 2 * SPECV_MAX_K + 1;
constexpr int kSplitReads = 16;  // reads of the published values before the fp64 fallback

// ------------------------------------------------------------ acceptance --
// Runs on the whole workgroup.  When `writer`, writes the accepted prefix and
// the padding of out_tokens (slot n is the draw's), out_n and out_logz (the
// other workgroups of a split sequence compute the same record and write
// nothing).  Returns the record.
template <int DT, int NW>
__device__ inline SeqRec accept_scan(const Params& p, long s, bool writer) {
  constexpr int kRowsPerWave = (kRowsMax + NW - 1) / NW;  // rows each wave folds, at most
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, nrows = 2 * K + 1, np = p.nch1 * kWaves;  // kWaves: the sweep's waves per chunk
  const int kb = seq_kb(p, s);  // the sequence's own draft count
  __shared__ double sL[kRowsMax];  // log2 sum_v 2^(x_v c) of each row
  __shared__ SeqRec sRec;
  // rows the sequence uses: target rows 0..kb, draft rows 0..kb-1
  auto used = [&](int i) { return i <= K ? i <= kb : i - K - 1 < kb; };

  // wave 0 starts the draft-token gathers at once: they do not need the normalisers
  int xk = 0;
  bool valid = true;
  float xp = 0.f, xq = 0.f;
  if (w == 0 && lane < kb) {
    xk = p.x[s * K + lane];
    valid = xk >= 0 && xk < p.V;
    const int xs = valid ? xk : 0;
    xp = Elt<DT>::at(row_ptr<DT>(p.lp, s * (K + 1) + lane, p.V), xs);
    xq = Elt<DT>::at(row_ptr<DT>(p.lq, s * K + lane, p.V), xs);
  }

  // each wave folds its rows; the partial loads of the first 64 per row go out together
  float ml[kRowsPerWave];
  double sl[kRowsPerWave];
  {
    float2 q[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int i = w + r * NW;
      q[r] = (i < nrows && used(i) && lane < np) ? p.part[(s * nrows + i) * np + lane] : make_float2(-INFINITY, 0.f);
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
      const int i = w + r * NW;
      if (i < nrows && used(i)) fold_partial(ml[r], sl[r], p.part[(s * nrows + i) * np + j]);
    }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = w + r * NW;
    if (i >= nrows) break;  // uniform over the wave
    if (!used(i)) continue;
    const double lz2 = wave_log2z(ml[r], sl[r]);
    if (lane == 0) {
      sL[i] = lz2;
      if (p.out_logz && writer) p.out_logz[s * nrows + i] = static_cast<float>(lz2 * M_LN2);
    }
  }
  __syncthreads();
  if (w == 0) {
    bool accept = false;
    if (lane < kb && valid) {
      const double c = p.c;
      // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
      const double lr = (static_cast<double>(xp) * c - sL[lane]) - (static_cast<double>(xq) * c - sL[K + 1 + lane]);
      const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
      accept = static_cast<double>(p.ua[s * K + lane]) < thr;
    }
    const uint64_t lim = (kb >= 64) ? ~0ull : ((1ull << kb) - 1ull);
    const uint64_t rejected = ~static_cast<uint64_t>(__ballot(accept)) & lim;
    const int n = rejected ? __ffsll(static_cast<unsigned long long>(rejected)) - 1 : kb;
    const bool bad = __builtin_amdgcn_readlane(valid ? 1 : 0, n < kb ? n : 0) == 0 && n < kb;
    if (writer && lane <= K && lane != n) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : -1;
    if (lane == 0) {
      if (writer) p.out_n[s] = n;
      SeqRec r;
      r.n = n;
      r.kb = kb;
      r.flags = bad ? SPECV_FLAG_BAD_DRAFT : 0;
      r.seq = static_cast<int32_t>(s);
      r.lzp = sL[n];
      r.lzq = n < kb ? sL[K + 1 + n] : 0.0;
      sRec = r;
    }
  }
  __syncthreads();
  return sRec;
}

// Whole wave: log2 sum_v 2^(x_v c) of row i of sequence s, folded from the
// sweep's partials in accept_scan's order (lane l takes partials l, l + 64,
// ...), so the value is bit for bit the one accept_scan computes for it.
__device__ inline double fold_row(const Params& p, long s, int nrows, int i, int np) {
  const int lane = threadIdx.x % kWave;
  const float2* base = p.part + (s * nrows + i) * np;
  float ml = -INFINITY;
  double sl = 0.0;
  for (int j = lane; j < np; j += kWave) fold_partial(ml, sl, base[j]);
  return wave_log2z(ml, sl);
}

// After the sweep's rounds, for a sequence decided before the last round:
// n = kbs[s] (its first rejection, or K_b with every draft accepted).
// k_round_accept ran the acceptance tests of those positions on the same
// partials with the same fold and test, so accept_scan would find the same n;
// the record needs only the normalisers of the decisive rows (folded as
// accept_scan folds them) and the tokens before n.  Wave 0 does it all, one
// memory round trip instead of accept_scan's gathers and folds of every row.
// Writes and returns what accept_scan would (there is no log Z to write:
// calls that ask for it take the one-sweep path).
template <int DT>
__device__ inline SeqRec decided_scan(const Params& p, long s, int n, bool writer) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int K = p.K, nrows = 2 * K + 1, np = p.nch1 * kWaves;
  const int kb = seq_kb(p, s);
  __shared__ SeqRec sRecD;
  if (w == 0) {
    const int xk = (lane <= n && lane < kb) ? p.x[s * K + lane] : 0;
    const double lzp = fold_row(p, s, nrows, n, np);
    const double lzq = n < kb ? fold_row(p, s, nrows, K + 1 + n, np) : 0.0;  // uniform
    const bool valid = xk >= 0 && xk < p.V;
    const bool bad = n < kb && __builtin_amdgcn_readlane(valid ? 1 : 0, n < kb ? n : 0) == 0;
    if (writer && lane <= K && lane != n) p.out_tokens[s * (K + 1) + lane] = lane < n ? xk : -1;
    if (lane == 0) {
      if (writer) p.out_n[s] = n;
      SeqRec r;
      r.n = n;
      r.kb = kb;
      r.flags = bad ? SPECV_FLAG_BAD_DRAFT : 0;
      r.seq = static_cast<int32_t>(s);
      r.lzp = lzp;
      r.lzq = lzq;
      sRecD = r;
    }
  }
  __syncthreads();
  return sRecD;
}

// ------------------------------------------------------------------ draw --
// fp32 weights scaled by the common factor 2^Fp: P' = 2^(x c - Wp) and
// Q' = 2^((y c - Wq) - D), with Wp, Wq = rint(L') whole, Fp, Fq the remaining
// fractions and D = Fq - Fp, so both references keep the fp32 accuracy of
// the fractions, not of L'.  A common factor leaves the draw unchanged (it
// normalises by its own sums), and -inf logits give weights of exactly 0.
struct FastWeight {
  float c, Wp, Wq, D;
  __device__ float P(float x) const { return ex2(fmaf(x, c, -Wp)); }
  __device__ float Q(float x) const { return ex2(fmaf(x, c, -Wq) - D); }
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

// A pointer that is the same in every lane, moved to scalar registers so that
// address arithmetic on it stays scalar.
template <class T>
__device__ inline const T* uniform_ptr(const T* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Segment geometry of a row: units of PV elements, wave iterations of
// 64 x U units, segments of `iters` iterations, at most kMaxSegs segments.
template <int DT, bool VEC>
struct Geometry {
  static constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  static constexpr int U = draw_lane_units(VEC);
  static constexpr int kIterUnits = kWave * U;
  long units;
  int iters, nseg;
  __device__ explicit Geometry(int V) {
    const SegGeom sg = seg_geom(V, PV, VEC);
    units = sg.units;
    iters = sg.iters;
    nseg = sg.nseg;
  }
};

// One wave iteration at unit `base`: this lane's units base + i*64 + lane
// (i < U) of the target row (and of the draft row unless BONUS), held raw
// and widened one unit at a time.  NT: non-temporal loads, for the stream,
// which reads each unit once (the sharp workload's step 719.8 -> 694.9 us);
// the rescan of one segment keeps ordinary loads.  Bit i of `live` says whether unit i lies
// inside the row.  Vector path: units are addressed from the iteration's
// scalar base with 32-bit offsets, and a unit past the row's end reads the
// row's last unit again (its sums must be skipped, or its elements masked).
// Scalar path: elements past the end read as -inf.
template <int DT, bool VEC, bool BONUS>
struct Iter {
  using G = Geometry<DT, VEC>;
  static constexpr int NR = VEC ? G::U : 1;
  static constexpr int NS = VEC ? 1 : G::U;
  uint4 rp[NR], rq[NR];     // vector path: the raw units
  float xp[NS], xq[NS];     // scalar path: the elements
  uint32_t live;            // bit i: unit i lies inside the row

  template <bool NT = false>
  __device__ void load(const void* rowp, const void* rowq, long base, long units) {
    const uint32_t lane = threadIdx.x % kWave;
    const long rem = units - base;  // > 0
    const uint32_t in_row = static_cast<uint32_t>(rem < G::kIterUnits ? rem : G::kIterUnits);
    live = 0;
#pragma unroll
    for (int i = 0; i < G::U; ++i) live |= ((i * kWave + lane) < in_row ? 1u : 0u) << i;
    if constexpr (VEC) {
      // the iteration's base in scalar registers, a 32-bit offset per lane
      const uint4* bp = uniform_ptr(static_cast<const uint4*>(rowp) + base);
      const uint4* bq = BONUS ? nullptr : uniform_ptr(static_cast<const uint4*>(rowq) + base);
      const uint32_t last = in_row - 1;
#pragma unroll
      for (int i = 0; i < G::U; ++i) {
        const uint32_t off = min(static_cast<uint32_t>(i * kWave) + lane, last);
        if constexpr (NT) {
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bp) + off);
          rp[i] = make_uint4(a.x, a.y, a.z, a.w);
          if constexpr (!BONUS) {
            const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bq) + off);
            rq[i] = make_uint4(c.x, c.y, c.z, c.w);
          }
        } else {
          rp[i] = bp[off];
          if constexpr (!BONUS) rq[i] = bq[off];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::U; ++i) {
        xp[i] = load_masked<DT>(rowp, base + i * kWave + lane, units);
        if constexpr (!BONUS) xq[i] = load_masked<DT>(rowq, base + i * kWave + lane, units);
      }
    }
  }
  __device__ bool is_live(int i) const { return (live >> i) & 1u; }
  // unit i of the target (Q_ROW false) or draft (true) row; MASK: -inf when
  // the unit lies past the row's end (otherwise it may repeat the last unit)
  template <bool Q_ROW, bool MASK>
  __device__ void unit(int i, float (&e)[G::PV]) const {
    if constexpr (VEC) {
      Elt<DT>::unpack(Q_ROW ? rq[i] : rp[i], e);
      if (MASK && !is_live(i)) {
#pragma unroll
        for (int k = 0; k < G::PV; ++k) e[k] = -INFINITY;
      }
    } else {
      e[0] = Q_ROW ? xq[i] : xp[i];
    }
  }
};

// Stream the decisive row(s): segment masses into segA, fp64 lane totals of
// P' and Q'.  Per unit the sums are pairwise in fp32, then pairwise over the
// lane's U units; the residual mass of a lane is sum P' - sum min(P', Q').
// Segments come in blocks of NW (one per wave); workgroup `part` of a
// sequence split over `split` takes blocks part, part + split, ...  A
// segment's mass does not depend on which workgroup computes it.
template <int DT, bool VEC, bool BONUS, int NW>
__device__ inline void stream_row(const void* rp, const void* rq, const FastWeight& wt, const Geometry<DT, VEC>& g,
                                  int part, int split, float* segA, double& tsp, double& tsq) {
  using G = Geometry<DT, VEC>;
  const int lane = threadIdx.x % kWave, w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int j = part * NW + w; j < g.nseg; j += NW * split) {
    float a = 0.f;
    for (int it = 0; it < g.iters; ++it) {
      const long base = (static_cast<long>(j) * g.iters + it) * G::kIterUnits;
      if (base >= g.units) break;  // uniform over the wave
      Iter<DT, VEC, BONUS> t;
      t.template load<true>(rp, rq, base, g.units);
      float up[G::U], uq[G::U], um[G::U];
#pragma unroll
      for (int i = 0; i < G::U; ++i) {
        float ep[G::PV], sp[G::PV], sq[G::PV], sm[G::PV];
        t.template unit<false, false>(i, ep);
#pragma unroll
        for (int k = 0; k < G::PV; ++k) sp[k] = wt.P(ep[k]);
        if constexpr (!BONUS) {
          float eq[G::PV];
          t.template unit<true, false>(i, eq);
#pragma unroll
          for (int k = 0; k < G::PV; ++k) {
            sq[k] = wt.Q(eq[k]);
            sm[k] = fminf(sp[k], sq[k]);
          }
        }
#pragma unroll
        for (int h = G::PV / 2; h > 0; h >>= 1)
#pragma unroll
          for (int k = 0; k < h; ++k) {
            sp[k] += sp[k + h];
            if constexpr (!BONUS) {
              sq[k] += sq[k + h];
              sm[k] += sm[k + h];
            }
          }
        const bool in = t.is_live(i);  // a repeated last unit adds nothing
        up[i] = in ? sp[0] : 0.f;
        if constexpr (!BONUS) {
          uq[i] = in ? sq[0] : 0.f;
          um[i] = in ? sm[0] : 0.f;
        } else {
          uq[i] = um[i] = 0.f;
        }
      }
#pragma unroll
      for (int h = G::U / 2; h > 0; h >>= 1)
#pragma unroll
        for (int k = 0; k < h; ++k) {
          up[k] += up[k + h];
          uq[k] += uq[k + h];
          um[k] += um[k + h];
        }
      a += BONUS ? up[0] : up[0] - um[0];
      tsp += up[0];
      tsq += uq[0];
    }
    const float seg = wave_sum_f32(a);
    if (lane == 0) segA[j] = seg;
  }
}

// Certified bound on how far the fast draw's t - C(v) can be from the exact
// one (C a running sum of the residual, t = u Z), in the units of P'.
// Per weight, the exponent carries roundings that grow with its size |f|
// (c's own rounding, the fma, the subtraction of D; a common offset cancels
// when P' is normalised by its own sum), at most u (3 |f| + 1), and v_exp_f32
// one ulp (measured <= 0.78), so the relative error is <= u (2.7 + 2.08 |f|),
// u = 2^-24.  Summed over a row, sum P' |f| <= sum P' (log2 V + 1) (an entropy
// bound).  The fp32 sums (within a unit, over a lane's units, over the
// segment's iterations, the DPP wave sum), the residual's subtraction and the
// rescan's rounding add at most (13 + iters) u (SP + SQ).  So one running sum is off by
// R <= u (16 + iters + 2.1 (log2 V + 1)) (SP + SQ), and t by as much.  Taking
// rho as 1 moves each residual weight by at most |rho - 1| Q', so a running
// sum and Z by at most |SP - SQ|.  Both errors enter twice (t and C), and the
// whole carries a safety factor of 2.
__device__ inline double fast_bound(double SP, double SQ, int V, int iters, bool bonus) {
  const double u = 0x1p-24;
  const double R = u * (16.0 + iters + 2.1 * (log2(static_cast<double>(V)) + 1.0)) * (SP + SQ);
  return 2.0 * (2.0 * R + (bonus ? 0.0 : 2.0 * fabs(SP - SQ)));
}

// Wave 0: find the token of segment j whose running sum first exceeds t,
// given the mass `base` of the segments before it.  Weights are recomputed
// exactly as in stream_row; token order within an iteration is (unit i,
// lane, element k).
// Returns false when rounding leaves the crossing outside the segment.
template <int DT, bool VEC, bool BONUS>
__device__ inline bool rescan_segment(const void* rp, const void* rq, const FastWeight& wt,
                                      const Geometry<DT, VEC>& g, int j, double base, double t,
                                      int* token, double* lo, double* hi) {
  using G = Geometry<DT, VEC>;
  const int lane = threadIdx.x % kWave;
  for (int it = 0; it < g.iters; ++it) {
    const long ubase = (static_cast<long>(j) * g.iters + it) * G::kIterUnits;
    if (ubase >= g.units) break;
    Iter<DT, VEC, BONUS> tl;
    tl.load(rp, rq, ubase, g.units);
#pragma unroll
    for (int i = 0; i < G::U; ++i) {
      float wv[G::PV];
      {
        float ep[G::PV];
        tl.template unit<false, true>(i, ep);
#pragma unroll
        for (int k = 0; k < G::PV; ++k) wv[k] = wt.P(ep[k]);
        if constexpr (!BONUS) {
          float eq[G::PV];
          tl.template unit<true, true>(i, eq);
#pragma unroll
          for (int k = 0; k < G::PV; ++k) wv[k] = fmaxf(wv[k] - wt.Q(eq[k]), 0.f);
        }
      }
      double mine = 0.0;
#pragma unroll
      for (int k = 0; k < G::PV; ++k) mine += wv[k];
      const double inc = wave_inclusive_scan(mine);
      const double total = readlane_f64(inc, kWave - 1);
      const uint64_t hit = __ballot(base + inc > t);
      if (hit) {
        const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        int tk = -1;
        double tlo = 0.0, thi = 0.0;
        if (lane == L) {
          double run = base + inc - mine;
#pragma unroll
          for (int k = 0; k < G::PV; ++k) {
            const double before = run;
            run += wv[k];
            if (tk < 0 && wv[k] > 0.f && run > t) {
              tk = k;
              tlo = before;
              thi = run;
            }
          }
        }
        tk = __builtin_amdgcn_readlane(tk, L);
        if (tk < 0) return false;  // the lane's sum crossed t only by rounding
        *token = static_cast<int>((ubase + i * kWave + L) * G::PV + tk);
        *lo = readlane_f64(tlo, L);
        *hi = readlane_f64(thi, L);
        return true;
      }
      base += total;
    }
  }
  return false;
}

// Two block sums with one pair of barriers; each is summed in the same order
// as block_sum_n, so the results are bitwise the same.
template <int NW>
__device__ inline void block_sum2_n(double& a, double& b, double* lds /* >= 2 NW */) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) {
    lds[w] = a;
    lds[NW + w] = b;
  }
  __syncthreads();
  double ta = 0.0, tb = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    ta += lds[i];
    tb += lds[NW + i];
  }
  a = ta;
  b = tb;
}

// SPLIT: the sequence's stream is shared by p.split workgroups (`part` is
// this one's index), which exchange their results through the workspace.
template <int DT, bool VEC, bool BONUS, bool SPLIT, int NW>
__device__ inline void fast_draw(const Params& p, long s, const SeqRec& rec, int part) {
  using G = Geometry<DT, VEC>;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const G g(p.V);
  const FastWeight wt = fast_weight(p, rec);
  // rec comes from LDS: make the decisive row's index wave-uniform, so the
  // stream's addresses are formed in scalar registers
  const int n = __builtin_amdgcn_readfirstlane(rec.n);
  const void* rp = row_ptr<DT>(p.lp, s * (p.K + 1) + n, p.V);
  const void* rq = BONUS ? nullptr : row_ptr<DT>(p.lq, s * p.K + n, p.V);
  __shared__ float segA[kMaxSegs];
  __shared__ double lds[2 * NW];

  const int split = SPLIT ? p.split : 1;
  double tsp = 0.0, tsq = 0.0;
  stream_row<DT, VEC, BONUS, NW>(rp, rq, wt, g, part, split, segA, tsp, tsq);
  // the reductions' barriers also publish segA
  double SP = tsp, SQ = 0.0;
  if constexpr (BONUS) {
    SP = block_sum_n<NW>(tsp, lds);
  } else {
    SQ = tsq;
    block_sum2_n<NW>(SP, SQ, lds);
  }
  if (w != 0) return;

  // segments per lane, consecutive; wave scan of the lanes' masses
  constexpr int kPer = kMaxSegs / kWave;
  const int per = (g.nseg + kWave - 1) / kWave;
  float segv[SPLIT ? kPer : 1];  // split: this lane's segment masses, read from the workspace
  double mine = 0.0;
  if constexpr (SPLIT) {
    // publish this workgroup's segment masses and sums with device-scope
    // stores over the NaN the sweep left there, wait for them, and count this
    // workgroup done; the sequence's last workgroup makes the draw
    float* gseg = p.segm + s * g.nseg;
    double* gsum = p.spq + (s * kMaxSplit) * 2;
    for (int k = lane;; k += kWave) {  // this workgroup's k-th segment, in increasing order
      const int j = ((k / NW) * split + part) * NW + k % NW;
      if (j >= g.nseg) break;
      __hip_atomic_store(gseg + j, segA[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) {
      __hip_atomic_store(gsum + 2 * part, SP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(gsum + 2 * part + 1, SQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the stores have completed
    uint32_t prior = 0;
    if (lane == 0) prior = __hip_atomic_fetch_add(&p.vcount[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prior = __builtin_amdgcn_readlane(prior, 0);
    if (prior != static_cast<uint32_t>(split - 1)) return;  // uniform over the wave
    // the last one: every workgroup's masses and sums (device-scope loads).
    // Every other workgroup counted itself done only after its stores had
    // completed, so a value still NaN is one whose store is not yet visible
    // here: read again, a bounded number of times.  If one is still NaN the
    // sequence goes to the fp64 draw, which needs none of them, so the draw
    // never depends on when the other workgroups' stores become visible.
    bool seen = false;
    double psp = 0.0, psq = 0.0;
    for (int attempt = 0; attempt < kSplitReads && !seen; ++attempt) {  // uniform over the wave
      if (attempt > 0) __builtin_amdgcn_s_sleep(2);
      bool mine_seen = true;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int j = lane * per + k;
        segv[k] = (k < per && j < g.nseg) ? __hip_atomic_load(gseg + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                          : 0.f;
        mine_seen &= !isnan(segv[k]);
      }
      if (lane < split) {
        psp = __hip_atomic_load(gsum + 2 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        psq = __hip_atomic_load(gsum + 2 * lane + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine_seen &= !(isnan(psp) || isnan(psq));
      }
      seen = __ballot(!mine_seen) == 0;
    }
    if (!seen) {  // uniform
      if (lane == 0) {
        if (p.out_flags) p.out_flags[s] = rec.flags | SPECV_FLAG_FP64;
        const uint32_t slot = atomicAdd(&p.qcount[0], 1u);
        p.queue[p.seq0 + slot] = rec;
      }
      return;
    }
    SP = wave_sum(psp);
    SQ = BONUS ? 0.0 : wave_sum(psq);
#pragma unroll
    for (int k = 0; k < kPer; ++k) mine += segv[k];  // adding the zeros past `per` changes nothing
  } else {
    for (int k = 0; k < per; ++k) {
      const int j = lane * per + k;
      if (j < g.nseg) mine += segA[j];
    }
  }
  const double inc = wave_inclusive_scan(mine);
  const double Z = readlane_f64(inc, kWave - 1);
  const double t = static_cast<double>(p.ur[s]) * Z;
  const uint64_t hit = __ballot(inc > t);
  bool certain = false;
  int token = -1;
  if (Z > 0.0 && hit) {
    const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    int jseg = -1;
    double jbase = 0.0;
    if (lane == L) {
      double run = inc - mine;
      if constexpr (SPLIT) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int j = lane * per + k;
          if (jseg < 0 && k < per && j < g.nseg) {
            if (run + segv[k] > t) jseg = j;
            else run += segv[k];
          }
        }
      } else {
        for (int k = 0; k < per && jseg < 0; ++k) {
          const int j = lane * per + k;
          if (j < g.nseg) {
            if (run + segA[j] > t) jseg = j;
            else run += segA[j];
          }
        }
      }
      jbase = run;
    }
    jseg = __builtin_amdgcn_readlane(jseg, L);  // L is uniform (from a ballot)
    jbase = readlane_f64(jbase, L);
    double lo = 0.0, hi = 0.0;
    if (jseg >= 0 && rescan_segment<DT, VEC, BONUS>(rp, rq, wt, g, jseg, jbase, t, &token, &lo, &hi))
      certain = fmin(t - lo, hi - t) > fast_bound(SP, SQ, p.V, g.iters, BONUS);
  }
  if (lane == 0) {
    if (p.out_flags) p.out_flags[s] = rec.flags | (certain ? 0 : SPECV_FLAG_FP64);
    if (certain) p.out_tokens[s * (p.K + 1) + rec.n] = token;
    if (p.xeager > 0) {  // every sequence's outcome, by sequence (see eager_chunks)
      SeqRec q = rec;
      if (certain) q.seq = -1;
      p.queue[s] = q;
    } else if (!certain) {
      const uint32_t slot = atomicAdd(&p.qcount[0], 1u);
      p.queue[p.seq0 + slot] = rec;
    }
  }
}

// Small batches leave most CUs idle while the fast draws run.  There
// (p.xeager > 0) workgroup nseq + e, e = i * xeager + part, computes the fp64
// draw's chunk sums of sequence seq0 + i for chunks part * xper .. + xper - 1,
// 128 threads per chunk, whether or not the fast draw will need them: the
// acceptance scan first (the same record as the sequence's own workgroup;
// it writes nothing), then the sums into xsum by sequence.  The fp64 draw
// then needs only its select (k_exact.hip), and the sums are those its own
// chunk kernel would compute.
template <int DT, bool VEC, int NW>
__device__ inline void eager_chunks(const Params& p, long e) {
  constexpr int kGroups = NW * kWave / kXBlock;
  const long local = e / p.xeager;
  const int part = static_cast<int>(e - local * p.xeager);
  const long s = p.seq0 + local;
  const int kd = p.vpre > 0 ? p.kbs[s] : p.vpre;
  const SeqRec rec = kd < p.vpre ? decided_scan<DT>(p, s, kd, false) : accept_scan<DT, NW>(p, s, false);
  const bool bonus = rec.n == rec.kb;
  const Rows<DT> rows = decisive_rows<DT>(p, s, rec);
  const ExactWeight wt = exact_weight(p, rec);
  const int grp = static_cast<int>(threadIdx.x / kXBlock);
  const int r0 = part * p.xper, r1 = min(p.R3, r0 + p.xper);
  double* out = p.xsum + s * p.R3 * 5;
  for (int r = r0; r < r1; r += kGroups) {  // the same trip count for every group
    const int rg = r + grp;
    exact_chunk_sums<DT, VEC>(p, rows, wt, bonus, rg < r1 ? rg : p.R3, rg < r1 ? out + rg * 5 : nullptr);
  }
}

// Workgroup g takes sequence seq0 + g (SPLIT: seq0 + g / split, part g % split).
// NW waves per workgroup: kVWaves (16), or kVWavesSmall (8) when the batch
// has more sequences than the device has CUs (see launch_verify_t).
template <int DT, bool VEC, bool SPLIT, int NW>
__global__ __launch_bounds__(NW * kWave) void k_verify(Params p) {
  long s = p.seq0 + blockIdx.x;
  int part = 0;
  if constexpr (!SPLIT && NW == kVWaves) {
    if (static_cast<long>(blockIdx.x) >= p.nseq) {  // xeager > 0 (uniform over the workgroup)
      eager_chunks<DT, VEC, NW>(p, blockIdx.x - p.nseq);
      return;
    }
  }
  if constexpr (SPLIT) {
    const uint32_t split = static_cast<uint32_t>(p.split);
    const uint32_t local = blockIdx.x / split;
    part = static_cast<int>(blockIdx.x - local * split);
    s = p.seq0 + local;
  }
  // uniform over the workgroup: a sequence decided before the last round
  // needs no acceptance scan
  const int kd = p.vpre > 0 ? p.kbs[s] : p.vpre;
  const SeqRec rec =
      kd < p.vpre ? decided_scan<DT>(p, s, kd, part == 0) : accept_scan<DT, NW>(p, s, part == 0);
  if (rec.n == rec.kb) fast_draw<DT, VEC, true, SPLIT, NW>(p, s, rec, part);
  else fast_draw<DT, VEC, false, SPLIT, NW>(p, s, rec, part);
}

// One 1024-thread workgroup of k_verify fills a CU (its registers), so a
// batch of more sequences than CUs would run in generations that each wait
// for their slowest sequence, every workgroup's acceptance and select phases
// exposed.  There (p.vwaves == kVWavesSmall) 512-thread workgroups let two
// sequences share a CU, one's latency phases overlapping the other's stream.
// Segment masses do not depend on which wave computes them, so both shapes
// draw the same tokens.
template <int DT, bool VEC>
void launch_verify_t(const Params& p, hipStream_t st) {
  const unsigned n = static_cast<unsigned>(p.nseq);
  if (p.split > 1)
    hipLaunchKernelGGL((k_verify<DT, VEC, true, kVWaves>), dim3(n * static_cast<unsigned>(p.split)), dim3(kVBlock), 0,
                       st, p);
  else if (p.vwaves == kVWavesSmall)
    hipLaunchKernelGGL((k_verify<DT, VEC, false, kVWavesSmall>), dim3(n), dim3(kVWavesSmall * kWave), 0, st, p);
  else  // and the chunk-sum workgroups when xeager > 0
    hipLaunchKernelGGL((k_verify<DT, VEC, false, kVWaves>), dim3(n * (1u + static_cast<unsigned>(p.xeager))),
                       dim3(kVBlock), 0, st, p);
}

}  // namespace

hipError_t launch_verify(const Params& p, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (p.vec) launch_verify_t<1, true>(p, st);
    else launch_verify_t<1, false>(p, st);
  } else {
    if (p.vec) launch_verify_t<0, true>(p, st);
    else launch_verify_t<0, false>(p, st);
  }
  return hipGetLastError();
}

}  // namespace sv
