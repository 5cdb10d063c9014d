// The fp64 draw, for the sequences whose fast draw could not be certified.
//
// The draw is the same inverse CDF as the fast one (the smallest token v
// whose running sum C(v) of w exceeds t = u Z; w = max(0, p_n - q_n) after a
// rejection at n < K, w = p_K after K acceptances), with fp64 weights
// P(v) = exp(x/T - L'p), Q(v) = exp(y/T - L'q) normalised by their own sums:
// w = max(0, P - rho Q) / sum P with rho = sum P / sum Q.
//
// Two kernels walk the queue the fast draw filled (each entry is the
// sequence's whole record, read together with the queue's length); rows of
// at most two chunks take one kernel that does both (k_exact_solo), and on
// small batches k_verify's spare workgroups have already computed every
// sequence's chunk sums, so the select runs alone (k_exact_select_seq):
//   exact_chunks (queued sequences x chunks of ch3 >= 1024 tokens): per chunk
//        sum P, sum Q, A = sum max(0, P - Q), G = sum_{P > Q} Q and
//        H = sum_{near flip} Q, the Q-mass within a relative kKappa of P = Q.
//        The chunk's residual mass at the exact rho is A - (rho - 1) G up to
//        the mass of tokens whose sign flips, which is at most |rho - 1| H.
//   exact_select (one workgroup per queued sequence): rho and the corrected
//        chunk sums give Z and the chunk holding t; that chunk is rescanned
//        (lane-contiguous runs, fp64 scan over 128 threads) with the exact
//        rho.  When t may lie before the located chunk (within the
//        corrections' error) the rescan starts from the first chunk; when rho
//        leaves the linearisation window the total is recomputed exactly
//        first.
// Per weight the error is ~1e-16 relative (exp_f64), so the token matches the
// exact inverse CDF unless t lies within ~1e-12 of an edge.  Past the end the
// draw takes the last token with positive weight; a residual of zero mass
// (p == q to rounding) falls back to p_n and sets a flag.
#include "sv_device.h"
#include "sv_exact.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr unsigned kExactSeqs = 32;              // queued sequences the kernels cover per pass, at least
constexpr unsigned kExactMaxGroups = 8192;       // chunk workgroups per pass, at most (beyond kExactSeqs rows)
constexpr unsigned kSoloSeqs = 256;              // queued sequences k_exact_solo covers per pass
constexpr int kMaxPer = (kMaxDrawChunks + kWave - 1) / kWave;  // chunks per lane in the select

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
// A queued sequence's chunk sums as wave 0 holds them: lane l owns chunks
// l*per .. l*per + per - 1 (per <= kMaxPer), 0 past the row.  They live at
// the sequence's queue slot (not its index), so the select can load them
// together with the queue entry instead of after it.
struct ChunkSums {
  double v[kMaxPer][5];
};

__device__ inline ChunkSums load_chunk_sums(const Params& p, long slot) {
  ChunkSums cv;
  const double* base = p.xsum + (p.seq0 + slot) * p.R3 * 5;
  const int lane = threadIdx.x % kWave, per = (p.R3 + kWave - 1) / kWave;
  // branch-free: every lane loads (outside the row, the first chunk's sums
  // again) and masks, so all loads are in flight together.  Relaxed atomic
  // loads, which the compiler keeps where they are written: callers load
  // these ahead of the test that decides whether they are needed.
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int c = lane * per + k;
    const bool in = threadIdx.x < kWave && k < per && c < p.R3;
#pragma unroll
    for (int f = 0; f < 5; ++f) {
      const double x = __hip_atomic_load(base + (in ? c : 0) * 5 + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      cv.v[k][f] = in ? x : 0.0;
    }
  }
  return cv;
}

// The draw for one queued sequence from its chunk sums (whole workgroup;
// cv matters in wave 0 only).  Thread 0 gets the token and whether the
// zero-mass fallback was used.
template <int DT, bool VEC>
__device__ inline void select_exact(const Params& p, const Rows<DT>& rows, const ExactWeight& wt, bool bonus,
                                    const ChunkSums& cv, double ur, int* token, bool* zw_zero) {
  const int lane = threadIdx.x % kWave;
  __shared__ double s_rho, s_t;
  __shared__ double s_base;
  __shared__ int s_chunk, s_usep, s_exact_total;
  if (threadIdx.x < kWave) {
    const int per = (p.R3 + kWave - 1) / kWave;
    auto cs = [&](int k, int f) { return cv.v[k][f]; };
    double sp_l = 0.0, sq_l = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      sp_l += cs(k, 0);
      if (!bonus) sq_l += cs(k, 1);
    }
    const double SP = wave_sum(sp_l);
    double rho = 1.0;
    int usep = 1;
    // chunk k's mass: the residual corrected to first order in rho - 1 (and
    // its error bound), or p's mass for a bonus or zero-residual draw
    auto mass = [&](int k, bool use_p) {
      return use_p ? cs(k, 0) : fmax(cs(k, 2) - (rho - 1.0) * cs(k, 3), 0.0);
    };
    auto merr = [&](int k, bool use_p) { return use_p ? 0.0 : fabs(rho - 1.0) * cs(k, 4); };
    if (!bonus) {
      const double SQ = wave_sum(sq_l);
      rho = SP / SQ;
      double z_l = 0.0;
#pragma unroll
      for (int k = 0; k < kMaxPer; ++k) z_l += mass(k, false);
      usep = !(wave_sum(z_l) > 0.0);  // p == q to rounding: draw from p_n instead
    }
    const bool use_p = bonus || usep;
    double v = 0.0, err = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      v += mass(k, use_p);
      err += merr(k, use_p);
    }
    const double inc = wave_inclusive_scan(v);
    const double err_inc = wave_inclusive_scan(err);
    const double z = readlane_f64(inc, kWave - 1);
    const double t = ur * z;
    const uint64_t hit = __ballot(inc > t);
    const uint64_t pos = __ballot(v > 0.0);
    // the lane holding the crossing (or, past the end, the last mass) finds its chunk
    const int L = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1
                      : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
    int rc = 0;
    double base = 0.0, err_before = 0.0;
    if (lane == L) {
      // the chunk where the running mass passes t; if rounding finds none in
      // this lane (or past the end), the lane's last chunk with mass
      double run = inc - v, erun = err_inc - err;
      int last = lane * per;
      double run_last = run, erun_last = erun;
      rc = -1;
#pragma unroll
      for (int k = 0; k < kMaxPer; ++k) {  // chunks past the row have no mass
        const int c = lane * per + k;
        const double m = mass(k, use_p);
        if (rc < 0 && k < per && c < p.R3) {
          if (hit && run + m > t) {
            rc = c;
          } else {
            if (m > 0.0) {
              last = c;
              run_last = run;
              erun_last = erun;
            }
            run += m;
            erun += merr(k, use_p);
          }
        }
      }
      if (rc < 0) {
        rc = last;
        run = run_last;
        erun = erun_last;
      }
      base = run;
      err_before = erun;
    }
    rc = __builtin_amdgcn_readlane(rc, L);  // L is uniform (from ballots)
    base = readlane_f64(base, L);
    err_before = readlane_f64(err_before, L);
    // t may lie before the located chunk when it is within the base's error,
    // and the first-order correction needs rho near 1
    const bool bad_rho = !bonus && !usep && !(fabs(rho - 1.0) <= kKappa);
    const bool near_edge = hit && t - base <= err_before + 1e-14 * z;
    if (bad_rho || near_edge) {
      rc = 0;
      base = 0.0;
    }
    if (lane == 0) {
      s_rho = rho;
      s_t = bad_rho ? ur : (hit || near_edge ? t : INFINITY);
      s_base = base;
      s_chunk = rc;
      s_usep = usep;
      s_exact_total = bad_rho;
    }
  }
  __shared__ double lds[kXWaves];
  __shared__ int s_j, s_jlast;
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
      wv[k] = (bonus || usep) ? P : fmax(P - rho * wt.Q(eq[k]), 0.0);
    }
  };

  if (s_exact_total) {  // rare: exact total over every chunk, then t
    double z = 0.0;
    for (long r0 = 0; r0 < p.V; r0 += kRound) {
      double wv[kRun], mine = 0.0;
      weights(r0 + static_cast<long>(threadIdx.x) * kRun, p.V, wv);
#pragma unroll
      for (int k = 0; k < kRun; ++k) mine += wv[k];
      z += block_sum_n<kXWaves>(mine, lds);
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
      double run = base + block_exclusive_scan_n<kXWaves>(mine, lds, &total);
      int found = -1, lastpos = -1;
#pragma unroll
      for (int k = 0; k < kRun; ++k) {
        if (wv[k] > 0.0) lastpos = static_cast<int>(v0 + k);
        run += wv[k];
        if (found < 0 && wv[k] > 0.0 && run > t) found = static_cast<int>(v0 + k);
      }
      // one LDS atomic per wave: the wave's first crossing and last positive weight
      const int fw = wave_min_i32(found >= 0 ? found : 0x7fffffff);
      const int lw = wave_max_i32(lastpos);
      if (lane == 0) {
        if (fw != 0x7fffffff) atomicMin(&s_j, fw);
        if (lw >= 0) atomicMax(&s_jlast, lw);
      }
      __syncthreads();
      if (s_j != 0x7fffffff) break;  // uniform: every lane reads the same LDS value
      base += total;
    }
    if (s_j != 0x7fffffff || t == INFINITY) break;  // found, or the past-the-end rule applies
  }
  if (threadIdx.x == 0) {
    *token = s_j != 0x7fffffff ? s_j : s_jlast;
    *zw_zero = usep && !bonus;
  }
}

// ---------------------------------------------------------------- kernels --
// Queue entry `slot`, read before the queue's length is known so that both
// loads are in flight together: the index is clamped into the queue's storage
// (branch-free), and the entry is used only when slot < count.  The loops
// test `first.seq >= 0` (true for every live entry) with a non-short-circuit &
// in their condition, which keeps the compiler from moving this load behind
// the test of the count.
__device__ inline SeqRec entry_ahead(const Params& p, long slot) {
  return p.queue[p.seq0 + min(slot, static_cast<long>(p.nseq) - 1)];
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kXBlock) void k_exact_chunks(Params p) {
  const SeqRec first = entry_ahead(p, blockIdx.x / p.R3);
  const long count = static_cast<long>(p.qcount[0]);
  for (long item = blockIdx.x; (item < count * p.R3) & (first.seq >= 0); item += gridDim.x) {
    SeqRec rec = first;
    if (item != blockIdx.x) rec = p.queue[p.seq0 + item / p.R3];
    const long s = rec.seq;
    const int r = static_cast<int>(item % p.R3);
    const bool bonus = rec.n == rec.kb;
    exact_chunk_sums<DT, VEC>(p, decisive_rows<DT>(p, s, rec), exact_weight(p, rec), bonus, r,
                              p.xsum + ((p.seq0 + item / p.R3) * p.R3 + r) * 5);  // by queue slot
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kXBlock) void k_exact_select(Params p) {
  const SeqRec first = entry_ahead(p, blockIdx.x);
  const long count = static_cast<long>(p.qcount[0]);
  // the first entry's chunk sums, loaded with the entry (slot clamped like it)
  const ChunkSums first_cv = load_chunk_sums(p, min(static_cast<long>(blockIdx.x), static_cast<long>(p.nseq) - 1));
  for (long e = blockIdx.x; (e < count) & (first.seq >= 0); e += gridDim.x) {
    SeqRec rec = first;
    ChunkSums cv = first_cv;
    if (e != blockIdx.x) {
      rec = p.queue[p.seq0 + e];
      cv = load_chunk_sums(p, e);
    }
    const long s = rec.seq;
    const bool bonus = rec.n == rec.kb;
    __syncthreads();  // shared scalars of the previous entry are no longer read
    int token;
    bool zw_zero;
    select_exact<DT, VEC>(p, decisive_rows<DT>(p, s, rec), exact_weight(p, rec), bonus, cv,
                          static_cast<double>(p.ur[s]), &token, &zw_zero);
    if (threadIdx.x == 0) {
      p.out_tokens[s * (p.K + 1) + rec.n] = token;
      if (p.out_flags && zw_zero) p.out_flags[s] |= SPECV_FLAG_ZW_ZERO;
    }
  }
}

// After k_verify computed every sequence's chunk sums (p.xeager > 0): one
// workgroup per sequence of the launch, whose record (seq < 0: the fast draw
// stood) and chunk sums are read together, by sequence.
template <int DT, bool VEC>
__global__ __launch_bounds__(kXBlock) void k_exact_select_seq(Params p) {
  const long b = blockIdx.x;
  const SeqRec rec = p.queue[p.seq0 + b];
  const ChunkSums cv = load_chunk_sums(p, b);
  if (rec.seq < 0) return;  // uniform
  const long s = rec.seq;
  const bool bonus = rec.n == rec.kb;
  int token;
  bool zw_zero;
  select_exact<DT, VEC>(p, decisive_rows<DT>(p, s, rec), exact_weight(p, rec), bonus, cv,
                        static_cast<double>(p.ur[s]), &token, &zw_zero);
  if (threadIdx.x == 0) {
    p.out_tokens[s * (p.K + 1) + rec.n] = token;
    if (p.out_flags && zw_zero) p.out_flags[s] |= SPECV_FLAG_ZW_ZERO;
  }
}

// Rows of at most kSoloMaxChunks chunks (V <= 2048): one workgroup per
// queued sequence computes every chunk's sums itself, into LDS, and makes
// the draw, so the fp64 draw takes one launch (its fixed cost is most of a
// call on such small rows).  The sums and the draw are those of the two
// kernels above.
template <int DT, bool VEC>
__global__ __launch_bounds__(kXBlock) void k_exact_solo(Params p) {
  const SeqRec first = entry_ahead(p, blockIdx.x);
  const long count = static_cast<long>(p.qcount[0]);
  __shared__ double s_cs[kSoloMaxChunks][5];
  const int lane = threadIdx.x % kWave, per = (p.R3 + kWave - 1) / kWave;
  for (long e = blockIdx.x; (e < count) & (first.seq >= 0); e += gridDim.x) {
    SeqRec rec = first;
    if (e != blockIdx.x) rec = p.queue[p.seq0 + e];
    const long s = rec.seq;
    const bool bonus = rec.n == rec.kb;
    const Rows<DT> rows = decisive_rows<DT>(p, s, rec);
    const ExactWeight wt = exact_weight(p, rec);
    __syncthreads();  // the previous entry's reads of s_cs are done
    for (int r = 0; r < p.R3; ++r) exact_chunk_sums<DT, VEC>(p, rows, wt, bonus, r, s_cs[r]);
    __syncthreads();
    ChunkSums cv;  // as load_chunk_sums lays them out (a bonus draw has sum P only)
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int c = lane * per + k;
      const bool in = threadIdx.x < kWave && k < per && c < p.R3;
#pragma unroll
      for (int f = 0; f < 5; ++f) cv.v[k][f] = (in && (f == 0 || !bonus)) ? s_cs[in ? c : 0][f] : 0.0;
    }
    int token;
    bool zw_zero;
    select_exact<DT, VEC>(p, rows, wt, bonus, cv, static_cast<double>(p.ur[s]), &token, &zw_zero);
    if (threadIdx.x == 0) {
      p.out_tokens[s * (p.K + 1) + rec.n] = token;
      if (p.out_flags && zw_zero) p.out_flags[s] |= SPECV_FLAG_ZW_ZERO;
    }
  }
}

template <int DT, bool VEC>
void launch_all(const Params& p, hipStream_t st) {
  const dim3 block(kXBlock);
  const unsigned ns = static_cast<unsigned>(p.nseq);
  if (p.xeager > 0) {
    hipLaunchKernelGGL((k_exact_select_seq<DT, VEC>), dim3(ns), block, 0, st, p);
    return;
  }
  if (p.R3 <= kSoloMaxChunks) {
    hipLaunchKernelGGL((k_exact_solo<DT, VEC>), dim3(ns < kSoloSeqs ? ns : kSoloSeqs), block, 0, st, p);
    return;
  }
  // grids cover up to max(kExactSeqs, min(B / 4, kExactMaxGroups / chunks))
  // queued sequences in one pass (more are walked in passes); idle
  // workgroups exit at once, but each still costs a dispatch and a load.
  // Sequences whose residuals are flat queue a fifth of their draws or more:
  // against a 32-sequence grid, a B / 4 grid measured 161.2 -> 128.6 us per
  // call at B = 1024 (K = 5, V = 32000, bf16) and 333.1 -> 263.7 at B = 2048,
  // B = 1024 of the T = 0.7, V = 128256 recipe 463.0 -> 454.7, B = 256
  // within noise; the cap on workgroups keeps a batch that queues nothing
  // (B = 1024, V = 256000, fp32: 250 chunks a row) at its 32-sequence grid.
  const unsigned cap = kExactMaxGroups / static_cast<unsigned>(p.R3);
  const unsigned want = ns / 4 < cap ? ns / 4 : cap;
  const unsigned cover = want > kExactSeqs ? want : kExactSeqs;
  const unsigned nx = ns < cover ? ns : cover;
  hipLaunchKernelGGL((k_exact_chunks<DT, VEC>), dim3(nx * p.R3), block, 0, st, p);
  hipLaunchKernelGGL((k_exact_select<DT, VEC>), dim3(nx), block, 0, st, p);
}

}  // namespace

hipError_t launch_exact(const Params& p, int dtype, hipStream_t st) {
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
