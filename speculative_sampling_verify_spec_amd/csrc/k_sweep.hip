// Row sweeps: the one pass over every logit that the verify step needs.
//
// Sampling mode: each wave reduces its share of one chunk of one row to a
// pair (R, s): R a whole number (stored as float) and s = sum 2^(x*c - R),
// c = log2(e) / T, so the share's sum of 2^(x*c) is s * 2^R.  The normalisers
// log2 Z of the target and draft distributions p and q are combined from
// these pairs afterwards with exact power-of-two rescales.
// Greedy mode: each wave reduces its share of a chunk to (largest logit,
// lowest index holding it).
//
// Per element the sampling sweep spends one bf16 widen (exact), half a
// v_max3_f32, one fma t = x*c - R (R = rint(max * c), so t <= 0.5 and the
// fma's single rounding is the only error in the exponent), one v_exp_f32 and
// one add; the greedy sweep a widen and a compare-select.  Both are HBM-bound:
// every row is read once with 16-byte non-temporal loads (4 fp32 or 8 bf16
// values per lane, coalesced across the wave), all of a lane's loads issued
// before it computes.  A row is split into chunks of equal size, one
// workgroup each, so no workgroup gets a short tail; each wave writes its own
// partial, so no workgroup barrier holds finished waves back.
//
// Rounds.  On large inputs, unless every row's normaliser is asked for, the
// sweep runs in rounds of levels (see round_begin): acceptance stops at the
// first rejection ([B] "多 Token 验证：左到右，遇错即停"), so rows past it are
// never needed.  A round's grid is (chunks, round slots, sequences); between
// rounds k_round_accept tests the levels just swept and lowers a rejected
// sequence's last level to sweep, which the next round's workgroups compare
// with one scalar load before leaving.  Rows of levels past a rejection keep
// stale partials, which only ever decide tests after the first failing one.
#include <hip/hip_ext.h>

#include "sv_device.h"

namespace sv {

namespace {

// Row `row` of the sampling sweep: K+1 target rows then K draft rows per
// sequence.  32-bit division: row counts are checked on the host.
template <int DT>
__device__ inline const void* sweep_row(const Params& p, uint32_t row) {
  const uint32_t per_seq = 2u * p.K + 1u;
  const uint32_t s = row / per_seq;
  const uint32_t j = row - s * per_seq;
  return j <= static_cast<uint32_t>(p.K) ? row_ptr<DT>(p.lp, static_cast<long>(s) * (p.K + 1) + j, p.V)
                                         : row_ptr<DT>(p.lq, static_cast<long>(s) * p.K + (j - p.K - 1), p.V);
}

// Row j of sequence s (target rows 0..K, then draft rows), for the 3-D grid:
// both candidate addresses are formed and one is selected, so the two base
// pointers load with the other kernel arguments.
template <int DT>
__device__ inline const void* sweep_row(const Params& p, uint32_t s, uint32_t j) {
  const void* t = row_ptr<DT>(p.lp, static_cast<long>(s) * (p.K + 1) + j, p.V);
  const void* d = row_ptr<DT>(p.lq, static_cast<long>(s) * p.K + (static_cast<long>(j) - p.K - 1), p.V);
  return j <= static_cast<uint32_t>(p.K) ? t : d;
}

// Where a workgroup's chunk lies.  The 3-D grid (chunks, round slots,
// sequences) serves rounds and per-sequence draft counts: no divisions,
// which matters there because the workgroups of skipped rows only test a
// count and leave (143.8 -> 131.7 us per ragged step at the headline shape).
// Slot y < lv1 - lv0 of a round is target row lv0 + y; the rest are the
// draft rows of the round's levels (none in the arg-max sweep).  The full
// sweep keeps a one-dimensional grid over (row, chunk), which measured
// faster for full sweeps (150.8 against 152.4 us, and 193.7 against 196.3
// for the arg-max sweep), with the prologue it was tuned with: a shorter
// one, without the never-true test of the counts, measured 0.3-0.8 us
// slower per step (its loads start earlier).
struct SweepPos {
  uint32_t chunk, row;  // row: the launch-wide row index (sequence * rows per sequence + j)
  uint32_t seq, j;      // 3-D grid only: the sequence and its row j (target k: k; draft k: K + 1 + k)
  int level;            // 3-D grid only: the row's level
  bool draft;           // 3-D grid only: a draft row
};

template <bool G3, bool ARGMAX>
__device__ inline SweepPos sweep_pos(const Params& p) {
  const uint32_t per_seq = ARGMAX ? p.K + 1u : 2u * p.K + 1u;
  SweepPos q;
  if constexpr (G3) {
    const int nt = p.lv1 - p.lv0, y = static_cast<int>(blockIdx.y);
    q.chunk = blockIdx.x;
    q.seq = static_cast<uint32_t>(p.seq0) + blockIdx.z;
    q.draft = !ARGMAX && y >= nt;
    q.level = p.lv0 + (q.draft ? y - nt : y);
    q.j = static_cast<uint32_t>(q.draft ? p.K + 1 + q.level : q.level);
    q.row = q.seq * per_seq + q.j;
  } else {
    const uint32_t local = blockIdx.x / static_cast<uint32_t>(p.nch1);
    q.chunk = blockIdx.x - local * static_cast<uint32_t>(p.nch1);
    q.row = static_cast<uint32_t>(p.seq0) * per_seq + local;
    q.seq = q.j = 0;
    q.level = 0;
    q.draft = false;
  }
  return q;
}

// Block 0 of a launch (both grid shapes).
__device__ inline bool first_block() { return (blockIdx.x | blockIdx.y | blockIdx.z) == 0; }

// Block 0 of the sampling sweep resets, for the launch's sequences, the
// state that the kernels after it fill: the fp64 draw's queue counter and,
// when the fast draw is split, its per-sequence counts (0) and published
// values (NaN: "not yet").
__device__ inline void reset_state(const Params& p) {
  if (threadIdx.x == 0) p.qcount[0] = 0u;
  if (p.split > 1) {
    for (int i = threadIdx.x; i < p.nseq; i += kBlock) p.vcount[p.seq0 + i] = 0u;
    const long nsegs = static_cast<long>(p.nseq) * p.nseg, nsums = static_cast<long>(p.nseq) * kMaxSplit * 2;
    for (long i = threadIdx.x; i < nsegs; i += kBlock) p.segm[static_cast<long>(p.seq0) * p.nseg + i] = NAN;
    for (long i = threadIdx.x; i < nsums; i += kBlock) p.spq[static_cast<long>(p.seq0) * kMaxSplit * 2 + i] = NAN;
  }
}

// This lane's elements of chunk `chunk` of a row (units of 16 bytes when VEC,
// single elements otherwise), loaded without branches.  Bit i of `live` says
// whether slot i lies inside the chunk.  VEC: units are addressed from the
// chunk's (scalar) base with 32-bit lane offsets, and a slot past the chunk's
// end reads the chunk's last unit again (real values of the same chunk, so
// they leave its maximum unchanged; sums must skip them).  Scalar path:
// elements past the end read as -inf.  Returns the chunk's unit range.
template <int DT, bool VEC, bool ARGMAX, bool LARGE>
__device__ inline void load_chunk(const Params& p, const void* r, uint32_t chunk,
                                  float (&e)[kSweepElems<DT, VEC, ARGMAX, LARGE>()], uint32_t& live, long& lo,
                                  long& hi) {
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  constexpr int IT = kSweepElems<DT, VEC, ARGMAX, LARGE>() / PV;
  static_assert(IT <= 32, "one live bit per slot");
  lo = static_cast<long>(chunk) * p.cq + min(static_cast<int>(chunk), p.cr);
  hi = lo + p.cq + (static_cast<int>(chunk) < p.cr ? 1 : 0);
  const uint32_t n = static_cast<uint32_t>(hi - lo);  // cq or cq + 1 units
  live = 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const uint32_t u = threadIdx.x + i * kBlock;
    // slots that every chunk fills (a test uniform over the launch) are live everywhere
    live |= (((i + 1) * kBlock <= p.cq || u < n) ? 1u : 0u) << i;
  }
  if constexpr (VEC) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* base = static_cast<const u32x4*>(r) + lo;
    u32x4 raw[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t u = threadIdx.x + i * kBlock;
      raw[i] = __builtin_nontemporal_load(base + ((i + 1) * kBlock <= p.cq ? u : min(u, n - 1)));
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) Elt<DT>::unpack(make_uint4(raw[i].x, raw[i].y, raw[i].z, raw[i].w), &e[i * PV]);
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) e[i] = load_masked<DT>(r, lo + threadIdx.x + static_cast<long>(i) * kBlock, hi);
  }
}

// G3: the 3-D grid of rounds and per-sequence draft counts (a separate
// instantiation, so that the full sweep carries no code for them ahead of
// its loads).
template <int DT, bool VEC, bool LARGE, bool G3>
__global__ __launch_bounds__(kBlock) void k_sweep_lse(Params p) {
  constexpr int N = kSweepElems<DT, VEC, false, LARGE>();
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  const SweepPos q = sweep_pos<G3, false>(p);
  const uint32_t chunk = q.chunk, row = q.row;
  // Rows past a sequence's own draft count are not read, and in a later
  // round neither are those of a sequence that has rejected.  In the 3-D
  // kernel the count test comes before any store, so the compiler may read
  // the count with a scalar load, which later workgroups find in the scalar
  // cache, and block 0 of round 0 resets the state at its end (it holds a
  // sequence's target row 0, which is always read).  The one-dimensional
  // kernel keeps the order it was tuned with: reset first, then a test of
  // the counts, which is never true as launched.
  if constexpr (G3) {
    const int kb = sweep_kb(p, q.seq);
    if (q.draft ? q.level >= kb : q.level > kb) return;
  } else {
    if (first_block()) reset_state(p);
    if (p.kb) {
      const uint32_t per_seq = 2u * p.K + 1u, s = row / per_seq, j = row - s * per_seq;
      const int kb = seq_kb(p, s);
      if (j <= static_cast<uint32_t>(p.K) ? j > static_cast<uint32_t>(kb) : j - p.K - 1 >= static_cast<uint32_t>(kb))
        return;
    }
  }
  const float c = p.c;
  float e[N];
  uint32_t live;
  long lo, hi;
  const void* r = G3 ? sweep_row<DT>(p, q.seq, q.j) : sweep_row<DT>(p, row);
  load_chunk<DT, VEC, false, LARGE>(p, r, chunk, e, live, lo, hi);

  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) m = fmaxf(m, e[k]);
  float R = -INFINITY, s = 0.f;
  if (m != -INFINITY) {
    R = rintf(m * c);
#pragma unroll
    for (int i = 0; i < N / PV; ++i) {
      float t[PV];
#pragma unroll
      for (int k = 0; k < PV; ++k) t[k] = ex2(fmaf(e[i * PV + k], c, -R));
      // pairwise within a 16-byte unit, then one add into the running sum
#pragma unroll
      for (int w = PV / 2; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) t[k] += t[k + w];
      s += ((live >> i) & 1u) ? t[0] : 0.f;
    }
  }

  // wave merge: exact power-of-two rescale to the wave's largest R, fp64 sum
  const float M = wave_max(R);
  const double sd = (R == -INFINITY) ? 0.0 : static_cast<double>(ldexpf(s, static_cast<int>(fmaxf(R - M, -200.f))));
  const double S = wave_sum(sd);
  if (threadIdx.x % kWave == 0)
    p.part[(static_cast<long>(row) * p.nch1 + chunk) * kWaves + threadIdx.x / kWave] = make_float2(M, static_cast<float>(S));
  if (G3 && p.lv0 == 0 && first_block()) reset_state(p);
}

// TREE: a later round of token-tree rows (3-D grid, slots = nodes lv0..lv1-1):
// a node's row is read when k_tree_round marked it.
template <int DT, bool VEC, bool LARGE, bool G3, bool TREE = false>
__global__ __launch_bounds__(kBlock) void k_sweep_argmax(Params p) {
  constexpr int N = kSweepElems<DT, VEC, true, LARGE>();
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  const SweepPos q = sweep_pos<G3, true>(p);  // target rows only
  const uint32_t chunk = q.chunk, row = q.row;
  // target rows past a sequence's own draft count are not read, nor, in a
  // later round, those of a sequence whose drafts stopped matching
  if constexpr (TREE) {
    if (!p.tneed[static_cast<long>(q.seq) * (p.K + 1) + q.level]) return;
  } else if constexpr (G3) {
    if (q.level > sweep_kb(p, q.seq)) return;
  } else if (p.kb) {  // never true as launched; see sweep_pos
    const uint32_t s = row / (p.K + 1u), j = row - s * (p.K + 1u);
    if (j > static_cast<uint32_t>(seq_kb(p, s))) return;
  }
  float e[N];
  uint32_t live;
  long lo, hi;
  load_chunk<DT, VEC, true, LARGE>(p, row_ptr<DT>(p.lp, row, p.V), chunk, e, live, lo, hi);
  // the lane's largest value, then the lowest index holding it (a backward
  // pass of selects over the lane's elements, which it visits in increasing
  // index order); repeated tail units carry their real index
  float bv = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) bv = fmaxf(bv, e[k]);
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = N / PV - 1; i >= 0; --i) {
    const long u = lo + threadIdx.x + static_cast<long>(i) * kBlock;
    const long ur = ((live >> i) & 1u) ? u : hi - 1;  // the unit actually read
#pragma unroll
    for (int k = PV - 1; k >= 0; --k) bi = e[i * PV + k] == bv ? static_cast<int>(ur * PV + k) : bi;
  }
  wave_argmax(bv, bi);
  if (threadIdx.x % kWave == 0)
    p.part[(static_cast<long>(row) * p.nch1 + chunk) * kWaves + threadIdx.x / kWave] = make_float2(bv, __int_as_float(bi));
}

}  // namespace

// Events, when given, are recorded as part of the dispatch itself (no
// separate marker packet, so no bubble between kernels).
template <typename Kern>
hipError_t launch_evented(Kern k, const dim3& grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1, const Params& p) {
  if (e0 || e1) hipExtLaunchKernelGGL(k, grid, dim3(kBlock), 0, st, e0, e1, 0, p);
  else hipLaunchKernelGGL(k, grid, dim3(kBlock), 0, st, p);
  return hipGetLastError();
}

// 3-D grids are (chunks, round slots, sequences), at most kMaxGridZ
// sequences per launch, so larger batches are swept in slices (events, when
// given, bracket all of them); the full sweep's grid is one-dimensional.
constexpr long kMaxGridZ = 65535;

template <typename Kern>
hipError_t launch_grid(Kern k, bool g3, unsigned slots, const Params& p, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1) {
  if (!g3)
    return launch_evented(k, dim3(static_cast<unsigned>(static_cast<long>(p.nseq) * slots * p.nch1)), st, e0, e1, p);
  Params q = p;
  for (long s0 = 0; s0 < p.nseq; s0 += kMaxGridZ) {
    q.seq0 = static_cast<int>(p.seq0 + s0);
    q.nseq = static_cast<int>(p.nseq - s0 < kMaxGridZ ? p.nseq - s0 : kMaxGridZ);
    const dim3 grid(static_cast<unsigned>(p.nch1), slots, static_cast<unsigned>(q.nseq));
    const hipError_t r = launch_evented(k, grid, st, s0 == 0 ? e0 : nullptr, s0 + kMaxGridZ >= p.nseq ? e1 : nullptr, q);
    if (r != hipSuccess) return r;
  }
  return hipSuccess;
}

// Round slots: the target rows of levels lv0..lv1-1, then (sampling) the
// draft rows among them (levels below K); the full sweep: every row.
inline unsigned sweep_slots(const Params& p, bool argmax) {
  if (!p.grid3) return argmax ? p.K + 1u : 2u * p.K + 1u;
  const int drafts = (p.lv1 < p.K ? p.lv1 : p.K) - p.lv0;
  return static_cast<unsigned>(p.lv1 - p.lv0 + (argmax || drafts < 0 ? 0 : drafts));
}

template <int DT, bool G3>
hipError_t launch_lse(const Params& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const unsigned slots = sweep_slots(p, false);
  if (!p.vec) return launch_grid(k_sweep_lse<DT, false, false, G3>, G3, slots, p, st, e0, e1);
  if (p.sweep_large) return launch_grid(k_sweep_lse<DT, true, true, G3>, G3, slots, p, st, e0, e1);
  return launch_grid(k_sweep_lse<DT, true, false, G3>, G3, slots, p, st, e0, e1);
}

template <int DT, bool G3>
hipError_t launch_argmax(const Params& p, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const unsigned slots = sweep_slots(p, true);
  if (!p.vec) return launch_grid(k_sweep_argmax<DT, false, false, G3>, G3, slots, p, st, e0, e1);
  if (p.sweep_large) return launch_grid(k_sweep_argmax<DT, true, true, G3>, G3, slots, p, st, e0, e1);
  return launch_grid(k_sweep_argmax<DT, true, false, G3>, G3, slots, p, st, e0, e1);
}

template <int DT>
hipError_t launch_argmax_tree(const Params& p, hipStream_t st) {
  const unsigned slots = static_cast<unsigned>(p.lv1 - p.lv0);
  if (!p.vec) return launch_grid(k_sweep_argmax<DT, false, false, true, true>, true, slots, p, st, nullptr, nullptr);
  if (p.sweep_large)
    return launch_grid(k_sweep_argmax<DT, true, true, true, true>, true, slots, p, st, nullptr, nullptr);
  return launch_grid(k_sweep_argmax<DT, true, false, true, true>, true, slots, p, st, nullptr, nullptr);
}

hipError_t launch_sweep_lse(const Params& p, int dtype, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const bool g3 = p.grid3 != 0;
  if (dtype == 1) return g3 ? launch_lse<1, true>(p, st, e0, e1) : launch_lse<1, false>(p, st, e0, e1);
  return g3 ? launch_lse<0, true>(p, st, e0, e1) : launch_lse<0, false>(p, st, e0, e1);
}

hipError_t launch_sweep_argmax(const Params& p, int dtype, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const bool g3 = p.grid3 != 0;
  if (dtype == 1) return g3 ? launch_argmax<1, true>(p, st, e0, e1) : launch_argmax<1, false>(p, st, e0, e1);
  return g3 ? launch_argmax<0, true>(p, st, e0, e1) : launch_argmax<0, false>(p, st, e0, e1);
}

hipError_t launch_sweep_argmax_tree(const Params& p, int dtype, hipStream_t st) {
  return dtype == 1 ? launch_argmax_tree<1>(p, st) : launch_argmax_tree<0>(p, st);
}

}  // namespace sv
