// Between two rounds of the row sweep: the acceptance tests of the levels
// the round just swept, one wave per sequence, so that the next round reads
// no row of a sequence that has already rejected ([B] "多 Token 验证：左到右，
// 遇错即停": drafts are checked left to right and checking stops at the first
// rejection).
//
// For sequence s the wave tests levels lv0..lv1-1 that are below its draft
// count K_b (or below the level where an earlier round found its first
// rejection), with the same fold of the sweep partials and the same test as
// the acceptance scan after the sweep (sampling: u_k < min(1, p_k(x_k) /
// q_k(x_k)) as an fp64 log2 ratio; greedy: x_k equal to the first arg-max of
// target row k).  It writes kbs[s], the last level the sweep still reads for
// s: K_b while every test so far passed, else the level of the first
// rejection.  The acceptance scan after the last round repeats every test
// from the partials, so nothing else depends on these values.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

// A lane's partial at index i of a row, by a relaxed atomic load: the
// compiler keeps such loads where they are written, so all of them go out
// together at the kernel's start.
__device__ inline float2 load_partial(const float2* row, int i) {
  const uint64_t b = __hip_atomic_load(reinterpret_cast<const uint64_t*>(row + i), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(b)), __uint_as_float(static_cast<uint32_t>(b >> 32)));
}

// Whole wave: log2 sum_v 2^(x_v c) of a row of np partials from the lane's
// partials lane and lane + 64 (q0, q1, loaded ahead) and, past 128, the rest;
// folded in the acceptance scan's order (lane l: l, l + 64, ...), so the
// value is the one it computes, bit for bit.
__device__ inline double fold_row(const float2* row, int np, float2 q0, float2 q1) {
  const int lane = threadIdx.x % kWave;
  float ml = -INFINITY;
  double sl = 0.0;
  if (lane < np) fold_partial(ml, sl, q0);
  if (lane + kWave < np) fold_partial(ml, sl, q1);
  for (int i = lane + 2 * kWave; i < np; i += kWave) fold_partial(ml, sl, row[i]);
  return wave_log2z(ml, sl);
}

// Whole wave: the first arg-max of a row of (max, index bits) partials, the
// same way.
__device__ inline int row_argmax(const float2* row, int np, float2 q0, float2 q1) {
  const int lane = threadIdx.x % kWave;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (lane < np) argmax_merge(bv, bi, q0.x, __float_as_int(q0.y));
  if (lane + kWave < np) argmax_merge(bv, bi, q1.x, __float_as_int(q1.y));
  for (int i = lane + 2 * kWave; i < np; i += kWave) argmax_merge(bv, bi, row[i].x, __float_as_int(row[i].y));
  wave_argmax(bv, bi);
  return bi;
}

// One wave per sequence, without branches on the sequence's state: every
// load goes out at once (its count, kbs, the draft tokens and uniforms of the
// round's levels, the first 128 partials of each of their rows), then only
// the logits at the draft tokens, which wait for the tokens.  Levels a
// sequence no longer sweeps are folded from stale partials (harmless) and
// masked out of the ballot.
template <int DT, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_round_accept(Params p) {
  const int lane = threadIdx.x % kWave;
  // the wave's sequence, in scalar registers (its count and kbs are scalar loads)
  const long local = static_cast<long>(blockIdx.x) * (blockDim.x / kWave) +
                     __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  if (local >= p.nseq) return;  // uniform over the wave
  const long s = p.seq0 + local;
  const int K = p.K, np = p.nch1 * kWaves;
  const int a = p.lv0, nr = p.lv1 - p.lv0;  // the round's levels: a .. a + nr - 1, all below K
  // the count and kbs by vector loads (a scalar load in flight would hold back
  // the first use of the kernel's arguments: scalar loads complete in any
  // order), unconditional (without per-sequence counts, kbs stands in as an
  // address); used only after every load has gone out
  const int kbr = __hip_atomic_load((p.kb ? p.kb : p.kbs) + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int kbs = __hip_atomic_load(p.kbs + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int li = a + min(lane, nr - 1);  // lane i < nr: level a + i
  const int xk = p.x[s * K + li];
  const uint32_t per_seq = GREEDY ? K + 1u : 2u * K + 1u;
  const int i0 = min(lane, np - 1), i1 = min(lane + kWave, np - 1);
  float2 qt[kMaxRoundLevels][2], qd[kMaxRoundLevels][2];  // partials of target and draft rows
  const float2* rt[kMaxRoundLevels];
  const float2* rd[kMaxRoundLevels];
#pragma unroll
  for (int i = 0; i < kMaxRoundLevels; ++i) {
    const int lv = a + min(i, nr - 1);
    rt[i] = p.part + (s * per_seq + lv) * np;
    rd[i] = p.part + (s * per_seq + (GREEDY ? lv : K + 1 + lv)) * np;
    qt[i][0] = load_partial(rt[i], i0);
    qt[i][1] = load_partial(rt[i], i1);
    if constexpr (!GREEDY) {
      qd[i][0] = load_partial(rd[i], i0);
      qd[i][1] = load_partial(rd[i], i1);
    }
  }
  const float u = GREEDY ? 0.f : p.ua[s * K + li];
  __builtin_amdgcn_sched_barrier(0);
  const int kb = p.kb ? min(max(kbr, 0), K) : K;
  const int cur = p.lv0 == 0 ? kb : kbs;  // the last level still swept so far
  const int e = min(p.lv1, cur);          // levels a..e-1 are tested here
  const int nl = max(e - a, 0);   // at most nr
  bool pass = false;
  if constexpr (GREEDY) {
    int am = -1;
#pragma unroll
    for (int i = 0; i < kMaxRoundLevels; ++i) {
      if (i < nr) {  // uniform
        const int ai = row_argmax(rt[i], np, qt[i][0], qt[i][1]);
        if (lane == i) am = ai;
      }
    }
    pass = xk == am;
  } else {
    const bool valid = xk >= 0 && xk < p.V;
    const int xs = valid ? xk : 0;
    const float xp = Elt<DT>::at(row_ptr<DT>(p.lp, s * (K + 1) + li, p.V), xs);
    const float xq = Elt<DT>::at(row_ptr<DT>(p.lq, s * K + li, p.V), xs);
    double lzp = 0.0, lzq = 0.0;  // lane i: log2 Z of target row a + i and of draft row a + i
#pragma unroll
    for (int i = 0; i < kMaxRoundLevels; ++i) {
      if (i < nr) {  // uniform
        const double zp = fold_row(rt[i], np, qt[i][0], qt[i][1]);
        const double zq = fold_row(rd[i], np, qd[i][0], qd[i][1]);
        if (lane == i) {
          lzp = zp;
          lzq = zq;
        }
      }
    }
    const double c = p.c;
    // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
    const double lr = (static_cast<double>(xp) * c - lzp) - (static_cast<double>(xq) * c - lzq);
    const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
    pass = valid && static_cast<double>(u) < thr;
  }
  const uint64_t failed = __ballot(lane < nl && !pass);
  const int last = failed ? a + __ffsll(static_cast<unsigned long long>(failed)) - 1 : cur;
  if (lane == 0) p.kbs[s] = last;
}

}  // namespace

hipError_t launch_round_accept(const Params& p, int dtype, bool greedy, hipStream_t st) {
  // one wave per workgroup, spread over the CUs (interleaved A/B against four
  // sequences per 256-thread workgroup, us per step: headline 138.75 ->
  // 138.62, greedy 81.00 -> 80.72, headline at B = 96 76.10 -> 75.80)
  const dim3 grid(static_cast<unsigned>(p.nseq)), block(kWave);
  if (greedy) hipLaunchKernelGGL((k_round_accept<0, true>), grid, block, 0, st, p);
  else if (dtype == 1) hipLaunchKernelGGL((k_round_accept<1, false>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_round_accept<0, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
