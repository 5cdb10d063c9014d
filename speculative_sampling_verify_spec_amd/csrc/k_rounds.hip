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

// Whole wave: fold the partials of row j of sequence s (rows per sequence:
// per_seq) into log2 sum_v 2^(x_v c).  The loads of lanes lane and lane + 64
// go out together.
__device__ inline double row_log2z(const Params& p, long s, uint32_t per_seq, int j, int np) {
  const int lane = threadIdx.x % kWave;
  const float2* base = p.part + (s * per_seq + j) * np;
  float ml = -INFINITY;
  double sl = 0.0;
  const float2 q0 = base[lane < np ? lane : np - 1];
  const float2 q1 = base[lane + kWave < np ? lane + kWave : np - 1];
  if (lane < np) fold_partial(ml, sl, q0);
  if (lane + kWave < np) fold_partial(ml, sl, q1);
  for (int i = lane + 2 * kWave; i < np; i += kWave) fold_partial(ml, sl, base[i]);
  return wave_log2z(ml, sl);
}

// Whole wave: the first arg-max of target row j of sequence s (greedy layout).
__device__ inline int row_argmax(const Params& p, long s, int j, int np) {
  const int lane = threadIdx.x % kWave;
  const float2* base = p.part + (s * (p.K + 1u) + j) * np;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = lane; i < np; i += kWave) argmax_merge(bv, bi, base[i].x, __float_as_int(base[i].y));
  wave_argmax(bv, bi);
  return bi;
}

template <int DT, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_round_accept(Params p) {
  const int lane = threadIdx.x % kWave;
  const long local = static_cast<long>(blockIdx.x) * kWaves + threadIdx.x / kWave;
  if (local >= p.nseq) return;  // uniform over the wave
  const long s = p.seq0 + local;
  const int K = p.K, np = p.nch1 * kWaves;
  const int kb = seq_kb(p, s);
  const int cur = p.lv0 == 0 ? kb : p.kbs[s];  // the last level still swept so far
  const int a = p.lv0, e = min(p.lv1, cur);      // levels a..e-1 are tested here
  int last = cur;
  if (e > a) {  // uniform over the wave
    const int nl = e - a;  // at most kMaxRoundLevels
    const int li = lane < nl ? a + lane : a;
    const int xk = p.x[s * K + li];
    bool pass = false;
    if constexpr (GREEDY) {
      int am = -1;
      for (int i = 0; i < nl; ++i) {
        const int ai = row_argmax(p, s, a + i, np);
        if (lane == i) am = ai;
      }
      pass = xk == am;
    } else {
      const float u = p.ua[s * K + li];
      const bool valid = xk >= 0 && xk < p.V;
      const int xs = valid ? xk : 0;
      const float xp = Elt<DT>::at(row_ptr<DT>(p.lp, s * (K + 1) + li, p.V), xs);
      const float xq = Elt<DT>::at(row_ptr<DT>(p.lq, s * K + li, p.V), xs);
      const uint32_t per_seq = 2u * K + 1u;
      double lzp = 0.0, lzq = 0.0;  // lane i: log2 Z of target row a + i and of draft row a + i
      for (int i = 0; i < nl; ++i) {
        const double zp = row_log2z(p, s, per_seq, a + i, np);
        const double zq = row_log2z(p, s, per_seq, K + 1 + a + i, np);
        if (lane == i) {
          lzp = zp;
          lzq = zq;
        }
      }
      if (valid) {
        const double c = p.c;
        // log2 p(x) - log2 q(x); -inf - -inf gives NaN, which rejects
        const double lr = (static_cast<double>(xp) * c - lzp) - (static_cast<double>(xq) * c - lzq);
        const double thr = lr >= 0.0 ? 1.0 : exp2(lr);
        pass = static_cast<double>(u) < thr;
      }
    }
    const uint64_t failed = __ballot(lane < nl && !pass);
    if (failed) last = a + __ffsll(static_cast<unsigned long long>(failed)) - 1;
  }
  if (lane == 0) p.kbs[s] = last;
}

}  // namespace

hipError_t launch_round_accept(const Params& p, int dtype, bool greedy, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((p.nseq + kWaves - 1) / kWaves)), block(kBlock);
  if (greedy) hipLaunchKernelGGL((k_round_accept<0, true>), grid, block, 0, st, p);
  else if (dtype == 1) hipLaunchKernelGGL((k_round_accept<1, false>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((k_round_accept<0, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
