// The replacement / bonus draw, fp32 fast path with a certified margin.
//
// After n acceptances the emitted token is drawn from w = max(0, p_n - q_n)
// (n < K) or w = p_K (n == K) by inverse CDF: the smallest token v whose
// running sum C(v) exceeds t = u * Z, Z the total weight.  Only the one
// decisive row (pair) per sequence is reread.
//
// Pass 1 (all workgroups): workgroup (s, r) sums w over chunk r of sequence
// s's decisive row(s) and stores the sum; the last workgroup of s to arrive
// (arrival counter, release/acquire fences) finalises.
// Finalise: one wave scans the chunk sums to find the chunk holding t, the
// workgroup rescans that chunk (contiguous runs per lane, fp64 block scan)
// and finds v.  The answer is certified when t lies further than the fast
// path's error bound from both ends of v's interval; otherwise the sequence
// is queued for the fp64 refine, which recomputes the draw from scratch.
//
// Fast-path values: p(v) = 2^((x - m) c - L) with m, L the row maximum and
// log2 normaliser from the sweep; bonus draws use the unnormalised 2^((x - m) c)
// and their own total, which cancels the normaliser's error.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

template <int DT>
struct DrawRow {
  const void* rp;
  const void* rq;  // null for a bonus draw
  float mp, mq, lp2, lq2, c;

  __device__ float weight(long v) const {
    const float xp = Elt<DT>::at(rp, v);
    if (!rq) return ex2((xp - mp) * c);
    const float xq = Elt<DT>::at(rq, v);
    const float P = ex2((xp - mp) * c - lp2);
    const float Q = ex2((xq - mq) * c - lq2);
    return fmaxf(P - Q, 0.f);
  }
  __device__ float weight_vals(float xp, float xq) const {
    if (!rq) return ex2((xp - mp) * c);
    const float P = ex2((xp - mp) * c - lp2);
    const float Q = ex2((xq - mq) * c - lq2);
    return fmaxf(P - Q, 0.f);
  }
};

__device__ inline void enqueue_refine(const Params& p, long s) {
  const uint32_t slot = atomicAdd(p.list_count, 1u);
  p.list[slot] = static_cast<int32_t>(s);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_draw(Params p) {
  const long s = blockIdx.x / p.R3;
  const int r = blockIdx.x % p.R3;
  const SeqRec rec = p.rec[s];
  const int K = p.K, n = rec.n;
  const bool bonus = n == K;

  if (p.policy == SPECV_DRAW_FP64) {
    if (r == 0 && threadIdx.x == 0) {
      if (p.out_flags) p.out_flags[s] = rec.flags;
      enqueue_refine(p, s);
    }
    return;
  }

  DrawRow<DT> row;
  row.rp = row_ptr<DT>(p.lp, s * (K + 1) + n, p.V);
  row.rq = bonus ? nullptr : row_ptr<DT>(p.lq, s * K + n, p.V);
  row.mp = rec.mp;
  row.mq = rec.mq;
  row.lp2 = static_cast<float>(rec.lp2);
  row.lq2 = static_cast<float>(rec.lq2);
  row.c = p.c;

  // ---- pass 1: this chunk's weight
  const long lo = static_cast<long>(r) * p.ch3;
  const long hi = min(static_cast<long>(p.V), lo + p.ch3);
  float acc = 0.f;
  if constexpr (VEC) {
    constexpr int PV = Elt<DT>::kPerVec;
    for (long vi = lo / PV + threadIdx.x; vi < hi / PV; vi += kBlock) {
      float ep[PV], eq[PV];
      Elt<DT>::unpack(load16(row.rp, vi), ep);
      if (row.rq) Elt<DT>::unpack(load16(row.rq, vi), eq);
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < PV; ++k) t += row.weight_vals(ep[k], row.rq ? eq[k] : 0.f);
      acc += t;
    }
  } else {
    for (long v = lo + threadIdx.x; v < hi; v += kBlock) acc += row.weight(v);
  }
  __shared__ double lds[kWaves];
  __shared__ int s_last;
  const double chunk_sum = block_sum(static_cast<double>(acc), lds);
  if (threadIdx.x == 0) {
    p.csum[s * p.R3 + r] = chunk_sum;
    __threadfence();
    s_last = atomicAdd(&p.cnt_draw[s], 1u) == static_cast<uint32_t>(p.R3 - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- finalise: locate the chunk holding t
  __shared__ double s_t, s_z, s_base;
  __shared__ int s_chunk;
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x < kWave) {
    const double v = lane < p.R3 ? p.csum[s * p.R3 + lane] : 0.0;
    const double inc = wave_inclusive_scan(v);
    double excl = __shfl_up(inc, 1, kWave);
    if (lane == 0) excl = 0.0;
    const double z = __shfl(inc, kWave - 1, kWave);
    const double t = static_cast<double>(p.ur[s]) * z;
    const uint64_t hit = __ballot(lane < p.R3 && inc > t);
    const int rc = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : -1;
    const double base = __shfl(excl, rc < 0 ? 0 : rc, kWave);
    if (lane == 0) {
      s_t = t;
      s_z = z;
      s_base = base;
      s_chunk = (z > 0.0) ? rc : -1;
    }
  }
  __syncthreads();
  const int rc = s_chunk;
  if (rc < 0) {  // no positive weight or t beyond the total: let fp64 decide
    if (threadIdx.x == 0) {
      if (p.out_flags) p.out_flags[s] = rec.flags;
      enqueue_refine(p, s);
    }
    return;
  }

  // ---- rescan chunk rc: lane-contiguous runs, fp64 block scan
  const long clo = static_cast<long>(rc) * p.ch3;
  const long chi = min(static_cast<long>(p.V), clo + p.ch3);
  const int ept = p.ch3 / kBlock;
  const long mylo = min(chi, clo + static_cast<long>(threadIdx.x) * ept);
  const long myhi = min(chi, mylo + ept);
  double mine = 0.0;
  for (long v = mylo; v < myhi; ++v) mine += row.weight(v);
  double total;
  double run = s_base + block_exclusive_scan(mine, lds, &total);
  const double t = s_t;
  __shared__ int s_j;
  __shared__ double s_lo, s_hi;
  if (threadIdx.x == 0) s_j = 0x7fffffff;
  __syncthreads();
  long found = -1;
  double flo = 0.0, fhi = 0.0;
  for (long v = mylo; v < myhi; ++v) {
    const double before = run;
    const float wv = row.weight(v);
    run += wv;
    if (wv > 0.f && run > t) {
      found = v;
      flo = before;
      fhi = run;
      break;
    }
  }
  if (found >= 0) atomicMin(&s_j, static_cast<int>(found));
  __syncthreads();
  if (found >= 0 && found == s_j) {
    s_lo = flo;
    s_hi = fhi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (p.out_flags) p.out_flags[s] = rec.flags;
    const int j = s_j;
    bool ok = j != 0x7fffffff;
    if (ok && p.policy == SPECV_DRAW_CERTIFIED) {
      const double margin = fmin(t - s_lo, s_hi - t);
      const double bound = bonus ? p.e_rel_bonus * s_z : p.e_abs_res;
      ok = margin > bound;
    }
    if (ok) p.out_tokens[s * (K + 1) + n] = j;
    else enqueue_refine(p, s);
  }
}

}  // namespace

hipError_t launch_draw(const Params& p, int dtype, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(static_cast<long>(p.B) * p.R3)), block(kBlock);
  if (dtype == 1) {
    if (p.vec) hipLaunchKernelGGL((k_draw<1, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_draw<1, false>), grid, block, 0, st, p);
  } else {
    if (p.vec) hipLaunchKernelGGL((k_draw<0, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_draw<0, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace sv
