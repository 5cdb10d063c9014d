// The replacement / bonus draw, fp32 fast path with a certified margin.
//
// After n acceptances the emitted token is drawn from w = max(0, p_n - q_n)
// (n < K) or w = p_K (n == K) by inverse CDF: the smallest token v whose
// running sum C(v) exceeds t = u * Z, Z the total weight.  Only the one
// decisive row (pair) per sequence is reread.
//
// draw_chunks (B x R3 workgroups): workgroup (s, r) sums w over chunk r of
//   sequence s's decisive row(s).
// draw_select (one workgroup per sequence, after a kernel boundary so no
//   in-kernel cross-workgroup publication is needed): one wave scans the
//   chunk sums to find the chunk holding t; the workgroup rescans that chunk
//   in rounds of 8 elements per lane (one fp64 block scan per round) and finds
//   v.  The answer is certified when t lies further than the fast path's error
//   bound from both ends of v's interval; otherwise the sequence is queued for
//   the fp64 refine, which recomputes the draw from scratch.
//
// Fast-path values: p(v) = 2^(x c - L) with L the row's log2 normaliser from
// the sweep, split into a whole part and a fraction; bonus draws use the
// unnormalised 2^(x c - whole) and their own total, which cancels the
// normaliser's error.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kRun = 8;                    // elements per lane per rescan round
constexpr int kRound = kBlock * kRun;      // 2048 elements per round

template <int DT>
struct DrawRow {
  const void* rp;
  const void* rq;  // null for a bonus draw
  float mp, mq, lp2, lq2, c;

  // p(v) = 2^(x c - whole - fraction); a bonus draw keeps the unnormalised
  // 2^(x c - whole) and divides by its own total instead
  __device__ float weight(float xp, float xq) const {
    if (!rq) return ex2(fmaf(xp, c, -mp));
    const float P = ex2(fmaf(xp, c, -mp) - lp2);
    const float Q = ex2(fmaf(xq, c, -mq) - lq2);
    return fmaxf(P - Q, 0.f);
  }
};

template <int DT>
__device__ inline DrawRow<DT> draw_row(const Params& p, long s, const SeqRec& rec) {
  DrawRow<DT> row;
  const bool bonus = rec.n == p.K;
  row.rp = row_ptr<DT>(p.lp, s * (p.K + 1) + rec.n, p.V);
  row.rq = bonus ? nullptr : row_ptr<DT>(p.lq, s * p.K + rec.n, p.V);
  row.mp = rec.mp;
  row.mq = rec.mq;
  row.lp2 = static_cast<float>(rec.lp2);
  row.lq2 = static_cast<float>(rec.lq2);
  row.c = p.c;
  return row;
}

// kRun consecutive logits starting at element v0 (v0 a multiple of kRun);
// elements at or past V read as -inf and weigh 0.
template <int DT, bool VEC>
__device__ inline void load_run(const void* row, long v0, int V, float* e) {
  if constexpr (VEC) {
    constexpr int PV = Elt<DT>::kPerVec;
    if (v0 + kRun <= V) {
#pragma unroll
      for (int i = 0; i < kRun / PV; ++i) Elt<DT>::unpack(load16(row, v0 / PV + i), e + i * PV);
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < kRun; ++k) e[k] = v0 + k < V ? Elt<DT>::at(row, v0 + k) : -INFINITY;
}

__device__ inline void enqueue_refine(const Params& p, long s) {
  const uint32_t slot = atomicAdd(p.list_count, 1u);
  p.list[slot] = static_cast<int32_t>(s);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_draw_chunks(Params p) {
  if (p.policy == SPECV_DRAW_FP64) return;
  const long s = blockIdx.x / p.R3;
  const int r = blockIdx.x % p.R3;
  const SeqRec rec = p.rec[s];
  const DrawRow<DT> row = draw_row<DT>(p, s, rec);
  const long lo = static_cast<long>(r) * p.ch3;
  const long hi = min(static_cast<long>(p.V), lo + p.ch3);
  // rounds of U units per lane (16-byte units when VEC), loads issued branch-free
  constexpr int PV = VEC ? Elt<DT>::kPerVec : 1;
  constexpr int U = VEC ? 4 : 8;
  const long ulo = lo / PV, uhi = hi / PV;  // VEC: lo and hi are multiples of PV
  float acc = 0.f;
  for (long r0 = ulo; r0 < uhi; r0 += static_cast<long>(kBlock) * U) {
    if constexpr (VEC) {
      uint4 rp[U], rq[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        const long uu = u < uhi ? u : uhi - 1;
        rp[i] = load16(row.rp, uu);
        if (row.rq) rq[i] = load16(row.rq, uu);
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (r0 + threadIdx.x + static_cast<long>(i) * kBlock < uhi) {
          float ep[PV], eq[PV];
          Elt<DT>::unpack(rp[i], ep);
          if (row.rq) Elt<DT>::unpack(rq[i], eq);
          float t = 0.f;
#pragma unroll
          for (int k = 0; k < PV; ++k) t += row.weight(ep[k], row.rq ? eq[k] : 0.f);
          acc += t;
        }
      }
    } else {
      float ep[U], eq[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const long u = r0 + threadIdx.x + static_cast<long>(i) * kBlock;
        ep[i] = load_masked<DT>(row.rp, u, uhi);
        eq[i] = row.rq ? load_masked<DT>(row.rq, u, uhi) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) acc += row.weight(ep[i], eq[i]);  // -inf logits weigh 0
    }
  }
  __shared__ double lds[kWaves];
  const double chunk_sum = block_sum(static_cast<double>(acc), lds);
  if (threadIdx.x == 0) p.csum[s * p.R3 + r] = chunk_sum;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_draw_select(Params p) {
  const long s = blockIdx.x;
  const SeqRec rec = p.rec[s];
  if (p.policy == SPECV_DRAW_FP64) {
    if (threadIdx.x == 0) {
      if (p.out_flags) p.out_flags[s] = rec.flags;
      enqueue_refine(p, s);
    }
    return;
  }
  const int K = p.K, n = rec.n;
  const bool bonus = n == K;
  const DrawRow<DT> row = draw_row<DT>(p, s, rec);

  // ---- locate the chunk holding t
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
  __shared__ double lds[kWaves];
  __shared__ int s_j;
  __shared__ double s_lo, s_hi;
  if (threadIdx.x == 0) s_j = 0x7fffffff;
  __syncthreads();
  const int rc = s_chunk;
  if (rc < 0) {  // no positive weight, or t at or past the total: fp64 decides
    if (threadIdx.x == 0) {
      if (p.out_flags) p.out_flags[s] = rec.flags;
      enqueue_refine(p, s);
    }
    return;
  }

  // ---- rescan chunk rc in rounds; lane l owns kRun consecutive elements per round
  const long clo = static_cast<long>(rc) * p.ch3;
  const long chi = min(static_cast<long>(p.V), clo + p.ch3);
  const double t = s_t;
  double base = s_base;
  for (long r0 = clo; r0 < chi; r0 += kRound) {
    const long v0 = r0 + static_cast<long>(threadIdx.x) * kRun;
    float wv[kRun];
    {
      float ep[kRun], eq[kRun];
      load_run<DT, VEC>(row.rp, v0, p.V, ep);
      if (row.rq) load_run<DT, VEC>(row.rq, v0, p.V, eq);
#pragma unroll
      for (int k = 0; k < kRun; ++k) wv[k] = (v0 + k < chi) ? row.weight(ep[k], row.rq ? eq[k] : 0.f) : 0.f;
    }
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) mine += wv[k];
    double total;
    double run = base + block_exclusive_scan(mine, lds, &total);
    long found = -1;
    double flo = 0.0, fhi = 0.0;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const double before = run;
      run += wv[k];
      if (found < 0 && wv[k] > 0.f && run > t && before <= t) {
        found = v0 + k;
        flo = before;
        fhi = run;
      }
    }
    if (found >= 0) atomicMin(&s_j, static_cast<int>(found));
    __syncthreads();
    if (found >= 0 && found == s_j) {
      s_lo = flo;
      s_hi = fhi;
    }
    __syncthreads();
    if (s_j != 0x7fffffff) break;  // uniform: every lane reads the same LDS value
    base += total;
  }
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
  const dim3 g1(static_cast<unsigned>(static_cast<long>(p.B) * p.R3)), g2(static_cast<unsigned>(p.B)), block(kBlock);
  if (dtype == 1) {
    if (p.vec) {
      hipLaunchKernelGGL((k_draw_chunks<1, true>), g1, block, 0, st, p);
      hipLaunchKernelGGL((k_draw_select<1, true>), g2, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((k_draw_chunks<1, false>), g1, block, 0, st, p);
      hipLaunchKernelGGL((k_draw_select<1, false>), g2, block, 0, st, p);
    }
  } else {
    if (p.vec) {
      hipLaunchKernelGGL((k_draw_chunks<0, true>), g1, block, 0, st, p);
      hipLaunchKernelGGL((k_draw_select<0, true>), g2, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((k_draw_chunks<0, false>), g1, block, 0, st, p);
      hipLaunchKernelGGL((k_draw_select<0, false>), g2, block, 0, st, p);
    }
  }
  return hipGetLastError();
}

}  // namespace sv
