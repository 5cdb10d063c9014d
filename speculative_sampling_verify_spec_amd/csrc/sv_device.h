// Device-side helpers shared by the libspecverify kernels: element loads for
// fp32 / bf16 rows, wave and workgroup reductions, and an fp64 block scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {

// ---------------------------------------------------------------- loads --
// DT 0: fp32 logits; DT 1: bf16 logits (raw 16-bit patterns).
template <int DT> struct Elt;

template <> struct Elt<0> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  static constexpr int kBytes = 4;
  __device__ static float at(const void* row, long i) { return static_cast<const float*>(row)[i]; }
  __device__ static void unpack(const uint4& v, float* e) {
    e[0] = __uint_as_float(v.x); e[1] = __uint_as_float(v.y);
    e[2] = __uint_as_float(v.z); e[3] = __uint_as_float(v.w);
  }
};

template <> struct Elt<1> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  __device__ static float at(const void* row, long i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[i]) << 16);
  }
  // bf16 -> fp32 is exact: the 16 bits become the high half of the fp32 word.
  __device__ static void unpack(const uint4& v, float* e) {
    e[0] = __uint_as_float(v.x << 16); e[1] = __uint_as_float(v.x & 0xffff0000u);
    e[2] = __uint_as_float(v.y << 16); e[3] = __uint_as_float(v.y & 0xffff0000u);
    e[4] = __uint_as_float(v.z << 16); e[5] = __uint_as_float(v.z & 0xffff0000u);
    e[6] = __uint_as_float(v.w << 16); e[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

// Sequence s's draft count: its own (clamped to [0, K]) or K.
__device__ inline int seq_kb(const Params& p, long s) {
  return p.kb ? min(max(p.kb[s], 0), p.K) : p.K;
}

// The last level the sweep reads for sequence s: its draft count, or, in a
// round after the first, the level of its first rejection once it has
// rejected (written by k_round_accept).
__device__ inline int sweep_kb(const Params& p, long s) {
  return p.lv0 > 0 ? p.kbs[s] : seq_kb(p, s);
}

template <int DT>
__device__ inline const void* row_ptr(const void* base, long row, int V) {
  return static_cast<const char*>(base) + row * static_cast<long>(V) * Elt<DT>::kBytes;
}

__device__ inline uint4 load16(const void* row, long vec_index) {
  return static_cast<const uint4*>(row)[vec_index];
}

__device__ inline uint4 load16_nt(const void* row, long vec_index) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(static_cast<const u32x4*>(row) + vec_index);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Branch-free masked loads: the address is clamped into [0, last] so the load
// is always legal and can be issued together with its neighbours; lanes past
// the end get -inf.  (A guarded load compiles to a branch and a wait per load,
// which leaves one load in flight per wave.)
template <int DT>
__device__ inline float load_masked(const void* row, long i, long end) {
  const bool ok = i < end;
  const float v = Elt<DT>::at(row, ok ? i : end - 1);
  return ok ? v : -INFINITY;
}

// Raw hardware exp2 (v_exp_f32).  Arguments below -126 give 0 or a denormal;
// callers only feed it values <= 0 whose tiny results do not matter.
__device__ inline float ex2(float t) { return __builtin_amdgcn_exp2f(t); }

// exp(y) in fp64 for the exact draw (about 20 instructions against roughly a
// hundred for the general library routine).  Cody-Waite reduction
// y = k ln2 + r with ln2 split into a high part whose low 21 mantissa bits are
// zero (so k * hi is exact) and the rounded remainder; then the degree-12
// Taylor polynomial of e^r on |r| <= ln2/2 (truncation below 1.7e-16
// relative) by Horner's rule, and an exact scale by 2^k.  Arguments below
// -745.5 (where e^y underflows to zero) and NaN return 0.  The constants come
// in `e` (kernel arguments, hence scalar registers).
__device__ inline double exp_f64(double y, const ExpConsts& e) {
  if (!(y > -745.5)) return 0.0;
  const double k = rint(y * e.log2e);
  double r = fma(-k, e.ln2_hi, y);
  r = fma(-k, e.ln2_lo, r);
  double q = e.inv_fact[0];
#pragma unroll
  for (int i = 1; i < 11; ++i) q = fma(q, r, e.inv_fact[i]);
  q = fma(q, r, 1.0);
  q = fma(q, r, 1.0);
  return ldexp(q, static_cast<int>(k));
}

// ----------------------------------------------------------- reductions --
// Cross-lane steps by DPP (data-parallel primitives: a VALU operand read from
// another lane of the same row of 16, or broadcast between rows), which take
// a few cycles where an LDS permute takes tens.  Lanes outside the row/bank
// masks, and sources outside the row, give 0.  All 64 lanes must be active.
template <int CTRL, int ROW_MASK, int BANK_MASK = 0xf>
__device__ inline int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, true);
}
template <int CTRL, int ROW_MASK, int BANK_MASK = 0xf>
__device__ inline double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROW_MASK, BANK_MASK>(static_cast<int>(b));
  const int hi = dpp_i32<CTRL, ROW_MASK, BANK_MASK>(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
__device__ inline double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Wave reductions: butterflies within each row of 16 lanes (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror), then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3, so lane
// 63 holds the result, which every lane gets as a scalar.  Fixed order, so
// deterministic.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_i32<0xb1, 0xf>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i32<0x4e, 0xf>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i32<0x141, 0xf>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i32<0x140, 0xf>(__float_as_int(v))));
  // rows outside the broadcast masks take 0 from the DPP; max with the value itself keeps them
  const float b15 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xa, 0xf, false));
  v = fmaxf(v, b15);
  const float b31 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xc, 0xf, false));
  v = fmaxf(v, b31);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One step of an order-independent reduction: lanes outside the row mask
// see their own value, which leaves them unchanged.
template <int CTRL, int ROW_MASK>
__device__ inline int dpp_keep(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}

template <typename Op>
__device__ inline int wave_reduce_i32(int v, Op op) {
  v = op(v, dpp_keep<0xb1, 0xf>(v));
  v = op(v, dpp_keep<0x4e, 0xf>(v));
  v = op(v, dpp_keep<0x141, 0xf>(v));
  v = op(v, dpp_keep<0x140, 0xf>(v));
  v = op(v, dpp_keep<0x142, 0xa>(v));
  v = op(v, dpp_keep<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline int wave_min_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return min(a, b); });
}

__device__ inline int wave_max_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return max(a, b); });
}

__device__ inline double wave_sum(double v) {
  v += dpp_f64<0xb1, 0xf>(v);
  v += dpp_f64<0x4e, 0xf>(v);
  v += dpp_f64<0x141, 0xf>(v);
  v += dpp_f64<0x140, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  return readlane_f64(v, 63);
}

// fp32 sum over a whole wave (all 64 lanes active) by DPP: butterflies within
// rows of 16 lanes, then two row broadcasts; fixed order, so deterministic.
// Every lane gets the total (lane 63's value, read as a scalar).
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

__device__ inline float wave_sum_f32(float v) {
  v += dpp_f32<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141, 0xf>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xf>(v);  // row_mirror: every lane holds its row's sum
  v += dpp_f32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds the total
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// (value, index) arg-max merge: larger value wins, equal values keep the lower index.
__device__ inline void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <int CTRL, int ROW_MASK>
__device__ inline void argmax_step(float& v, int& i) {
  const float v2 = __int_as_float(dpp_keep<CTRL, ROW_MASK>(__float_as_int(v)));
  const int i2 = dpp_keep<CTRL, ROW_MASK>(i);
  argmax_merge(v, i, v2, i2);
}

// Every lane gets the wave's (largest value, lowest index holding it); the
// merge is a total order, so the DPP order gives the same answer as any other.
__device__ inline void wave_argmax(float& v, int& i) {
  argmax_step<0xb1, 0xf>(v, i);
  argmax_step<0x4e, 0xf>(v, i);
  argmax_step<0x141, 0xf>(v, i);
  argmax_step<0x140, 0xf>(v, i);
  argmax_step<0x142, 0xa>(v, i);
  argmax_step<0x143, 0xc>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// ------------------------------------------------------ sweep partials --
// Fold one lane's (R, s) sweep partial into its running pair (ml, sl):
// exact power-of-two rescales, fp64 sums.  Any float pair is safe here (the
// shift counts are clamped to [-1000, 0]), so stale partials of rows a call
// did not sweep give meaningless but harmless values.
__device__ inline void fold_partial(float& ml, double& sl, float2 q) {
  if (q.x == -INFINITY) return;
  if (q.x > ml) {
    sl = ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - q.x, -1000.f)));
    ml = q.x;
  }
  sl += ldexp(static_cast<double>(q.y), static_cast<int>(fmaxf(q.x - ml, -1000.f)));
}

// log2 sum 2^(x c) of a row from the lanes' running pairs (whole wave).  The
// exponent of the sum is exact (frexp); its mantissa's log2 comes from
// v_log_f32, good to ~1e-7 absolute, which is all the uses of the normaliser
// need (the acceptance test's near-tie window is 1e-5 and the draw normalises
// by its own sums).
__device__ inline double wave_log2z(float ml, double sl) {
  const float M = wave_max(ml);
  const double S = wave_sum(ml == -INFINITY ? 0.0 : ldexp(sl, static_cast<int>(fmaxf(ml - M, -1000.f))));
  int e;
  const double m = frexp(S, &e);  // S = m 2^e, m in [1/2, 1)
  return static_cast<double>(M) + e + __builtin_amdgcn_logf(static_cast<float>(m));
}

// Workgroup-wide sum of one double per thread over NW waves; every thread
// gets the total.
template <int NW>
__device__ inline double block_sum_n(double v, double* lds /* >= NW */) {
  v = wave_sum(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += lds[i];
  return t;
}

__device__ inline double block_sum(double v, double* lds /* >= kWaves */) { return block_sum_n<kWaves>(v, lds); }

__device__ inline float block_max(float v, float* lds /* >= kWaves */) {
  v = wave_max(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = fmaxf(t, lds[i]);
  return t;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline double wave_inclusive_scan(double v) {
  // within each row of 16: the sum of the last four lanes (row_shr 1..3 of
  // the inputs), then + the value 4 lanes back (lanes 4..15), then + the
  // value 8 lanes back (lanes 8..15); then the rows' totals by broadcast
  double s = v;
  s += dpp_f64<0x111, 0xf>(v);
  s += dpp_f64<0x112, 0xf>(v);
  s += dpp_f64<0x113, 0xf>(v);
  s += dpp_f64<0x114, 0xf, 0xe>(s);
  s += dpp_f64<0x118, 0xf, 0xc>(s);
  s += dpp_f64<0x142, 0xa>(s);  // rows 1 and 3: + lane 15 of the row before
  s += dpp_f64<0x143, 0xc>(s);  // rows 2 and 3: + lane 31
  return s;
}

// Exclusive prefix sum of one double per thread over a workgroup of NW
// waves, in thread order.  Returns the exclusive prefix; *total gets the
// block total.
template <int NW>
__device__ inline double block_exclusive_scan_n(double v, double* lds /* >= NW */, double* total) {
  const double inc = wave_inclusive_scan(v);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  double excl = __shfl_up(inc, 1, kWave);
  if (lane == 0) excl = 0.0;
  __syncthreads();
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  double before = 0.0, all = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += lds[i];
    all += lds[i];
  }
  *total = all;
  return before + excl;
}

}  // namespace sv
