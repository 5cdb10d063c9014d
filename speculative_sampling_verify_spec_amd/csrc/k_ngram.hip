// n-gram (prompt-lookup) draft proposer, one workgroup per history ([D]
// "Спекулятивное декодирование на n-граммах": when the latest tokens repeat
// an earlier n-gram, propose what followed it; [A]: Prompt Lookup takes the
// draft from the context itself).
//
// For a history h[0..L), an occurrence of the size-n suffix ends at e
// (1 <= e <= L - 1, so a token follows it) where h[e-n..e) == h[L-n..L).
// Ends are visited in rounds of 4096, sixteen per thread; a round's tokens and
// the 16 before them are staged in LDS by coalesced loads (the next round's
// loads issued before this round's work).  Each thread first compares the
// last token of its ends with the suffix's (one compare per end, a bit mask);
// size 1 is counted from the mask, and only the ends that passed go on to the
// remaining comparisons, whose run of matches m(e) is counted for every size
// n <= m(e) in per-thread registers (count and latest end per size, compiled
// for the largest size in use); waves reduce them and LDS atomics gather one
// value per wave.
// Thread 0 takes the largest n in [n_min, n_max] seen at least min_hits
// times, and the workgroup writes h[e*..min(e* + K, L)) for its latest end
// e*, then -1 up to K.  Without such an n the proposal is empty.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kNgBlock = 256;
constexpr int kNgPer = 16;                       // ends per thread per round
constexpr int kNgRound = kNgBlock * kNgPer;

template <int NM>
__global__ __launch_bounds__(kNgBlock) void k_ngram(const int32_t* hist, const int32_t* lengths, int Lmax,
                                                    int n_min, int n_max, int min_hits, int K,
                                                    int32_t* out_draft, int32_t* out_count) {
  const long b = blockIdx.x;
  const int32_t* h = hist + b * static_cast<long>(Lmax);
  const int L = min(max(lengths[b], 0), Lmax);
  const int lane = threadIdx.x % kWave;
  __shared__ int32_t suf[SPECV_MAX_NGRAM];  // suf[j] = h[L-1-j]
  __shared__ int cnt[SPECV_MAX_NGRAM + 1], last[SPECV_MAX_NGRAM + 1];
  __shared__ int s_e;
  if (threadIdx.x < SPECV_MAX_NGRAM) suf[threadIdx.x] = threadIdx.x < L ? h[L - 1 - threadIdx.x] : 0;
  if (threadIdx.x <= SPECV_MAX_NGRAM) {
    cnt[threadIdx.x] = 0;
    last[threadIdx.x] = -1;
  }
  __syncthreads();
  const int jmax = min(n_max, L);  // the suffix has L tokens at most; n_max <= NM
  int32_t sf[NM];                  // the suffix in registers (the same for every lane)
#pragma unroll
  for (int j = 0; j < NM; ++j) sf[j] = suf[j];
  int c[NM], l[NM];  // per size n + 1: ends seen, the latest one (ends increase along a thread's walk)
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    c[n] = 0;
    l[n] = -1;
  }
  // rounds of kNgRound ends; the round's tokens and the NM before them are
  // staged in LDS (coalesced loads), so matches are measured without
  // dependent global loads
  __shared__ int32_t win[kNgRound + SPECV_MAX_NGRAM];
  // this round's tokens (from base - 1 on) and the NM before them, loaded one
  // round ahead so that the loads of round r + 1 overlap the work of round r
  auto fetch = [&](int base, int32_t (&v)[kNgPer], int32_t& hv) {
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) {
      const int i = base - 1 + r * kNgBlock + threadIdx.x;  // >= 0
      v[r] = i < L ? h[i] : 0;
    }
    const int i = base - 1 - NM + static_cast<int>(threadIdx.x);
    hv = (threadIdx.x < NM && i >= 0 && i < L) ? h[i] : 0;
  };
  int32_t v[kNgPer], hv = 0;
  if (L > 1) fetch(1, v, hv);
  for (int base = 1; base < L; base += kNgRound) {
    const int w0 = base - 1 - NM;  // win[k] = h[w0 + k]
    int32_t nv[kNgPer], nhv = 0;
    if (base + kNgRound < L) fetch(base + kNgRound, nv, nhv);  // uniform
    __syncthreads();  // the previous round is done with win
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) win[NM + r * kNgBlock + threadIdx.x] = v[r];
    if (threadIdx.x < NM) win[threadIdx.x] = hv;
    __syncthreads();
    // first tokens: bit r of `first` says whether end r's last token equals
    // the suffix's (m(e) >= 1: e < L, and the suffix has a token); that token,
    // h[e - 1], is the thread's own v[r]
    uint32_t first = 0;
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) {
      const int e = base + r * kNgBlock + threadIdx.x;
      first |= ((e < L && jmax > 0 && v[r] == sf[0]) ? 1u : 0u) << r;
    }
    // size 1 straight from the bits (ends increase with r)
    c[0] += __popc(first);
    if (first) l[0] = base + (31 - __clz(first)) * kNgBlock + threadIdx.x;
    // longer sizes: only the ends whose last token matched, in increasing order
    uint32_t more = NM > 1 ? first : 0u;
    while (more) {
      const int r = __builtin_ctz(more);
      more &= more - 1u;
      const int e = base + r * kNgBlock + threadIdx.x;
      const int k = e - 1 - w0;
      // match length m(e): trailing ones of the NM comparisons (j = 0 matched),
      // cut to the sizes that exist (j < jmax and h[e-1-j] inside the history)
      uint32_t bits = 1u;
#pragma unroll
      for (int j = 1; j < NM; ++j) bits |= (win[k - j] == sf[j] ? 1u : 0u) << j;
      bits &= (1u << min(jmax, e)) - 1u;
      const int m = __builtin_ctz(~bits);
#pragma unroll
      for (int n = 1; n < NM; ++n) {
        c[n] += m > n ? 1 : 0;
        l[n] = m > n ? e : l[n];
      }
    }
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) v[r] = nv[r];
    hv = nhv;
  }
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    if (n < n_max) {  // uniform
      int cs = c[n], ls = l[n];
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        cs += __shfl_xor(cs, o, kWave);
        ls = max(ls, __shfl_xor(ls, o, kWave));
      }
      if (lane == 0 && cs > 0) {
        atomicAdd(&cnt[n + 1], cs);
        atomicMax(&last[n + 1], ls);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int e = -1;
    for (int n = n_max; n >= n_min; --n) {
      if (cnt[n] >= min_hits && cnt[n] > 0) {
        e = last[n];
        break;
      }
    }
    s_e = e;
    out_count[b] = e < 0 ? 0 : min(K, L - e);
  }
  __syncthreads();
  const int e = s_e;
  if (threadIdx.x < K) {
    const int i = threadIdx.x;
    out_draft[b * K + i] = (e >= 0 && e + i < L) ? h[e + i] : -1;
  }
}

}  // namespace

hipError_t launch_ngram(const int32_t* hist, const int32_t* lengths, int B, int Lmax, int n_min, int n_max,
                        int min_hits, int K, int32_t* out_draft, int32_t* out_count, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(B)), block(kNgBlock);
  // counters for the sizes in use only (registers, fully unrolled)
  if (n_max <= 4)
    hipLaunchKernelGGL(k_ngram<4>, grid, block, 0, st, hist, lengths, Lmax, n_min, n_max, min_hits, K, out_draft,
                       out_count);
  else if (n_max <= 8)
    hipLaunchKernelGGL(k_ngram<8>, grid, block, 0, st, hist, lengths, Lmax, n_min, n_max, min_hits, K, out_draft,
                       out_count);
  else
    hipLaunchKernelGGL(k_ngram<SPECV_MAX_NGRAM>, grid, block, 0, st, hist, lengths, Lmax, n_min, n_max, min_hits,
                       K, out_draft, out_count);
  return hipGetLastError();
}

}  // namespace sv
