// n-gram (prompt-lookup) draft proposer, one workgroup per history ([D]
// "Спекулятивное декодирование на n-граммах": when the latest tokens repeat
// an earlier n-gram, propose what followed it; [A]: Prompt Lookup takes the
// draft from the context itself).
//
// For a history h[0..L), an occurrence of the size-n suffix ends at e
// (1 <= e <= L - 1, so a token follows it) where h[e-n..e) == h[L-n..L).
// Ends are visited in rounds of 4096, sixteen per thread; a round's tokens and
// the 16 before them are staged in LDS from registers filled by coalesced
// loads: 16-byte vectors of four consecutive tokens per lane when the rows
// allow it (L_max a multiple of 4, an aligned history), which measured far
// faster than one token per lane, else single tokens.  The suffix is loaded
// first, then the first four rounds (histories up to 16385 tokens) all before
// the first round, so that rounds do not wait for memory one after another;
// longer histories load their later rounds one at a time.
// Each thread compares the last token of each of its ends with the suffix's
// last token, and the token before it with the suffix's second-last (from
// the thread's own registers inside a 16-byte vector, else from LDS): two bit
// masks per thread, which count sizes 1 and 2.  Only the ends that matched
// both go on to the remaining comparisons, whose run of matches m(e) is
// counted for every size n <= m(e) in per-thread registers (count and latest
// end per size, compiled for the largest size in use);
// DPP wave reductions and LDS atomics gather one value per wave.
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
constexpr int kNgPre = 4;                        // rounds loaded before the first (histories up to 16385 tokens)

// Offset within a round of thread t's r-th token (and end): VEC4, the four
// tokens of vector r / 4 (vectors of a round 1024 tokens apart); otherwise
// every 256th token.  Both increase with r.
template <bool VEC4>
__device__ inline int ng_off(int r, int t) {
  return VEC4 ? (r >> 2) * (kNgBlock * 4) + 4 * t + (r & 3) : r * kNgBlock + t;
}

template <int NM, bool VEC4>
__global__ __launch_bounds__(kNgBlock) void k_ngram(const int32_t* hist, const int32_t* lengths, int Lmax,
                                                    int n_min, int n_max, int min_hits, int K,
                                                    int32_t* out_draft, int32_t* out_count) {
  const long b = blockIdx.x;
  const int32_t* h = hist + b * static_cast<long>(Lmax);
  const int t = static_cast<int>(threadIdx.x);
  const int lane = t % kWave;
  const int L_raw = lengths[b];
  // Memory order.  All history loads are branch-free (indices clamped;
  // tokens at or past L, and before the history, are never counted): a load
  // under a branch makes the compiler wait for every load in flight.  After
  // the length (a scalar load):
  //  - the suffix, by one vector load ahead of all others (lane j < NM reads
  //    h[L-1-j]); vector loads complete in order, so waiting for it waits
  //    for nothing else;
  //  - the tokens of rounds 0 .. kNgPre - 1, clamped to the last token, all
  //    issued before the first round, so that no round waits for memory
  //    once the one before it is done.
  // round pr's tokens h[pr * kNgRound + ng_off(r, t)], and the NM before it.
  // VEC4: a vector starting past the clamp reads the clamp's vector instead
  // (rows are whole vectors); all its tokens lie past L and are never used.
  int32_t v[kNgPre][kNgPer], hv[kNgPre];
  auto load_round = [&](int pr, int clamp_to) {
    if constexpr (VEC4) {
      const int4* h4 = reinterpret_cast<const int4*>(h);
#pragma unroll
      for (int q = 0; q < kNgPer / 4; ++q) {
        const int4 x = h4[min(pr * kNgRound + ng_off<true>(4 * q, t), clamp_to & ~3) / 4];
        v[pr][4 * q] = x.x;
        v[pr][4 * q + 1] = x.y;
        v[pr][4 * q + 2] = x.z;
        v[pr][4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kNgPer; ++r) v[pr][r] = h[min(pr * kNgRound + ng_off<false>(r, t), clamp_to)];
    }
  };
  hv[0] = 0;  // before the history
  const int L = min(max(L_raw, 0), Lmax);
  const int last_tok = max(L - 1, 0);
  const int32_t sx = h[max(L - 1 - min(lane, NM - 1), 0)];
  __builtin_amdgcn_sched_barrier(0);
  load_round(0, last_tok);
#pragma unroll
  for (int pr = 1; pr < kNgPre; ++pr) {
    load_round(pr, last_tok);
    hv[pr] = h[min(max(pr * kNgRound - NM + t, 0), last_tok)];  // used by threads < NM
  }
  __shared__ int cnt[SPECV_MAX_NGRAM + 1], last[SPECV_MAX_NGRAM + 1];
  __shared__ int s_e;
  if (t <= SPECV_MAX_NGRAM) {  // published by the barriers below
    cnt[t] = 0;
    last[t] = -1;
  }
  int32_t sf[NM];  // sf[j] = h[L-1-j], the suffix
#pragma unroll
  for (int j = 0; j < NM; ++j) sf[j] = j < L ? __builtin_amdgcn_readlane(sx, j) : 0;
  const int jmax = min(n_max, L);  // the suffix has L tokens at most; n_max <= NM
  int c[NM], l[NM];  // per size n + 1: ends seen, the latest one (ends increase along a thread's walk)
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    c[n] = 0;
    l[n] = -1;
  }
  // One round: ends base .. base + kNgRound - 1, from the thread's tokens vr
  // (vr[r] = h[base - 1 + ng_off(r, t)]) and hvr (the NM tokens before the
  // round, threads < NM), staged in LDS so that matches are measured without
  // dependent global loads.
  __shared__ __align__(16) int32_t win[kNgRound + SPECV_MAX_NGRAM];
  auto round = [&](int base, const int32_t (&vr)[kNgPer], int32_t hvr) {
    const int w0 = base - 1 - NM;  // win[k] = h[w0 + k]
    __syncthreads();  // the previous round is done with win
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) win[NM + ng_off<VEC4>(r, t)] = vr[r];
    if (t < NM) win[t] = hvr;
    __syncthreads();
    // first tokens: bit r of `first` says whether end r's last token equals
    // the suffix's (m(e) >= 1: e < L, and the suffix has a token); that token,
    // h[e - 1], is the thread's own vr[r]
    uint32_t first = 0;
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) first |= (vr[r] == sf[0] ? 1u : 0u) << r;
    // ends at or past L (the last round only; uniform test), or no suffix
    if (base + kNgRound > L || jmax <= 0) {
      uint32_t live = 0;
#pragma unroll
      for (int r = 0; r < kNgPer; ++r) live |= (base + ng_off<VEC4>(r, t) < L && jmax > 0 ? 1u : 0u) << r;
      first &= live;
    }
    // size 1 straight from the bits (ends increase with r)
    c[0] += __popc(first);
    if (first) l[0] = base + ng_off<VEC4>(31 - __clz(first), t);
    // size 2 likewise: the token before each end's last one, h[e - 2], is the
    // thread's own vr[r - 1] within a vector, else the window's (end 1 has none)
    uint32_t second = 0;
    if (NM > 1 && jmax > 1) {  // uniform
#pragma unroll
      for (int r = 0; r < kNgPer; ++r) {
        const int32_t pv = (VEC4 && (r & 3)) ? vr[r > 0 ? r - 1 : 0] : win[NM - 1 + ng_off<VEC4>(r, t)];
        second |= (pv == sf[1] ? 1u : 0u) << r;
      }
      second &= first;
      if (base == 1 && t == 0) second &= ~1u;
      c[1] += __popc(second);
      if (second) l[1] = base + ng_off<VEC4>(31 - __clz(second), t);
    }
    // longer sizes: only the ends whose last two tokens matched, in increasing order
    uint32_t more = NM > 2 ? second : 0u;
    while (more) {
      const int r = __builtin_ctz(more);
      more &= more - 1u;
      const int e = base + ng_off<VEC4>(r, t);
      const int k = e - 1 - w0;
      // match length m(e): trailing ones of the NM comparisons (j = 0, 1
      // matched), cut to the sizes that exist (j < jmax and h[e-1-j] inside
      // the history)
      uint32_t bits = 3u;
#pragma unroll
      for (int j = 2; j < NM; ++j) bits |= (win[k - j] == sf[j] ? 1u : 0u) << j;
      bits &= (1u << min(jmax, e)) - 1u;
      const int m = __builtin_ctz(~bits);
#pragma unroll
      for (int n = 2; n < NM; ++n) {
        c[n] += m > n ? 1 : 0;
        l[n] = m > n ? e : l[n];
      }
    }
  };
#pragma unroll
  for (int pr = 0; pr < kNgPre; ++pr) {
    const int base = 1 + pr * kNgRound;
    if (base < L) round(base, v[pr], hv[pr]);  // uniform
  }
  // histories longer than kNgPre rounds: the rest, one round at a time
  for (int base = 1 + kNgPre * kNgRound; base < L; base += kNgRound) {
    int32_t vt[kNgPer];
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) vt[r] = h[min(base - 1 + ng_off<VEC4>(r, t), L - 1)];
    round(base, vt, h[min(max(base - 1 - NM + t, 0), L - 1)]);
  }
  // per size: the wave's count and latest end (DPP reductions, lane 63 holds
  // the result), one LDS atomic per wave
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    if (n < n_max) {  // uniform
      const int cs = wave_reduce_i32(c[n], [](int a, int x) { return a + x; });
      const int ls = wave_reduce_i32(l[n], [](int a, int x) { return max(a, x); });
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
  if (static_cast<int>(threadIdx.x) < K) {
    const int i = threadIdx.x;
    out_draft[b * K + i] = (e >= 0 && e + i < L) ? h[e + i] : -1;
  }
}

}  // namespace

template <bool VEC4>
void launch_ngram_t(const int32_t* hist, const int32_t* lengths, int B, int Lmax, int n_min, int n_max,
                    int min_hits, int K, int32_t* out_draft, int32_t* out_count, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(B)), block(kNgBlock);
  // counters for the sizes in use only (registers, fully unrolled)
  if (n_max <= 4)
    hipLaunchKernelGGL((k_ngram<4, VEC4>), grid, block, 0, st, hist, lengths, Lmax, n_min, n_max, min_hits, K,
                       out_draft, out_count);
  else if (n_max <= 8)
    hipLaunchKernelGGL((k_ngram<8, VEC4>), grid, block, 0, st, hist, lengths, Lmax, n_min, n_max, min_hits, K,
                       out_draft, out_count);
  else
    hipLaunchKernelGGL((k_ngram<SPECV_MAX_NGRAM, VEC4>), grid, block, 0, st, hist, lengths, Lmax, n_min, n_max,
                       min_hits, K, out_draft, out_count);
}

hipError_t launch_ngram(const int32_t* hist, const int32_t* lengths, int B, int Lmax, int n_min, int n_max,
                        int min_hits, int K, int32_t* out_draft, int32_t* out_count, hipStream_t st) {
  // whole 16-byte vectors per row: an aligned history and L_max a multiple of 4
  if (reinterpret_cast<uintptr_t>(hist) % 16 == 0 && Lmax % 4 == 0)
    launch_ngram_t<true>(hist, lengths, B, Lmax, n_min, n_max, min_hits, K, out_draft, out_count, st);
  else
    launch_ngram_t<false>(hist, lengths, B, Lmax, n_min, n_max, min_hits, K, out_draft, out_count, st);
  return hipGetLastError();
}

}  // namespace sv
