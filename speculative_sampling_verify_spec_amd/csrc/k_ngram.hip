// n-gram (prompt-lookup) draft proposer, one workgroup per history ([D]
// "Спекулятивное декодирование на n-граммах": when the latest tokens repeat
// an earlier n-gram, propose what followed it; [A]: Prompt Lookup takes the
// draft from the context itself).
//
// For a history h[0..L), an occurrence of the size-n suffix ends at e
// (1 <= e <= L - 1, so a token follows it) where h[e-n..e) == h[L-n..L).
// Thread t visits ends e = 1 + t, 1 + t + 1024, ... and measures the match
// length m(e) by comparing backwards with the suffix (held in LDS; almost
// every end fails at the first token).  Per size n it counts ends with
// m(e) >= n and keeps the latest one; waves reduce, LDS atomics gather.
// Thread 0 takes the largest n in [n_min, n_max] seen at least min_hits
// times, and the workgroup writes h[e*..min(e* + K, L)) for its latest end
// e*, then -1 up to K.  Without such an n the proposal is empty.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kNgBlock = 1024;
constexpr int kNgWaves = kNgBlock / kWave;

__global__ __launch_bounds__(kNgBlock) void k_ngram(const int32_t* hist, const int32_t* lengths, int Lmax,
                                                    int n_min, int n_max, int min_hits, int K,
                                                    int32_t* out_draft, int32_t* out_count) {
  const long b = blockIdx.x;
  const int32_t* h = hist + b * static_cast<long>(Lmax);
  const int L = min(max(lengths[b], 0), Lmax);
  const int lane = threadIdx.x % kWave;
  __shared__ int32_t suf[SPECV_MAX_NGRAM];  // suf[j] = h[L-1-j]
  __shared__ int cnt[SPECV_MAX_NGRAM + 1], last[SPECV_MAX_NGRAM + 1];
  __shared__ int s_e, s_n;
  if (threadIdx.x < SPECV_MAX_NGRAM) suf[threadIdx.x] = threadIdx.x < L ? h[L - 1 - threadIdx.x] : 0;
  if (threadIdx.x <= SPECV_MAX_NGRAM) {
    cnt[threadIdx.x] = 0;
    last[threadIdx.x] = -1;
  }
  __syncthreads();
  const int jmax = min(n_max, L);  // the suffix has L tokens at most
  int c[SPECV_MAX_NGRAM], l[SPECV_MAX_NGRAM];
#pragma unroll
  for (int n = 0; n < SPECV_MAX_NGRAM; ++n) {
    c[n] = 0;
    l[n] = -1;
  }
  for (int e = 1 + threadIdx.x; e < L; e += kNgBlock) {
    int m = 0;
    while (m < jmax && m < e && h[e - 1 - m] == suf[m]) ++m;
#pragma unroll
    for (int n = 0; n < SPECV_MAX_NGRAM; ++n) {  // size n + 1
      if (m > n) {
        ++c[n];
        l[n] = e;  // ends increase along a thread's walk
      }
    }
  }
#pragma unroll
  for (int n = 0; n < SPECV_MAX_NGRAM; ++n) {
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
    int e = -1, size = 0;
    for (int n = n_max; n >= n_min; --n) {
      if (cnt[n] >= min_hits && cnt[n] > 0) {
        e = last[n];
        size = n;
        break;
      }
    }
    s_e = e;
    s_n = size;
    out_count[b] = e < 0 ? 0 : min(K, L - e);
  }
  __syncthreads();
  const int e = s_e;
  if (threadIdx.x < K) {
    const int i = threadIdx.x;
    out_draft[b * K + i] = (e >= 0 && e + i < L) ? h[e + i] : -1;
  }
  (void)kNgWaves;
}

}  // namespace

hipError_t launch_ngram(const int32_t* hist, const int32_t* lengths, int B, int Lmax, int n_min, int n_max,
                        int min_hits, int K, int32_t* out_draft, int32_t* out_count, hipStream_t st) {
  hipLaunchKernelGGL(k_ngram, dim3(static_cast<unsigned>(B)), dim3(kNgBlock), 0, st, hist, lengths, Lmax, n_min,
                     n_max, min_hits, K, out_draft, out_count);
  return hipGetLastError();
}

}  // namespace sv
