// n-gram map: the hash-table form of the prompt-lookup proposer ([D]
// "Спекулятивное декодирование на n-граммах": its map variants key a hash
// table by the current n-gram of size N and keep what followed it, so that a
// lookup replaces the linear scan of the history).
//
// One table per sequence in device memory, kept by the caller from call to
// call: open addressing with linear probing over `capacity` slots (a power of
// two).  A slot holds {key, count, end}: the 64-bit key of an n-gram and its
// size, the number of its occurrences that a token follows, and the latest
// such occurrence's end e (h[e-n..e) is the n-gram, h[e] the token after it).
// The table's first 16 bytes hold a flag, set when an insert found no free
// slot within kMaxProbe probes (the table is then too small for the history).
//
// One workgroup per sequence and call:
//  - A sequence whose previous length is 0 gets its table cleared, and is
//    built from its whole history.
//  - Insert every n-gram of a size n in [n_min, n_max] that ends at e in
//    [max(n, L_old), L_new - 1], i.e. whose following token arrived since the
//    previous call: compare-and-swap the key into its slot, then add 1 to the
//    count and raise the end to e.  Thread t takes ends L_old + t, + 256, ...;
//    the keys of all sizes ending at e come out of one pass over the tokens
//    before e, and their first probes go out together.
//  - Propose: lane j of wave 0 looks up the suffix of size n = n_max - j as
//    the previous calls left it, before any count changes, and adds this
//    call's own occurrences of it (counted in LDS while the keys are made);
//    the largest n counted at least min_hits times wins, and the draft is
//    h[end..min(end + K, L_new)).  That is the scan's proposal (k_ngram.hip)
//    for the same history, as long as no two different n-grams of one history
//    share a key (about N^2 / 2^65 for N of them).
//  - A decode step adds a few ends, one per thread: the keys go into their
//    slots before the barrier that ends the lookups, and only the counts and
//    ends after it, so the lookups, the draft's loads and the inserts overlap.
// Atomics have workgroup scope (performed in the L2 of the workgroup's XCD):
// one table is touched by one workgroup per call, and the end of a kernel
// publishes it to the next call's workgroup, on whichever XCD that runs.
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kMapBlock = 256;
constexpr int kMaxProbe = 64;
constexpr int kMaxN = SPECV_MAX_NGRAM;
constexpr uint64_t kKeySeed = 0x243F6A8885A308D3ull;  // any odd start value

struct NgSlot {
  unsigned long long key;  // 0: empty
  int count;
  int end;
};
static_assert(sizeof(NgSlot) == 16, "slot layout");

// Rolling part of the key: tokens folded in from the one just before e
// backwards (xor, multiply by an odd constant, xor-shift), so that one pass
// over h[e-1], h[e-2], ... gives the keys of every size ending at e.
__device__ inline uint64_t ng_step(uint64_t s, int32_t tok) {
  s ^= static_cast<uint32_t>(tok);
  s *= 0x9E3779B97F4A7C15ull;
  return s ^ (s >> 29);
}

// The key of the size-n n-gram whose rolling part is s: the size mixed in,
// then the xor-shift-multiply avalanche of the splitmix64 generator's output
// step.  0 marks an empty slot and is mapped to 1.
__device__ inline unsigned long long ng_key(uint64_t s, int n) {
  uint64_t z = s + static_cast<uint64_t>(n) * 0xD1B54A32D192ED03ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z ? z : 1ull;
}

__device__ inline unsigned long long cas_key(NgSlot* sl, unsigned long long key) {
  unsigned long long expected = 0ull;
  __hip_atomic_compare_exchange_strong(&sl->key, &expected, key, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
  return expected;  // the key found there (0 if the slot was empty and is now ours)
}

// Insert key into its slot: the first probe's CAS result `o` is given; probe
// on past other keys.  Returns the slot, or -1 when none was free within
// kMaxProbe probes.
__device__ inline int probe_insert(NgSlot* slots, unsigned mask, unsigned long long key, unsigned long long o) {
  unsigned slot = static_cast<unsigned>(key) & mask;
  for (int probe = 1; o != 0ull && o != key && probe < kMaxProbe; ++probe) {
    slot = (slot + 1u) & mask;
    o = cas_key(&slots[slot], key);
  }
  return (o == 0ull || o == key) ? static_cast<int>(slot) : -1;
}

__device__ inline void count_occurrence(NgSlot* sl, int e) {
  __hip_atomic_fetch_add(&sl->count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __hip_atomic_fetch_max(&sl->end, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The keys of the n-grams of sizes 1..NM ending at e (tokens h[e-1],
// h[e-2], ..., loads clamped to the history's start).
template <int NM>
__device__ inline void keys_at(const int32_t* h, int e, unsigned long long (&key)[NM]) {
  int32_t tok[NM];
#pragma unroll
  for (int j = 0; j < NM; ++j) tok[j] = h[max(e - 1 - j, 0)];
  uint64_t s = kKeySeed;
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    s = ng_step(s, tok[j]);
    key[j] = ng_key(s, j + 1);
  }
}

// NM: the largest size the kernel is compiled for (n_max <= NM).
template <int NM>
__global__ __launch_bounds__(kMapBlock) void k_ngram_map(char* tables, int cap, const int32_t* hist, int Lmax,
                                                         const int32_t* len_old, const int32_t* len_new,
                                                         int n_min, int n_max, int min_hits, int K,
                                                         int32_t* out_draft, int32_t* out_count,
                                                         int32_t* out_status) {
  const long b = blockIdx.x;
  const int t = static_cast<int>(threadIdx.x), lane = t % kWave, w = t / kWave;
  const int32_t* h = hist + b * static_cast<long>(Lmax);
  char* base = tables + b * (16 + 16 * static_cast<long>(cap));
  int* full = reinterpret_cast<int*>(base);
  NgSlot* slots = reinterpret_cast<NgSlot*>(base + 16);
  const unsigned mask = static_cast<unsigned>(cap) - 1u;
  const int L = min(max(len_new[b], 0), Lmax);
  const int L0 = min(max(len_old[b], 0), L);
  const bool fresh = L0 == 0;  // uniform: a new history, whose table is cleared and built whole
  // this call's occurrences of the suffix of each size (index n - 1): count and latest end
  __shared__ int s_cnt[NM], s_end[NM];
  __shared__ int s_full;  // an insert of this call found no free slot
  if (t < NM) {
    s_cnt[t] = 0;
    s_end[t] = 0;
  }
  if (t == 0) s_full = 0;
  // a decode step adds few ends, at most one per thread: their keys are made
  // now, with the suffix's keys (the loads of both in flight together), in
  // the threads that use them: wave 0 (the lookups) and those with an end
  auto in_use = [&](int m, int e) { return m >= n_min && m <= n_max && m <= e; };
  const int e_lo = max(L0, n_min);
  const bool one_pass = L - e_lo <= kMapBlock;  // uniform
  const int e1 = e_lo + t;
  const bool has = one_pass && e1 < L;
  unsigned long long skey[NM], ik[NM];
  if (w == 0 || has || !one_pass) {
    keys_at<NM>(h, L, skey);
    keys_at<NM>(h, has ? e1 : 1, ik);
  }
  if (fresh) {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) *reinterpret_cast<uint4*>(base) = zero;
    for (long i = t; i < cap; i += kMapBlock) reinterpret_cast<uint4*>(slots)[i] = zero;
  }
  __syncthreads();  // LDS counters set; a cleared table's stores are in L2

  // The suffix's entries as the previous calls left them: lane j of wave 0
  // looks up size n = n_max - j (key and count/end read together).  Keys
  // this call inserts may land in empty slots meanwhile, with count 0, which
  // changes no lookup's result; counts change only after the next barrier.
  const int n = n_max - lane;
  const bool active = w == 0 && n >= n_min && n >= 1 && n <= L;
  unsigned long long key = 0ull;
#pragma unroll
  for (int j = 0; j < NM; ++j) key = j + 1 == n ? skey[j] : key;
  int cnt = 0, end = 0;
  int was_full = 0;  // the flag as the previous calls left it (a build starts clear)
  auto lookup = [&]() {
    if (w == 0 && !fresh) was_full = __hip_atomic_load(full, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (!active || fresh) return;
    unsigned slot = static_cast<unsigned>(key) & mask;
    for (int probe = 0; probe < kMaxProbe; ++probe) {
      const unsigned long long k = __hip_atomic_load(&slots[slot].key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const unsigned long long ce = __hip_atomic_load(reinterpret_cast<unsigned long long*>(&slots[slot].count),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (k == key) {
        cnt = static_cast<int>(static_cast<uint32_t>(ce));
        end = static_cast<int>(static_cast<uint32_t>(ce >> 32));
        return;
      }
      if (k == 0ull) return;
      slot = (slot + 1u) & mask;
    }
  };
  // this call's n-grams equal to the suffix of their size, counted in LDS
  auto match = [&](const unsigned long long (&k)[NM], int e) {
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (in_use(j + 1, e) && k[j] == skey[j]) {
        atomicAdd(&s_cnt[j], 1);
        atomicMax(&s_end[j], e);
      }
    }
  };
  if (one_pass) {
    // keys into their slots (first probes together), then the lookups
    unsigned long long o[NM];
#pragma unroll
    for (int j = 0; j < NM; ++j) o[j] = has && in_use(j + 1, e1) ? cas_key(&slots[ik[j] & mask], ik[j]) : 0ull;
    lookup();
    int slot[NM];
#pragma unroll
    for (int j = 0; j < NM; ++j) slot[j] = -1;
    if (has) {
      match(ik, e1);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (!in_use(j + 1, e1)) continue;
        slot[j] = probe_insert(slots, mask, ik[j], o[j]);
        if (slot[j] < 0) {
          s_full = 1;
          __hip_atomic_fetch_or(full, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    __syncthreads();  // the lookups and the LDS counts are done: counts may change now
#pragma unroll
    for (int j = 0; j < NM; ++j)
      if (slot[j] >= 0) count_occurrence(&slots[slot[j]], e1);
  } else {  // a build, or a long update: the lookups, then every insert
    lookup();
    __syncthreads();
    for (int e = e_lo + t; e < L; e += kMapBlock) {
      unsigned long long k[NM], o[NM];
      keys_at<NM>(h, e, k);
      match(k, e);
#pragma unroll
      for (int j = 0; j < NM; ++j) o[j] = in_use(j + 1, e) ? cas_key(&slots[k[j] & mask], k[j]) : 0ull;
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (!in_use(j + 1, e)) continue;
        const int sl = probe_insert(slots, mask, k[j], o[j]);
        if (sl >= 0) {
          count_occurrence(&slots[sl], e);
        } else {
          s_full = 1;
          __hip_atomic_fetch_or(full, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    __syncthreads();  // the LDS counts and the overflow flag are final
  }

  if (w != 0) return;
  // the answer: the previous calls' entry plus this call's occurrences
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    if (j + 1 == n) {
      cnt += s_cnt[j];
      end = max(end, s_end[j]);
    }
  }
  const int overflow = __builtin_amdgcn_readfirstlane(was_full) | s_full;
  const uint64_t won = __ballot(active && cnt >= min_hits && cnt > 0);
  int e0 = 0, count = 0;
  if (won && !overflow) {  // uniform
    e0 = __builtin_amdgcn_readlane(end, __ffsll(static_cast<unsigned long long>(won)) - 1);
    count = min(K, L - e0);
  }
  if (lane < K) out_draft[b * K + lane] = lane < count ? h[max(min(e0 + lane, L - 1), 0)] : -1;
  if (lane == 0) {
    out_count[b] = count;
    if (out_status) out_status[b] = overflow ? SPECV_NGRAM_MAP_FULL : 0;
  }
}

}  // namespace

hipError_t launch_ngram_map(void* tables, int capacity, const int32_t* hist, const int32_t* len_old,
                            const int32_t* len_new, int B, int Lmax, int n_min, int n_max, int min_hits, int K,
                            int32_t* out_draft, int32_t* out_count, int32_t* out_status, hipStream_t s) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(B)), dim3(kMapBlock), 0, s, static_cast<char*>(tables),
                       capacity, hist, Lmax, len_old, len_new, n_min, n_max, min_hits, K, out_draft, out_count,
                       out_status);
  };
  if (n_max <= 4) go(k_ngram_map<4>);
  else if (n_max <= 8) go(k_ngram_map<8>);
  else go(k_ngram_map<kMaxN>);
  return hipGetLastError();
}

}  // namespace sv
