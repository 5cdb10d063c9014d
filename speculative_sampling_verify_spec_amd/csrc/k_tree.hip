// Token trees (at most 64 nodes, one per lane of a wave): greedy verification
// and the tree attention mask with depth position ids.
//
// A tree is parents[N] (parents[0] = -1, parents[v] < v) and a token per
// node; node 0 holds the committed root token, and row v of the logits scores
// the token after node v.  Lane v builds the set of node v's ancestors
// (itself included) as a 64-bit mask by pointer jumping: six rounds of
// "take the set of the node 2^r steps up" cover any depth below 64.  Then:
//  - mask ([C] "5.3 Medusa, EAGLE và MTP", sections 3.1 and 8): row v sees
//    exactly the nodes of its set; position id ([C] 3.2) = depth = size - 1;
//  - greedy verification ([C] 9.1; [A] "Token tree": the deepest accepted
//    branch is the round's output): node v passes its edge test when its
//    token is the first arg-max of its parent's row, and is accepted when
//    every node of its set passes (the root passes).  The deepest accepted
//    node d (lowest index among equals) gives the output: the tokens of its
//    set after the root, in depth order, then the arg-max of row d.
// A node whose parent is not in [0, v) has an empty chain: it sees only
// itself, has depth 0 and is never accepted (its edge test fails).
#include "sv_device.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int kTreeBlock = 1024;
constexpr int kTreeWaves = kTreeBlock / kWave;

// Lane v < n: the ancestor set of node v of tree `par` (n <= 64 nodes),
// its validity (parent in [0, v)) and its depth.
__device__ inline void ancestor_sets(const int32_t* par, int n, uint64_t& set, bool& valid, int& depth) {
  const int v = threadIdx.x % kWave;
  const int pv = v < n ? par[v] : -1;
  valid = v == 0 || (v < n && pv >= 0 && pv < v);
  set = v < n ? (1ull << v) : 0ull;
  int jump = (v < n && v > 0 && valid) ? pv : -1;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const uint64_t up = __shfl(set, jump < 0 ? v : jump, kWave);
    const int jj = __shfl(jump, jump < 0 ? v : jump, kWave);
    if (jump >= 0) {
      set |= up;
      jump = jj;
    }
  }
  depth = __popcll(set) - 1;
}

__global__ __launch_bounds__(kTreeBlock) void k_tree_scan(Params p) {
  const long s = blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int N = p.K + 1, np = p.nch1 * kWaves;  // kWaves: the sweep's waves per chunk
  __shared__ int sA[kWave];
  for (int i = w; i < N; i += kTreeWaves) {  // arg-max of every node's row from the sweep's partials
    const float2* pr = p.part + (s * N + i) * np;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < np; j += kWave) argmax_merge(bv, bi, pr[j].x, __float_as_int(pr[j].y));
    wave_argmax(bv, bi);
    if (lane == 0) sA[i] = bi;
  }
  __syncthreads();
  if (w != 0) return;

  uint64_t set;
  bool valid;
  int depth;
  ancestor_sets(p.parents + s * N, N, set, valid, depth);
  const int v = lane;
  const int tok = v < N ? p.x[s * N + v] : 0;
  const int pv = v < N ? p.parents[s * N + v] : -1;
  const bool edge_ok = v == 0 || (v < N && valid && tok == sA[pv]);
  const uint64_t ok = static_cast<uint64_t>(__ballot(edge_ok || v >= N));
  const bool accepted = v < N && (set & ~ok) == 0;
  // deepest accepted node, lowest index among equals (the root always qualifies)
  const int key = wave_max_i32(accepted ? (depth << 8) | (kWave - 1 - v) : -1);
  const int d = kWave - 1 - (key & 0xff), dd = key >> 8;  // uniform
  const uint64_t path = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(set >> 32), d))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(set), d));
  int32_t* ot = p.out_tokens + s * N;
  int32_t* op = p.out_path ? p.out_path + s * N : nullptr;
  if (v < N && ((path >> v) & 1ull)) {  // a node of the path: its token and index at its depth
    if (v != 0) ot[depth - 1] = tok;
    if (op) op[depth] = v;
  }
  if (v < N && v > dd) {
    ot[v] = -1;
    if (op) op[v] = -1;
  }
  if (v == 0) {
    ot[dd] = sA[d];
    p.out_n[s] = dd;
  }
}

// Between two rounds of a tree's rows (token trees read in rounds by depth):
// rows of depth < d0 have been swept where needed, which decides the edge
// test of every node of depth <= d0.  The nodes the next round reads are
// those of depth in [d0, d1) whose ancestors of depth <= d0 (itself included
// at depth d0) are all accepted: a row is needed only once its node is
// accepted, and a round reads its deeper rows ahead of their own tests.
// Rows of shallower nodes that were not swept hold stale arg-maxes; they can
// only decide the tests of children whose parent is not accepted, which
// acceptance masks (the same holds in k_tree_scan after the last round).
__global__ __launch_bounds__(kTreeBlock) void k_tree_round(Params p, int d0, int d1) {
  const long s = blockIdx.x;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int N = p.K + 1, np = p.nch1 * kWaves;
  __shared__ int sA[kWave];
  uint64_t set;
  bool valid;
  int depth;
  ancestor_sets(p.parents + s * N, N, set, valid, depth);  // in every wave: which rows are shallow
  const uint64_t shallow = static_cast<uint64_t>(__ballot(lane < N && depth < d0));
  for (int i = w; i < N; i += kTreeWaves) {
    if (!((shallow >> i) & 1ull)) continue;  // uniform over the wave
    const float2* pr = p.part + (s * N + i) * np;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < np; j += kWave) argmax_merge(bv, bi, pr[j].x, __float_as_int(pr[j].y));
    wave_argmax(bv, bi);
    if (lane == 0) sA[i] = bi;
  }
  __syncthreads();
  if (w != 0) return;
  const int v = lane;
  const int tok = v < N ? p.x[s * N + v] : 0;
  const int pv = v < N ? p.parents[s * N + v] : -1;
  const int pa = (v > 0 && v < N && valid) ? pv : 0;  // a parent in [0, v), or 0 (read and unused)
  const bool tested = v < N && depth <= d0;
  const bool edge_ok = v == 0 || (tested && valid && tok == sA[pa]);
  // nodes deeper than d0 lie in no set of a node of depth <= d0
  const uint64_t ok = static_cast<uint64_t>(__ballot(edge_ok || !tested));
  const uint64_t acc = static_cast<uint64_t>(__ballot(tested && (set & ~ok) == 0));
  const uint64_t upto = static_cast<uint64_t>(__ballot(tested));
  const bool need = v < N && depth >= d0 && depth < d1 && (set & upto & ~acc) == 0;
  if (v < N) p.tneed[s * N + v] = need ? 1 : 0;
}

__global__ __launch_bounds__(kWave) void k_tree_mask(const int32_t* parents, int N, uint8_t* out_mask,
                                                     int32_t* out_depth) {
  const long s = blockIdx.x;
  uint64_t set;
  bool valid;
  int depth;
  ancestor_sets(parents + s * N, N, set, valid, depth);
  const int v = threadIdx.x;
  if (v < N) {
    if (out_depth) out_depth[s * N + v] = depth;
    if (out_mask) {
      uint8_t* row = out_mask + (s * N + v) * N;
      for (int u = 0; u < N; ++u) row[u] = static_cast<uint8_t>((set >> u) & 1ull);
    }
  }
}

}  // namespace

hipError_t launch_tree_scan(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_scan, dim3(static_cast<unsigned>(p.nseq)), dim3(kTreeBlock), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_tree_round(const Params& p, int d0, int d1, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_round, dim3(static_cast<unsigned>(p.nseq)), dim3(kTreeBlock), 0, st, p, d0, d1);
  return hipGetLastError();
}

hipError_t launch_tree_mask(const int32_t* parents, int B, int N, uint8_t* out_mask, int32_t* out_depth,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_tree_mask, dim3(static_cast<unsigned>(B)), dim3(kWave), 0, st, parents, N, out_mask,
                     out_depth);
  return hipGetLastError();
}

}  // namespace sv
