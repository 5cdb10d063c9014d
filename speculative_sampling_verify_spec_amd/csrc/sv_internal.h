// Internal definitions shared by the libspecverify host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;   // threads per workgroup in every kernel
constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxDrawChunks = 256;   // fp64 draw chunks per row: one wave combines them, 4 per lane
constexpr int kXBlock = 128;          // threads that compute one fp64 draw chunk's sums
constexpr int kSoloMaxChunks = 2;     // rows of at most this many fp64 draw chunks: one fp64 launch (k_exact_solo)
constexpr int kEagerMaxRounds = 4;    // k_verify's chunk-sum workgroups: at most this many chunks per group of 128 threads
// Rows of at most kShortMaxV tokens (two fp64 draw chunks of 1024) take one
// launch for the whole step in sampling mode (k_short), at any batch size
// unless spec_short_max_seqs limits it.  Measured (us per call, one launch
// against the general path): K = 4, V = 1000 fp32: B = 1 6.1 / 11.4,
// B = 256 7.5 / 22.7, B = 4096 60.2 / 174.6, B = 16384 227 / 508; V = 2000
// fp32, B = 8192: 251 / 298; K = 5, V = 2048 bf16, B = 8192: 234 / 402.
constexpr int kShortMaxV = kSoloMaxChunks * 1024;

// Elements one lane of a row sweep holds: 16-byte units on the vector path,
// sixteen single elements on the scalar path.  The vector path has two
// shapes.  The large one (14 units for the log-sum-exp sweep, 16 for the
// arg-max sweep: the fastest of 6 to 18 on large launches, where fewer,
// larger workgroups beat higher occupancy) serves launches of at least
// kSweepLargeMinGroups workgroups; smaller launches, which the large shape
// would fill only a few times over, take 6 units.
template <int DT, bool VEC, bool ARGMAX, bool LARGE>
constexpr int kSweepElems() {
  return VEC ? (LARGE ? (ARGMAX ? 16 : 14) : 6) * (DT == 1 ? 8 : 4) : 16;
}
constexpr long kSweepLargeMinGroups = 6144;

// Early exit.  Acceptance stops at a sequence's first rejection n, and only
// the rows of levels 0..n are needed (level k < K_b: target row k and draft
// row k; level K_b: the bonus target row).  On inputs of at least
// kRoundsMinBytes the sweep therefore runs in rounds over levels [lv0, lv1):
// [0, 1), [1, 3), [3, K + 1).  After each round but the last,
// k_round_accept tests the levels it swept (at most kMaxRoundLevels) and
// writes each sequence's last level still to sweep; the next round's
// workgroups of a sequence that has rejected leave at once.  Smaller inputs
// take one sweep of every row: there the extra launches cost more than the
// rows they save.
constexpr int kMaxRounds = 3;
constexpr int kMaxRoundLevels = 2;  // levels of a round that another round follows
__host__ __device__ constexpr int round_begin(int r) { return r == 0 ? 0 : (r == 1 ? 1 : 3); }
// Token trees read their rows in the same rounds, by depth: the root, then
// depths 1-2, then the rest (a node's row is needed only once the node is
// accepted, and acceptance descends from the root).
constexpr double kRoundsMinBytes = 256.0 * (1 << 20);

// The fast draw (k_verify) streams a sequence's decisive row(s) in wave
// iterations of 64 lanes x kDrawLaneUnits units (16-byte vectors, or single
// elements on the scalar path), grouped into at most kMaxSegs segments of
// whole iterations.  Host and kernel share this geometry: the host sizes the
// split workspace and picks the split from it.
constexpr int kVerifyBlock = 1024;            // threads per k_verify workgroup
constexpr int kVerifyWaves = kVerifyBlock / kWave;
constexpr int kVerifyWavesSmall = 8;  // k_verify's waves per workgroup for batches of more sequences than CUs
constexpr int kMaxSegs = 1024;                // segments per row, at most
__host__ __device__ constexpr int draw_lane_units(bool vec) { return vec ? 2 : 8; }

struct SegGeom {
  long units;  // units of the row (vectors on the vector path, else elements)
  int iters;   // wave iterations per segment
  int nseg;    // segments
};

__host__ __device__ inline SegGeom seg_geom(int V, int per_vec, bool vec) {
  SegGeom g;
  g.units = vec ? V / per_vec : V;  // vector path: V is a multiple of per_vec
  const long iter_units = static_cast<long>(kWave) * draw_lane_units(vec);
  const long total = g.units > 0 ? (g.units + iter_units - 1) / iter_units : 1;  // at least one iteration
  g.iters = static_cast<int>((total + kMaxSegs - 1) / kMaxSegs);
  g.nseg = static_cast<int>((total + g.iters - 1) / g.iters);
  return g;
}

// When the batch leaves CUs idle, each sequence's fast draw is split over up
// to kMaxSplit workgroups (one CU each), which stream interleaved blocks of
// kVerifyWaves segments; the last of them to finish draws.  Only batches of
// at most kSplitMaxSeqs sequences are split.
constexpr int kMaxSplit = 16;
constexpr int kSplitMaxSeqs = 128;
// Rows of fewer blocks are not split: the exchange through the workspace
// costs about what streaming two blocks in one workgroup instead of two
// saves (measured at V = 32000).
constexpr int kSplitMinBlocks = 3;

// Per-sequence record of the acceptance scan; the fast draw puts it, with the
// sequence's index, in the fp64 draw's queue, so that one 32-byte load gives
// that draw everything it needs.
struct SeqRec {
  int32_t n;       // accepted draft tokens
  int32_t kb;      // the sequence's draft count (n == kb: bonus draw)
  int32_t flags;   // SPECV_FLAG_* set so far
  int32_t seq;     // the sequence (in a queue entry)
  double lzp, lzq; // log2 sum_v 2^(x_v c) of the decisive target / draft row (fp32-accurate)
};
static_assert(sizeof(SeqRec) == 32, "SeqRec layout");

// Constants of the fp64 exp: the Cody-Waite split of ln 2 and the Taylor
// coefficients 1/n!.  They travel as kernel arguments, so the kernels read
// them from scalar registers instead of rebuilding 64-bit literals per use.
struct ExpConsts {
  double log2e;
  double ln2_hi;        // ln 2 with its low 21 mantissa bits zero: k * ln2_hi is exact for |k| < 2^21
  double ln2_lo;        // ln 2 - ln2_hi, rounded
  double inv_fact[11];  // 1/12!, 1/11!, ..., 1/2!
};

inline ExpConsts make_exp_consts() {
  ExpConsts e{};
  e.log2e = 1.4426950408889634;
  e.ln2_hi = 0x1.62e42fee00000p-1;
  e.ln2_lo = 0x1.a39ef35793c76p-33;
  double f = 1.0;
  for (int n = 2; n <= 12; ++n) {
    f *= n;
    e.inv_fact[12 - n] = 1.0 / f;  // exact factorials; one rounding each
  }
  return e;
}

// Everything a kernel needs, passed by value.
struct Params {
  const void* lp;            // [B][K+1][V] target logits
  const void* lq;            // [B][K][V] draft logits (sampling only)
  const int32_t* x;          // [B][K] draft tokens
  const float* ua;           // [B][K]
  const float* ur;           // [B]
  const int32_t* kb;         // [B] per-sequence draft counts, or null (all K)
  const int32_t* parents;    // token trees: [B][N] parent of each node (x holds the node tokens, K = N - 1)
  int32_t* out_path;         // token trees: [B][N] node indices of the accepted path, or null
  unsigned long long* stats; // [2K] per-position counters to add to, or null
  int B, K, V;
  int vec;                   // 1: 16-byte vector loads are legal for every row
  float c;                   // log2(e) / T rounded to fp32
  double inv_t;              // 1 / T in fp64 (exact draw)
  ExpConsts ec;              // fp64 exp constants (exact draw)
  int32_t* out_tokens;       // [B][K+1]
  int32_t* out_n;            // [B]
  float* out_logz;           // [B][2K+1] or null
  int32_t* out_flags;        // [B] or null
  // workspace
  float2* part;              // [rows][nch1][kWaves] (R, s) sweep partials, or (max, index bits) in greedy mode
  double* xsum;              // [B][R3][5] exact draw chunk sums (by queue slot; by sequence if xeager)
  uint32_t* qcount;          // [1] sequences queued for the exact draw
  SeqRec* queue;             // [B] their records (from the first sequence of the launch on; by sequence if xeager)
  int nch1, ch1;             // sweep chunks per row, elements per sweep chunk (at most)
  int cq, cr;                // sweep chunk c spans c*cq + min(c, cr) .. + cq + (c < cr) units
  int sweep_large;           // the sweep runs its large shape (see kSweepElems)
  int grid3;                 // the sweep's grid: 0 one-dimensional over every row; 1 (chunks, round
                             // slots, sequences) over the rows of levels lv0..lv1-1 each sequence uses
  int lv0, lv1;              // grid3: the levels the launch covers (target rows lv0..lv1-1, and the
                             // draft rows among them); lv0 > 0: skip the rows past kbs[s]
  int32_t* kbs;              // [B] rounds: the last level still to sweep per sequence (k_round_accept)
  uint8_t* tneed;            // token trees in rounds: [B][N] 1 where the round sweeps the node's row (k_tree_round)
  int vwaves;                // k_verify's waves per workgroup when unsplit: kVerifyWaves or kVerifyWavesSmall
  int vpre;                  // k_verify, rounds: the last round's first level (sequences with kbs below it
                             // were decided earlier); 0 after a one-sweep call
  int R3, ch3;               // fp64 draw chunks per row, elements per chunk
  int xeager;                // > 0: k_verify launches xeager more workgroups per sequence that compute the
                             // fp64 draw's chunk sums of every sequence (xper chunks each) into xsum by
                             // sequence, and the fast draw leaves every sequence's record in queue[s]
                             // (seq < 0: drawn); 0: sums of queued sequences only, by queue slot
  int xper;                  // xeager: chunks per workgroup
  int seq0, nseq;            // the sequences a launch covers
  int split;                 // workgroups per sequence in k_verify (1: no split)
  int nseg;                  // segments of the fast draw's row stream (seg_geom)
  float* segm;               // split: [B][nseg] segment masses of the fast draw (NaN until published)
  double* spq;               // split: [B][kMaxSplit][2] sum P', sum Q' of each workgroup (NaN until published)
  uint32_t* vcount;          // split: [B] workgroups of the sequence done streaming
};

// Workspace layout (byte offsets), shared by spec_verify_workspace_size and the launcher.
struct Layout {
  size_t part, kbs, tneed, xsum, queue, qcount, segm, spq, vcount, total;
  int nch1, ch1, cq, cr, R3, ch3;
  int sweep_large;  // the sweep's large shape (see kSweepElems)
};

Layout make_layout(int B, int K, int V, int dtype, bool vec, bool greedy, bool tree);

// Launchers (one per kernel), defined next to their kernels.
hipError_t launch_sweep_lse(const Params& p, int dtype, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_sweep_argmax(const Params& p, int dtype, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_verify(const Params& p, int dtype, hipStream_t s);
hipError_t launch_exact(const Params& p, int dtype, hipStream_t s);
hipError_t launch_short(const Params& p, int dtype, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_greedy_scan(const Params& p, hipStream_t s);
hipError_t launch_round_accept(const Params& p, int dtype, bool greedy, hipStream_t s);
hipError_t launch_position_stats(const Params& p, hipStream_t s);
hipError_t launch_validate(const Params& p, int dtype, bool greedy, unsigned long long* dbg, hipStream_t s);
// whether validation is on (read from SPECV_DEBUG at the first use); with
// set_to, sets it and returns the previous value
bool debug_enabled_flag(int* set_to);
unsigned long long* debug_counters_ptr();  // the current device's counters, or null
hipError_t launch_tree_scan(const Params& p, hipStream_t s);
hipError_t launch_tree_round(const Params& p, int d0, int d1, hipStream_t s);
hipError_t launch_sweep_argmax_tree(const Params& p, int dtype, hipStream_t s);
hipError_t launch_ngram(const int32_t* hist, const int32_t* lengths, int B, int Lmax, int n_min, int n_max,
                        int min_hits, int K, int32_t* out_draft, int32_t* out_count, hipStream_t s);
hipError_t launch_ngram_map(void* tables, int capacity, const int32_t* hist, const int32_t* len_old,
                            const int32_t* len_new, int B, int Lmax, int n_min, int n_max, int min_hits, int K,
                            int32_t* out_draft, int32_t* out_count, int32_t* out_status, hipStream_t s);
hipError_t launch_tree_mask(const int32_t* parents, int B, int N, uint8_t* out_mask, int32_t* out_depth,
                            hipStream_t s);

}  // namespace sv
