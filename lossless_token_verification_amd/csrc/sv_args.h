// Argument blocks, workspace layout and device helpers of the verification,
// KV-rollback and LM-head kernels (everything but the row-statistics stream):
// device-scope publication, paged-KV rollback of one sequence, Philox4x32-10.
#pragma once

#include "sv_common.h"

namespace sv {

constexpr int kMaxPositions = 64;      // k + 1 <= 64
// Draw tiles of the largest vocabulary (fp32 has the most tiles).
constexpr int kMaxTiles = kMaxVocab / (kWave * 4);

constexpr uint32_t kFlagTokenRange = 1u;
constexpr uint32_t kFlagTemperature = 2u;


// Workspace: [flags (256 B)] [two slice counters: 8 B per sequence]
// [tile sums: 2 * B * nt floats] [partials: rows * nc], each area padded to
// 256 B.
constexpr size_t kFlagsBytes = 256;
// Draw tiles each workgroup of a verification sums, at most: two rows per tile
// for a single draw, three for the hierarchy's joint draw of y and z (the
// plan takes fewer when that leaves the launch short of workgroups).
constexpr int kTilesPerSlice = 128;
constexpr int kTilesPerSliceJoint = 64;
constexpr int kMinTilesPerSlice = 8;
constexpr int64_t kVerifyWorkgroups = 1024;

// The verification launches (stage 1 with its draw, stage-2 draw).
struct VerifyArgs {
  int32_t hier;            // 0: single stage (q = exit 0, p = exit 1); 1: L_d, L_i, L_f
  int32_t B, k, V, dtype, nc, window;
  int32_t nt, ns, tps;     // draw tiles per row, slices per sequence, tiles per slice
  int64_t ld;
  const void* exit_ptr[3];
  int32_t exit_row0[3];
  const Partial* partials;
  float* tsum[2];          // [B, nt] tile sums of each stage's draw
  int32_t* cnt[2];         // [B] slices done: cnt[0] joint or single draw, cnt[1] the
                           // hierarchy's stage-2 draw before a1
  const int32_t* tokens;
  const float* temperature;
  uint32_t key0, key1, offset;
  int32_t* accept_len;        // a (single) or a1 (hier)
  int32_t* accept_len_final;  // a2 (hier) or NULL
  int32_t* out_tokens;
  int32_t* num_emitted;
  int32_t* num_drop;
  float* diag_uniforms;
  double* diag_probs;
  double* row_log2z;         // [rows]: merged z = c + log2 S per row (NaN: greedy); NULL: none
  int32_t* row_argmax;       // [rows]: greedy argmax (-1: sampled); NULL: none
  double* diag_draws;
  uint32_t* flags;
  // LM-head path: logits at the drafted tokens come from `gath` (one per row,
  // NULL: read from the logit rows), the draws read the recomputed stopped
  // rows of `draw_rows` ([2B, draw_ld] fp32: p row 2b, q row 2b + 1), and a
  // first pass with `decide_only` writes each sequence's stopped rows to
  // `stop_rows` (greedy sequences are finished there).
  const float* gath;
  const float* draw_rows;
  int64_t draw_ld;
  int32_t decide_only;
  int32_t* stop_rows;
  // Lazy final exit: a first pass with `stage1_only` runs stage 1 over the
  // positions below stage1_window (the only L_d / L_i rows streamed so far).
  // Where it fixes a1 (a rejection there, or a window that covers every
  // draft) it writes lazy_a1 = a1 and lists the L_f rows 0..a1; otherwise it
  // writes lazy_a1 = -1 and lists the remaining L_d / L_i rows and every L_f
  // row.  Row ids are global, appended to row_list_out at an atomically
  // advanced *row_count_out.  The verification then merges L_f rows 0..a1
  // where lazy_a1 >= 0, every row otherwise.  NULL lazy_a1: every row.
  int32_t stage1_only;
  int32_t* lazy_a1;
  int32_t* row_list_out;
  int32_t* row_count_out;
  int32_t stage1_window;
  // Flush of pending tentative tokens: a single-stage chain per sequence over
  // its n = flush_lim[b] + 1 pending tokens (0: the sequence is not flushed),
  // q = exit 0 (the pending L_i rows), p = exit 1 (the final exit), Philox
  // stage 1, no bonus.  NULL: an ordinary verification.
  const int32_t* flush_lim;
  // optional paged-KV rollback of every sequence once its result is known
  int32_t* kv_table;       // [B, kv_max_blocks] or NULL
  int32_t* kv_lens;        // [B]
  int32_t* kv_freed;       // [B, kv_max_freed] or NULL
  int32_t* kv_num_freed;   // [B]
  int32_t kv_max_blocks, kv_block_size, kv_max_freed;
};

struct PackArgs {
  int32_t B, k;
  const int32_t* out_tokens;
  const int32_t* num_emitted;
  int32_t* packed;
  int32_t* cu_offsets;
};

struct KvArgs {
  int32_t B, max_blocks, block_size, max_freed;
  int32_t* table;
  int32_t* lens;
  const int32_t* drop;
  int32_t* freed;
  int32_t* num_freed;
};

// LM-head GEMM: logits[r, v] = sum_i A[r, i] * W[v, i] for bf16 A rows
// (hidden states) and a bf16 head W [V, ldw], fp32 accumulation on MFMA.
// Row r of A is draft row r (r < m_draft: a_draft + r * d) or target row
// r - m_draft (a_target); with `a_rows`, GEMM row r takes A row a_rows[r]
// (-1: the row is skipped).  Epilogues:
//  - stats: partial softmax statistics of every (row, N tile), in the Partial
//    format of the row-statistics kernel;
//  - rows: the fp32 logits themselves, out[r * ldo + v].
// Draft row b*k + j and target row b*(k+1) + j, j < k, hold drafted token
// tokens[b*k + j]; the merge forms the logit there into gath[r].
struct GemmArgs {
  const uint16_t* a_draft;
  const uint16_t* a_target;
  const int32_t* a_rows;
  const uint16_t* w;
  int64_t ldw;
  int32_t M, m_draft, V, d, B, k;
  int32_t n_tiles;          // N tiles of the grid (vocabulary tiles)
  const int32_t* tokens;
  const float* temperature;
  Partial* partials;        // [M, n_tiles]
  float* gath;              // [M]
  float* out;               // [M, ldo]
  int64_t ldo;
};
// Merges the n partials of each of `rows` rows into one (nc = 1 format) and
// writes each row's drafted-token logit (GemmArgs.gath).  The first
// workgroups also zero `clear_words` and the flag word (the counters of the
// verification launches that follow).
struct MergeArgs {
  const Partial* in;
  Partial* out;
  int32_t rows, n;
  int32_t* clear_words;
  int32_t n_clear;
  uint32_t* flags;
};
constexpr int kGemmMT = 192;   // rows per GEMM workgroup tile (statistics GEMM)
constexpr int kGemmRowsMT = 256;  // rows per tile of the recompute GEMM (2B rows)
constexpr int kGemmNT = 384;   // vocabulary entries per GEMM workgroup tile (statistics GEMM)
constexpr int kGemmRowsNT = 256;  // and per tile of the recompute GEMM
constexpr int kGemmWM = 2;     // wavefronts of a GEMM workgroup along rows
constexpr int kGemmWN = 4;     // and along the vocabulary
constexpr int kGemmKT = 64;    // hidden elements per pipeline step
constexpr int kHiddenMultiple = 64;   // the LM-head call's hidden size is a multiple of this
static_assert(kHiddenMultiple % kGemmKT == 0, "whole pipeline steps");

hipError_t launch_lmhead_stats(const GemmArgs& a, hipStream_t st, hipEvent_t ev_start = nullptr,
                               hipEvent_t ev_stop = nullptr);
hipError_t launch_lmhead_rows(const GemmArgs& a, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, const GemmArgs& g, hipStream_t st);

// By-products of a verification call: the entropy of every streamed row
// (from the chunk partials and their T), and per tested position the
// acceptance mass beta = sum min(p, q) with the largest entries of the
// residual max(0, p - q).  The outcome export is one pass over the rows of
// every position (each workgroup one 64 KiB chunk of q, p and, for the
// hierarchy, L_f) writing a PairPart per (sequence, stage, position, chunk),
// then one wavefront per (sequence, stage, position) merging them.
constexpr int kTopM = 8;       // residual tokens one position can export
struct PairPart {
  double beta;                 // sum over the chunk of min(p, q)
  float mass[kTopM];           // the chunk's largest residuals, largest first
  int32_t tok[kTopM];          // their tokens (-1: none)
};
static_assert(sizeof(PairPart) == 72, "PairPart layout");
struct ByArgs {
  int32_t B, k, V, dtype, nc, hier;
  int64_t ld;
  const void* exit_ptr[3];
  int32_t exit_pos[3], exit_row0[3];
  const Partial* partials;
  const double* tpart;         // entropy partials or NULL
  const float* temperature;
  int32_t rows;                // rows of every exit
  float* entropy;              // [rows] or NULL
  PairPart* pair;              // [B, 2, k+1, nc] workspace
  float* beta;                 // [B, 2, k+1] or NULL
  int32_t* top_tok;            // [B, 2, k+1, top_m] or NULL
  float* top_mass;             // [B, 2, k+1, top_m] or NULL
  int32_t top_m;
};
// Pending tentative tokens across calls: a round appends each active
// sequence's stage-1 output (a1 accepted drafts and y) and the L_i rows it was
// tested or drawn under; a flush verifies them against the final exit.
struct PendArgs {
  int32_t B, k, V, dtype, cap, nch;   // nch: 64 KiB chunks per row
  int64_t ld;
  const void* li;            // [B, k+1, ld] L_i logits of the round
  const int32_t* active;     // [B] or NULL (every sequence)
  const int32_t* a1;         // [B] stage-1 accept counts
  const int32_t* t_out;      // [B, k+1] stage-1 output tokens
  int32_t* count;            // [B] pending tokens
  int32_t* tokens;           // [B, cap]
  void* rows;                // [B, cap, ld]
  int32_t min_pending;       // flush threshold
  int32_t* lim;              // [B] flush: last pending position, -1 = not flushed
  int32_t row0_q, row0_p;    // flush: first global row of the pending rows and of L_f
  int32_t* row_list;         // flush: the rows to stream (pending rows, then L_f rows,
  int32_t* row_count;        //   of each flushed sequence in order) and their number
  int32_t* arrive;           // [B] round: workgroups of the append done so far (zeroed
                             //   by the round's statistics launch)
  uint32_t* flags;
};
constexpr uint32_t kFlagPendingFull = 4u;
hipError_t launch_pending_append(const PendArgs& a, hipStream_t st);
hipError_t launch_flush_prep(const PendArgs& a, hipStream_t st);

hipError_t launch_entropy(const ByArgs& a, hipStream_t st);
hipError_t launch_outcome(const ByArgs& a, hipStream_t st);

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st);
hipError_t launch_pack(const PackArgs& a, hipStream_t st);
hipError_t launch_kv_truncate(const KvArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// device helpers

// Tile sums pass between the workgroups of one launch without cache-wide
// fences: writers store them with device-scope atomic stores (written through
// to the coherent level) and wait for the stores to complete before counting
// themselves done; the last workgroup reads them with device-scope atomic
// loads.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this wavefront issued has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Rolls back the paged-KV state of one sequence: drops its last `drop` slots,
// moves the ids of blocks left without a slot to freed[] in ascending logical
// order (-1 padded) and clears their table entries.  A sequence whose drop is
// outside [0, L], whose L exceeds the table, or that would free more than
// max_freed blocks is left unchanged and gets num_freed = -1.  One thread.
__device__ __forceinline__ void kv_rollback_one(int32_t* row, int32_t* len, int64_t drop,
                                                int32_t* freed, int32_t* num_freed,
                                                int max_blocks, int block_size, int max_freed) {
  const int64_t L = *len;
  const int64_t bs = block_size;
  const int64_t used = (L + bs - 1) / bs;
  const int64_t keep = (L - drop + bs - 1) / bs;
  const bool ok = drop >= 0 && drop <= L && used <= max_blocks && used - keep <= max_freed;
  if (!ok) {
    for (int i = 0; i < max_freed; ++i) freed[i] = -1;
    *num_freed = -1;
    return;
  }
  const int n = static_cast<int>(used - keep);
  for (int i = 0; i < n; ++i) {
    freed[i] = row[keep + i];
    row[keep + i] = -1;
  }
  for (int i = n; i < max_freed; ++i) freed[i] = -1;
  *num_freed = n;
  *len = static_cast<int32_t>(L - drop);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiply S-box; the key is bumped by the Weyl constants before every
// round after the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t m0 = static_cast<uint64_t>(0xD2511F53u) * x.x;
    const uint64_t m1 = static_cast<uint64_t>(0xCD9E8D57u) * x.z;
    const uint32_t hi0 = static_cast<uint32_t>(m0 >> 32), lo0 = static_cast<uint32_t>(m0);
    const uint32_t hi1 = static_cast<uint32_t>(m1 >> 32), lo1 = static_cast<uint32_t>(m1);
    x = make_uint4(hi1 ^ x.y ^ k0, lo1, hi0 ^ x.w ^ k1, lo0);
  }
  return x;
}

// 24-bit uniform in [0, 1 - 2^-24] from a 32-bit word (exact in float).
__device__ __forceinline__ float uniform24(uint32_t w) {
  return static_cast<float>(w >> 8) * 5.9604644775390625e-08f;
}

}  // namespace sv
