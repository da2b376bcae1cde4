/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) batched lossless token
 * verification library (libspecverify.so).
 *
 * What it computes
 * ----------------
 * Speculative decoding lets a cheap draft propose tokens that the expensive
 * target verifies in parallel ("Technische Zusammenfassung: HiSpec:
 * Hierarchische spekulatives Decodieren fuer LLMs", gist.science 2510.01336,
 * section 1 "Problemstellung"; "Speculative Speculative Decoding",
 * gist.science 2603.03251, Technische Zusammenfassung section 1).  Verification
 * is lossless when it applies the standard speculative-sampling rule, whose
 * proof the HiSpec summary invokes for each of its stages (section 2, bullet
 * "Verlustfreie Garantie"):
 *
 *   - drafted token x at position j is accepted with probability
 *     min(1, p_j(x) / q_j(x)), p = target distribution, q = draft distribution;
 *   - at the first rejection a token is resampled from norm(max(0, p_j - q_j)),
 *     the residual proportional to target minus draft (SSD summary section 3.B);
 *   - when every draft is accepted a bonus token is drawn from the next target
 *     row (SSD summary section 2, item 1).
 *
 * spec_verify_hier adds HiSpec's two-stage verification L_d -> L_i -> L_f
 * (HiSpec summary section 2 "Kernmechanismus", bullets "Verlustfreie Garantie"
 * and "Dynamische Verifizierungsrichtlinie"): the intermediate exit L_i
 * verifies the drafts of the shallow exit L_d and tentatively accepts them, the
 * final exit L_f then verifies the tentative tokens in windows of N_i
 * positions.  kv_blocktable_truncate drops the KV slots of rejected tokens from
 * a paged block table without recomputation or padding (HiSpec summary
 * section 2, bullets "Wiederverwendung von KV-Cache ..." and "Unterstuetzung
 * fuer Batch-Inferenz").
 *
 * spec_verify_tentative_round / _flush spread the same two stages over calls:
 * rounds of intermediate verification append their tentatively accepted tokens
 * to a caller-owned pending state until N_i are pending, then a flush verifies
 * them against the final exit (HiSpec summary, section 2, bullet "Dynamische
 * Verifizierungsrichtlinie").  On request the dense calls also return by-
 * products of the same rows: the entropy of every row, and per tested position
 * the acceptance probability and the likeliest correction tokens
 * (spec_verify_diag).
 *
 * Distributions are softmax(logits / temperature) per row, computed from the
 * logits inside the library; temperature 0 means greedy (one-hot at the
 * lowest-index maximum), which reduces the rule to an argmax prefix match.
 *
 * Uniforms come from Philox4x32-10 (Salmon et al., SC'11): one block per
 * (position j, sequence b, stage s, call offset) with counter
 * (j, b, s, offset) and key (seed low 32 bits, seed high 32 bits).  Word 0
 * gives the accept uniform u = (w0 >> 8) * 2^-24, word 1 the draw uniform
 * v = (w1 >> 8) * 2^-24.  Stage 0 is the single stage and stage 1 of the
 * hierarchy, stage 1 is its second stage.  Same inputs, seed and offset give
 * bit-identical outputs.
 *
 * Conventions
 * -----------
 * Ownership: every data pointer is caller-owned device memory (or host memory
 * where stated).  The library never allocates, frees or keeps device memory;
 * scratch comes from the caller's workspace, sized by
 * spec_verify_workspace_bytes.  Inputs are read-only; outputs are written.
 *
 * Layout: logits are row-major [B, P, V] (P = k for the draft exit, k + 1 for
 * the others), element type float32 or bfloat16, consecutive (b, j) rows
 * row_stride elements apart (row_stride >= V; 0 means V).  Rows that start on
 * a 16-byte boundary are streamed with 128-bit loads, other rows with scalar
 * loads (correct, slower).  Tokens and counts are int32.
 *
 * Asynchrony: calls enqueue work on hip_stream (a hipStream_t; NULL = the null
 * stream) and return without synchronising; outputs are valid once the stream
 * has reached that point.  spec_verify_device_status synchronises.
 *
 * Errors: every call returns an SV_* status.  Arguments are validated on the
 * host before any launch; a failing call launches nothing and writes nothing,
 * and spec_verify_last_error() (thread-local) describes the failure.  No C++
 * exception crosses this interface.  Data problems only visible on the device
 * (a token outside [0, V), a negative or NaN temperature) do not fail the call:
 * the token is rejected (it has probability 0), the sequence is treated as
 * greedy, and a bit is set in the workspace flags (spec_verify_device_status).
 *
 * Thread safety: calls are reentrant; concurrent calls must use distinct
 * workspaces and outputs.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_VERIFY_ABI_VERSION 4

/* Status codes. */
#define SV_OK 0
#define SV_ERR_INVALID_ARG 1 /* NULL pointer, negative size, row_stride < V, window < 1 ... */
#define SV_ERR_UNSUPPORTED 2 /* dtype, k > SV_MAX_DRAFT, V > SV_MAX_VOCAB            */
#define SV_ERR_MISALIGNED 3  /* pointer not aligned to its element size               */
#define SV_ERR_WORKSPACE 4   /* workspace NULL, too small, or not 256-byte aligned     */
#define SV_ERR_DEVICE 5      /* a HIP call failed; its text is in spec_verify_last_error */

/* Element types of logits. */
#define SV_DTYPE_F32 0
#define SV_DTYPE_BF16 1

/* Limits. */
#define SV_MAX_DRAFT 63        /* k + 1 positions fit one 64-lane wavefront */
#define SV_MAX_VOCAB (1 << 20) /* inverse-CDF tile sums stay in LDS          */
#define SV_MAX_HIDDEN (1 << 16) /* hidden size of the LM-head path            */
#define SV_MAX_TOP_M 8          /* residual tokens per position in the export */

/* Device flags (spec_verify_device_status). */
#define SV_FLAG_TOKEN_RANGE 1u /* a drafted token outside [0, V) was rejected        */
#define SV_FLAG_TEMPERATURE 2u /* a negative or NaN temperature was treated as 0    */
#define SV_FLAG_PENDING_FULL 4u /* a round's output did not fit the pending capacity */

typedef struct {
  int32_t batch;      /* B >= 0 sequences (0: nothing to do)                  */
  int32_t num_draft;  /* k in [0, SV_MAX_DRAFT] drafted tokens per sequence    */
  int32_t vocab;      /* V in [1, SV_MAX_VOCAB]                                 */
  int32_t dtype;      /* SV_DTYPE_F32 or SV_DTYPE_BF16 (all exits alike)       */
  int64_t row_stride; /* elements between consecutive rows; 0 => V             */
  uint64_t seed;      /* Philox key: low 32 bits = k0, high 32 bits = k1       */
  uint32_t offset;    /* Philox counter word 3: a call / step index            */
  uint32_t reserved;  /* must be 0                                             */
} spec_verify_desc;

/* Optional per-call diagnostics and by-products.  Every field is a device
 * pointer (or, for the events, a hipEvent_t handle) or NULL; a NULL field is
 * not computed.  Entries that do not apply (untested positions, stages
 * without a draw) are NaN.  Stage index 0 = single stage / hierarchy stage 1,
 * 1 = hierarchy stage 2.
 *
 * By-products (spec_verify_single, spec_verify_hier, spec_verify_hier_rollback;
 * the lazy and LM-head calls return SV_ERR_UNSUPPORTED when one is set):
 *   entropy   the Shannon entropy in nats of every streamed row's distribution
 *             (softmax at the sequence's temperature; 0 for greedy sequences),
 *             rows in the workspace's order: exit 0 [B, k], then exit 1
 *             [B, k+1], then exit 2 [B, k+1].  The entropy of the draft's
 *             distribution is what entropy-driven adaptive draft lengths use
 *             ("Optimierung der Inferenzgeschwindigkeit von Sprachmodellen
 *             durch spekulative Dekodierung", mind-verse.de, paragraphs on
 *             SVIP).  It costs one multiply-add per streamed element.
 *   accept_mass, residual_tokens, residual_mass: the verification-outcome
 *             export of every tested position (q, p) = (draft or L_d, target
 *             or L_i) row j < k for stage 0 and (L_i, L_f) row j <= k for
 *             stage 1: beta = sum_v min(p_v, q_v), the probability that the
 *             rule accepts there, and the top_m largest r_v of the residual
 *             r = max(0, p - q) (ties: lower token first; r_v > 0 only;
 *             padded with token -1, mass 0), r_v being the probability of
 *             rejecting there and emitting v.  These are the likely outcomes
 *             of a verification that a speculation cache prepares for
 *             ("Speculative Speculative Decoding", gist.science 2603.03251,
 *             section 2 items 1-2, section 3.A and 3.B).  It re-reads the
 *             rows of every tested position once more after the statistics.
 *
 * Row statistics (spec_verify_single, spec_verify_hier,
 * spec_verify_hier_rollback; SV_ERR_UNSUPPORTED from the lazy and LM-head
 * calls): row_log2z and row_argmax give every row's merged softmax statistics
 * in the order of the entropy field, so that a caller can form any
 * probability of any row from the logits; written by the verification launch
 * at no extra stream cost.
 */
typedef struct {
  float* uniforms;   /* [B, 2, k+1, 2]: (u, v) of each position                   */
  double* probs;     /* [B, 2, k+1, 2]: (p(t_j), q(t_j)) of each tested position    */
  double* draws;     /* [B, 2, 4]: (R, v*R, C(y-1), C(y)) of each stage's draw      */
  void* stats_begin; /* hipEvent_t (created by the caller) that takes the start
                        time of the row-statistics kernel (the HBM stream; the
                        lazy call: its first statistics kernel), or NULL.  The
                        kernel is launched with hipExtLaunchKernel, so the
                        event adds no marker packet to hip_stream             */
  void* stats_end;   /* hipEvent_t that takes its end time (the lazy call: the
                        end of its last statistics kernel), or NULL          */
  float* entropy;    /* [rows of every exit]: row entropies, nats                */
  float* accept_mass;          /* [B, 2, k+1]: beta of each tested position      */
  int32_t* residual_tokens;    /* [B, 2, k+1, top_m]: largest residual tokens    */
  float* residual_mass;        /* [B, 2, k+1, top_m]: their r_v                  */
  int32_t top_m;               /* 1..SV_MAX_TOP_M when either residual field is set */
  double* row_log2z;           /* [rows of every exit]: the merged normalizer of each
                                  row in the kernel's base-2 units, z = c + log2 S, so
                                  that P_v = 2^(l_v * s - z) with s = log2(e) / tau
                                  rounded to float; NaN for greedy rows             */
  int32_t* row_argmax;         /* [rows of every exit]: greedy rows' argmax (lowest
                                  index on ties); -1 for sampled rows               */
} spec_verify_diag;

/* Version of this header's ABI (SPEC_VERIFY_ABI_VERSION). */
int32_t spec_verify_abi_version(void);

/* Static text for a status code. */
const char* spec_verify_status_string(int32_t status);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* spec_verify_last_error(void);

/* Workspace bytes a call needs: num_exits = 2 (spec_verify_single) or 3
 * (spec_verify_hier).  It holds the flag word, per-sequence counters, draw
 * tile sums, the chunk partials of every row and the by-products' scratch
 * (entropy partials, outcome-export partials).  0 if the descriptor is
 * invalid.  Pure host code. */
size_t spec_verify_workspace_bytes(const spec_verify_desc* desc, int32_t num_exits);

/* Host-side validation of a descriptor, window and workspace size, exactly as
 * the verify calls perform it (no pointers checked).  Pure host code: callable
 * without a GPU.  window is ignored for num_exits = 2. */
int32_t spec_verify_validate(const spec_verify_desc* desc, int32_t num_exits, int32_t window,
                             size_t workspace_bytes);

/* Single-stage verify: draft q vs target p (standard rule, bonus from p_k).
 *   draft_logits   [B, k, V]   device, read-only
 *   target_logits  [B, k+1, V] device, read-only
 *   draft_tokens   [B, k]      device int32
 *   temperature    [B]         device float32, NULL => all 1.0; 0 => greedy
 *   accept_len     [B]         out: accepted drafts a in [0, k]
 *   out_tokens     [B, k+1]    out: the a accepted drafts then the correction
 *                              or bonus token; -1 after the a+1 emitted tokens
 *   num_emitted    [B]         out: a + 1
 *   num_drop       [B]         out or NULL: k - a drafted KV slots to roll back
 *   packed_tokens  [B*(k+1)]   out or NULL: emitted tokens of all sequences
 *                              back to back (no padding)
 *   cu_offsets     [B+1]       out or NULL (required with packed_tokens):
 *                              sequence b's tokens are packed[cu[b] .. cu[b+1])
 *   workspace      device scratch, 256-byte aligned, >= spec_verify_workspace_bytes(desc, 2)
 *   diag           host pointer to a spec_verify_diag, or NULL
 */
int32_t spec_verify_single(const spec_verify_desc* desc, const void* draft_logits,
                           const void* target_logits, const int32_t* draft_tokens,
                           const float* temperature, int32_t* accept_len, int32_t* out_tokens,
                           int32_t* num_emitted, int32_t* num_drop, int32_t* packed_tokens,
                           int32_t* cu_offsets, void* workspace, size_t workspace_bytes,
                           const spec_verify_diag* diag, void* hip_stream);

/* Hierarchical verify L_d -> L_i -> L_f.
 * Stage 1: the standard rule with q = L_d rows 0..k-1, p = L_i rows 0..k; it
 *   yields a1 accepted drafts and one L_i token (correction, or the bonus from
 *   L_i row k), the tentative sequence t of length a1 + 1.
 * Stage 2: the standard rule with t as the draft, q = L_i and p = L_f rows
 *   0..a1, visited in windows of `window` positions; a2 = first rejection
 *   (else a1 + 1).  On a rejection the L_f correction is drawn from
 *   max(0, L_f - L_i) at a2; no L_f bonus is drawn (L_f's distribution after
 *   t is not an input).
 * Emitted: n = min(a1, a2) + 1 tokens; num_drop = k - (n - 1).
 *   ld_logits [B, k, V], li_logits and lf_logits [B, k+1, V]: device, read-only
 *   accept_len_inter [B] out: a1;  accept_len_final [B] out: a2
 *   other arguments as for spec_verify_single; workspace sized with num_exits = 3
 */
int32_t spec_verify_hier(const spec_verify_desc* desc, int32_t window, const void* ld_logits,
                         const void* li_logits, const void* lf_logits,
                         const int32_t* draft_tokens, const float* temperature,
                         int32_t* accept_len_inter, int32_t* accept_len_final,
                         int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                         int32_t* packed_tokens, int32_t* cu_offsets, void* workspace,
                         size_t workspace_bytes, const spec_verify_diag* diag,
                         void* hip_stream);

/* Paged-KV rollback after verification.  Sequence b holds seq_lens[b] KV slots
 * in blocks of block_size slots listed by block_table[b, 0..max_blocks) (-1 =
 * empty).  Its last num_drop[b] slots are dropped: the new length is
 * L' = L - num_drop; logical blocks ceil(L'/bs) .. ceil(L/bs)-1 no longer hold
 * a slot, so their ids are written to freed_blocks[b, ...] in ascending
 * logical order (-1 padded to max_freed), num_freed[b] is their count, and
 * their table entries become -1.  Partly used blocks are kept.
 *   block_table  [B, max_blocks] device int32, in/out
 *   seq_lens     [B]             device int32, in/out
 *   num_drop     [B]             device int32 (e.g. the verify call's num_drop)
 *   freed_blocks [B, max_freed]  device int32, out (may be NULL if max_freed == 0)
 *   num_freed    [B]             device int32, out
 * A sequence whose num_drop lies outside [0, L], whose L exceeds
 * max_blocks * block_size, or that would free more than max_freed blocks is
 * left unchanged and gets num_freed[b] = -1.
 */
int32_t kv_blocktable_truncate(int32_t batch, int32_t max_blocks, int32_t block_size,
                               int32_t* block_table, int32_t* seq_lens,
                               const int32_t* num_drop, int32_t* freed_blocks,
                               int32_t max_freed, int32_t* num_freed, void* hip_stream);

/* spec_verify_hier followed by kv_blocktable_truncate with its num_drop, in the
 * same launches: each sequence's paged-KV state is rolled back as soon as its
 * result is known (HiSpec summary section 2: entries of discarded tokens are
 * removed before the next phase, per-sequence lengths without padding).
 * Arguments as for the two calls; num_drop may be NULL; the rollback's
 * num_drop is the call's own.  A workspace sized for spec_verify_hier. */
int32_t spec_verify_hier_rollback(const spec_verify_desc* desc, int32_t window,
                                  const void* ld_logits, const void* li_logits,
                                  const void* lf_logits, const int32_t* draft_tokens,
                                  const float* temperature, int32_t* accept_len_inter,
                                  int32_t* accept_len_final, int32_t* out_tokens,
                                  int32_t* num_emitted, int32_t* num_drop, int32_t max_blocks,
                                  int32_t block_size, int32_t* block_table, int32_t* seq_lens,
                                  int32_t* freed_blocks, int32_t max_freed, int32_t* num_freed,
                                  void* workspace, size_t workspace_bytes,
                                  const spec_verify_diag* diag, void* hip_stream);

/* spec_verify_hier_rollback without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing: its
 * workspace is a static array of SV_NOALLOC_SCRATCH_BYTES in the library's
 * device code, one per GPU, held until the process ends (the first call on a
 * GPU looks up that GPU's copy; the GPU is hip_stream's, or the current device
 * for the null stream).  Arguments, results and errors as for
 * spec_verify_hier_rollback; a call whose workspace (spec_verify_workspace_bytes
 * with num_exits = 3) exceeds SV_NOALLOC_SCRATCH_BYTES fails with
 * SV_ERR_WORKSPACE and launches nothing.  Every call on one GPU uses the same
 * array, which keeps the last call's contents (the call itself clears what must
 * start at zero): calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined results. */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t spec_verify_hier_rollback_noalloc(const spec_verify_desc* desc, int32_t window,
                                          const void* ld_logits, const void* li_logits,
                                          const void* lf_logits, const int32_t* draft_tokens,
                                          const float* temperature, int32_t* accept_len_inter,
                                          int32_t* accept_len_final, int32_t* out_tokens,
                                          int32_t* num_emitted, int32_t* num_drop,
                                          int32_t max_blocks, int32_t block_size,
                                          int32_t* block_table, int32_t* seq_lens,
                                          int32_t* freed_blocks, int32_t max_freed,
                                          int32_t* num_freed, const spec_verify_diag* diag,
                                          void* hip_stream);

/* Workspace bytes of spec_verify_lmhead_single (0 if desc or hidden is
 * invalid). */
size_t spec_verify_lmhead_workspace_bytes(const spec_verify_desc* desc, int32_t hidden);

/* Single-stage verify whose logits come from a linear LM head shared by the
 * draft and final exits: in an early-exit model each exit turns its hidden
 * state into a token distribution (HiSpec summary, section 2
 * "Kernmechanismus"); here q at drafted position j is the softmax of
 * h_draft[b, j] . W^T and p the softmax of h_target[b, j] . W^T.  The rule is
 * then exactly spec_verify_single's.  The logits are formed on the matrix
 * cores (bf16 products, fp32 sums) and the logit matrix is never stored: the
 * softmax statistics are reduced from each output tile, the logits at the
 * drafted tokens are formed as dot products (fp32 sums), and after the
 * decisions only the rows each sequence draws from (p at the stop position
 * and, for a correction, q there) are recomputed, into the workspace.
 *   desc           dtype must be SV_DTYPE_BF16; vocab = V; row_stride = the
 *                  head's row stride in elements (0 => hidden), a multiple
 *                  of 8
 *   hidden         d, a multiple of 64 in [64, SV_MAX_HIDDEN]
 *   h_draft        [B, k, d]   device bf16, read-only (draft exit at the k
 *                              drafted positions; may be NULL if k == 0)
 *   h_target       [B, k+1, d] device bf16, read-only (final exit)
 *   w_vocab        [V, row_stride] device bf16, read-only: row v is the
 *                  d-vector of vocabulary entry v (a linear layer's weight)
 *   the three must be 16-byte aligned; other arguments as for
 *   spec_verify_single (diag.stats_begin/end bracket the statistics GEMM)
 *   workspace      >= spec_verify_lmhead_workspace_bytes(desc, hidden): about
 *                  B*(2k+1)*ceil(V/384)*16 bytes of tile statistics plus
 *                  2*B*V*4 bytes of recomputed rows
 * Errors as for spec_verify_single; a bf16 requirement or hidden size outside
 * the limits is SV_ERR_UNSUPPORTED.
 */
int32_t spec_verify_lmhead_single(const spec_verify_desc* desc, int32_t hidden,
                                  const void* h_draft, const void* h_target,
                                  const void* w_vocab, const int32_t* draft_tokens,
                                  const float* temperature, int32_t* accept_len,
                                  int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                                  int32_t* packed_tokens, int32_t* cu_offsets, void* workspace,
                                  size_t workspace_bytes, const spec_verify_diag* diag,
                                  void* hip_stream);

/* spec_verify_hier_rollback with a lazy final exit: the L_f rows past each
 * sequence's stage-1 stop are never read.  Stage 2 only tests tentative tokens
 * t_0..t_a1, so it reads L_f rows 0..a1 alone (HiSpec summary, section 2
 * "Kernmechanismus": the intermediate exit discards tokens early, before the
 * final exit verifies them).  Stage 1 is streamed window by window in the
 * same way: the L_d / L_i rows past the first `window` positions are read only
 * for sequences that accepted every draft in that window.  The launches:
 * statistics of the L_d and L_i rows of the first `window` positions; stage 1
 * over them per sequence, which lists the rows still needed (L_f rows 0..a1
 * where a draft was rejected in the window, otherwise the remaining L_d /
 * L_i rows and every L_f row); statistics of the listed rows; then the
 * verification.  Results are bit-identical to spec_verify_hier_rollback's;
 * the bytes read depend on the data.  Same arguments and workspace; the
 * by-product fields of diag are rejected (SV_ERR_UNSUPPORTED). */
int32_t spec_verify_hier_rollback_lazy(const spec_verify_desc* desc, int32_t window,
                                       const void* ld_logits, const void* li_logits,
                                       const void* lf_logits, const int32_t* draft_tokens,
                                       const float* temperature, int32_t* accept_len_inter,
                                       int32_t* accept_len_final, int32_t* out_tokens,
                                       int32_t* num_emitted, int32_t* num_drop,
                                       int32_t max_blocks, int32_t block_size,
                                       int32_t* block_table, int32_t* seq_lens,
                                       int32_t* freed_blocks, int32_t max_freed,
                                       int32_t* num_freed, void* workspace,
                                       size_t workspace_bytes, const spec_verify_diag* diag,
                                       void* hip_stream);

/* Pending tentative tokens of every sequence, carried across calls (caller-
 * owned device memory, zero the counts before the first round).  HiSpec
 * accumulates tentatively accepted tokens, N_i = 4 by default, before the
 * full model verifies them (HiSpec summary, section 2, bullet "Dynamische
 * Verifizierungsrichtlinie"): a round runs the intermediate verification
 * L_d -> L_i and appends its output to this state, a flush verifies the state
 * against the final exit L_f. */
typedef struct {
  int32_t* count;    /* [B] pending tokens per sequence, 0..capacity             */
  int32_t* tokens;   /* [B, capacity] the pending tokens, in order              */
  void* rows;        /* [B, capacity, row_stride] logits of the desc's dtype: the
                        L_i row each pending token was accepted or drawn under */
  int32_t capacity;  /* 1..SV_MAX_DRAFT                                          */
} spec_verify_pending;

/* Workspace bytes of spec_verify_tentative_round and _flush for this desc
 * (num_draft = drafts per round) and capacity; 0 if either is invalid. */
size_t spec_verify_tentative_workspace_bytes(const spec_verify_desc* desc, int32_t capacity);

/* One intermediate verification round: stage 1 of the hierarchy (the standard
 * rule, q = L_d, p = L_i, Philox stage 0) for every sequence, then, for every
 * active sequence, its output t = (x_0..x_{a1-1}, y) is appended to the
 * pending tokens and the L_i rows 0..a1 to the pending rows.
 *   desc         B, k = drafts of this round, V, dtype, row_stride (also the
 *                pending rows' stride), seed, offset (use a fresh offset per
 *                call: the Philox counter is (j, b, stage, offset))
 *   ld_logits    [B, k, V], li_logits [B, k+1, V], draft_tokens [B, k],
 *   temperature  as for spec_verify_hier
 *   active       [B] int32 device, 0 = leave this sequence's state alone; NULL
 *                = every sequence
 *   pending      the state (appended in place)
 *   accept_len   [B] out: a1 of every sequence (active or not)
 *   num_drop     [B] out or NULL: k - a1, the drafts discarded by this round
 *                (their KV entries in the layers up to L_i are stale)
 * A sequence whose output does not fit its remaining capacity gets what fits
 * and sets SV_FLAG_PENDING_FULL.  Errors as for spec_verify_hier; capacity
 * outside [1, SV_MAX_DRAFT] is SV_ERR_UNSUPPORTED. */
int32_t spec_verify_tentative_round(const spec_verify_desc* desc, const void* ld_logits,
                                    const void* li_logits, const int32_t* draft_tokens,
                                    const float* temperature, const int32_t* active,
                                    const spec_verify_pending* pending, int32_t* accept_len,
                                    int32_t* num_drop, void* workspace, size_t workspace_bytes,
                                    void* hip_stream);

/* Full verification of the pending tokens of every sequence holding at least
 * max(1, min_pending) of them (the others are left alone): stage 2 of the
 * hierarchy across calls -- the standard rule over t_0..t_{c-1} with q = the
 * pending L_i rows and p = the final exit's rows, Philox stage 1 -- gives a2 =
 * the first rejection (else c); on a rejection the correction z is drawn from
 * norm(max(0, p - q)) at a2 and t_0..t_{a2-1}, z are emitted, otherwise all c
 * pending tokens (no bonus, as in spec_verify_hier).  The flushed sequences'
 * counts become 0.  Only the rows of pending positions are read.
 *   desc         as for the rounds (num_draft is not used here)
 *   lf_logits    [B, capacity+1, V] device: row j is the final exit's row at
 *                pending position j (rows past the count are not read)
 *   min_pending  the window N_i (>= 0)
 *   accept_len   [B] out: a2, or -1 for a sequence not flushed
 *   out_tokens   [B, capacity+1] out: emitted tokens, -1 padded
 *   num_emitted  [B] out: 0 for a sequence not flushed
 *   num_drop     [B] out or NULL: pending tokens discarded (c - a2 on a
 *                rejection, else 0): their KV entries in every layer are stale
 * A round followed by a flush with the same offset gives exactly the results
 * of spec_verify_hier. */
int32_t spec_verify_tentative_flush(const spec_verify_desc* desc, const void* lf_logits,
                                    const float* temperature, int32_t min_pending,
                                    const spec_verify_pending* pending, int32_t* accept_len,
                                    int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* Synchronises hip_stream, then copies the device flags (SV_FLAG_*) of the
 * last verify call that used `workspace` into *flags_out (host). */
int32_t spec_verify_device_status(const void* workspace, uint32_t* flags_out, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
