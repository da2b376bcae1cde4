// C ABI of libspecverify.so: host-side validation, workspace layout and the
// launch sequence of each call.  See include/spec_verify.h for the contract.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "spec_verify.h"
#include "sv_args.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Plan {
  int num_exits = 0;
  int64_t rows_total = 0;
  int nc = 0;
  int64_t ld = 0;
  size_t ws_bytes = 0;
  size_t seq_bytes = 0;   // per-sequence slice counters and stage-1 counts
  size_t tile_bytes = 0;  // draw tile sums of both stages
  size_t part_bytes = 0;  // chunk partials
  size_t tpart_bytes = 0; // entropy partials (one double per chunk partial)
  size_t pair_bytes = 0;  // outcome-export partials, B * 2 * (k+1) * nc
  int nt = 0;             // draw tiles per row
  int ns = 0;             // slices (workgroups) per sequence
  int tps = 0;            // draw tiles per slice
  int32_t exit_pos[3] = {0, 0, 0};
  int32_t exit_row0[3] = {0, 0, 0};
};

// Validates the descriptor and derives the launch plan.  Pure host code.
int32_t make_plan(const spec_verify_desc* d, int32_t num_exits, Plan* p) {
  if (!d) return fail(SV_ERR_INVALID_ARG, "desc is NULL");
  if (num_exits != 2 && num_exits != 3) return fail(SV_ERR_INVALID_ARG, "num_exits must be 2 or 3");
  if (d->reserved != 0) return fail(SV_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->batch < 0) return fail(SV_ERR_INVALID_ARG, "batch < 0");
  if (d->num_draft < 0) return fail(SV_ERR_INVALID_ARG, "num_draft < 0");
  if (d->num_draft > SV_MAX_DRAFT)
    return fail(SV_ERR_UNSUPPORTED, "num_draft > " + std::to_string(SV_MAX_DRAFT));
  if (d->vocab < 1) return fail(SV_ERR_INVALID_ARG, "vocab < 1");
  if (d->vocab > SV_MAX_VOCAB)
    return fail(SV_ERR_UNSUPPORTED, "vocab > " + std::to_string(SV_MAX_VOCAB));
  if (d->dtype != SV_DTYPE_F32 && d->dtype != SV_DTYPE_BF16)
    return fail(SV_ERR_UNSUPPORTED, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  const int64_t ld = d->row_stride == 0 ? d->vocab : d->row_stride;
  if (ld < d->vocab) return fail(SV_ERR_INVALID_ARG, "row_stride < vocab");
  if (ld > (int64_t(1) << 40)) return fail(SV_ERR_INVALID_ARG, "row_stride too large");
  const int k = d->num_draft;
  p->num_exits = num_exits;
  p->exit_pos[0] = k;
  p->exit_pos[1] = k + 1;
  p->exit_pos[2] = num_exits == 3 ? k + 1 : 0;
  const int64_t B = d->batch;
  p->exit_row0[0] = 0;
  p->rows_total = B * k;
  for (int e = 1; e < num_exits; ++e) {
    if (p->rows_total > INT32_MAX) break;
    p->exit_row0[e] = static_cast<int32_t>(p->rows_total);
    p->rows_total += B * (k + 1);
  }
  const int ce = sv::chunk_elems(d->dtype);
  p->nc = (d->vocab + ce - 1) / ce;
  if (p->rows_total > INT32_MAX || p->rows_total * p->nc > INT32_MAX)
    return fail(SV_ERR_UNSUPPORTED, "batch too large for one call");
  p->ld = ld;
  const int te = sv::tile_elems(d->dtype);
  p->nt = (d->vocab + te - 1) / te;
  // Draw tiles per slice: about kVerifyWorkgroups workgroups in the
  // verification launch (small batches or short rows get more slices per
  // sequence, so the draws still spread over the chip), between kMinTilesPerSlice
  // and the most one slice's LDS staging takes (fewer for the hierarchy's
  // three-row joint draw).
  {
    const int64_t cap = num_exits == 3 ? sv::kTilesPerSliceJoint : sv::kTilesPerSlice;
    const int64_t want = (static_cast<int64_t>(p->nt) * B + sv::kVerifyWorkgroups - 1) /
                         sv::kVerifyWorkgroups;
    p->tps = static_cast<int>(std::min(cap, std::max<int64_t>(sv::kMinTilesPerSlice, want)));
  }
  p->ns = (p->nt + p->tps - 1) / p->tps;
  if (B * p->ns > INT32_MAX) return fail(SV_ERR_UNSUPPORTED, "batch too large for one call");
  // two slice counters and the lazy call's stage-1 counts per sequence, then
  // its row list: a count and up to B * (3k + 2) row ids (per sequence at most
  // the L_d / L_i rows past the stage-1 window and every L_f row, or L_f rows
  // 0..a1)
  p->seq_bytes = B > 0 ? ((static_cast<size_t>(B) * (3 * k + 5) + 1) * sizeof(int32_t) + 255) /
                             256 * 256
                       : 0;
  p->tile_bytes = (static_cast<size_t>(B) * 2 * p->nt * sizeof(float) + 255) / 256 * 256;
  const size_t n_part = static_cast<size_t>(p->rows_total) * p->nc;
  p->part_bytes = (n_part * sizeof(sv::Partial) + 255) / 256 * 256;
  p->tpart_bytes = (n_part * sizeof(double) + 255) / 256 * 256;
  p->pair_bytes = static_cast<size_t>(B) * 2 * (k + 1) * p->nc * sizeof(sv::PairPart);
  p->ws_bytes = sv::kFlagsBytes + p->seq_bytes + p->tile_bytes + p->part_bytes + p->tpart_bytes +
                p->pair_bytes;
  return SV_OK;
}

int32_t check_workspace(const Plan& p, const void* ws, size_t bytes) {
  if (!ws) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned_to(ws, 256)) return fail(SV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (bytes < p.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "workspace has " + std::to_string(bytes) + " bytes, needs " +
                                      std::to_string(p.ws_bytes));
  return SV_OK;
}

int32_t check_logits(const void* ptr, int rows, int dtype, const char* name) {
  if (rows == 0) return SV_OK;
  if (!ptr) return fail(SV_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned_to(ptr, sv::elem_bytes(dtype)))
    return fail(SV_ERR_MISALIGNED, std::string(name) + " not aligned to its element size");
  return SV_OK;
}

int32_t check_i32(const void* ptr, bool required, const char* name) {
  if (!ptr) return required ? fail(SV_ERR_INVALID_ARG, std::string(name) + " is NULL") : SV_OK;
  if (!aligned_to(ptr, 4)) return fail(SV_ERR_MISALIGNED, std::string(name) + " not 4-byte aligned");
  return SV_OK;
}

bool wants_outcome(const spec_verify_diag* d) {
  return d && (d->accept_mass || d->residual_tokens || d->residual_mass);
}
bool wants_byproducts(const spec_verify_diag* d) { return d && (d->entropy || wants_outcome(d)); }
bool wants_row_stats(const spec_verify_diag* d) { return d && (d->row_log2z || d->row_argmax); }

int32_t check_diag(const spec_verify_diag* diag) {
  if (!diag) return SV_OK;
  if (diag->uniforms && !aligned_to(diag->uniforms, 4))
    return fail(SV_ERR_MISALIGNED, "diag.uniforms not 4-byte aligned");
  if (diag->probs && !aligned_to(diag->probs, 8))
    return fail(SV_ERR_MISALIGNED, "diag.probs not 8-byte aligned");
  if (diag->draws && !aligned_to(diag->draws, 8))
    return fail(SV_ERR_MISALIGNED, "diag.draws not 8-byte aligned");
  if (diag->entropy && !aligned_to(diag->entropy, 4))
    return fail(SV_ERR_MISALIGNED, "diag.entropy not 4-byte aligned");
  if (diag->accept_mass && !aligned_to(diag->accept_mass, 4))
    return fail(SV_ERR_MISALIGNED, "diag.accept_mass not 4-byte aligned");
  if (diag->residual_tokens && !aligned_to(diag->residual_tokens, 4))
    return fail(SV_ERR_MISALIGNED, "diag.residual_tokens not 4-byte aligned");
  if (diag->residual_mass && !aligned_to(diag->residual_mass, 4))
    return fail(SV_ERR_MISALIGNED, "diag.residual_mass not 4-byte aligned");
  if (diag->row_log2z && !aligned_to(diag->row_log2z, 8))
    return fail(SV_ERR_MISALIGNED, "diag.row_log2z not 8-byte aligned");
  if (diag->row_argmax && !aligned_to(diag->row_argmax, 4))
    return fail(SV_ERR_MISALIGNED, "diag.row_argmax not 4-byte aligned");
  if ((diag->residual_tokens || diag->residual_mass) &&
      (diag->top_m < 1 || diag->top_m > SV_MAX_TOP_M))
    return fail(SV_ERR_INVALID_ARG, "diag.top_m must be in [1, " + std::to_string(SV_MAX_TOP_M) + "]");
  return SV_OK;
}

int32_t device_error(hipError_t e, const char* what) {
  return fail(SV_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define SV_TRY(expr)              \
  do {                            \
    const int32_t _s = (expr);    \
    if (_s != SV_OK) return _s;   \
  } while (0)

struct KvRollback {
  int32_t max_blocks, block_size, max_freed;
  int32_t* table;
  int32_t* lens;
  int32_t* freed;
  int32_t* num_freed;
};

int32_t check_kv(int32_t batch, int32_t max_blocks, int32_t block_size, const int32_t* table,
                 const int32_t* lens, const int32_t* drop, bool drop_required,
                 const int32_t* freed, int32_t max_freed, const int32_t* num_freed) {
  if (batch < 0) return fail(SV_ERR_INVALID_ARG, "batch < 0");
  if (max_blocks < 0) return fail(SV_ERR_INVALID_ARG, "max_blocks < 0");
  if (block_size < 1) return fail(SV_ERR_INVALID_ARG, "block_size < 1");
  if (max_freed < 0) return fail(SV_ERR_INVALID_ARG, "max_freed < 0");
  const bool any = batch > 0;
  SV_TRY(check_i32(table, any && max_blocks > 0, "block_table"));
  SV_TRY(check_i32(lens, any, "seq_lens"));
  SV_TRY(check_i32(drop, any && drop_required, "num_drop"));
  SV_TRY(check_i32(freed, any && max_freed > 0, "freed_blocks"));
  SV_TRY(check_i32(num_freed, any, "num_freed"));
  return SV_OK;
}

// Arguments of the lazy final exit's stage-1 pass: one workgroup per
// sequence decides stage 1 from the L_d and L_i statistics.
sv::VerifyArgs stage1_args(const spec_verify_desc* desc, const Plan& p, const void* const* logits,
                           const sv::Partial* partials, const int32_t* tokens,
                           const float* temperature, uint32_t* flags) {
  sv::VerifyArgs va{};
  va.hier = 1;
  va.B = desc->batch;
  va.k = desc->num_draft;
  va.V = desc->vocab;
  va.dtype = desc->dtype;
  va.nc = p.nc;
  va.window = 1;
  va.nt = p.nt;
  va.ns = 1;
  va.tps = p.tps;
  va.ld = p.ld;
  for (int e = 0; e < 3; ++e) {
    va.exit_ptr[e] = logits[e];
    va.exit_row0[e] = p.exit_row0[e];
  }
  va.partials = partials;
  va.tokens = tokens;
  va.temperature = temperature;
  va.key0 = static_cast<uint32_t>(desc->seed & 0xffffffffu);
  va.key1 = static_cast<uint32_t>(desc->seed >> 32);
  va.offset = desc->offset;
  va.flags = flags;
  return va;
}

int32_t run_verify(const spec_verify_desc* desc, int32_t num_exits, int32_t window,
                   const void* const* logits, const int32_t* tokens, const float* temperature,
                   int32_t* accept_len, int32_t* accept_len_final, int32_t* out_tokens,
                   int32_t* num_emitted, int32_t* num_drop, int32_t* packed, int32_t* cu_offsets,
                   void* workspace, size_t workspace_bytes, const spec_verify_diag* diag,
                   void* hip_stream, const KvRollback* kv = nullptr, bool lazy = false,
                   bool clear_round = false) {
  Plan p;
  SV_TRY(make_plan(desc, num_exits, &p));
  if (num_exits == 3 && window < 1) return fail(SV_ERR_INVALID_ARG, "window < 1");
  static const char* names[3] = {"draft/L_d logits", "target/L_i logits", "L_f logits"};
  for (int e = 0; e < num_exits; ++e)
    SV_TRY(check_logits(logits[e], desc->batch * p.exit_pos[e], desc->dtype, names[e]));
  const bool any = desc->batch > 0;
  SV_TRY(check_i32(tokens, any && desc->num_draft > 0, "draft_tokens"));
  if (temperature && !aligned_to(temperature, 4))
    return fail(SV_ERR_MISALIGNED, "temperature not 4-byte aligned");
  SV_TRY(check_i32(accept_len, any, "accept_len"));
  if (num_exits == 3) SV_TRY(check_i32(accept_len_final, any, "accept_len_final"));
  SV_TRY(check_i32(out_tokens, any, "out_tokens"));
  SV_TRY(check_i32(num_emitted, any, "num_emitted"));
  SV_TRY(check_i32(num_drop, false, "num_drop"));
  SV_TRY(check_i32(packed, false, "packed_tokens"));
  SV_TRY(check_i32(cu_offsets, packed != nullptr, "cu_offsets"));
  if (cu_offsets && !packed) return fail(SV_ERR_INVALID_ARG, "cu_offsets without packed_tokens");
  SV_TRY(check_diag(diag));
  if (lazy && (wants_byproducts(diag) || wants_row_stats(diag)))
    return fail(SV_ERR_UNSUPPORTED,
                "the lazy final exit does not stream every row: no by-products or row statistics");
  SV_TRY(check_workspace(p, workspace, workspace_bytes));
  if (kv)
    SV_TRY(check_kv(desc->batch, kv->max_blocks, kv->block_size, kv->table, kv->lens, nullptr,
                    false, kv->freed, kv->max_freed, kv->num_freed));
  if (!any) return SV_OK;

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  int32_t* seqw = reinterpret_cast<int32_t*>(ws + sv::kFlagsBytes);
  float* tsum = reinterpret_cast<float*>(ws + sv::kFlagsBytes + p.seq_bytes);
  char* part_base = ws + sv::kFlagsBytes + p.seq_bytes + p.tile_bytes;
  sv::Partial* partials = reinterpret_cast<sv::Partial*>(part_base);
  double* tpart = reinterpret_cast<double*>(part_base + p.part_bytes);
  sv::PairPart* pair = reinterpret_cast<sv::PairPart*>(part_base + p.part_bytes + p.tpart_bytes);
  const bool want_entropy = diag && diag->entropy;
  const int B = desc->batch;
  hipError_t err;

  sv::StatsArgs sa{};
  for (int e = 0; e < 3; ++e) {
    sa.exit_ptr[e] = e < num_exits ? logits[e] : nullptr;
    sa.exit_pos[e] = p.exit_pos[e];
    sa.exit_row0[e] = e < num_exits ? p.exit_row0[e] : INT32_MAX;
  }
  sa.num_exits = num_exits;
  sa.V = desc->vocab;
  sa.nc = p.nc;
  sa.dtype = desc->dtype;
  sa.ld = p.ld;
  sa.temperature = temperature;
  sa.partials = partials;
  sa.clear_words = seqw;   // slice counters (and, lazy, the stage-1 counts and list count)
  // (a tentative round: its append's arrival counters in the third block)
  sa.n_clear = lazy ? 3 * B + 1 : (clear_round ? 3 * B : 2 * B);
  sa.flags = flags;
  sa.tpart = want_entropy ? tpart : nullptr;
  int32_t* lazy_a1 = lazy ? seqw + 2 * B : nullptr;
  const int k = desc->num_draft;
  int32_t* list_count = seqw + 3 * B;   // lazy: rows listed by the window pass
  int32_t* row_list = seqw + 3 * B + 1;
  // lazy: the stage-1 window, rows j < r0 of L_d and j < r1 of L_i (with the
  // bonus row when the window covers every draft)
  const int r0 = std::min(std::max(window, 1), k), r1 = r0 + (r0 == k ? 1 : 0);
  hipEvent_t ev_begin = diag ? static_cast<hipEvent_t>(diag->stats_begin) : nullptr;
  hipEvent_t ev_end = diag ? static_cast<hipEvent_t>(diag->stats_end) : nullptr;
  if (!lazy) {
    err = sv::launch_stats(sa, p.rows_total, st, ev_begin, ev_end);
    if (err != hipSuccess) return device_error(err, "row statistics launch");
  } else {
    // the L_d and L_i rows of the first N_i positions; stage 1 on them lists
    // the rows still needed (L_f rows 0..a1, or, for a sequence that accepted
    // all N_i drafts, the rest of its L_d / L_i rows and all of its L_f rows),
    // which the list-mode statistics then stream
    sv::StatsArgs sw = sa;
    sw.win_b = B;
    sw.win_r0 = r0;
    sw.win_r1 = r1;
    err = sv::launch_stats(sw, static_cast<int64_t>(B) * (r0 + r1), st, ev_begin, nullptr);
    if (err != hipSuccess) return device_error(err, "row statistics launch");
  }
  sv::VerifyArgs va{};
  if (lazy) {
    va = stage1_args(desc, p, logits, partials, tokens, temperature, flags);
    va.stage1_only = 1;
    va.stage1_window = r0;
    va.lazy_a1 = lazy_a1;
    va.row_list_out = row_list;
    va.row_count_out = list_count;
    err = sv::launch_verify(va, st);
    if (err != hipSuccess) return device_error(err, "stage-1 launch");
    sv::StatsArgs sl = sa;   // the listed rows only
    sl.n_clear = 0;
    sl.row_list = row_list;
    sl.row_count = list_count;
    const int64_t per_seq = std::max(3 * k, k + 1);
    err = sv::launch_stats_list(sl, static_cast<int64_t>(B) * per_seq * p.nc, st, nullptr, ev_end);
    if (err != hipSuccess) return device_error(err, "listed row statistics launch");
  }

  va = sv::VerifyArgs{};
  va.lazy_a1 = lazy_a1;
  va.hier = num_exits == 3;
  va.B = B;
  va.k = desc->num_draft;
  va.V = desc->vocab;
  va.dtype = desc->dtype;
  va.nc = p.nc;
  va.window = num_exits == 3 ? window : 1;
  va.nt = p.nt;
  va.ns = p.ns;
  va.tps = p.tps;
  va.ld = p.ld;
  for (int e = 0; e < 3; ++e) {
    va.exit_ptr[e] = e < num_exits ? logits[e] : nullptr;
    va.exit_row0[e] = e < num_exits ? p.exit_row0[e] : 0;
  }
  va.partials = partials;
  for (int s = 0; s < 2; ++s) {
    va.tsum[s] = tsum + static_cast<size_t>(s) * B * p.nt;
    va.cnt[s] = seqw + s * B;
  }
  va.tokens = tokens;
  va.temperature = temperature;
  va.key0 = static_cast<uint32_t>(desc->seed & 0xffffffffu);
  va.key1 = static_cast<uint32_t>(desc->seed >> 32);
  va.offset = desc->offset;
  va.accept_len = accept_len;
  va.accept_len_final = num_exits == 3 ? accept_len_final : nullptr;
  va.out_tokens = out_tokens;
  va.num_emitted = num_emitted;
  va.num_drop = num_drop;
  va.diag_uniforms = diag ? diag->uniforms : nullptr;
  va.diag_probs = diag ? diag->probs : nullptr;
  va.diag_draws = diag ? diag->draws : nullptr;
  va.row_log2z = diag ? diag->row_log2z : nullptr;
  va.row_argmax = diag ? diag->row_argmax : nullptr;
  va.flags = flags;
  if (kv) {
    va.kv_table = kv->table;
    va.kv_lens = kv->lens;
    va.kv_freed = kv->freed;
    va.kv_num_freed = kv->num_freed;
    va.kv_max_blocks = kv->max_blocks;
    va.kv_block_size = kv->block_size;
    va.kv_max_freed = kv->max_freed;
  }
  err = sv::launch_verify(va, st);
  if (err != hipSuccess) return device_error(err, "verify launch");

  if (packed) {
    sv::PackArgs pa{desc->batch, desc->num_draft, out_tokens, num_emitted, packed, cu_offsets};
    err = sv::launch_pack(pa, st);
    if (err != hipSuccess) return device_error(err, "pack launch");
  }

  if (wants_byproducts(diag)) {
    sv::ByArgs ba{};
    ba.B = B;
    ba.k = desc->num_draft;
    ba.V = desc->vocab;
    ba.dtype = desc->dtype;
    ba.nc = p.nc;
    ba.hier = num_exits == 3;
    ba.ld = p.ld;
    for (int e = 0; e < 3; ++e) {
      ba.exit_ptr[e] = e < num_exits ? logits[e] : nullptr;
      ba.exit_pos[e] = p.exit_pos[e];
      ba.exit_row0[e] = e < num_exits ? p.exit_row0[e] : INT32_MAX;
    }
    ba.partials = partials;
    ba.tpart = tpart;
    ba.temperature = temperature;
    ba.rows = static_cast<int32_t>(p.rows_total);
    ba.entropy = diag->entropy;
    ba.pair = pair;
    ba.beta = diag->accept_mass;
    ba.top_tok = diag->residual_tokens;
    ba.top_mass = diag->residual_mass;
    ba.top_m = (diag->residual_tokens || diag->residual_mass) ? diag->top_m : 0;
    if (want_entropy && p.rows_total > 0) {
      err = sv::launch_entropy(ba, st);
      if (err != hipSuccess) return device_error(err, "entropy launch");
    }
    if (wants_outcome(diag)) {
      err = sv::launch_outcome(ba, st);
      if (err != hipSuccess) return device_error(err, "outcome export launch");
    }
  }
  return SV_OK;
}

// Workspace and launch plan of the LM-head path.
struct LmPlan {
  int64_t M = 0;          // GEMM rows: B*k draft rows, then B*(k+1) target rows
  int n_tiles = 0;        // vocabulary tiles of the GEMM
  int nt = 0, ns = 0;     // draw tiles per recomputed row and slices per sequence
  int64_t ldw = 0, ldo = 0;
  size_t seq_bytes = 0, tile_bytes = 0, part_bytes = 0, merged_bytes = 0, gath_bytes = 0,
         stop_bytes = 0, rows_bytes = 0, ws_bytes = 0;
};

size_t pad256(size_t n) { return (n + 255) / 256 * 256; }

int32_t make_lm_plan(const spec_verify_desc* d, int32_t hidden, LmPlan* p) {
  if (!d) return fail(SV_ERR_INVALID_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(SV_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->batch < 0) return fail(SV_ERR_INVALID_ARG, "batch < 0");
  if (d->num_draft < 0) return fail(SV_ERR_INVALID_ARG, "num_draft < 0");
  if (d->num_draft > SV_MAX_DRAFT)
    return fail(SV_ERR_UNSUPPORTED, "num_draft > " + std::to_string(SV_MAX_DRAFT));
  if (d->vocab < 1) return fail(SV_ERR_INVALID_ARG, "vocab < 1");
  if (d->vocab > SV_MAX_VOCAB)
    return fail(SV_ERR_UNSUPPORTED, "vocab > " + std::to_string(SV_MAX_VOCAB));
  if (d->dtype != SV_DTYPE_BF16)
    return fail(SV_ERR_UNSUPPORTED, "the LM-head path takes bf16 hidden states and head");
  if (hidden < sv::kHiddenMultiple || hidden % sv::kHiddenMultiple != 0 || hidden > SV_MAX_HIDDEN)
    return fail(SV_ERR_UNSUPPORTED, "hidden must be a multiple of 64 in [64, " +
                                        std::to_string(SV_MAX_HIDDEN) + "]");
  const int64_t ldw = d->row_stride == 0 ? hidden : d->row_stride;
  if (ldw < hidden) return fail(SV_ERR_INVALID_ARG, "row_stride < hidden");
  if (ldw % 8 != 0) return fail(SV_ERR_MISALIGNED, "row_stride not a multiple of 8");
  if (ldw > (int64_t(1) << 40)) return fail(SV_ERR_INVALID_ARG, "row_stride too large");
  const int64_t B = d->batch, k = d->num_draft;
  p->M = B * (2 * k + 1);
  p->n_tiles = (d->vocab + sv::kGemmNT - 1) / sv::kGemmNT;
  if (p->M > INT32_MAX / 2 || p->M * p->n_tiles > INT32_MAX)
    return fail(SV_ERR_UNSUPPORTED, "batch too large for one call");
  const int te = sv::tile_elems(SV_DTYPE_F32);   // draws read fp32 recomputed rows
  p->nt = (d->vocab + te - 1) / te;
  p->ns = (p->nt + sv::kTilesPerSlice - 1) / sv::kTilesPerSlice;
  p->ldw = ldw;
  p->ldo = (static_cast<int64_t>(d->vocab) + 3) / 4 * 4;
  p->seq_bytes = pad256(static_cast<size_t>(B) * 2 * sizeof(int32_t));
  p->tile_bytes = pad256(static_cast<size_t>(B) * 2 * p->nt * sizeof(float));
  p->part_bytes = pad256(static_cast<size_t>(p->M) * p->n_tiles * sizeof(sv::Partial));
  p->merged_bytes = pad256(static_cast<size_t>(p->M) * sizeof(sv::Partial));
  p->gath_bytes = pad256(static_cast<size_t>(p->M) * sizeof(float));
  p->stop_bytes = pad256(static_cast<size_t>(B) * 2 * sizeof(int32_t));
  p->rows_bytes = static_cast<size_t>(B) * 2 * p->ldo * sizeof(float);
  p->ws_bytes = sv::kFlagsBytes + p->seq_bytes + p->tile_bytes + p->part_bytes +
                p->merged_bytes + p->gath_bytes + p->stop_bytes + p->rows_bytes;
  return SV_OK;
}

int32_t run_lmhead(const spec_verify_desc* desc, int32_t hidden, const void* h_draft,
                   const void* h_target, const void* w_vocab, const int32_t* tokens,
                   const float* temperature, int32_t* accept_len, int32_t* out_tokens,
                   int32_t* num_emitted, int32_t* num_drop, int32_t* packed,
                   int32_t* cu_offsets, void* workspace, size_t workspace_bytes,
                   const spec_verify_diag* diag, void* hip_stream) {
  LmPlan p;
  SV_TRY(make_lm_plan(desc, hidden, &p));
  const int B = desc->batch, k = desc->num_draft;
  const bool any = B > 0;
  if (any) {
    if (k > 0 && !h_draft) return fail(SV_ERR_INVALID_ARG, "h_draft is NULL");
    if (!h_target) return fail(SV_ERR_INVALID_ARG, "h_target is NULL");
    if (!w_vocab) return fail(SV_ERR_INVALID_ARG, "w_vocab is NULL");
    if ((k > 0 && !aligned_to(h_draft, 16)) || !aligned_to(h_target, 16) ||
        !aligned_to(w_vocab, 16))
      return fail(SV_ERR_MISALIGNED, "hidden states and head must be 16-byte aligned");
  }
  SV_TRY(check_i32(tokens, any && k > 0, "draft_tokens"));
  if (temperature && !aligned_to(temperature, 4))
    return fail(SV_ERR_MISALIGNED, "temperature not 4-byte aligned");
  SV_TRY(check_i32(accept_len, any, "accept_len"));
  SV_TRY(check_i32(out_tokens, any, "out_tokens"));
  SV_TRY(check_i32(num_emitted, any, "num_emitted"));
  SV_TRY(check_i32(num_drop, false, "num_drop"));
  SV_TRY(check_i32(packed, false, "packed_tokens"));
  SV_TRY(check_i32(cu_offsets, packed != nullptr, "cu_offsets"));
  if (cu_offsets && !packed) return fail(SV_ERR_INVALID_ARG, "cu_offsets without packed_tokens");
  SV_TRY(check_diag(diag));
  if (wants_byproducts(diag) || wants_row_stats(diag))
    return fail(SV_ERR_UNSUPPORTED,
                "the LM-head path stores no logit rows: no by-products or row statistics");
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned_to(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < p.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, needs " + std::to_string(p.ws_bytes));
  if (!any) return SV_OK;

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = ws + off;
    off += n;
    return q;
  };
  uint32_t* flags = reinterpret_cast<uint32_t*>(take(sv::kFlagsBytes));
  int32_t* seqw = reinterpret_cast<int32_t*>(take(p.seq_bytes));
  float* tsum = reinterpret_cast<float*>(take(p.tile_bytes));
  sv::Partial* part = reinterpret_cast<sv::Partial*>(take(p.part_bytes));
  sv::Partial* merged = reinterpret_cast<sv::Partial*>(take(p.merged_bytes));
  float* gath = reinterpret_cast<float*>(take(p.gath_bytes));
  int32_t* stop_rows = reinterpret_cast<int32_t*>(take(p.stop_bytes));
  float* rows = reinterpret_cast<float*>(take(p.rows_bytes));
  hipError_t err;

  sv::GemmArgs g{};
  g.a_draft = static_cast<const uint16_t*>(h_draft);
  g.a_target = static_cast<const uint16_t*>(h_target);
  g.w = static_cast<const uint16_t*>(w_vocab);
  g.ldw = p.ldw;
  g.M = static_cast<int32_t>(p.M);
  g.m_draft = B * k;
  g.V = desc->vocab;
  g.d = hidden;
  g.B = B;
  g.k = k;
  g.n_tiles = p.n_tiles;
  g.tokens = tokens;
  g.temperature = temperature;
  g.partials = part;
  g.gath = gath;
  err = sv::launch_lmhead_stats(g, st, diag ? static_cast<hipEvent_t>(diag->stats_begin) : nullptr,
                                diag ? static_cast<hipEvent_t>(diag->stats_end) : nullptr);
  if (err != hipSuccess) return device_error(err, "LM-head statistics launch");

  sv::MergeArgs ma{part, merged, g.M, p.n_tiles, seqw, 2 * B, flags};
  err = sv::launch_merge(ma, g, st);
  if (err != hipSuccess) return device_error(err, "merge launch");

  sv::VerifyArgs va{};
  va.hier = 0;
  va.B = B;
  va.k = k;
  va.V = desc->vocab;
  va.dtype = SV_DTYPE_F32;   // the draws read fp32 recomputed rows
  va.nc = 1;
  va.window = 1;
  va.nt = p.nt;
  va.ns = 1;                 // decisions: one workgroup per sequence
  va.tps = sv::kTilesPerSlice;
  va.ld = p.ldo;
  va.exit_row0[0] = 0;
  va.exit_row0[1] = B * k;
  va.partials = merged;
  for (int s = 0; s < 2; ++s) {
    va.tsum[s] = tsum + static_cast<size_t>(s) * B * p.nt;
    va.cnt[s] = seqw + s * B;
  }
  va.tokens = tokens;
  va.temperature = temperature;
  va.key0 = static_cast<uint32_t>(desc->seed & 0xffffffffu);
  va.key1 = static_cast<uint32_t>(desc->seed >> 32);
  va.offset = desc->offset;
  va.accept_len = accept_len;
  va.out_tokens = out_tokens;
  va.num_emitted = num_emitted;
  va.num_drop = num_drop;
  va.diag_uniforms = diag ? diag->uniforms : nullptr;
  va.diag_probs = diag ? diag->probs : nullptr;
  va.diag_draws = diag ? diag->draws : nullptr;
  va.flags = flags;
  va.gath = gath;
  va.decide_only = 1;
  va.stop_rows = stop_rows;
  err = sv::launch_verify(va, st);
  if (err != hipSuccess) return device_error(err, "decision launch");

  sv::GemmArgs r = g;
  r.a_rows = stop_rows;
  r.n_tiles = (desc->vocab + sv::kGemmRowsNT - 1) / sv::kGemmRowsNT;
  r.M = 2 * B;
  r.out = rows;
  r.ldo = p.ldo;
  r.partials = nullptr;
  r.gath = nullptr;
  err = sv::launch_lmhead_rows(r, st);
  if (err != hipSuccess) return device_error(err, "LM-head row recompute launch");

  va.ns = p.ns;
  va.decide_only = 0;
  va.draw_rows = rows;
  va.draw_ld = p.ldo;
  err = sv::launch_verify(va, st);
  if (err != hipSuccess) return device_error(err, "draw launch");

  if (packed) {
    sv::PackArgs pa{B, k, out_tokens, num_emitted, packed, cu_offsets};
    err = sv::launch_pack(pa, st);
    if (err != hipSuccess) return device_error(err, "pack launch");
  }
  return SV_OK;
}

// Cross-call tentative buffering: a round is the single-stage verification of
// (L_d, L_i) followed by the append to the pending state; a flush streams the
// pending rows and the final exit's rows of the pending positions, then runs
// the verification kernel in flush mode.
struct TentPlan {
  Plan round, flush;           // flush: k = capacity
  size_t round_extra = 0, flush_extra = 0, ws_bytes = 0;
};

int32_t make_tent_plan(const spec_verify_desc* d, int32_t capacity, TentPlan* t) {
  SV_TRY(make_plan(d, 2, &t->round));
  if (capacity < 1 || capacity > SV_MAX_DRAFT)
    return fail(SV_ERR_UNSUPPORTED, "pending capacity must be in [1, " + std::to_string(SV_MAX_DRAFT) + "]");
  spec_verify_desc f = *d;
  f.num_draft = capacity;
  SV_TRY(make_plan(&f, 2, &t->flush));
  const size_t B = static_cast<size_t>(d->batch);
  // round: stage-1 output tokens [B, k+1] and counts [B]; flush: limits [B]
  t->round_extra = pad256(B * (d->num_draft + 1) * sizeof(int32_t)) + pad256(B * sizeof(int32_t));
  t->flush_extra = pad256(B * sizeof(int32_t)) +
                   pad256((B * 2 * static_cast<size_t>(capacity) + 1) * sizeof(int32_t));
  t->ws_bytes = std::max(pad256(t->round.ws_bytes) + t->round_extra,
                         pad256(t->flush.ws_bytes) + t->flush_extra);
  return SV_OK;
}

int32_t check_pending(const spec_verify_pending* pd, int32_t batch, int32_t dtype) {
  if (!pd) return fail(SV_ERR_INVALID_ARG, "pending is NULL");
  if (batch == 0) return SV_OK;
  SV_TRY(check_i32(pd->count, true, "pending.count"));
  SV_TRY(check_i32(pd->tokens, true, "pending.tokens"));
  if (!pd->rows) return fail(SV_ERR_INVALID_ARG, "pending.rows is NULL");
  if (!aligned_to(pd->rows, sv::elem_bytes(dtype)))
    return fail(SV_ERR_MISALIGNED, "pending.rows not aligned to its element size");
  return SV_OK;
}

int32_t run_round(const spec_verify_desc* desc, const void* ld, const void* li,
                  const int32_t* tokens, const float* temperature, const int32_t* active,
                  const spec_verify_pending* pending, int32_t* accept_len, int32_t* num_drop,
                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!pending) return fail(SV_ERR_INVALID_ARG, "pending is NULL");
  TentPlan t;
  SV_TRY(make_tent_plan(desc, pending->capacity, &t));
  SV_TRY(check_pending(pending, desc->batch, desc->dtype));
  SV_TRY(check_i32(active, false, "active"));
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < t.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, needs " + std::to_string(t.ws_bytes));
  char* ws = static_cast<char*>(workspace);
  const size_t off = pad256(t.round.ws_bytes);
  const int B = desc->batch, k = desc->num_draft;
  int32_t* t_out = reinterpret_cast<int32_t*>(ws + off);
  int32_t* n_out = reinterpret_cast<int32_t*>(ws + off + pad256(static_cast<size_t>(B) * (k + 1) * 4));
  const void* logits[3] = {ld, li, nullptr};
  SV_TRY(run_verify(desc, 2, 1, logits, tokens, temperature, accept_len, nullptr, t_out, n_out,
                    num_drop, nullptr, nullptr, workspace, t.round.ws_bytes, nullptr, hip_stream,
                    nullptr, false, true));
  if (B == 0) return SV_OK;
  sv::PendArgs pa{};
  pa.B = B;
  pa.k = k;
  pa.V = desc->vocab;
  pa.dtype = desc->dtype;
  pa.cap = pending->capacity;
  pa.nch = t.round.nc;
  pa.ld = t.round.ld;
  pa.li = li;
  pa.active = active;
  pa.a1 = accept_len;
  pa.t_out = t_out;
  pa.count = pending->count;
  pa.tokens = pending->tokens;
  pa.rows = pending->rows;
  pa.flags = reinterpret_cast<uint32_t*>(ws);
  // the third block of per-sequence words (cleared by the statistics launch)
  pa.arrive = reinterpret_cast<int32_t*>(ws + sv::kFlagsBytes) + 2 * B;
  const hipError_t err = sv::launch_pending_append(pa, static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return device_error(err, "pending append launch");
  return SV_OK;
}

int32_t run_flush(const spec_verify_desc* desc, const void* lf, const float* temperature,
                  int32_t min_pending, const spec_verify_pending* pending, int32_t* accept_len,
                  int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop, void* workspace,
                  size_t workspace_bytes, void* hip_stream) {
  if (!pending) return fail(SV_ERR_INVALID_ARG, "pending is NULL");
  TentPlan t;
  SV_TRY(make_tent_plan(desc, pending->capacity, &t));
  const Plan& p = t.flush;
  const int B = desc->batch, cap = pending->capacity;
  SV_TRY(check_pending(pending, B, desc->dtype));
  if (min_pending < 0) return fail(SV_ERR_INVALID_ARG, "min_pending < 0");
  SV_TRY(check_logits(lf, B * (cap + 1), desc->dtype, "lf_logits"));
  if (temperature && !aligned_to(temperature, 4))
    return fail(SV_ERR_MISALIGNED, "temperature not 4-byte aligned");
  const bool any = B > 0;
  SV_TRY(check_i32(accept_len, any, "accept_len"));
  SV_TRY(check_i32(out_tokens, any, "out_tokens"));
  SV_TRY(check_i32(num_emitted, any, "num_emitted"));
  SV_TRY(check_i32(num_drop, false, "num_drop"));
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned_to(workspace, 256)) return fail(SV_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < t.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, needs " + std::to_string(t.ws_bytes));
  if (!any) return SV_OK;

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  int32_t* seqw = reinterpret_cast<int32_t*>(ws + sv::kFlagsBytes);
  float* tsum = reinterpret_cast<float*>(ws + sv::kFlagsBytes + p.seq_bytes);
  sv::Partial* partials =
      reinterpret_cast<sv::Partial*>(ws + sv::kFlagsBytes + p.seq_bytes + p.tile_bytes);
  int32_t* lim = reinterpret_cast<int32_t*>(ws + pad256(p.ws_bytes));
  int32_t* row_count = reinterpret_cast<int32_t*>(ws + pad256(p.ws_bytes) +
                                                  pad256(static_cast<size_t>(B) * sizeof(int32_t)));
  int32_t* row_list = row_count + 1;
  hipError_t err;

  sv::PendArgs pa{};
  pa.B = B;
  pa.cap = cap;
  pa.count = pending->count;
  pa.min_pending = min_pending;
  pa.lim = lim;
  pa.row0_q = p.exit_row0[0];
  pa.row0_p = p.exit_row0[1];
  pa.row_list = row_list;
  pa.row_count = row_count;
  err = sv::launch_flush_prep(pa, st);
  if (err != hipSuccess) return device_error(err, "flush prep launch");

  const void* exits[2] = {pending->rows, lf};
  sv::StatsArgs sa{};
  for (int e = 0; e < 3; ++e) {
    sa.exit_ptr[e] = e < 2 ? exits[e] : nullptr;
    sa.exit_pos[e] = p.exit_pos[e];
    sa.exit_row0[e] = e < 2 ? p.exit_row0[e] : INT32_MAX;
  }
  sa.num_exits = 2;
  sa.V = desc->vocab;
  sa.nc = p.nc;
  sa.dtype = desc->dtype;
  sa.ld = p.ld;
  sa.temperature = temperature;
  sa.partials = partials;
  sa.clear_words = seqw;
  sa.n_clear = 2 * B;
  sa.flags = flags;
  sa.row_list = row_list;   // the pending rows and L_f rows of the flushed sequences
  sa.row_count = row_count;
  sa.cached_loads = 1;       // the verification below reads the pending rows again
  err = sv::launch_stats_list(sa, p.rows_total * p.nc, st);
  if (err != hipSuccess) return device_error(err, "row statistics launch");

  sv::VerifyArgs va{};
  va.hier = 0;
  va.B = B;
  va.k = cap;
  va.V = desc->vocab;
  va.dtype = desc->dtype;
  va.nc = p.nc;
  va.window = 1;
  va.nt = p.nt;
  va.ns = p.ns;
  va.tps = p.tps;
  va.ld = p.ld;
  for (int e = 0; e < 3; ++e) {
    va.exit_ptr[e] = e < 2 ? exits[e] : nullptr;
    va.exit_row0[e] = e < 2 ? p.exit_row0[e] : 0;
  }
  va.partials = partials;
  for (int s = 0; s < 2; ++s) {
    va.tsum[s] = tsum + static_cast<size_t>(s) * B * p.nt;
    va.cnt[s] = seqw + s * B;
  }
  va.tokens = pending->tokens;
  va.temperature = temperature;
  va.key0 = static_cast<uint32_t>(desc->seed & 0xffffffffu);
  va.key1 = static_cast<uint32_t>(desc->seed >> 32);
  va.offset = desc->offset;
  va.accept_len = accept_len;
  va.out_tokens = out_tokens;
  va.num_emitted = num_emitted;
  va.num_drop = num_drop;
  va.flags = flags;
  va.flush_lim = lim;
  err = sv::launch_verify(va, st);
  if (err != hipSuccess) return device_error(err, "flush verify launch");
  return SV_OK;
}

}  // namespace

namespace {

// Scratch of spec_verify_hier_rollback_noalloc, for callers that cannot
// allocate: one array per GPU the library runs on, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is
// a stand-in, not a device address): the first call on a device looks up that
// device's copy with hipGetSymbolAddress and keeps the address.
constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the scratch array on the GPU that runs `st` (the current
// device for the null stream).
int32_t scratch_address(hipStream_t st, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  int dev = cur;
  if (st) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(st, &d);
    if (e != hipSuccess) return device_error(e, "hipStreamGetDevice");
    dev = d;
  }
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SV_ERR_UNSUPPORTED, "device index " + std::to_string(dev) +
                                        " beyond the scratch table of the no-allocation call");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return device_error(e, "hipSetDevice");
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess && r != hipSuccess) e = r;
    }
    if (e != hipSuccess) return device_error(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SV_ERR_DEVICE, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

}  // namespace

extern "C" {

int32_t spec_verify_abi_version(void) { return SPEC_VERIFY_ABI_VERSION; }

const char* spec_verify_status_string(int32_t status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_MISALIGNED: return "SV_ERR_MISALIGNED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_DEVICE: return "SV_ERR_DEVICE";
    default: return "SV_ERR_UNKNOWN";
  }
}

const char* spec_verify_last_error(void) { return g_last_error.c_str(); }

size_t spec_verify_workspace_bytes(const spec_verify_desc* desc, int32_t num_exits) {
  Plan p;
  const std::string keep = g_last_error;
  const int32_t s = make_plan(desc, num_exits, &p);
  g_last_error = keep;
  return s == SV_OK ? p.ws_bytes : 0;
}

int32_t spec_verify_validate(const spec_verify_desc* desc, int32_t num_exits, int32_t window,
                             size_t workspace_bytes) {
  Plan p;
  SV_TRY(make_plan(desc, num_exits, &p));
  if (num_exits == 3 && window < 1) return fail(SV_ERR_INVALID_ARG, "window < 1");
  if (workspace_bytes < p.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                      " bytes, needs " + std::to_string(p.ws_bytes));
  return SV_OK;
}

int32_t spec_verify_single(const spec_verify_desc* desc, const void* draft_logits,
                           const void* target_logits, const int32_t* draft_tokens,
                           const float* temperature, int32_t* accept_len, int32_t* out_tokens,
                           int32_t* num_emitted, int32_t* num_drop, int32_t* packed_tokens,
                           int32_t* cu_offsets, void* workspace, size_t workspace_bytes,
                           const spec_verify_diag* diag, void* hip_stream) {
  const void* logits[3] = {draft_logits, target_logits, nullptr};
  return run_verify(desc, 2, 1, logits, draft_tokens, temperature, accept_len, nullptr, out_tokens,
                    num_emitted, num_drop, packed_tokens, cu_offsets, workspace, workspace_bytes,
                    diag, hip_stream);
}

int32_t spec_verify_hier(const spec_verify_desc* desc, int32_t window, const void* ld_logits,
                         const void* li_logits, const void* lf_logits,
                         const int32_t* draft_tokens, const float* temperature,
                         int32_t* accept_len_inter, int32_t* accept_len_final,
                         int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                         int32_t* packed_tokens, int32_t* cu_offsets, void* workspace,
                         size_t workspace_bytes, const spec_verify_diag* diag,
                         void* hip_stream) {
  const void* logits[3] = {ld_logits, li_logits, lf_logits};
  return run_verify(desc, 3, window, logits, draft_tokens, temperature, accept_len_inter,
                    accept_len_final, out_tokens, num_emitted, num_drop, packed_tokens,
                    cu_offsets, workspace, workspace_bytes, diag, hip_stream);
}

int32_t kv_blocktable_truncate(int32_t batch, int32_t max_blocks, int32_t block_size,
                               int32_t* block_table, int32_t* seq_lens,
                               const int32_t* num_drop, int32_t* freed_blocks,
                               int32_t max_freed, int32_t* num_freed, void* hip_stream) {
  SV_TRY(check_kv(batch, max_blocks, block_size, block_table, seq_lens, num_drop, true,
                  freed_blocks, max_freed, num_freed));
  if (batch == 0) return SV_OK;
  sv::KvArgs a{batch, max_blocks, block_size, max_freed, block_table, seq_lens,
               num_drop, freed_blocks, num_freed};
  const hipError_t err = sv::launch_kv_truncate(a, static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return device_error(err, "kv truncate launch");
  return SV_OK;
}

int32_t spec_verify_hier_rollback(const spec_verify_desc* desc, int32_t window,
                                  const void* ld_logits, const void* li_logits,
                                  const void* lf_logits, const int32_t* draft_tokens,
                                  const float* temperature, int32_t* accept_len_inter,
                                  int32_t* accept_len_final, int32_t* out_tokens,
                                  int32_t* num_emitted, int32_t* num_drop, int32_t max_blocks,
                                  int32_t block_size, int32_t* block_table, int32_t* seq_lens,
                                  int32_t* freed_blocks, int32_t max_freed, int32_t* num_freed,
                                  void* workspace, size_t workspace_bytes,
                                  const spec_verify_diag* diag, void* hip_stream) {
  const void* logits[3] = {ld_logits, li_logits, lf_logits};
  KvRollback kv{max_blocks, block_size, max_freed, block_table, seq_lens, freed_blocks, num_freed};
  return run_verify(desc, 3, window, logits, draft_tokens, temperature, accept_len_inter,
                    accept_len_final, out_tokens, num_emitted, num_drop, nullptr, nullptr,
                    workspace, workspace_bytes, diag, hip_stream, &kv);
}

size_t spec_verify_lmhead_workspace_bytes(const spec_verify_desc* desc, int32_t hidden) {
  LmPlan p;
  const std::string keep = g_last_error;
  const int32_t s = make_lm_plan(desc, hidden, &p);
  g_last_error = keep;
  return s == SV_OK ? p.ws_bytes : 0;
}

int32_t spec_verify_lmhead_single(const spec_verify_desc* desc, int32_t hidden,
                                  const void* h_draft, const void* h_target,
                                  const void* w_vocab, const int32_t* draft_tokens,
                                  const float* temperature, int32_t* accept_len,
                                  int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                                  int32_t* packed_tokens, int32_t* cu_offsets, void* workspace,
                                  size_t workspace_bytes, const spec_verify_diag* diag,
                                  void* hip_stream) {
  return run_lmhead(desc, hidden, h_draft, h_target, w_vocab, draft_tokens, temperature,
                    accept_len, out_tokens, num_emitted, num_drop, packed_tokens, cu_offsets,
                    workspace, workspace_bytes, diag, hip_stream);
}

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
                                          void* hip_stream) {
  Plan p;
  SV_TRY(make_plan(desc, 3, &p));
  if (p.ws_bytes > kScratchBytes)
    return fail(SV_ERR_WORKSPACE, "the call needs " + std::to_string(p.ws_bytes) +
                                      " bytes of scratch; the no-allocation call holds " +
                                      std::to_string(kScratchBytes));
  void* ws = nullptr;
  SV_TRY(scratch_address(static_cast<hipStream_t>(hip_stream), &ws));
  const void* logits[3] = {ld_logits, li_logits, lf_logits};
  KvRollback kv{max_blocks, block_size, max_freed, block_table, seq_lens, freed_blocks, num_freed};
  return run_verify(desc, 3, window, logits, draft_tokens, temperature, accept_len_inter,
                    accept_len_final, out_tokens, num_emitted, num_drop, nullptr, nullptr, ws,
                    kScratchBytes, diag, hip_stream, &kv);
}

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
                                       void* hip_stream) {
  const void* logits[3] = {ld_logits, li_logits, lf_logits};
  KvRollback kv{max_blocks, block_size, max_freed, block_table, seq_lens, freed_blocks, num_freed};
  return run_verify(desc, 3, window, logits, draft_tokens, temperature, accept_len_inter,
                    accept_len_final, out_tokens, num_emitted, num_drop, nullptr, nullptr,
                    workspace, workspace_bytes, diag, hip_stream, &kv, true);
}

size_t spec_verify_tentative_workspace_bytes(const spec_verify_desc* desc, int32_t capacity) {
  TentPlan t;
  const std::string keep = g_last_error;
  const int32_t s = make_tent_plan(desc, capacity, &t);
  g_last_error = keep;
  return s == SV_OK ? t.ws_bytes : 0;
}

int32_t spec_verify_tentative_round(const spec_verify_desc* desc, const void* ld_logits,
                                    const void* li_logits, const int32_t* draft_tokens,
                                    const float* temperature, const int32_t* active,
                                    const spec_verify_pending* pending, int32_t* accept_len,
                                    int32_t* num_drop, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  return run_round(desc, ld_logits, li_logits, draft_tokens, temperature, active, pending,
                   accept_len, num_drop, workspace, workspace_bytes, hip_stream);
}

int32_t spec_verify_tentative_flush(const spec_verify_desc* desc, const void* lf_logits,
                                    const float* temperature, int32_t min_pending,
                                    const spec_verify_pending* pending, int32_t* accept_len,
                                    int32_t* out_tokens, int32_t* num_emitted, int32_t* num_drop,
                                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run_flush(desc, lf_logits, temperature, min_pending, pending, accept_len, out_tokens,
                   num_emitted, num_drop, workspace, workspace_bytes, hip_stream);
}

int32_t spec_verify_device_status(const void* workspace, uint32_t* flags_out, void* hip_stream) {
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!flags_out) return fail(SV_ERR_INVALID_ARG, "flags_out is NULL");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t err = hipStreamSynchronize(st);
  if (err != hipSuccess) return device_error(err, "stream synchronize");
  err = hipMemcpy(flags_out, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (err != hipSuccess) return device_error(err, "flags copy");
  return SV_OK;
}

}  // extern "C"
