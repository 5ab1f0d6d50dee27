// C ABI of libsv: host-side validation, workspace carving, split choice and
// dispatch to the HIP launchers. No device memory is allocated or freed here and
// nothing synchronises; every entry point validates what the host can see before
// it enqueues anything.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "api_internal.h"
#include "internal.h"
#include "sv.h"

namespace {

thread_local std::string g_last_error;

sv_status fail(sv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sv_status ok() {
  g_last_error.clear();
  return SV_OK;
}

sv_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxBlocksPerSeq = 16384;
constexpr int kMaxDraft = 16;
constexpr int kMaxRows = 128;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Alignment the kernels rely on: data arrays, outputs and workspaces are read and
// written with 16-byte vector accesses and LDS-DMA, int32 and float-scalar arrays with
// 4-byte ones. NULL (an absent optional buffer) passes.
struct Buf {
  const void* p;
  const char* name;
  uintptr_t align;
};

sv_status check_alignment(std::initializer_list<Buf> bufs, const char* what) {
  for (const Buf& b : bufs)
    if (b.p && (reinterpret_cast<uintptr_t>(b.p) & (b.align - 1)) != 0)
      return fail(SV_ERR_UNSUPPORTED, "%s: %s is not %zu-byte aligned", what, b.name,
                  static_cast<size_t>(b.align));
  return SV_OK;
}

// Validates the shape; `what` names the entry point for the message.
sv_status check_shape(const sv_shape* s, const char* what) {
  if (!s) return fail(SV_ERR_NULL_ARG, "%s: shape is NULL", what);
  if (s->num_seqs < 0) return fail(SV_ERR_BAD_SHAPE, "%s: num_seqs < 0", what);
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0)
    return fail(SV_ERR_BAD_SHAPE, "%s: head counts must be positive", what);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(SV_ERR_BAD_SHAPE, "%s: num_q_heads (%d) not a multiple of num_kv_heads (%d)",
                what, s->num_q_heads, s->num_kv_heads);
  if (s->max_blocks_per_seq <= 0 || s->num_phys_blocks <= 0)
    return fail(SV_ERR_BAD_SHAPE, "%s: max_blocks_per_seq and num_phys_blocks must be positive",
                what);
  if (s->num_draft <= 0) return fail(SV_ERR_BAD_SHAPE, "%s: num_draft must be positive", what);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", what, s->head_dim);
  if (s->block_size != 32 && s->block_size != 64 && s->block_size != 128)
    return fail(SV_ERR_UNSUPPORTED, "%s: block_size %d not in {32, 64, 128}", what,
                s->block_size);
  if (s->num_draft > kMaxDraft)
    return fail(SV_ERR_UNSUPPORTED, "%s: num_draft %d > %d", what, s->num_draft, kMaxDraft);
  const int group = s->num_q_heads / s->num_kv_heads;
  if (static_cast<int64_t>(s->num_draft) * group > kMaxRows)
    return fail(SV_ERR_UNSUPPORTED, "%s: num_draft * group = %d > %d", what,
                s->num_draft * group, kMaxRows);
  if (s->dtype != SV_F32 && s->dtype != SV_BF16)
    return fail(SV_ERR_UNSUPPORTED, "%s: dtype %d not supported", what, s->dtype);
  if (s->max_blocks_per_seq > kMaxBlocksPerSeq)
    return fail(SV_ERR_UNSUPPORTED, "%s: max_blocks_per_seq %d > %d", what,
                s->max_blocks_per_seq, kMaxBlocksPerSeq);
  return SV_OK;
}

sv_status check_budget(const sv_budget* b, const char* what) {
  if (!b) return fail(SV_ERR_NULL_ARG, "%s: budget is NULL", what);
  if (b->dense_ctx_tokens < 0 || b->min_blocks < 0 || b->frac_per_mille < 0 ||
      b->frac_per_mille > 1000)
    return fail(SV_ERR_BAD_SHAPE, "%s: budget fields out of range", what);
  if ((b->keep_first != 0 && b->keep_first != 1) || (b->keep_last != 0 && b->keep_last != 1))
    return fail(SV_ERR_BAD_SHAPE, "%s: keep_first / keep_last must be 0 or 1", what);
  if (b->min_blocks < b->keep_first + b->keep_last)
    return fail(SV_ERR_BAD_SHAPE, "%s: min_blocks %d smaller than the forced blocks", what,
                b->min_blocks);
  return SV_OK;
}

sv_status check_kmax(const sv_shape* s, int32_t k_max, const char* what) {
  if (k_max <= 0 || k_max > s->max_blocks_per_seq)
    return fail(SV_ERR_BAD_SHAPE, "%s: k_max %d not in [1, max_blocks_per_seq=%d]", what, k_max,
                s->max_blocks_per_seq);
  return SV_OK;
}

// A selection keeps min(k, k_max) blocks, the forced ones among them, so k_max must
// hold the forced blocks.
sv_status check_select_kmax(const sv_budget* b, int32_t k_max, const char* what) {
  if (k_max < b->keep_first + b->keep_last)
    return fail(SV_ERR_BAD_SHAPE, "%s: k_max %d smaller than the forced blocks", what, k_max);
  return SV_OK;
}

// Split count. Library choice: a grid that is resident at once (256 workgroups when
// each needs a CU: 128 padded rows or fp32; else 384 of the 512 slots of two per CU,
// or all 512 for long streams), but no more splits than about one per four tiles, so
// the per-workgroup prologue and the merge stay small next to the stream.
int resolve_splits(const sv_shape* s, int32_t k_max, int32_t num_splits) {
  const int tt = sv::attn_tile_tokens(s->block_size, s->dtype == SV_BF16,
                                     s->num_draft * (s->num_q_heads / s->num_kv_heads));
  const int64_t ctx_tiles = static_cast<int64_t>(k_max) * (s->block_size / tt);
  int64_t want = num_splits;
  if (want <= 0) {
    const int64_t units = static_cast<int64_t>(s->num_seqs) * s->num_kv_heads;
    const int64_t rows = static_cast<int64_t>(s->num_draft) * (s->num_q_heads / s->num_kv_heads);
    // One workgroup per CU for the builds that take a CU alone (128 rows, fp32). The
    // others (64 KB ring, two fit a CU) get three workgroups for every two CUs, or two
    // per CU when each split would still stream 16 tiles or more. A workgroup keeps one
    // tile in flight, so long streams are bound by each workgroup's latency and gain
    // from more workgroups, while short ones are bound by the launch's fixed cost, where
    // more splits only add partials to write and merge.
    const bool one_per_cu = rows > 64 || s->dtype != SV_BF16;
    if (units <= 0) {
      want = 1;
    } else if (one_per_cu) {
      want = sv::kAttnCUs / units - 1;
    } else {
      want = sv::kAttnCUs * 3 / 2 / units - 1;
      if (want >= 1 && ctx_tiles >= 16 * want) {
        // keep a count that merged inside the launch (at most 31 context splits) there
        int64_t two = sv::kAttnCUs * 2 / units - 1;
        if (want < sv::kMaxInKernelParts && two >= sv::kMaxInKernelParts)
          two = sv::kMaxInKernelParts - 1;
        want = two;
      }
    }
    const int64_t by_tiles = (ctx_tiles + 3) / 4;
    if (want > by_tiles) want = by_tiles;
  }
  if (want > ctx_tiles) want = ctx_tiles;
  // A split may straddle one block boundary at each end: keep it within the
  // attention kernel's descriptor table.
  const int64_t min_splits = (k_max + sv::kAttnMaxBlocksPerSplit - 2) / (sv::kAttnMaxBlocksPerSplit - 1);
  if (want < min_splits) want = min_splits;
  if (want < 1) want = 1;
  return static_cast<int>(want);
}

size_t select_ws_layout(const sv_shape* s, size_t* scores_off) {
  const size_t units = static_cast<size_t>(s->num_seqs) * s->num_kv_heads;
  *scores_off = 0;
  return align_up(units * s->max_blocks_per_seq * sizeof(float));
}

// Compute units and wall-clock rate (kHz) of the current device, cached per device.
struct DeviceInfo {
  int cus;
  int wall_khz;
};

DeviceInfo device_info() {
  static std::atomic<int> cus_cache[64];
  static std::atomic<int> khz_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return DeviceInfo{sv::kAttnCUs, 100000};
  int n = cus_cache[dev].load(std::memory_order_relaxed);
  int khz = khz_cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = sv::kAttnCUs;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
      khz = 100000;   // the 100 MHz constant clock of CDNA GPUs
    khz_cache[dev].store(khz, std::memory_order_relaxed);
    cus_cache[dev].store(n, std::memory_order_relaxed);
  }
  return DeviceInfo{n, khz};
}

// Bytes of the merge lines at the start of an attention workspace (one per unit).
size_t merge_lines_bytes(const sv_shape* s) {
  const size_t units = static_cast<size_t>(s->num_seqs) * s->num_kv_heads;
  return align_up(units * sv::kTicketStride * sizeof(uint32_t));
}

// Region after the merge lines: [partial O][partial (m, l)] when there is more than one
// split, then (fused calls only) the block scores. Offsets are relative to its start.
struct RestLayout {
  size_t o_off, ml_off, scores_off, attn_end, fused_end;
};

RestLayout rest_layout(const sv_shape* s, int splits) {
  RestLayout r{};
  const size_t rows = static_cast<size_t>(s->num_draft) * (s->num_q_heads / s->num_kv_heads);
  const size_t units = static_cast<size_t>(s->num_seqs) * s->num_kv_heads;
  if (splits > 1) {
    const size_t parts = static_cast<size_t>(splits) + 1;   // + the draft-only split
    r.o_off = 0;
    r.ml_off = align_up(units * parts * rows * s->head_dim * sizeof(float));
    r.attn_end = r.ml_off + align_up(units * parts * rows * 2 * sizeof(float));
  }
  r.scores_off = r.attn_end;
  size_t sc_off;
  r.fused_end = r.scores_off + select_ws_layout(s, &sc_off);
  return r;
}

// Attention workspace: [merge lines: units x 256 B][partial O][partial (m, l)]; nothing
// with one split.
size_t attn_ws_bytes(const sv_shape* s, int splits) {
  return splits <= 1 ? 0 : merge_lines_bytes(s) + rest_layout(s, splits).attn_end;
}

// Workspace of sv_select_and_attend: [merge lines][partials][scores]. The merge lines are
// reserved even with one split, so the scores never land on them whatever split
// counts calls on one workspace use.
size_t fused_ws_bytes(const sv_shape* s, int splits) {
  return merge_lines_bytes(s) + rest_layout(s, splits).fused_end;
}

sv::SelectParams select_params(const sv_shape* shape, const sv_budget* budget, const void* q,
                               const float* repr_pool, const int32_t* block_table,
                               const int32_t* ctx_lens, int32_t k_max, int32_t* idx,
                               int32_t* cnt) {
  sv::SelectParams p{};
  p.q = q;
  p.repr_pool = repr_pool;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.idx = idx;
  p.cnt = cnt;
  p.B = shape->num_seqs;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.G = shape->num_q_heads / shape->num_kv_heads;
  p.D = shape->head_dim;
  p.T = shape->num_draft;
  p.bs = shape->block_size;
  p.NB = shape->max_blocks_per_seq;
  p.P = shape->num_phys_blocks;
  p.k_max = k_max;
  p.dense_ctx = budget->dense_ctx_tokens;
  p.min_blocks = budget->min_blocks;
  p.frac_per_mille = budget->frac_per_mille;
  p.keep_first = budget->keep_first;
  p.keep_last = budget->keep_last;
  p.xcd_group = sv::xcd_groupable(p.B * p.Hkv) ? 1 : 0;
  return p;
}

// Attention parameters; `lines` and `rest` are the merge lines and the region after
// them (both unused with one split).
sv::AttnParams attn_params(const sv_shape* shape, const void* q, const void* k_draft,
                           const void* v_draft, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* ctx_lens, int32_t k_max,
                           float scale, int splits, void* out, float* lse, void* lines,
                           void* rest) {
  const RestLayout rl = rest_layout(shape, splits);
  char* w = static_cast<char*>(rest);
  const bool parts = splits > 1;
  sv::AttnParams p{};
  p.q = q;
  p.k_draft = k_draft;
  p.v_draft = v_draft;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.out = out;
  p.lse = lse;
  p.part_o = parts ? reinterpret_cast<float*>(w + rl.o_off) : nullptr;
  p.part_ml = parts ? reinterpret_cast<float*>(w + rl.ml_off) : nullptr;
  p.B = shape->num_seqs;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.G = shape->num_q_heads / shape->num_kv_heads;
  p.D = shape->head_dim;
  p.T = shape->num_draft;
  p.bs = shape->block_size;
  p.NB = shape->max_blocks_per_seq;
  p.P = shape->num_phys_blocks;
  p.k_max = k_max;
  p.S = splits;
  p.R = shape->num_draft * p.G;
  p.xcd_group = sv::xcd_groupable(p.B * p.Hkv) ? 1 : 0;
  p.tickets = parts ? static_cast<uint32_t*>(lines) : nullptr;
  const DeviceInfo dev = device_info();
  p.merge = sv::attn_merge_mode(splits, p.B * p.Hkv, p.R, shape->dtype == SV_BF16, dev.cus);
  p.merge_wait_ticks = static_cast<uint32_t>(static_cast<int64_t>(dev.wall_khz) *
                                             sv::kMergeWaitUs / 1000);
  p.scale_log2 = scale * 1.44269504088896340736f;
  return p;
}

}  // namespace

namespace sv {

sv_status fail_status(sv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sv_status check_select_and_attend(const sv_shape* shape, const sv_budget* budget, const void* q,
                                  const float* repr_pool, const void* k_draft,
                                  const void* v_draft, const int32_t* draft_mask,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  int32_t k_max, float scale, int32_t num_splits, int32_t* idx,
                                  int32_t* cnt, void* out, float* lse, const char* what) {
  if (sv_status st = check_shape(shape, what)) return st;
  if (sv_status st = check_budget(budget, what)) return st;
  if (sv_status st = check_kmax(shape, k_max, what)) return st;
  if (sv_status st = check_select_kmax(budget, k_max, what)) return st;
  if (num_splits < 0) return fail(SV_ERR_BAD_SHAPE, "%s: num_splits < 0", what);
  if (!(scale > 0.0f) || scale == __builtin_inff())
    return fail(SV_ERR_BAD_SHAPE, "%s: scale must be finite and positive", what);
  if (shape->num_seqs == 0) return SV_OK;
  if (!q || !repr_pool || !k_draft || !v_draft || !k_pool || !v_pool || !block_table ||
      !ctx_lens || !idx || !cnt || !out)
    return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
  return check_alignment({{q, "q", 16}, {repr_pool, "repr_pool", 16}, {k_draft, "k_draft", 16},
                          {v_draft, "v_draft", 16}, {k_pool, "k_pool", 16},
                          {v_pool, "v_pool", 16}, {out, "out", 16}, {lse, "lse", 4},
                          {draft_mask, "draft_mask", 4}, {block_table, "block_table", 4},
                          {ctx_lens, "ctx_lens", 4}, {idx, "idx", 4}, {cnt, "cnt", 4}},
                         what);
}

int resolve_splits_checked(const sv_shape* shape, int32_t k_max, int32_t num_splits) {
  return resolve_splits(shape, k_max, num_splits);
}

size_t fused_rest_bytes(const sv_shape* shape, int splits) {
  return rest_layout(shape, splits).fused_end;
}

sv_status select_and_attend_into(const sv_shape* shape, const sv_budget* budget, const void* q,
                                 const float* repr_pool, const void* k_draft,
                                 const void* v_draft, const int32_t* draft_mask,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* ctx_lens,
                                 int32_t k_max, float scale, int splits, int32_t* idx,
                                 int32_t* cnt, void* out, float* lse, void* lines, void* rest,
                                 hipStream_t st, const char* what) {
  const bool bf16 = shape->dtype == SV_BF16;
  float* scores = reinterpret_cast<float*>(static_cast<char*>(rest) +
                                           rest_layout(shape, splits).scores_off);
  SelectParams sp = select_params(shape, budget, q, repr_pool, block_table, ctx_lens, k_max, idx,
                                  cnt);
  sp.scores = scores;
  sp.scores_requested = 0;
  AttnParams ap = attn_params(shape, q, k_draft, v_draft, k_pool, v_pool, block_table, ctx_lens,
                              k_max, scale, splits, out, lse, lines, rest);
  ap.idx = idx;
  ap.cnt = cnt;
  ap.draft_mask = draft_mask;
  hipError_t e = launch_score(sp, bf16, st);
  if (e != hipSuccess) return from_hip(e, what);
  if (shape->max_blocks_per_seq <= kWaveTopkMaxBlocks) {
    // Budget + top-k run inside the attention workgroups.
    ap.scores = scores;
    ap.idx_out = idx;
    ap.cnt_out = cnt;
    ap.dense_ctx = budget->dense_ctx_tokens;
    ap.min_blocks = budget->min_blocks;
    ap.frac_per_mille = budget->frac_per_mille;
    ap.keep_first = budget->keep_first;
    ap.keep_last = budget->keep_last;
  } else {
    e = launch_topk(sp, st);
    if (e != hipSuccess) return from_hip(e, what);
  }
  return from_hip(launch_attn(ap, bf16, st), what);
}

}  // namespace sv

extern "C" {

int32_t sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_str(int32_t status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL_ARG: return "SV_ERR_NULL_ARG";
    case SV_ERR_BAD_SHAPE: return "SV_ERR_BAD_SHAPE";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    default: return "SV_ERR_UNKNOWN";
  }
}

const char* sv_last_error(void) { return g_last_error.c_str(); }

int32_t sv_budget_blocks(const sv_budget* budget, int32_t ctx_len, int32_t block_size) {
  if (!budget || ctx_len < 0 || block_size <= 0) return -1;
  if (budget->dense_ctx_tokens < 0 || budget->min_blocks < 0 || budget->frac_per_mille < 0 ||
      budget->frac_per_mille > 1000 ||
      budget->min_blocks < (budget->keep_first != 0) + (budget->keep_last != 0))
    return -1;
  const int64_t nb = (static_cast<int64_t>(ctx_len) + block_size - 1) / block_size;
  if (ctx_len <= budget->dense_ctx_tokens) return static_cast<int32_t>(nb);
  int64_t k = (static_cast<int64_t>(budget->frac_per_mille) * nb + 999) / 1000;
  if (k < budget->min_blocks) k = budget->min_blocks;
  if (k > nb) k = nb;
  return static_cast<int32_t>(k);
}

sv_status sv_block_repr(const sv_shape* shape, const void* k_new, const void* v_new,
                        int32_t n_new_max, const int32_t* n_new, const int32_t* ctx_before,
                        const int32_t* ctx_after, const int32_t* block_table, void* k_pool,
                        void* v_pool, float* repr_pool, void* stream) {
  const char* what = "sv_block_repr";
  if (sv_status st = check_shape(shape, what)) return st;
  if (n_new_max < 0) return fail(SV_ERR_BAD_SHAPE, "%s: n_new_max < 0", what);
  if (n_new_max > 0 && shape->num_seqs > 0) {
    if (!k_new || !v_new || !n_new || !ctx_before || !block_table || !k_pool || !v_pool ||
        !repr_pool)
      return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
    if (sv_status st = check_alignment(
            {{k_new, "k_new", 16}, {v_new, "v_new", 16}, {k_pool, "k_pool", 16},
             {v_pool, "v_pool", 16}, {repr_pool, "repr_pool", 16}, {n_new, "n_new", 4},
             {ctx_before, "ctx_before", 4}, {ctx_after, "ctx_after", 4},
             {block_table, "block_table", 4}},
            what))
      return st;
  }
  if (n_new_max > static_cast<int64_t>(shape->max_blocks_per_seq) * shape->block_size)
    return fail(SV_ERR_BAD_SHAPE, "%s: n_new_max exceeds the sequence capacity", what);
  sv::ReprParams p{k_new, v_new, n_new, ctx_before, ctx_after, block_table, k_pool, v_pool,
                   repr_pool,
                   shape->num_seqs, shape->num_kv_heads, shape->head_dim, shape->block_size,
                   shape->max_blocks_per_seq, shape->num_phys_blocks, n_new_max};
  return from_hip(sv::launch_block_repr(p, shape->dtype == SV_BF16,
                                        static_cast<hipStream_t>(stream)),
                  what);
}

size_t sv_select_workspace_bytes(const sv_shape* shape, int32_t k_max) {
  (void)k_max;
  if (check_shape(shape, "sv_select_workspace_bytes") != SV_OK) return 0;
  size_t off;
  return select_ws_layout(shape, &off);
}

sv_status sv_select_blocks(const sv_shape* shape, const sv_budget* budget, const void* q,
                           const float* repr_pool, const int32_t* block_table,
                           const int32_t* ctx_lens, int32_t k_max, int32_t* idx, int32_t* cnt,
                           float* scores, void* ws, size_t ws_bytes, void* stream) {
  const char* what = "sv_select_blocks";
  if (sv_status st = check_shape(shape, what)) return st;
  if (sv_status st = check_budget(budget, what)) return st;
  if (sv_status st = check_kmax(shape, k_max, what)) return st;
  if (sv_status st = check_select_kmax(budget, k_max, what)) return st;
  if (shape->num_seqs == 0) return ok();
  if (!q || !repr_pool || !block_table || !ctx_lens || !idx || !cnt)
    return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
  if (sv_status st = check_alignment({{q, "q", 16}, {repr_pool, "repr_pool", 16},
                                      {ws, "ws", 16}, {scores, "scores", 4},
                                      {block_table, "block_table", 4},
                                      {ctx_lens, "ctx_lens", 4}, {idx, "idx", 4},
                                      {cnt, "cnt", 4}},
                                     what))
    return st;
  size_t scores_off;
  const size_t need = select_ws_layout(shape, &scores_off);
  if (!ws || ws_bytes < need)
    return fail(SV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  char* w = static_cast<char*>(ws);
  sv::SelectParams p = select_params(shape, budget, q, repr_pool, block_table, ctx_lens, k_max,
                                     idx, cnt);
  p.scores = scores ? scores : reinterpret_cast<float*>(w + scores_off);
  p.scores_requested = scores != nullptr;
  return from_hip(sv::launch_select(p, shape->dtype == SV_BF16, static_cast<hipStream_t>(stream)),
                  what);
}

int32_t sv_attn_num_splits(const sv_shape* shape, int32_t k_max, int32_t num_splits) {
  if (check_shape(shape, "sv_attn_num_splits") != SV_OK) return 0;
  if (check_kmax(shape, k_max, "sv_attn_num_splits") != SV_OK) return 0;
  return resolve_splits(shape, k_max, num_splits);
}

size_t sv_attn_workspace_bytes(const sv_shape* shape, int32_t k_max, int32_t num_splits) {
  if (check_shape(shape, "sv_attn_workspace_bytes") != SV_OK) return 0;
  if (check_kmax(shape, k_max, "sv_attn_workspace_bytes") != SV_OK) return 0;
  return attn_ws_bytes(shape, resolve_splits(shape, k_max, num_splits));
}

sv_status sv_attn_plan_query(const sv_shape* shape, int32_t k_max, int32_t num_splits,
                             sv_attn_plan* plan) {
  const char* what = "sv_attn_plan_query";
  if (sv_status st = check_shape(shape, what)) return st;
  if (sv_status st = check_kmax(shape, k_max, what)) return st;
  if (num_splits < 0) return fail(SV_ERR_BAD_SHAPE, "%s: num_splits < 0", what);
  if (!plan) return fail(SV_ERR_NULL_ARG, "%s: plan is NULL", what);
  const bool bf16 = shape->dtype == SV_BF16;
  const int rows = shape->num_draft * (shape->num_q_heads / shape->num_kv_heads);
  const int units = shape->num_seqs * shape->num_kv_heads;
  const int splits = resolve_splits(shape, k_max, num_splits);
  plan->num_splits = splits;
  plan->workgroups = (splits > 1 ? splits + 1 : 1) * units;
  plan->tile_tokens = sv::attn_tile_tokens(shape->block_size, bf16, rows);
  plan->padded_rows = plan->tile_tokens == 128 ? 128 : sv::attn_padded_rows(rows);
  plan->ring_kb = plan->tile_tokens == 128 ? 128 : sv::attn_ring_kb(splits, units, rows, bf16);
  switch (sv::attn_merge_mode(splits, units, rows, bf16, device_info().cus)) {
    case sv::kMergeNone: plan->merge_mode = SV_MERGE_NONE; break;
    case sv::kMergeWait: plan->merge_mode = SV_MERGE_IN_LAUNCH_WAIT; break;
    case sv::kMergeLast: plan->merge_mode = SV_MERGE_IN_LAUNCH_LAST; break;
    default: plan->merge_mode = SV_MERGE_KERNEL; break;
  }
  return ok();
}

sv_status sv_sparse_verify_attn(const sv_shape* shape, const void* q, const void* k_draft,
                                const void* v_draft, const int32_t* draft_mask,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* ctx_lens,
                                const int32_t* idx, const int32_t* cnt, int32_t k_max,
                                float scale, int32_t num_splits, void* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  const char* what = "sv_sparse_verify_attn";
  if (sv_status st = check_shape(shape, what)) return st;
  if (sv_status st = check_kmax(shape, k_max, what)) return st;
  if (num_splits < 0) return fail(SV_ERR_BAD_SHAPE, "%s: num_splits < 0", what);
  if (!(scale > 0.0f) || scale == __builtin_inff())
    return fail(SV_ERR_BAD_SHAPE, "%s: scale must be finite and positive", what);
  if (shape->num_seqs == 0) return ok();
  if (!q || !k_draft || !v_draft || !k_pool || !v_pool || !block_table || !ctx_lens || !idx ||
      !cnt || !out)
    return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
  if (sv_status st = check_alignment(
          {{q, "q", 16}, {k_draft, "k_draft", 16}, {v_draft, "v_draft", 16},
           {k_pool, "k_pool", 16}, {v_pool, "v_pool", 16}, {out, "out", 16}, {ws, "ws", 16},
           {lse, "lse", 4}, {block_table, "block_table", 4}, {ctx_lens, "ctx_lens", 4},
           {idx, "idx", 4}, {cnt, "cnt", 4}, {draft_mask, "draft_mask", 4}},
          what))
    return st;
  const int splits = resolve_splits(shape, k_max, num_splits);
  const size_t need = attn_ws_bytes(shape, splits);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  char* w = static_cast<char*>(ws);
  sv::AttnParams p = attn_params(shape, q, k_draft, v_draft, k_pool, v_pool, block_table,
                                 ctx_lens, k_max, scale, splits, out, lse, w,
                                 need ? w + merge_lines_bytes(shape) : nullptr);
  p.idx = idx;
  p.cnt = cnt;
  p.draft_mask = draft_mask;
  return from_hip(sv::launch_attn(p, shape->dtype == SV_BF16, static_cast<hipStream_t>(stream)),
                  what);
}

size_t sv_select_and_attend_workspace_bytes(const sv_shape* shape, int32_t k_max,
                                            int32_t num_splits) {
  if (check_shape(shape, "sv_select_and_attend_workspace_bytes") != SV_OK) return 0;
  if (check_kmax(shape, k_max, "sv_select_and_attend_workspace_bytes") != SV_OK) return 0;
  return fused_ws_bytes(shape, resolve_splits(shape, k_max, num_splits));
}

sv_status sv_select_and_attend(const sv_shape* shape, const sv_budget* budget, const void* q,
                               const float* repr_pool, const void* k_draft, const void* v_draft,
                               const int32_t* draft_mask, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               int32_t k_max, float scale, int32_t num_splits, int32_t* idx,
                               int32_t* cnt, void* out, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
  const char* what = "sv_select_and_attend";
  if (sv_status st = sv::check_select_and_attend(shape, budget, q, repr_pool, k_draft, v_draft,
                                                 draft_mask, k_pool, v_pool, block_table,
                                                 ctx_lens, k_max, scale, num_splits, idx, cnt,
                                                 out, lse, what))
    return st;
  if (shape->num_seqs == 0) return ok();
  const int splits = resolve_splits(shape, k_max, num_splits);
  const size_t need = fused_ws_bytes(shape, splits);
  if (!ws || ws_bytes < need)
    return fail(SV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (sv_status st = check_alignment({{ws, "ws", 16}}, what)) return st;
  char* w = static_cast<char*>(ws);
  return sv::select_and_attend_into(shape, budget, q, repr_pool, k_draft, v_draft, draft_mask,
                                    k_pool, v_pool, block_table, ctx_lens, k_max, scale, splits,
                                    idx, cnt, out, lse, w, w + merge_lines_bytes(shape),
                                    static_cast<hipStream_t>(stream), what);
}

}  // extern "C"

namespace {

sv_status check_ffn_shape(const sv_ffn_shape* s, const char* what) {
  if (!s) return fail(SV_ERR_NULL_ARG, "%s: shape is NULL", what);
  if (s->num_tokens < 0 || s->d_model <= 0 || s->d_ffn <= 0)
    return fail(SV_ERR_BAD_SHAPE, "%s: sizes must be positive (num_tokens >= 0)", what);
  if (s->dtype != SV_BF16)
    return fail(SV_ERR_UNSUPPORTED, "%s: dtype %d not supported (bf16 only)", what, s->dtype);
  if (s->num_tokens > 16)
    return fail(SV_ERR_UNSUPPORTED, "%s: num_tokens %d > 16", what, s->num_tokens);
  if (s->d_model % 512 != 0)
    return fail(SV_ERR_UNSUPPORTED, "%s: d_model %d not a multiple of 512", what, s->d_model);
  if (static_cast<int64_t>(s->d_ffn) * s->d_model * 2 >= (int64_t{1} << 31))
    return fail(SV_ERR_UNSUPPORTED, "%s: a %d x %d weight matrix is 2 GiB or more", what,
                s->d_ffn, s->d_model);
  const int64_t np = sv::ffn_padded_tokens(s->num_tokens);
  if (np * s->d_model * 2 > 128 * 1024)
    return fail(SV_ERR_UNSUPPORTED, "%s: %d padded tokens x d_model %d exceed the 128 KB LDS stage",
                what, static_cast<int>(np), s->d_model);
  return SV_OK;
}

struct FfnLayout {
  size_t mask_off, h_off, part_off, total;
};

FfnLayout ffn_layout(const sv_ffn_shape* s) {
  FfnLayout l{};
  const size_t f = static_cast<size_t>(s->d_ffn);
  const size_t np = static_cast<size_t>(sv::ffn_padded_tokens(s->num_tokens));
  l.mask_off = 0;
  l.h_off = align_up(f * sizeof(uint32_t));
  l.part_off = l.h_off + align_up(f * 16 * sizeof(float));
  l.total = l.part_off + align_up(static_cast<size_t>(sv::ffn_ranges(s->d_ffn, s->d_model)) * np *
                                  s->d_model * sizeof(float));
  return l;
}

}  // namespace

extern "C" {

size_t sv_sparse_ffn_workspace_bytes(const sv_ffn_shape* shape) {
  if (check_ffn_shape(shape, "sv_sparse_ffn_workspace_bytes") != SV_OK) return 0;
  return ffn_layout(shape).total;
}

sv_status sv_sparse_ffn(const sv_ffn_shape* shape, const void* x, const void* w_gate,
                        const void* w_up, const void* w_down_t, float tau, void* y,
                        uint32_t* keep_bits, void* ws, size_t ws_bytes, void* stream) {
  const char* what = "sv_sparse_ffn";
  if (sv_status st = check_ffn_shape(shape, what)) return st;
  if (!(tau >= 0.0f) || tau == __builtin_inff())
    return fail(SV_ERR_BAD_SHAPE, "%s: tau must be finite and >= 0", what);
  if (shape->num_tokens == 0) return ok();
  if (!x || !w_gate || !w_up || !w_down_t || !y)
    return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
  if (sv_status st = check_alignment({{x, "x", 16}, {w_gate, "w_gate", 16}, {w_up, "w_up", 16},
                                      {w_down_t, "w_down_t", 16}, {y, "y", 16}, {ws, "ws", 16},
                                      {keep_bits, "keep_bits", 4}},
                                     what))
    return st;
  const FfnLayout l = ffn_layout(shape);
  if (!ws || ws_bytes < l.total)
    return fail(SV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", what, l.total,
                ws ? ws_bytes : static_cast<size_t>(0));
  char* w = static_cast<char*>(ws);
  sv::FfnParams p{};
  p.x = x;
  p.w_gate = w_gate;
  p.w_up = w_up;
  p.w_down_t = w_down_t;
  p.y = y;
  p.mask = reinterpret_cast<uint32_t*>(w + l.mask_off);
  p.h = reinterpret_cast<float*>(w + l.h_off);
  p.part = reinterpret_cast<float*>(w + l.part_off);
  p.keep_out = keep_bits;
  p.tau = tau;
  p.N = shape->num_tokens;
  p.Dm = shape->d_model;
  p.F = shape->d_ffn;
  p.dn_range = sv::ffn_range(p.F, p.Dm);
  p.dn_ranges = sv::ffn_ranges(p.F, p.Dm);
  return from_hip(sv::launch_ffn(p, static_cast<hipStream_t>(stream)), what);
}

sv_status sv_reuse_indices(const sv_shape* shape, int32_t k_max, const int32_t* prev_idx,
                           const int32_t* prev_cnt, int32_t* idx, int32_t* cnt, void* stream) {
  const char* what = "sv_reuse_indices";
  if (sv_status st = check_shape(shape, what)) return st;
  if (sv_status st = check_kmax(shape, k_max, what)) return st;
  if (shape->num_seqs == 0) return ok();
  if (!prev_idx || !prev_cnt || !idx || !cnt)
    return fail(SV_ERR_NULL_ARG, "%s: a required pointer is NULL", what);
  if (sv_status st = check_alignment({{prev_idx, "prev_idx", 4}, {prev_cnt, "prev_cnt", 4},
                                      {idx, "idx", 4}, {cnt, "cnt", 4}},
                                     what))
    return st;
  const int64_t units = static_cast<int64_t>(shape->num_seqs) * shape->num_kv_heads;
  const int64_t n_idx = units * k_max;
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
  };
  if (overlap(prev_idx, n_idx * 4, idx, n_idx * 4) || overlap(prev_cnt, units * 4, cnt, units * 4))
    return fail(SV_ERR_BAD_SHAPE, "%s: source and destination overlap", what);
  sv::ReuseParams p{prev_idx, prev_cnt, idx, cnt, n_idx, units};
  return from_hip(sv::launch_reuse(p, static_cast<hipStream_t>(stream)), what);
}

}  // extern "C"
