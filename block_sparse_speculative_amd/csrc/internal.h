// Internal declarations shared by the libsv translation units (host launchers and
// device helpers). Not part of the public ABI; see include/sv.h for that.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- launch parameters

struct ReprParams {
  const void* k_new;
  const void* v_new;
  const int32_t* n_new;
  const int32_t* ctx_before;
  const int32_t* ctx_after;   // valid tokens after the call, or null (= ctx_before + n_new)
  const int32_t* block_table;
  void* k_pool;
  void* v_pool;
  float* repr_pool;
  int32_t B, Hkv, D, bs, NB, P, n_new_max;
};

struct SelectParams {
  const void* q;
  const float* repr_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int32_t* idx;
  int32_t* cnt;
  float* scores;        // [B, Hkv, NB] (user buffer or workspace)
  int32_t xcd_group;    // nonzero: the workgroups of unit u have linear ids = u mod 8
  int32_t scores_requested;   // nonzero: write scores even where every block is kept
  int32_t B, Hq, Hkv, G, D, T, bs, NB, P, k_max;
  int32_t dense_ctx, min_blocks, frac_per_mille, keep_first, keep_last;
};

struct AttnParams {
  const void* q;
  const void* k_draft;
  const void* v_draft;
  const int32_t* draft_mask;   // [B][T] visibility bits among the drafts, or null (chain)
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* idx;   // selected blocks [units, k_max] (read unless `scores` is set)
  const int32_t* cnt;   // selected counts [units]
  const float* scores;  // fused select mode: block scores [units, NB], else null
  int32_t* idx_out;     // fused select mode: indices / counts written by split 0
  int32_t* cnt_out;
  void* out;
  float* lse;
  float* part_o;        // [units, S+1, R, D] unnormalised partial outputs
  float* part_ml;       // [units, S+1, R, 2]  (running max in log2 units, denominator)
  uint32_t* tickets;    // [units][kTicketStride] merge words (one 256-byte line per unit)
  int32_t merge;        // kMerge* mode
  uint32_t merge_wait_ticks;   // kMergeWait: wall-clock ticks a workgroup waits for its siblings
  int32_t xcd_group;    // nonzero: the workgroups of unit u have linear ids = u mod 8
  int32_t B, Hq, Hkv, G, D, T, bs, NB, P, k_max;
  int32_t S;            // context splits (a draft-only split is added when S > 1)
  int32_t R;
  float scale_log2;     // softmax scale * log2(e), > 0
  int32_t dense_ctx, min_blocks, frac_per_mille, keep_first, keep_last;   // fused select
};

struct ReuseParams {
  const int32_t* prev_idx;
  const int32_t* prev_cnt;
  int32_t* idx;
  int32_t* cnt;
  int64_t n_idx;
  int64_t n_cnt;
};

struct FfnParams {
  const void* x;          // [N, Dm] bf16
  const void* w_gate;     // [F, Dm] bf16
  const void* w_up;       // [F, Dm] bf16
  const void* w_down_t;   // [F, Dm] bf16 (down projection, channel-major)
  void* y;                // [N, Dm] bf16
  float* h;               // [F, 16] fp32: a * u of kept (channel, token), else 0
  uint32_t* mask;         // [F] bit t: token t keeps the channel
  uint32_t* keep_out;     // [F] copy of mask for the caller, or null
  float* part;            // [dn_ranges, NP, Dm] fp32 partial outputs of the down projection
  float tau;
  int32_t N, Dm, F;
  int32_t dn_range;       // channels per down-projection range (ffn_range)
  int32_t dn_ranges;      // ranges (ffn_ranges)
};

// ---------------------------------------------------------------- host launchers
// Each returns hipSuccess or the launch error; shapes are validated by the caller.

hipError_t launch_block_repr(const ReprParams& p, bool bf16, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, bool bf16, hipStream_t stream);   // score + top-k
hipError_t launch_score(const SelectParams& p, bool bf16, hipStream_t stream);
hipError_t launch_topk(const SelectParams& p, hipStream_t stream);
hipError_t launch_attn(const AttnParams& p, bool bf16, hipStream_t stream);
hipError_t launch_reuse(const ReuseParams& p, hipStream_t stream);
hipError_t launch_ffn(const FfnParams& p, hipStream_t stream);
int ffn_padded_tokens(int n);   // 8 or 16: token rows the FFN kernels are compiled for
int ffn_range(int f, int dm);   // channels per down-projection range
int ffn_ranges(int f, int dm);  // down-projection ranges

// How the split partials of a unit are combined.
enum : int32_t {
  kMergeNone = 0,       // one split: the workgroup writes the output
  kMergeWait = 1,       // in the launch: each workgroup waits (bounded) for its siblings and
                        // merges its slice of rows; one that gives up hands its slice to the
                        // last workgroup of the unit to arrive
  kMergeLast = 2,       // in the launch: the last workgroup of a unit to arrive merges every
                        // row; the others leave as soon as their partials are stored
  kMergeKernel = 3,     // a separate merge_kernel launch
};
// Merge mode for a launch (cus = compute units of the device): kMergeWait when the whole
// grid can be resident at once, kMergeLast when it cannot, kMergeKernel when a unit has
// more workgroups than the arrival word tracks.
int attn_merge_mode(int splits, int units, int rows, bool bf16, int cus);

// Tokens per attention tile (a tile never spans two blocks): for bf16, 128 when the
// blocks hold 128 tokens and a unit has more than 64 rows (fewer tile barriers for the
// compute-heavy 128-row units), else 64 for blocks of 64 or more tokens; 32 otherwise.
inline int attn_tile_tokens(int block_size, bool bf16, int rows) {
  if (bf16 && block_size >= 128 && rows > 64) return 128;
  return (bf16 && block_size >= 64) ? 64 : 32;
}

constexpr int kAttnCUs = 256;        // compute units of the MI355X
constexpr int kTicketStride = 64;    // uint32 per unit's merge line: one 256-byte line each
// In-launch merge words of a unit's line: the launch epoch (uint32 word 0) and two 64-bit
// arrival words (uint32 words 2-3 and 4-5), used by launches of even and odd epoch. An
// arrival word holds the number of workgroups that have stored their partial (low 32
// bits) and the slices handed to the last arriver (high 32 bits, bit s = split s), so a
// unit has at most kMaxInKernelParts workgroups.
constexpr int kEpochWord = 0;
constexpr int kArriveWord0 = 2;
constexpr int kMaxInKernelParts = 32;
constexpr int kMergeWaitUs = 50;     // longest wait of a workgroup for its siblings
constexpr int kXcds = 8;             // XCDs; workgroups are dispatched round-robin over them

// Whether the per-unit kernels can place each unit on one XCD.
inline bool xcd_groupable(int units) { return units % kXcds == 0; }

// LDS ring of one attention workgroup in KB: 128 when a workgroup has its CU to
// itself (the grid has at most one per CU, 128 padded rows = 8 waves, or fp32,
// whose registers allow one), else 64 so that two workgroups share a CU.
inline int attn_ring_kb(int splits, int units, int rows, bool bf16) {
  const int64_t wgs = static_cast<int64_t>(splits > 1 ? splits + 1 : 1) * units;
  return (!bf16 || wgs <= kAttnCUs || rows > 64) ? 128 : 64;
}

// Padded row count of the (draft token x GQA head) tile.
inline int attn_padded_rows(int rows) {
  return rows <= 16 ? 16 : rows <= 32 ? 32 : rows <= 64 ? 64 : 128;
}

constexpr int kSelectChunk = 128;     // blocks scored by one select workgroup (at most)
// Longest block-table row whose top-k one workgroup does with its keys in registers
// (the fused select-and-attend mode needs it; longer rows take the separate LDS
// top-k kernel).
constexpr int kWaveTopkMaxBlocks = 1024;
// Most selected blocks one attention split stages descriptors for (the split count
// is raised so that no split covers more).
constexpr int kAttnMaxBlocksPerSplit = 1024;
constexpr int kSelectThreads = 256;

}  // namespace sv
