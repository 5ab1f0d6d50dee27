/*
 * sv.h -- C ABI of the block-sparse multi-draft verification-attention library
 * (libsv.so, MI355X / gfx950).
 *
 * The method (arXiv 2512.21911 as described on the tutorial page "Accelerate
 * Speculative Decoding with Sparse Computation in Verification", section "Core
 * technique 1", and on its sciencestack page, Figure 1 caption): during the
 * verification pass of speculative decoding, every KV block carries a
 * representative key; the first draft token's query scores the representatives;
 * a piecewise budget keeps the top-k blocks; every draft token then attends over
 * the shared selected blocks plus the draft tokens up to itself; a layer may reuse
 * the previous layer's selection.
 *
 * Conventions for every entry point
 *  - Buffer pointers are DEVICE pointers unless stated otherwise. The caller
 *    allocates and owns every buffer, including workspaces. The library never
 *    allocates or frees device memory, never synchronises, and keeps no pointer
 *    after returning.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *    enqueued asynchronously on it, in call order.
 *  - Every entry point returns an sv_status. Arguments visible to the host are
 *    validated BEFORE anything is enqueued: a nonzero status means nothing was
 *    launched. sv_last_error() then holds a message (thread-local).
 *  - Values that live on the device (context lengths, block-table entries,
 *    indices) are preconditions the host cannot check. Kernels skip entries outside
 *    their valid range instead of reading out of bounds; results for such inputs
 *    are unspecified.
 *  - Alignment: the kernels read and write data arrays with 16-byte vector
 *    accesses and direct-to-LDS loads. Every element-typed or float array of a
 *    head or model dimension (q, drafts, pools, repr_pool, x, weights, out, y) and
 *    every workspace must be 16-byte aligned; int32 arrays, lse, scores and
 *    keep_bits 4-byte aligned. A misaligned pointer returns SV_ERR_UNSUPPORTED
 *    naming it. (hipMalloc and torch allocations are 256-byte aligned.)
 *  - Tensor layouts are dense row-major with the shapes given below.
 *      B   = num_seqs           Hq = num_q_heads      Hkv = num_kv_heads
 *      G   = Hq / Hkv (GQA group; query head h uses KV head h / G)
 *      D   = head_dim             bs = block_size       T  = num_draft
 *      NB  = max_blocks_per_seq   P  = num_phys_blocks
 *  - Paged KV pool (one pool per layer):
 *      k_pool    [P, Hkv, bs, D]  element type `dtype` (token-major in a block)
 *      v_pool    [P, Hkv, bs, D]  element type `dtype` (token-major in a block)
 *      repr_pool [P, Hkv, D]      float32, mean key of each block
 *    block_table [B, NB] int32 maps logical block j of sequence b to a physical
 *    block; only entries j < ceil(ctx_b / bs) are read.
 *
 * Supported envelope (else SV_ERR_UNSUPPORTED): D in {64, 128}; bs in {32, 64, 128};
 * 1 <= T <= 16; T*G <= 128; dtype in {SV_F32, SV_BF16}; NB <= 16384.
 */
#ifndef SV_H_
#define SV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 3

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_NULL_ARG = 1,     /* a required pointer is NULL                         */
  SV_ERR_BAD_SHAPE = 2,    /* sizes inconsistent or out of range                  */
  SV_ERR_UNSUPPORTED = 3,  /* outside the supported envelope                      */
  SV_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required          */
  SV_ERR_HIP = 5           /* a HIP launch or runtime call failed                 */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Problem sizes shared by all entry points (see the size names above). */
typedef struct sv_shape {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t num_phys_blocks;
  int32_t num_draft;
  int32_t dtype;           /* sv_dtype */
} sv_shape;

/* Piecewise block budget (tutorial page, "Core technique 1": a large budget for
 * short contexts and aggressive sparsity for long ones). With nb = ceil(ctx/bs):
 *   k = nb                                                    if ctx <= dense_ctx_tokens
 *   k = min(nb, max(min_blocks, ceil(frac_per_mille * nb / 1000)))   otherwise.
 * keep_first / keep_last force block 0 and block nb-1 into every sparse
 * selection; forced blocks count inside k. Requires dense_ctx_tokens >= 0,
 * 0 <= frac_per_mille <= 1000 and min_blocks >= keep_first + keep_last. */
typedef struct sv_budget {
  int32_t dense_ctx_tokens;
  int32_t min_blocks;
  int32_t frac_per_mille;
  int32_t keep_first;
  int32_t keep_last;
} sv_budget;

/* Library ABI version (SV_ABI_VERSION of the build). */
int32_t sv_abi_version(void);

/* Static, human-readable name of a status code. */
const char* sv_status_str(int32_t status);

/* Message describing the last failure of an entry point on this thread ("" if
 * none). Valid until the next call into the library on this thread. */
const char* sv_last_error(void);

/* Host-only, pure: the block budget k for one sequence (formula in sv_budget).
 * Returns -1 if `budget` is NULL or invalid, or if ctx_len < 0 or block_size <= 0. */
int32_t sv_budget_blocks(const sv_budget* budget, int32_t ctx_len, int32_t block_size);

/* KV append fused with the block-representative update (representative value of a
 * block: sciencestack page, Figure 1 caption; the pages leave it undefined and this
 * library takes the arithmetic mean of the block's keys over its valid tokens). The
 * same call rewrites tokens already in the cache, as the refresh after a periodic
 * full verification does (SpecPV page, highlights and introduction: periodic full
 * verification keeps errors from accumulating).
 *
 * For each sequence b, the n_new[b] tokens k_new[b, 0:n_new[b]] / v_new[...] are
 * written at logical positions ctx_before[b] .. ctx_before[b]+n_new[b]-1 of the
 * pool through block_table. The sequence then holds end_b valid tokens: ctx_after[b]
 * when ctx_after is given (tokens past the rewritten ones stay valid), else
 * ctx_before[b]+n_new[b] (an append). For every block touched, repr_pool receives the
 * float32 mean of ALL its valid keys (old and new). The summation order depends only
 * on the block's valid-token count, so a block's representative does not depend on
 * how its tokens arrived.
 *   k_new, v_new  [B, n_new_max, Hkv, D]  dtype
 *   n_new         [B] int32, 0 <= n_new[b] <= n_new_max      (device)
 *   ctx_before    [B] int32, ctx_before[b]+n_new[b] <= NB*bs (device)
 *   ctx_after     [B] int32 or NULL, ctx_before[b]+n_new[b] <= ctx_after[b] <= NB*bs
 *                 (device; values outside that range are clamped into it)
 *   block_table   [B, NB] int32                              (device)
 *   k_pool, v_pool, repr_pool  pool tensors (layouts above), updated in place.
 * n_new_max may be 0 (nothing is launched). */
sv_status sv_block_repr(const sv_shape* shape, const void* k_new, const void* v_new,
                        int32_t n_new_max, const int32_t* n_new, const int32_t* ctx_before,
                        const int32_t* ctx_after, const int32_t* block_table, void* k_pool,
                        void* v_pool, float* repr_pool, void* stream);

/* Bytes of workspace sv_select_blocks needs for this shape. */
size_t sv_select_workspace_bytes(const sv_shape* shape, int32_t k_max);

/* Block selection: GQA-batched scoring + piecewise budget + top-k
 * (tutorial page, "Core technique 1"; sciencestack page, Figure 1 caption: the
 * first draft token's query against each block representative, one shared set).
 *
 * For sequence b and KV head g, with nb = ceil(ctx_lens[b]/bs):
 *   score[j] = sum over the G query heads h of g of  q[b,0,h,:] . repr_pool[bt[b,j], g, :]
 * computed in float32 (unscaled). k = min(budget(ctx_lens[b]), k_max). If k >= nb
 * every block is selected; otherwise the forced blocks plus the k - |forced| best
 * other blocks by score (ties to the lower index; NaN ranks lowest).
 *   q          [B, T, Hq, D] dtype; only draft token 0 is read
 *   idx        [B, Hkv, k_max] int32 out: ascending logical indices, padded with -1
 *   cnt        [B, Hkv]        int32 out: number of selected blocks (= min(k, nb))
 *   scores     [B, Hkv, NB]    float32 out, optional (NULL): the block scores
 * With k_max >= budget(ctx_lens[b]) for every sequence (sv_budget_blocks gives it)
 * the selection is the method's; a smaller k_max caps the budget as above (a
 * sequence whose budget keeps every block then also gets the best k_max by score).
 * k_max < keep_first + keep_last is rejected (SV_ERR_BAD_SHAPE). `ws` must hold
 * sv_select_workspace_bytes() bytes (scratch for the scores when `scores` is NULL);
 * its contents need no initialisation. Two kernels are enqueued (scoring, then
 * budget + top-k). */
sv_status sv_select_blocks(const sv_shape* shape, const sv_budget* budget, const void* q,
                           const float* repr_pool, const int32_t* block_table,
                           const int32_t* ctx_lens, int32_t k_max, int32_t* idx,
                           int32_t* cnt, float* scores, void* ws, size_t ws_bytes,
                           void* stream);

/* Number of KV splits sv_sparse_verify_attn uses: `num_splits` if > 0 (clamped to
 * the work available), else the library's choice for this shape. The k_max * (bs/TT)
 * tile slots of a (sequence, KV head) are cut into that many balanced ranges, where
 * TT = 128 tokens for bf16 blocks of 128 tokens when T*G > 64, else 64 for bf16
 * blocks of 64 or more tokens, else 32. With more than one
 * split, one extra workgroup per (sequence, KV head) handles the draft tokens. */
int32_t sv_attn_num_splits(const sv_shape* shape, int32_t k_max, int32_t num_splits);

/* Bytes of workspace sv_sparse_verify_attn needs (0 when one split is used). */
size_t sv_attn_workspace_bytes(const sv_shape* shape, int32_t k_max, int32_t num_splits);

/* How the partials of a split (sequence, KV head) unit are combined. */
typedef enum sv_merge_mode {
  SV_MERGE_NONE = 0,            /* one split: no partials                                */
  SV_MERGE_IN_LAUNCH_WAIT = 1,  /* in the attention launch: the unit's workgroups wait,
                                   bounded in time, for each other and merge a slice of
                                   rows each (a workgroup whose wait runs out hands its
                                   slice to the last one to arrive)                       */
  SV_MERGE_IN_LAUNCH_LAST = 2,  /* in the attention launch: the last workgroup of the unit
                                   to arrive merges every row (grids that cannot be
                                   resident at once)                                      */
  SV_MERGE_KERNEL = 3           /* a second kernel (more than 32 workgroups per unit)     */
} sv_merge_mode;

/* Launch plan of the attention for a shape (host-only; reads the current device's
 * compute-unit count, 256 if there is no device). */
typedef struct sv_attn_plan {
  int32_t num_splits;    /* context splits (sv_attn_num_splits)                        */
  int32_t workgroups;    /* workgroups of the attention launch                         */
  int32_t tile_tokens;   /* tokens per KV tile                                         */
  int32_t padded_rows;   /* rows (draft token x GQA head) of a unit, padded            */
  int32_t ring_kb;       /* LDS ring of one workgroup in KB                            */
  int32_t merge_mode;    /* sv_merge_mode                                              */
} sv_attn_plan;

/* Fills *plan for sv_sparse_verify_attn / sv_select_and_attend with these arguments.
 * Returns the same status as those calls would for a bad shape, k_max or num_splits;
 * SV_ERR_NULL_ARG when plan is NULL. */
sv_status sv_attn_plan_query(const sv_shape* shape, int32_t k_max, int32_t num_splits,
                             sv_attn_plan* plan);

/* Multi-draft attention over the shared selected blocks (sciencestack page,
 * Figure 1 caption: all draft tokens use the same selected block set; abstract:
 * draft tokens are verified in one parallel pass).
 *
 * Draft token t of query head h (KV head g = h / G) attends over every valid
 * context token of the blocks idx[b, g, 0:cnt[b,g]] and over the draft tokens it
 * sees: drafts 0..t (a chain) when draft_mask is NULL, else every draft u whose bit
 * draft_mask[b, t] >> u & 1 is set, and always t itself. A draft tree (SpecPV page,
 * introduction: the EAGLE-3 drafter emits a tree of candidate tokens) is given by
 * setting the bits of t's ancestors (tree attention):
 *   out[b,t,h,:] = softmax_k(scale * q[b,t,h,:] . key_k) @ value_k
 *   lse[b,t,h]   = natural log of the softmax denominator (of the scaled logits)
 * Accumulation is float32; `out` is rounded to dtype (round to nearest even).
 *   q                 [B, T, Hq, D]   dtype
 *   k_draft, v_draft  [B, T, Hkv, D]  dtype (the draft tokens' own keys/values)
 *   draft_mask        [B, T] int32 (device) or NULL: visibility bits among the drafts;
 *                     bits at or above T are ignored
 *   k_pool, v_pool, block_table      as above
 *   ctx_lens [B] int32; idx [B, Hkv, k_max]; cnt [B, Hkv]   (device)
 *   out [B, T, Hq, D] dtype; lse [B, T, Hq] float32 or NULL
 * num_splits: 0 = library choice, else the number of KV splits (see
 * sv_attn_num_splits). With more than one split the partial results go to `ws`
 * (sv_attn_workspace_bytes() bytes; may be NULL when that is 0). Its first B*Hkv*256
 * bytes (rounded up to 256) are merge lines, one per (sequence, KV head): a launch
 * epoch and two arrival words. Zero-fill the workspace at allocation, and again
 * before a call with more (sequence, KV head) units than any earlier call on it; in
 * between leave those bytes to the library (zero-filling all of them again is also
 * valid; changing only some of them is not). How the partials are merged is given by
 * sv_attn_plan_query (sv_merge_mode); no workgroup waits for another without a time
 * bound, so the result does not depend on other work running on the device.
 * Calls that may run concurrently must not share a workspace. scale must be finite
 * and > 0. */
sv_status sv_sparse_verify_attn(const sv_shape* shape, const void* q, const void* k_draft,
                                const void* v_draft, const int32_t* draft_mask,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* ctx_lens,
                                const int32_t* idx, const int32_t* cnt, int32_t k_max,
                                float scale, int32_t num_splits, void* out, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace sv_select_and_attend needs for this shape. */
size_t sv_select_and_attend_workspace_bytes(const sv_shape* shape, int32_t k_max,
                                            int32_t num_splits);

/* One selecting layer in one call: exactly sv_select_blocks followed by
 * sv_sparse_verify_attn with the same arguments (same indices, counts, outputs and
 * LSE), in fewer launches (tutorial page, "Core technique 1": representative
 * scoring and top-k feed the sparse attention; sciencestack page, Figure 1
 * caption: the first draft token's query picks the blocks that all drafts share).
 *
 * Launches: the scoring kernel, then the attention kernel, whose context workgroups
 * each run the budget + top-k of their unit from the scores (exact, lowest index
 * wins ties) before streaming their share of the selected blocks; split 0 of each
 * unit writes idx / cnt. With NB > 1024 the separate top-k kernel runs between the
 * two instead. The split partials are merged as sv_attn_plan_query reports.
 *   arguments        as in sv_select_blocks and sv_sparse_verify_attn
 *   idx, cnt         outputs (as sv_select_blocks writes them)
 *   ws               sv_select_and_attend_workspace_bytes() bytes: the attention
 *                    workspace (merge lines first, reserved even with one split:
 *                    zero-fill at allocation and before a call with more units than
 *                    any earlier one, else leave them to the library), then the score
 *                    scratch. Calls that may run concurrently must not share it. */
sv_status sv_select_and_attend(const sv_shape* shape, const sv_budget* budget, const void* q,
                               const float* repr_pool, const void* k_draft, const void* v_draft,
                               const int32_t* draft_mask, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               int32_t k_max, float scale, int32_t num_splits, int32_t* idx,
                               int32_t* cnt, void* out, float* lse, void* ws, size_t ws_bytes,
                               void* stream);

/* Size of the device array sv_select_and_attend_static works in (one per device), and
 * the most (sequence, KV head) units a call of it may have. */
#define SV_STATIC_SCRATCH_BYTES (32u << 20)
#define SV_STATIC_SCRATCH_UNITS 2048

/* sv_select_and_attend for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * results and launches as sv_select_and_attend, minus the workspace: the partials,
 * merge lines and block scores live in a fixed array of SV_STATIC_SCRATCH_BYTES in
 * device memory that the library holds on each device it runs on until the process
 * ends. The call allocates nothing. It returns SV_ERR_WORKSPACE (nothing launched) when
 * num_seqs * num_kv_heads exceeds SV_STATIC_SCRATCH_UNITS or the partials and scores of
 * the call do not fit (use sv_select_and_attend then). Every call on a device shares
 * that device's array, so calls that may overlap on one device (other streams or
 * threads) race and must not be issued; consecutive calls on one stream are fine. */
sv_status sv_select_and_attend_static(const sv_shape* shape, const sv_budget* budget,
                                      const void* q, const float* repr_pool, const void* k_draft,
                                      const void* v_draft, const int32_t* draft_mask,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      int32_t k_max, float scale, int32_t num_splits,
                                      int32_t* idx, int32_t* cnt, void* out, float* lse,
                                      void* stream);

/* Sizes of the sparse FFN of a verification pass (the draft tokens' rows). */
typedef struct sv_ffn_shape {
  int32_t num_tokens;   /* N: rows (draft tokens) */
  int32_t d_model;      /* Dm */
  int32_t d_ffn;        /* F: channels of the FFN */
  int32_t dtype;        /* sv_dtype; SV_BF16 only */
} sv_ffn_shape;

/* Bytes of workspace sv_sparse_ffn needs (0 for an invalid shape). */
size_t sv_sparse_ffn_workspace_bytes(const sv_ffn_shape* shape);

/* Threshold-pruned gated FFN of the verification pass (tutorial page, "Core technique
 * 2": channels whose intermediate activation is below a threshold tau are pruned at
 * inference time; sciencestack page, Figure 1 caption: the pruned channels are set by
 * the output of the activation function and the threshold). With a = SiLU(x W_gate^T):
 *   token t keeps channel c   iff  |a[t, c]| >= tau
 *   y[t] = sum over channels c kept by t of  a[t, c] * (x[t] . w_up[c]) * w_down_t[c]
 * tau = 0 keeps every channel (the dense SwiGLU FFN). Only the w_up and w_down_t rows of
 * channels some token keeps are read. Accumulation is float32; y is rounded to bf16.
 *   x         [N, Dm] bf16
 *   w_gate    [F, Dm] bf16 (row c = channel c's gate weights); w_up likewise
 *   w_down_t  [F, Dm] bf16 (row c = channel c's output weights: the down projection
 *             stored channel-major, so a pruned channel's row is skipped whole)
 *   y         [N, Dm] bf16 out
 *   keep_bits [F] uint32 out or NULL: bit t of keep_bits[c] = token t keeps channel c
 *   ws        sv_sparse_ffn_workspace_bytes() bytes (no initialisation needed)
 * Envelope (else SV_ERR_UNSUPPORTED): bf16; N <= 16; d_model a multiple of 512 with
 * (N <= 8 ? 8 : 16) * d_model * 2 <= 128 KiB; each weight matrix under 2 GiB
 * (d_ffn * d_model * 2 < 2^31: the kernels address rows with 32-bit byte offsets). tau
 * must be finite and >= 0. Three kernels are enqueued on `stream`; with num_tokens = 0
 * nothing is enqueued and keep_bits is left as it was. */
sv_status sv_sparse_ffn(const sv_ffn_shape* shape, const void* x, const void* w_gate,
                        const void* w_up, const void* w_down_t, float tau, void* y,
                        uint32_t* keep_bits, void* ws, size_t ws_bytes, void* stream);

/* Inter-layer retrieval reuse (tutorial page, "Core technique 1": some layers take
 * the previous layer's retrieval result instead of selecting again; sciencestack
 * abstract: inter-layer retrieval reuse). Copies prev_idx [B, Hkv, k_max] and
 * prev_cnt [B, Hkv] into idx / cnt. Source and destination must not overlap
 * (SV_ERR_BAD_SHAPE otherwise). */
sv_status sv_reuse_indices(const sv_shape* shape, int32_t k_max, const int32_t* prev_idx,
                           const int32_t* prev_cnt, int32_t* idx, int32_t* cnt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_H_ */
