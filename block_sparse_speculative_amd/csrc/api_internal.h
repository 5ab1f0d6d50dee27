// Host-side pieces of the C ABI shared between its translation units (api.cpp and the
// static-scratch entry point). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv.h"

namespace sv {

// Records a failure message for sv_last_error() and returns `st`.
sv_status fail_status(sv_status st, const char* fmt, ...);

// Every host check of sv_select_and_attend except the workspace (shape, budget, k_max,
// num_splits, scale, pointers and their alignment). `what` names the entry point in the
// message.
sv_status check_select_and_attend(const sv_shape* shape, const sv_budget* budget, const void* q,
                                  const float* repr_pool, const void* k_draft,
                                  const void* v_draft, const int32_t* draft_mask,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  int32_t k_max, float scale, int32_t num_splits, int32_t* idx,
                                  int32_t* cnt, void* out, float* lse, const char* what);

// Split count the attention uses (sv_attn_num_splits without validation).
int resolve_splits_checked(const sv_shape* shape, int32_t k_max, int32_t num_splits);

// Bytes of the region after the merge lines that sv_select_and_attend needs
// (partials, then block scores).
size_t fused_rest_bytes(const sv_shape* shape, int splits);

// The launches of sv_select_and_attend, with its workspace given as the merge lines
// (one 256-byte line per (sequence, KV head) unit) and the region after them.
sv_status select_and_attend_into(const sv_shape* shape, const sv_budget* budget, const void* q,
                                 const float* repr_pool, const void* k_draft,
                                 const void* v_draft, const int32_t* draft_mask,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const int32_t* ctx_lens,
                                 int32_t k_max, float scale, int splits, int32_t* idx,
                                 int32_t* cnt, void* out, float* lse, void* lines, void* rest,
                                 hipStream_t stream, const char* what);

}  // namespace sv
