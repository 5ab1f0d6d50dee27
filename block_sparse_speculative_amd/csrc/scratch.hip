// sv_select_and_attend_static: sv_select_and_attend for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). Its workspace is a fixed array in device memory, `scratch`,
// defined below; each device the library runs on holds its own copy from module load
// until the process ends.
//
// Layout of `scratch`: merge lines for up to kScratchUnits (sequence, KV head) units
// (one 256-byte line each, at a fixed place), then the partials and block scores of
// the call. The array starts zeroed (static storage), and the in-launch merge leaves
// the lines consistent at the end of every launch (the arrival word of the next
// launch's epoch is cleared, the epoch advanced), whatever the unit and split counts
// of the calls; the lines never overlap the partials, so no call needs to clear them.
// Everything after the lines is written before it is read within a call.
//
// Every call on one device shares that device's array: calls that may overlap on one
// device (other streams, other threads) race and must not be issued.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "sv.h"

static constexpr size_t kScratchBytes = SV_STATIC_SCRATCH_BYTES;   // per device
static constexpr int kScratchUnits = SV_STATIC_SCRATCH_UNITS;      // merge lines reserved
static constexpr size_t kScratchLines = static_cast<size_t>(kScratchUnits) * 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of this device's `scratch`, looked up once per device with that
// device current (the host-side name of the array is not a device address).
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace

extern "C" {

sv_status sv_select_and_attend_static(const sv_shape* shape, const sv_budget* budget,
                                      const void* q, const float* repr_pool, const void* k_draft,
                                      const void* v_draft, const int32_t* draft_mask,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      int32_t k_max, float scale, int32_t num_splits,
                                      int32_t* idx, int32_t* cnt, void* out, float* lse,
                                      void* stream) {
  const char* what = "sv_select_and_attend_static";
  if (sv_status st = sv::check_select_and_attend(shape, budget, q, repr_pool, k_draft, v_draft,
                                                 draft_mask, k_pool, v_pool, block_table,
                                                 ctx_lens, k_max, scale, num_splits, idx, cnt,
                                                 out, lse, what))
    return st;
  if (shape->num_seqs == 0) return sv::fail_status(SV_OK, "");
  const int64_t units = static_cast<int64_t>(shape->num_seqs) * shape->num_kv_heads;
  if (units > kScratchUnits)
    return sv::fail_status(SV_ERR_WORKSPACE,
                           "%s: %lld (sequence, KV head) units exceed the static scratch's %d",
                           what, static_cast<long long>(units), kScratchUnits);
  const int splits = sv::resolve_splits_checked(shape, k_max, num_splits);
  const size_t need = sv::fused_rest_bytes(shape, splits);
  if (need > kScratchBytes - kScratchLines)
    return sv::fail_status(SV_ERR_WORKSPACE,
                           "%s: needs %zu bytes of scratch after the merge lines, the static "
                           "scratch has %zu (use sv_select_and_attend with a workspace)",
                           what, need, kScratchBytes - kScratchLines);
  void* base = nullptr;
  const hipError_t e = scratch_ptr(&base);
  if (e != hipSuccess || !base)
    return sv::fail_status(SV_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", what,
                           hipGetErrorString(e));
  char* w = static_cast<char*>(base);
  return sv::select_and_attend_into(shape, budget, q, repr_pool, k_draft, v_draft, draft_mask,
                                    k_pool, v_pool, block_table, ctx_lens, k_max, scale, splits,
                                    idx, cnt, out, lse, w, w + kScratchLines,
                                    static_cast<hipStream_t>(stream), what);
}

}  // extern "C"
