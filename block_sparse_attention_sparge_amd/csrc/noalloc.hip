// sparge_attn_topk_noalloc: the top-k call with its workspace in a fixed
// device array instead of a caller-supplied buffer, for callers that cannot
// allocate (code under graph capture, serving loops, harnesses that forbid it).
//
// `scratch` below is a file-scope device array. In host code its name is only
// a host-side stand-in, not a device address: the device address of each
// GPU's copy is obtained once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr, and only that pointer is ever handed to kernels.
#include <mutex>

#include "../../include/sparge.h"
#include "common.h"

namespace {

static __device__ __align__(256) char scratch[SPARGE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (resolved on the
// first call on that device). Returns nullptr if it cannot be resolved.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int sparge_attn_topk_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, double topk,
                                        uint16_t* out, int64_t B, int64_t H, int64_t N, int64_t D,
                                        const int64_t q_strides[3], const int64_t k_strides[3],
                                        const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                                        int is_causal, uint8_t* mask_out, void* stream) {
  // Every argument is checked on the host before any HIP call: the regular
  // call without a workspace runs all of its checks that precede the workspace
  // one and launches nothing, so any answer but SPARGE_ERR_WORKSPACE is final.
  const int rc = sparge_attn_topk(q, k, v, topk, out, B, H, N, D, q_strides, k_strides, v_strides,
                                  o_strides, scale, is_causal, mask_out, nullptr, 0, stream);
  if (rc != SPARGE_ERR_WORKSPACE) return rc;
  if (sparge_workspace_bytes(B, H, N, D, topk) > static_cast<size_t>(SPARGE_NOALLOC_SCRATCH_BYTES))
    return SPARGE_ERR_SCRATCH_LIMIT;
  void* ws = scratch_for_current_device();
  if (!ws) return SPARGE_ERR_LAUNCH;
  // every workspace byte the kernels read (pooled means, lists, counts) is
  // written earlier in the same call, so the array needs no clearing
  return sparge_attn_topk(q, k, v, topk, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides, scale,
                          is_causal, mask_out, ws, static_cast<size_t>(SPARGE_NOALLOC_SCRATCH_BYTES), stream);
}
