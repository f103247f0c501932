// Mask compaction: mask_id rows (uint8, nonzero = kept) -> ascending kept-block lists.
//
// Turns a user block mask (SpargeAttention Documentation, block_sparse_sage2_attn_cuda
// and "Mask Requirements") into the per-query-block list the attention kernel
// walks, so that masked tiles are never loaded. One wavefront per mask row:
// 64 bytes per step, a ballot and a prefix count place each kept id.
#include "common.h"

namespace sparge {
namespace {

__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__global__ __launch_bounds__(256) void compact_kernel(const uint8_t* __restrict__ mask,
                                                      int64_t rows, int64_t n_kb,
                                                      int32_t* __restrict__ kv_idx,
                                                      int32_t* __restrict__ kv_cnt) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* m = mask + row * n_kb;
  int32_t* out = kv_idx + row * n_kb;
  int64_t base = 0;
  for (int64_t j0 = 0; j0 < n_kb; j0 += 64) {
    const int64_t j = j0 + lane;
    const bool sel = (j < n_kb) && m[j] != 0;
    const uint64_t b = __ballot(sel);
    if (sel) out[base + count_below(b)] = static_cast<int32_t>(j);
    base += __popcll(b);
  }
  if (lane == 0) kv_cnt[row] = static_cast<int32_t>(base);
}

// Mask value check ("Mask Requirements": entries are 0 or 1). Workgroup w
// writes bad[w] = 1 if any byte it scanned is neither 0 nor 1, else 0: every
// slot is written by exactly one workgroup, so no zeroing pass and no atomics.
__global__ __launch_bounds__(256) void check_mask_kernel(const uint8_t* __restrict__ mask, int64_t n,
                                                         int32_t* __restrict__ bad) {
  int found = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    found |= mask[i] > 1;
  found = __syncthreads_or(found);
  if (threadIdx.x == 0) bad[blockIdx.x] = found ? 1 : 0;
}

}  // namespace

hipError_t launch_check_mask(const uint8_t* mask, int64_t n, int32_t* bad, int n_wg, hipStream_t stream) {
  void* args[] = {(void*)&mask, (void*)&n, (void*)&bad};
  return hipLaunchKernel(reinterpret_cast<const void*>(&check_mask_kernel), dim3(static_cast<uint32_t>(n_wg)),
                         dim3(256), args, 0, stream);
}

hipError_t launch_compact(const uint8_t* mask, int64_t rows, int64_t n_kb, int32_t* kv_idx,
                          int32_t* kv_cnt, hipStream_t stream) {
  void* args[] = {(void*)&mask, (void*)&rows, (void*)&n_kb, (void*)&kv_idx, (void*)&kv_cnt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&compact_kernel),
                         dim3(static_cast<uint32_t>((rows + 3) / 4)), dim3(256), args, 0, stream);
}

}  // namespace sparge
