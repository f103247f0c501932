// Token reordering: gather or scatter whole rows of a (B, H, N, D) bf16 tensor
// along the token axis by a permutation of [0, N).
//
// Used for the optional spatiotemporal token layouts (Official repository for
// AB-Attention, "Optional cube layout"; Attention Mechanisms (LightX2V), Sol-Attn
// on Wan2.1, "Tuning and implementation"): Q, K and V are reordered before the
// sparse attention so that 128-query and 64-key blocks cover compact video
// regions, and the output is restored afterwards. Pure data movement, bound by
// HBM bandwidth: every byte is read once and written once with 16-byte accesses,
// each row a contiguous 128- or 256-byte segment.
#include "common.h"

namespace sparge {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;

template <int D>
__global__ __launch_bounds__(kThreads) void permute_kernel(const uint16_t* __restrict__ x, Strides xs,
                                                           const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ out, Strides os,
                                                           int64_t H, int64_t N, int64_t n_row_blocks,
                                                           int inverse) {
  constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  constexpr int kRowsPerPass = kThreads / kChunks;  // rows one pass of the block covers
  const int64_t bh = blockIdx.x / n_row_blocks;
  const int64_t p0 = (blockIdx.x - bh * n_row_blocks) * kRowsPerBlock;
  const int64_t b = bh / H, h = bh - b * H;
  const uint16_t* xh = x + b * xs.b + h * xs.h;
  uint16_t* oh = out + b * os.b + h * os.h;
  const int c = threadIdx.x % kChunks;
#pragma unroll
  for (int pass = 0; pass < kRowsPerBlock / kRowsPerPass; ++pass) {
    const int64_t p = p0 + pass * kRowsPerPass + threadIdx.x / kChunks;
    if (p >= N) break;
    const int64_t target = perm[p];
    if (target < 0 || target >= N) continue;        // not a permutation entry: nothing moves
    const int64_t src = inverse ? p : target;
    const int64_t dst = inverse ? target : p;
    const uint4 v = *reinterpret_cast<const uint4*>(xh + src * xs.n + 8 * c);
    *reinterpret_cast<uint4*>(oh + dst * os.n + 8 * c) = v;
  }
}

}  // namespace

hipError_t launch_permute(const uint16_t* x, Strides xs, const int32_t* perm, uint16_t* out,
                          Strides os, int64_t B, int64_t H, int64_t N, int D, int inverse,
                          hipStream_t stream) {
  const int64_t n_row_blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  void* args[] = {(void*)&x, (void*)&xs, (void*)&perm, (void*)&out, (void*)&os,
                  (void*)&H, (void*)&N, (void*)&n_row_blocks, (void*)&inverse};
  const void* fn = D == 128 ? reinterpret_cast<const void*>(&permute_kernel<128>)
                            : reinterpret_cast<const void*>(&permute_kernel<64>);
  return hipLaunchKernel(fn, dim3(static_cast<uint32_t>(B * H * n_row_blocks)), dim3(kThreads), args, 0,
                         stream);
}

}  // namespace sparge
