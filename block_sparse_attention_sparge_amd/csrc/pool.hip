// Block-mean pooling: x (B, H, N, D) bf16 -> out (B, H, ceil(N/R), D) fp32, R = 128 or 64.
//
// First step of mask prediction: each block of R consecutive tokens is
// replaced by its mean (SpargeAttention Documentation, "Mask Requirements":
// 128-row query blocks and 64-row key blocks). A ragged last block is divided
// by the rows it really has.
//
// HBM-bound: every input byte is read once with 16-byte loads (a wavefront
// reads whole 256-byte rows), partial sums stay in registers, and one LDS
// reduction per block folds the row groups together.
#include "common.h"

namespace sparge {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int D, int R>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ x, int64_t H,
                                                   int64_t N, Strides s, int64_t nb,
                                                   float* __restrict__ out) {
  constexpr int kThreadsPerRow = D / 8;            // one 16-byte chunk per thread
  constexpr int kRowsPerPass = 256 / kThreadsPerRow;
  constexpr int kPasses = R / kRowsPerPass;
  static_assert(kPasses >= 1 && R % kRowsPerPass == 0, "block must be a whole number of passes");

  const int64_t w = blockIdx.x;
  const int64_t bh = w / nb;
  const int64_t blk = w - bh * nb;
  const int64_t b = bh / H, h = bh - (bh / H) * H;
  const int t = threadIdx.x;
  const int c8 = t % kThreadsPerRow;
  const int r0 = t / kThreadsPerRow;
  const int64_t lo = blk * R;
  const int64_t hi = (lo + R < N) ? lo + R : N;
  const uint16_t* base = x + b * s.b + h * s.h + c8 * 8;

  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  uint4 chunk[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t r = lo + r0 + p * kRowsPerPass;
    chunk[p] = (r < hi) ? *reinterpret_cast<const uint4*>(base + r * s.n) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    acc[0] += bf16_lo(chunk[p].x);
    acc[1] += bf16_hi(chunk[p].x);
    acc[2] += bf16_lo(chunk[p].y);
    acc[3] += bf16_hi(chunk[p].y);
    acc[4] += bf16_lo(chunk[p].z);
    acc[5] += bf16_hi(chunk[p].z);
    acc[6] += bf16_lo(chunk[p].w);
    acc[7] += bf16_hi(chunk[p].w);
  }

  __shared__ float part[kRowsPerPass][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) part[r0][c8 * 8 + j] = acc[j];
  __syncthreads();
  if (t < D) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < kRowsPerPass; ++r) sum += part[r][t];
    out[w * D + t] = sum / static_cast<float>(hi - lo);
  }
}

template <int D, int R>
hipError_t launch_pool_t(const uint16_t* x, int64_t B, int64_t H, int64_t N, Strides s,
                         float* out, hipStream_t stream) {
  const int64_t nb = (N + R - 1) / R;
  const int64_t grid = B * H * nb;
  void* args[] = {(void*)&x, (void*)&H, (void*)&N, (void*)&s, (void*)&nb, (void*)&out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&pool_kernel<D, R>), dim3((uint32_t)grid),
                         dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_pool(const uint16_t* x, int64_t B, int64_t H, int64_t N, int D, Strides s,
                       int block_rows, float* out, hipStream_t stream) {
  if (D == 128)
    return block_rows == 128 ? launch_pool_t<128, 128>(x, B, H, N, s, out, stream)
                             : launch_pool_t<128, 64>(x, B, H, N, s, out, stream);
  return block_rows == 128 ? launch_pool_t<64, 128>(x, B, H, N, s, out, stream)
                           : launch_pool_t<64, 64>(x, B, H, N, s, out, stream);
}

}  // namespace sparge
