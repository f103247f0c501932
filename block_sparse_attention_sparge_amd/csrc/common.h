// Internal declarations shared by the host API and the gfx950 kernels of libsparge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparge {

constexpr int kQBlock = 128;   // query rows per block
constexpr int kKBlock = 64;    // key rows per block
constexpr int kNumXcd = 8;     // MI355X: 8 accelerator complex dies, each with its own L2

// Shape of one (B, H, N, D) bf16 operand: element strides of the B, H, N axes.
struct Strides {
  int64_t b, h, n;
};

// Launchers. Each validates nothing (the C API has done it) and returns the
// launch status of its kernel(s).
hipError_t launch_pool(const uint16_t* x, int64_t B, int64_t H, int64_t N, int D, Strides s,
                       int block_rows, float* out, hipStream_t stream);

// k: the count of a row with all N_KB candidates (also the row stride of kv_idx).
// causal: row i ranks key blocks 0 .. (last row of block i) / 64 only and keeps
// the topk count of those (same rounding rule as the host's).
hipError_t launch_predict(const float* qbar, const float* kbar, int64_t BH, int64_t N, int D,
                          int64_t k, double topk, int causal, float scale, uint8_t* mask,
                          int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream);

// CDF-threshold selection: each row keeps its blocks in decreasing softmax
// probability until the running sum reaches tau (tau >= 1: every candidate);
// kv_idx rows are N_KB long, kv_cnt receives each row's count.
hipError_t launch_predict_cdf(const float* qbar, const float* kbar, int64_t BH, int64_t N, int D,
                              double tau, int causal, float scale, uint8_t* mask, int32_t* kv_idx,
                              int32_t* kv_cnt, hipStream_t stream);

hipError_t launch_compact(const uint8_t* mask, int64_t rows, int64_t n_kb, int32_t* kv_idx,
                          int32_t* kv_cnt, hipStream_t stream);

// bad[w] (w < n_wg) = 1 if workgroup w saw a mask byte other than 0 or 1, else 0.
constexpr int kCheckMaskWorkgroups = 1024;
hipError_t launch_check_mask(const uint8_t* mask, int64_t n, int32_t* bad, int n_wg, hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const int32_t* kv_idx;   // nullptr: dense
  const int32_t* kv_cnt;
  int64_t ld_idx;
  int64_t B, H, N;
  int D;
  Strides qs, ks, vs, os;
  float scale;
  int causal;              // 1: row r sees keys c <= r only
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// Gather (inverse = 0: out row p = x row perm[p]) or scatter (inverse = 1:
// out row perm[p] = x row p) of whole token rows; entries outside [0, N) move nothing.
hipError_t launch_permute(const uint16_t* x, Strides xs, const int32_t* perm, uint16_t* out,
                          Strides os, int64_t B, int64_t H, int64_t N, int D, int inverse,
                          hipStream_t stream);

}  // namespace sparge
