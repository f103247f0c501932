// C ABI of libsparge: argument validation, workspace carving and kernel dispatch.
//
// Every entry point validates all of its arguments on the host before making
// any HIP call, so rejected calls have no side effect and the error paths can
// be exercised without a GPU. See include/sparge.h for the contract.
#include "../../include/sparge.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <utility>
#include <vector>

#include "common.h"

using sparge::Strides;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;   // guards the size arithmetic below against overflow
constexpr size_t kAlign = 256;
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // elements between consecutive tokens
// the attention kernel computes key positions (block * 64 + 64) and query rows in 32 bits
constexpr int64_t kMaxAttnN = (int64_t(1) << 31) - 128;

bool valid_d(int64_t D) { return D == 64 || D == 128; }

int check_shape(int64_t B, int64_t H, int64_t N, int64_t D) {
  if (B < 1 || H < 1 || N < 1 || !valid_d(D)) return SPARGE_ERR_SHAPE;
  if (B > kMaxDim || H > kMaxDim || N > kMaxDim) return SPARGE_ERR_SHAPE;
  // grid sizes are 32-bit: B*H*ceil(N/64) key blocks must stay below 2^31
  const int64_t bh = B * H;
  if (bh > (int64_t(1) << 31) || bh * ((N + 63) / 64) >= (int64_t(1) << 31)) return SPARGE_ERR_SHAPE;
  return SPARGE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides of a bf16 operand: non-negative multiples of 8 elements.
int check_strides(const int64_t* s) {
  if (!s) return SPARGE_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] & 7) != 0 || s[i] > (int64_t(1) << 50)) return SPARGE_ERR_STRIDE;
  return SPARGE_OK;
}

// An output layout must not map two elements to the same address: sorted by
// stride, each axis must step past everything the smaller axes span.
bool non_overlapping(int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* s) {
  struct Ax { int64_t size, stride; };
  Ax ax[4] = {{B, s[0]}, {H, s[1]}, {N, s[2]}, {D, 1}};
  std::sort(ax, ax + 4, [](const Ax& a, const Ax& b) { return a.stride < b.stride; });
  int64_t span = 0;   // largest offset reachable with the smaller axes
  for (const Ax& a : ax) {
    if (a.size == 1) continue;
    if (a.stride <= span) return false;
    span += (a.size - 1) * a.stride;
  }
  return true;
}

// Byte range [lo, hi) touched by a (B, H, N, D) bf16 operand.
struct Range { uintptr_t lo, hi; };
Range range_bf16(const void* p, int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* s) {
  const int64_t last = (B - 1) * s[0] + (H - 1) * s[1] + (N - 1) * s[2] + (D - 1);
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(last + 1) * 2u};
}
Range range_bytes(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int topk_count(int64_t n_kb, double topk, int64_t* k) {
  if (!(topk > 0.0 && topk <= 1.0)) return SPARGE_ERR_TOPK;   // also rejects NaN
  const double x = topk * static_cast<double>(n_kb);
  const double r = std::nearbyint(x);
  int64_t kk = (std::fabs(x - r) <= 1e-9) ? static_cast<int64_t>(r) : static_cast<int64_t>(std::ceil(x));
  kk = std::max<int64_t>(1, std::min<int64_t>(n_kb, kk));
  *k = kk;
  return SPARGE_OK;
}

int64_t n_qblocks(int64_t N) { return (N + SPARGE_Q_BLOCK - 1) / SPARGE_Q_BLOCK; }
int64_t n_kblocks(int64_t N) { return (N + SPARGE_K_BLOCK - 1) / SPARGE_K_BLOCK; }
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layouts.
struct TopkWs {
  size_t qbar, kbar, idx, cnt, total;
};
TopkWs topk_layout(int64_t B, int64_t H, int64_t N, int64_t D, int64_t k) {
  TopkWs w;
  const size_t bh = static_cast<size_t>(B * H);
  w.qbar = 0;
  w.kbar = w.qbar + round_up(bh * n_qblocks(N) * D * sizeof(float));
  w.idx = w.kbar + round_up(bh * n_kblocks(N) * D * sizeof(float));
  w.cnt = w.idx + round_up(bh * n_qblocks(N) * k * sizeof(int32_t));
  w.total = w.cnt + round_up(bh * n_qblocks(N) * sizeof(int32_t));
  return w;
}
struct MaskWs {
  size_t idx, cnt, total;
};
MaskWs mask_layout(int64_t B, int64_t H, int64_t N) {
  MaskWs w;
  const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
  w.idx = 0;
  w.cnt = round_up(rows * n_kblocks(N) * sizeof(int32_t));
  w.total = w.cnt + round_up(rows * sizeof(int32_t));
  return w;
}

// Checks shared by every attention entry point.
int check_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int64_t B,
               int64_t H, int64_t N, int64_t D, const int64_t* qs, const int64_t* ks,
               const int64_t* vs, const int64_t* os) {
  if (!q || !k || !v || !out) return SPARGE_ERR_NULL;
  if (int rc = check_shape(B, H, N, D)) return rc;
  if (N > kMaxAttnN) return SPARGE_ERR_SHAPE;
  for (const int64_t* s : {qs, ks, vs, os})
    if (int rc = check_strides(s)) return rc;
  // the attention kernel addresses the rows of one 64-key tile with 32-bit byte offsets
  for (const int64_t* s : {qs, ks, vs})
    if (s[2] > kMaxRowStride) return SPARGE_ERR_STRIDE;
  // K and V tiles are read as 64 whole rows bounded by 64 token strides, so
  // their rows must not overlap (a token stride of at least D)
  if (ks[2] < D || vs[2] < D) return SPARGE_ERR_STRIDE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SPARGE_ERR_STRIDE;
  if (!non_overlapping(B, H, N, D, os)) return SPARGE_ERR_STRIDE;
  const Range ro = range_bf16(out, B, H, N, D, os);
  if (overlap(ro, range_bf16(q, B, H, N, D, qs)) || overlap(ro, range_bf16(k, B, H, N, D, ks)) ||
      overlap(ro, range_bf16(v, B, H, N, D, vs)))
    return SPARGE_ERR_ALIAS;
  return SPARGE_OK;
}

float resolve_scale(float scale, int64_t D) {
  return (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(static_cast<float>(D));
}

int status_of(hipError_t e) { return e == hipSuccess ? SPARGE_OK : SPARGE_ERR_LAUNCH; }

sparge::AttnArgs attn_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                           int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* qs,
                           const int64_t* ks, const int64_t* vs, const int64_t* os, float scale) {
  sparge::AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = out;
  a.kv_idx = nullptr; a.kv_cnt = nullptr; a.ld_idx = 0;
  a.B = B; a.H = H; a.N = N; a.D = static_cast<int>(D);
  a.qs = Strides{qs[0], qs[1], qs[2]};
  a.ks = Strides{ks[0], ks[1], ks[2]};
  a.vs = Strides{vs[0], vs[1], vs[2]};
  a.os = Strides{os[0], os[1], os[2]};
  a.scale = resolve_scale(scale, D);
  a.causal = 0;
  return a;
}

}  // namespace

extern "C" {

const char* sparge_status_string(int status) {
  switch (status) {
    case SPARGE_OK: return "ok";
    case SPARGE_ERR_NULL: return "a required pointer is NULL";
    case SPARGE_ERR_SHAPE: return "invalid shape (B, H, N >= 1; D in {64, 128}; size limits)";
    case SPARGE_ERR_TOPK: return "topk must be in (0, 1]";
    case SPARGE_ERR_STRIDE: return "invalid stride or alignment (multiples of 8 elements, 16-byte aligned, non-overlapping output)";
    case SPARGE_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case SPARGE_ERR_WORKSPACE: return "workspace missing or too small";
    case SPARGE_ERR_ARG: return "invalid argument";
    case SPARGE_ERR_LAUNCH: return "kernel launch failed";
    case SPARGE_ERR_MASK_VALUE: return "mask_id holds a value other than 0 or 1";
    case SPARGE_ERR_SCRATCH_LIMIT: return "the shape needs more workspace than the no-allocation call's fixed 128 MiB array";
    default: return "unknown status";
  }
}

int sparge_topk_count(int64_t n_kblocks_, double topk, int64_t* k_out) {
  if (!k_out) return SPARGE_ERR_NULL;
  if (n_kblocks_ < 1) return SPARGE_ERR_ARG;
  return topk_count(n_kblocks_, topk, k_out);
}

size_t sparge_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, double topk) {
  if (check_shape(B, H, N, D) != SPARGE_OK) return 0;
  if (topk < 0.0) return mask_layout(B, H, N).total;
  int64_t k = 0;
  if (topk_count(n_kblocks(N), topk, &k) != SPARGE_OK) return 0;
  return topk_layout(B, H, N, D, k).total;
}

int sparge_pool_blocks(const uint16_t* x, int64_t B, int64_t H, int64_t N, int64_t D,
                       const int64_t x_strides[3], int block_rows, float* out, void* stream) {
  if (!x || !out) return SPARGE_ERR_NULL;
  if (int rc = check_shape(B, H, N, D)) return rc;
  if (int rc = check_strides(x_strides)) return rc;
  if (!aligned16(x) || !aligned16(out)) return SPARGE_ERR_STRIDE;
  if (block_rows != SPARGE_Q_BLOCK && block_rows != SPARGE_K_BLOCK) return SPARGE_ERR_ARG;
  const size_t out_bytes = static_cast<size_t>(B * H * ((N + block_rows - 1) / block_rows) * D) * sizeof(float);
  if (overlap(range_bytes(out, out_bytes), range_bf16(x, B, H, N, D, x_strides))) return SPARGE_ERR_ALIAS;
  const Strides s{x_strides[0], x_strides[1], x_strides[2]};
  return status_of(sparge::launch_pool(x, B, H, N, static_cast<int>(D), s, block_rows, out,
                                       static_cast<hipStream_t>(stream)));
}

int sparge_predict_mask(const float* qbar, const float* kbar, int64_t B, int64_t H, int64_t N,
                        int64_t D, double topk, float scale, int is_causal, uint8_t* mask_id,
                        int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
  if (!qbar || !kbar || !kv_idx || !kv_cnt) return SPARGE_ERR_NULL;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (int rc = check_shape(B, H, N, D)) return rc;
  if (N > SPARGE_MAX_PREDICT_N) return SPARGE_ERR_SHAPE;
  int64_t k = 0;
  if (int rc = topk_count(n_kblocks(N), topk, &k)) return rc;
  const size_t bh = static_cast<size_t>(B * H);
  const size_t rows = bh * n_qblocks(N);
  const Range in_q = range_bytes(qbar, rows * D * sizeof(float));
  const Range in_k = range_bytes(kbar, bh * n_kblocks(N) * D * sizeof(float));
  const Range outs[3] = {range_bytes(kv_idx, rows * k * sizeof(int32_t)),
                         range_bytes(kv_cnt, rows * sizeof(int32_t)),
                         mask_id ? range_bytes(mask_id, rows * n_kblocks(N)) : Range{0, 0}};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], in_q) || overlap(outs[i], in_k)) return SPARGE_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return SPARGE_ERR_ALIAS;
  }
  return status_of(sparge::launch_predict(qbar, kbar, B * H, N, static_cast<int>(D), k, topk,
                                          is_causal, resolve_scale(scale, D), mask_id, kv_idx,
                                          kv_cnt, static_cast<hipStream_t>(stream)));
}

int sparge_compact_mask(const uint8_t* mask_id, int64_t B, int64_t H, int64_t N, int32_t* kv_idx,
                        int32_t* kv_cnt, void* stream) {
  if (!mask_id || !kv_idx || !kv_cnt) return SPARGE_ERR_NULL;
  if (int rc = check_shape(B, H, N, 64)) return rc;
  const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
  const Range in = range_bytes(mask_id, rows * n_kblocks(N));
  const Range oi = range_bytes(kv_idx, rows * n_kblocks(N) * sizeof(int32_t));
  const Range oc = range_bytes(kv_cnt, rows * sizeof(int32_t));
  if (overlap(in, oi) || overlap(in, oc) || overlap(oi, oc)) return SPARGE_ERR_ALIAS;
  return status_of(sparge::launch_compact(mask_id, static_cast<int64_t>(rows), n_kblocks(N), kv_idx,
                                          kv_cnt, static_cast<hipStream_t>(stream)));
}

int sparge_attn_from_list(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* kv_idx, const int32_t* kv_cnt, int64_t ld_idx,
                          uint16_t* out, int64_t B, int64_t H, int64_t N, int64_t D,
                          const int64_t q_strides[3], const int64_t k_strides[3],
                          const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                          int is_causal, void* stream) {
  if (int rc = check_attn(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides)) return rc;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (kv_idx) {
    if (!kv_cnt) return SPARGE_ERR_NULL;
    if (ld_idx < 1) return SPARGE_ERR_ARG;
    const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
    const Range ro = range_bf16(out, B, H, N, D, o_strides);
    if (overlap(ro, range_bytes(kv_idx, rows * ld_idx * sizeof(int32_t))) ||
        overlap(ro, range_bytes(kv_cnt, rows * sizeof(int32_t))))
      return SPARGE_ERR_ALIAS;
  }
  sparge::AttnArgs a = attn_args(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides, scale);
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_idx ? kv_cnt : nullptr;
  a.ld_idx = kv_idx ? ld_idx : 0;
  a.causal = is_causal;
  return status_of(sparge::launch_attention(a, static_cast<hipStream_t>(stream)));
}

int block_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint8_t* mask_id, uint16_t* out, int64_t B, int64_t H, int64_t N,
                      int64_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                      int is_causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_attn(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides)) return rc;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  sparge::AttnArgs a = attn_args(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides, scale);
  a.causal = is_causal;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!mask_id) return status_of(sparge::launch_attention(a, st));   // dense: no list needed

  const MaskWs w = mask_layout(B, H, N);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPARGE_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
  const Range rw = range_bytes(workspace, w.total);
  const Range ro = range_bf16(out, B, H, N, D, o_strides);
  const Range rm = range_bytes(mask_id, rows * n_kblocks(N));
  if (overlap(ro, rm) || overlap(rw, rm) || overlap(rw, ro) ||
      overlap(rw, range_bf16(q, B, H, N, D, q_strides)) ||
      overlap(rw, range_bf16(k, B, H, N, D, k_strides)) ||
      overlap(rw, range_bf16(v, B, H, N, D, v_strides)))
    return SPARGE_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  if (int rc = status_of(sparge::launch_compact(mask_id, static_cast<int64_t>(rows), n_kblocks(N),
                                                idx, cnt, st)))
    return rc;
  a.kv_idx = idx;
  a.kv_cnt = cnt;
  a.ld_idx = n_kblocks(N);
  return status_of(sparge::launch_attention(a, st));
}

int sparge_check_mask(const uint8_t* mask_id, int64_t B, int64_t H, int64_t N, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!mask_id) return SPARGE_ERR_NULL;
  if (int rc = check_shape(B, H, N, 64)) return rc;
  const size_t n = static_cast<size_t>(B * H * n_qblocks(N) * n_kblocks(N));
  // one flag per workgroup of 256 threads, each scanning >= 256 bytes
  const int n_wg = static_cast<int>(std::min<size_t>(sparge::kCheckMaskWorkgroups, (n + 255) / 256));
  const size_t need = static_cast<size_t>(n_wg) * sizeof(int32_t);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SPARGE_ERR_WORKSPACE;
  if (overlap(range_bytes(workspace, need), range_bytes(mask_id, n))) return SPARGE_ERR_ALIAS;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* bad = static_cast<int32_t*>(workspace);
  if (int rc = status_of(sparge::launch_check_mask(mask_id, static_cast<int64_t>(n), bad, n_wg, st)))
    return rc;
  std::vector<int32_t> host(static_cast<size_t>(n_wg));
  if (hipMemcpyAsync(host.data(), bad, need, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return SPARGE_ERR_LAUNCH;
  for (int32_t f : host)
    if (f) return SPARGE_ERR_MASK_VALUE;
  return SPARGE_OK;
}

int block_sparse_attn_checked(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint8_t* mask_id, uint16_t* out, int64_t B, int64_t H, int64_t N,
                              int64_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                              int is_causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_attn(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides)) return rc;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (mask_id) {
    const MaskWs w = mask_layout(B, H, N);
    if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPARGE_ERR_WORKSPACE;
    const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
    const Range rw = range_bytes(workspace, w.total);
    const Range rm = range_bytes(mask_id, rows * n_kblocks(N));
    const Range ro = range_bf16(out, B, H, N, D, o_strides);
    // every check block_sparse_attn makes, before anything is launched
    if (overlap(ro, rm) || overlap(rw, rm) || overlap(rw, ro) ||
        overlap(rw, range_bf16(q, B, H, N, D, q_strides)) ||
        overlap(rw, range_bf16(k, B, H, N, D, k_strides)) ||
        overlap(rw, range_bf16(v, B, H, N, D, v_strides)))
      return SPARGE_ERR_ALIAS;
    // the lists region of the workspace (rows * N_KB int32: four bytes per mask
    // byte, so never smaller than the check's flags) holds them until compaction
    // reuses it
    if (int rc = sparge_check_mask(mask_id, B, H, N, workspace, workspace_bytes, stream)) return rc;
  }
  return block_sparse_attn(q, k, v, mask_id, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides,
                           scale, is_causal, workspace, workspace_bytes, stream);
}

int sparge_attn_topk(const uint16_t* q, const uint16_t* k, const uint16_t* v, double topk,
                     uint16_t* out, int64_t B, int64_t H, int64_t N, int64_t D,
                     const int64_t q_strides[3], const int64_t k_strides[3],
                     const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                     int is_causal, uint8_t* mask_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (int rc = check_attn(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides)) return rc;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (N > SPARGE_MAX_PREDICT_N) return SPARGE_ERR_SHAPE;
  int64_t kk = 0;
  if (int rc = topk_count(n_kblocks(N), topk, &kk)) return rc;
  const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
  const Range ro = range_bf16(out, B, H, N, D, o_strides);
  const Range rq = range_bf16(q, B, H, N, D, q_strides);
  const Range rk = range_bf16(k, B, H, N, D, k_strides);
  const Range rv = range_bf16(v, B, H, N, D, v_strides);
  const Range rm = mask_out ? range_bytes(mask_out, rows * n_kblocks(N)) : Range{0, 0};
  if (mask_out && (overlap(rm, ro) || overlap(rm, rq) || overlap(rm, rk) || overlap(rm, rv)))
    return SPARGE_ERR_ALIAS;
  // the workspace comes last: every check before it concerns the caller's own buffers
  const TopkWs w = topk_layout(B, H, N, D, kk);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPARGE_ERR_WORKSPACE;
  const Range rw = range_bytes(workspace, w.total);
  if (overlap(rw, ro) || overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv) || overlap(rw, rm))
    return SPARGE_ERR_ALIAS;

  const float sc = resolve_scale(scale, D);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qbar = reinterpret_cast<float*>(ws + w.qbar);
  float* kbar = reinterpret_cast<float*>(ws + w.kbar);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  const Strides qs{q_strides[0], q_strides[1], q_strides[2]};
  const Strides ks{k_strides[0], k_strides[1], k_strides[2]};
  if (int rc = status_of(sparge::launch_pool(q, B, H, N, static_cast<int>(D), qs, SPARGE_Q_BLOCK, qbar, st))) return rc;
  if (int rc = status_of(sparge::launch_pool(k, B, H, N, static_cast<int>(D), ks, SPARGE_K_BLOCK, kbar, st))) return rc;
  if (int rc = status_of(sparge::launch_predict(qbar, kbar, B * H, N, static_cast<int>(D), kk, topk,
                                                is_causal, sc, mask_out, idx, cnt, st)))
    return rc;
  sparge::AttnArgs a = attn_args(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides, sc);
  a.kv_idx = idx;
  a.kv_cnt = cnt;
  a.ld_idx = kk;
  a.causal = is_causal;
  return status_of(sparge::launch_attention(a, st));
}

int sparge_token_permutation(int64_t n_text, int64_t T, int64_t Hh, int64_t Ww, int layout,
                             const int64_t cube[3], int32_t* perm) {
  if (!perm) return SPARGE_ERR_NULL;
  if (n_text < 0 || T < 1 || Hh < 1 || Ww < 1) return SPARGE_ERR_ARG;
  if (T > kMaxDim || Hh > kMaxDim || Ww > kMaxDim || n_text > kMaxDim) return SPARGE_ERR_ARG;
  const int64_t video = T * Hh * Ww;
  if (video > (int64_t(1) << 31) - 1 - n_text || T * Hh > kMaxDim) return SPARGE_ERR_ARG;
  if (layout != SPARGE_LAYOUT_RASTER && layout != SPARGE_LAYOUT_CUBE && layout != SPARGE_LAYOUT_MORTON)
    return SPARGE_ERR_ARG;
  if (layout == SPARGE_LAYOUT_CUBE && (!cube || cube[0] < 1 || cube[1] < 1 || cube[2] < 1))
    return SPARGE_ERR_ARG;
  if (layout == SPARGE_LAYOUT_MORTON && std::max({T, Hh, Ww}) > (int64_t(1) << 21)) return SPARGE_ERR_ARG;
  int64_t pos = 0;
  for (; pos < n_text; ++pos) perm[pos] = static_cast<int32_t>(pos);
  auto token = [&](int64_t t, int64_t h, int64_t w) { return n_text + (t * Hh + h) * Ww + w; };
  if (layout == SPARGE_LAYOUT_RASTER) {
    for (int64_t i = 0; i < video; ++i) perm[pos++] = static_cast<int32_t>(n_text + i);
  } else if (layout == SPARGE_LAYOUT_CUBE) {
    const int64_t ct = cube[0], ch = cube[1], cw = cube[2];
    for (int64_t t0 = 0; t0 < T; t0 += ct)
      for (int64_t h0 = 0; h0 < Hh; h0 += ch)
        for (int64_t w0 = 0; w0 < Ww; w0 += cw)
          for (int64_t t = t0; t < std::min(T, t0 + ct); ++t)
            for (int64_t h = h0; h < std::min(Hh, h0 + ch); ++h)
              for (int64_t w = w0; w < std::min(Ww, w0 + cw); ++w)
                perm[pos++] = static_cast<int32_t>(token(t, h, w));
  } else {
    // Z-order: bit b of w, h, t lands on bit 3b, 3b+1, 3b+2 of the key
    auto spread = [](uint64_t v) {
      uint64_t r = 0;
      for (int b = 0; b < 21; ++b) r |= ((v >> b) & 1u) << (3 * b);
      return r;
    };
    std::vector<std::pair<uint64_t, int32_t>> keyed;
    keyed.reserve(static_cast<size_t>(video));
    for (int64_t t = 0; t < T; ++t)
      for (int64_t h = 0; h < Hh; ++h)
        for (int64_t w = 0; w < Ww; ++w)
          keyed.emplace_back(spread(w) | (spread(h) << 1) | (spread(t) << 2),
                             static_cast<int32_t>(token(t, h, w)));
    std::sort(keyed.begin(), keyed.end());
    for (const auto& kv : keyed) perm[pos++] = kv.second;
  }
  return SPARGE_OK;
}

int sparge_permute_tokens(const uint16_t* x, const int32_t* perm, uint16_t* out, int64_t B, int64_t H,
                          int64_t N, int64_t D, const int64_t x_strides[3],
                          const int64_t out_strides[3], int inverse, void* stream) {
  if (!x || !perm || !out) return SPARGE_ERR_NULL;
  if (int rc = check_shape(B, H, N, D)) return rc;
  if (int rc = check_strides(x_strides)) return rc;
  if (int rc = check_strides(out_strides)) return rc;
  if (inverse != 0 && inverse != 1) return SPARGE_ERR_ARG;
  if (N > (int64_t(1) << 31) - 1) return SPARGE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return SPARGE_ERR_STRIDE;
  if (!non_overlapping(B, H, N, D, out_strides)) return SPARGE_ERR_STRIDE;
  const Range ro = range_bf16(out, B, H, N, D, out_strides);
  if (overlap(ro, range_bf16(x, B, H, N, D, x_strides)) ||
      overlap(ro, range_bytes(perm, static_cast<size_t>(N) * sizeof(int32_t))))
    return SPARGE_ERR_ALIAS;
  const Strides xs{x_strides[0], x_strides[1], x_strides[2]};
  const Strides os{out_strides[0], out_strides[1], out_strides[2]};
  return status_of(sparge::launch_permute(x, xs, perm, out, os, B, H, N, static_cast<int>(D), inverse,
                                          static_cast<hipStream_t>(stream)));
}

int sparge_predict_mask_cdf(const float* qbar, const float* kbar, int64_t B, int64_t H, int64_t N,
                            int64_t D, double tau, float scale, int is_causal, uint8_t* mask_id,
                            int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
  if (!qbar || !kbar || !kv_idx || !kv_cnt) return SPARGE_ERR_NULL;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (int rc = check_shape(B, H, N, D)) return rc;
  if (N > SPARGE_MAX_PREDICT_N) return SPARGE_ERR_SHAPE;
  if (!(tau > 0.0 && tau <= 1.0)) return SPARGE_ERR_TOPK;
  const size_t bh = static_cast<size_t>(B * H);
  const size_t rows = bh * n_qblocks(N);
  const Range in_q = range_bytes(qbar, rows * D * sizeof(float));
  const Range in_k = range_bytes(kbar, bh * n_kblocks(N) * D * sizeof(float));
  const Range outs[3] = {range_bytes(kv_idx, rows * n_kblocks(N) * sizeof(int32_t)),
                         range_bytes(kv_cnt, rows * sizeof(int32_t)),
                         mask_id ? range_bytes(mask_id, rows * n_kblocks(N)) : Range{0, 0}};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], in_q) || overlap(outs[i], in_k)) return SPARGE_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return SPARGE_ERR_ALIAS;
  }
  return status_of(sparge::launch_predict_cdf(qbar, kbar, B * H, N, static_cast<int>(D), tau, is_causal,
                                              resolve_scale(scale, D), mask_id, kv_idx, kv_cnt,
                                              static_cast<hipStream_t>(stream)));
}

int sparge_attn_cdf(const uint16_t* q, const uint16_t* k, const uint16_t* v, double tau, uint16_t* out,
                    int64_t B, int64_t H, int64_t N, int64_t D, const int64_t q_strides[3],
                    const int64_t k_strides[3], const int64_t v_strides[3], const int64_t o_strides[3],
                    float scale, int is_causal, uint8_t* mask_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (int rc = check_attn(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides)) return rc;
  if (is_causal != 0 && is_causal != 1) return SPARGE_ERR_ARG;
  if (N > SPARGE_MAX_PREDICT_N) return SPARGE_ERR_SHAPE;
  if (!(tau > 0.0 && tau <= 1.0)) return SPARGE_ERR_TOPK;
  const int64_t kk = n_kblocks(N);   // a row may keep every block
  const TopkWs w = topk_layout(B, H, N, D, kk);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPARGE_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * H * n_qblocks(N));
  const Range rw = range_bytes(workspace, w.total);
  const Range ro = range_bf16(out, B, H, N, D, o_strides);
  const Range rq = range_bf16(q, B, H, N, D, q_strides);
  const Range rk = range_bf16(k, B, H, N, D, k_strides);
  const Range rv = range_bf16(v, B, H, N, D, v_strides);
  if (overlap(rw, ro) || overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv)) return SPARGE_ERR_ALIAS;
  if (mask_out) {
    const Range rm = range_bytes(mask_out, rows * n_kblocks(N));
    if (overlap(rm, ro) || overlap(rm, rw) || overlap(rm, rq) || overlap(rm, rk) || overlap(rm, rv))
      return SPARGE_ERR_ALIAS;
  }
  const float sc = resolve_scale(scale, D);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qbar = reinterpret_cast<float*>(ws + w.qbar);
  float* kbar = reinterpret_cast<float*>(ws + w.kbar);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + w.idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  const Strides qs{q_strides[0], q_strides[1], q_strides[2]};
  const Strides ks{k_strides[0], k_strides[1], k_strides[2]};
  if (int rc = status_of(sparge::launch_pool(q, B, H, N, static_cast<int>(D), qs, SPARGE_Q_BLOCK, qbar, st))) return rc;
  if (int rc = status_of(sparge::launch_pool(k, B, H, N, static_cast<int>(D), ks, SPARGE_K_BLOCK, kbar, st))) return rc;
  if (int rc = status_of(sparge::launch_predict_cdf(qbar, kbar, B * H, N, static_cast<int>(D), tau, is_causal,
                                                    sc, mask_out, idx, cnt, st)))
    return rc;
  sparge::AttnArgs a = attn_args(q, k, v, out, B, H, N, D, q_strides, k_strides, v_strides, o_strides, sc);
  a.kv_idx = idx;
  a.kv_cnt = cnt;
  a.ld_idx = kk;
  a.causal = is_causal;
  return status_of(sparge::launch_attention(a, st));
}

}  // extern "C"
