// Block-sparse flash attention forward for gfx950 (MI355X).
//
// Non-causal softmax attention in which query block i (128 rows) visits only
// the 64-key blocks of its list (SpargeAttention Documentation,
// block_sparse_sage2_attn_cuda and "Mask Requirements": fixed 128x64 tiles).
// Skipped tiles are never loaded. Online softmax keeps a running max m and
// sum l per query row and rescales the output accumulator in registers.
//
// Work decomposition
//   one workgroup = one query block of one head, 4 wavefronts x 32 query rows.
//   Per 64-key tile, each wavefront computes S^T = K_tile Q_w^T (64 x 32) with
//   v_mfma_f32_32x32x16_bf16, so every lane ends up owning one query row
//   (lane % 32) and 32 of the tile's 64 scores. Row max / row sum need a single
//   exchange with the partner lane (lane ^ 32). The probabilities, rounded to
//   bf16, are already laid out as the B operand of O^T += V^T P^T, so they never
//   leave registers. V^T operands come straight from the row-major V tile with
//   the gfx950 transpose read ds_read_b64_tr_b16.
//   K rows are read in a permuted order (sigma below) so that the S^T
//   accumulator registers hold consecutive keys, matching the PV operand order.
//
// Memory
//   Q rows stay in registers for the whole walk. K and V tiles are staged
//   through LDS, double buffered: the global loads for tile t+1 are issued
//   before tile t is computed and land in the other LDS buffer afterwards
//   (one barrier per tile). Row pitches are padded (K: +16 B, V: +64 B) so the
//   two LDS read patterns spread over the banks.
//   Workgroups are numbered so that each of the 8 XCDs (each with its own L2)
//   walks a contiguous range of query blocks of the same head, and all XCDs
//   move through the heads together, keeping one head's K/V hot in the
//   last-level cache while neighbouring query blocks share tiles in L2.
#include "common.h"

namespace sparge {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
  static constexpr int kKPitch = D * 2 + 16;          // bytes per K row in LDS
  static constexpr int kVPitch = D * 2 + 64;          // bytes per V row in LDS
  static constexpr int kKBytes = kKBlock * kKPitch;
  static constexpr int kVBytes = kKBlock * kVPitch;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kLds = 2 * kStage;
  static constexpr int kChunksPerRow = D / 8;         // 16-byte chunks per row
  static constexpr int kChunksPerThread = kKBlock * kChunksPerRow / 256;
  static constexpr int kSteps = D / 16;               // k-steps of the QK^T product
  static constexpr int kDChunks = D / 32;             // 32-wide column chunks of O
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  int64_t ld_idx;
  int64_t H, N;
  int64_t n_qb, n_kb;
  int64_t per_xcd;     // query blocks per XCD slice of a head
  Strides qs, ks, vs, os;
  float c;             // scale * log2(e)
};

// Row of the K tile that feeds A-operand row m, chosen so that accumulator
// register i of lane (n, g) holds key 8g + i (i < 8) or 16 + 8g + (i - 8).
__device__ __forceinline__ int sigma(int m) {
  const int a = m >> 3, gg = (m >> 2) & 1, bb = m & 3;
  return 16 * (a >> 1) + 8 * gg + 4 * (a & 1) + bb;
}

// Key block visited at step tt. An id outside [0, n_kb) maps to a block past
// the end of the sequence: its keys load as zeros and are masked out, so a
// corrupt list entry contributes nothing instead of reading out of bounds.
__device__ __forceinline__ int64_t block_id(const int32_t* list, int tt, int64_t n_kb) {
  if (!list) return tt;
  const int64_t j = list[tt];
  return (j >= 0 && j < n_kb) ? j : n_kb;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* kh, const uint16_t* vh, int64_t kn,
                                          int64_t vn, int64_t N, int64_t j, int t,
                                          uint4 (&kr)[Cfg<D>::kChunksPerThread],
                                          uint4 (&vr)[Cfg<D>::kChunksPerThread]) {
#pragma unroll
  for (int e = 0; e < Cfg<D>::kChunksPerThread; ++e) {
    const int c = t + 256 * e;
    const int row = c / Cfg<D>::kChunksPerRow;
    const int col = (c % Cfg<D>::kChunksPerRow) * 8;
    const int64_t key = j * kKBlock + row;
    if (key < N) {
      kr[e] = load16(kh + key * kn + col);
      vr[e] = load16(vh + key * vn + col);
    } else {
      kr[e] = make_uint4(0, 0, 0, 0);
      vr[e] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(char* stage, int t,
                                           const uint4 (&kr)[Cfg<D>::kChunksPerThread],
                                           const uint4 (&vr)[Cfg<D>::kChunksPerThread]) {
#pragma unroll
  for (int e = 0; e < Cfg<D>::kChunksPerThread; ++e) {
    const int c = t + 256 * e;
    const int row = c / Cfg<D>::kChunksPerRow;
    const int colb = (c % Cfg<D>::kChunksPerRow) * 16;
    *reinterpret_cast<uint4*>(stage + row * Cfg<D>::kKPitch + colb) = kr[e];
    *reinterpret_cast<uint4*>(stage + Cfg<D>::kKBytes + row * Cfg<D>::kVPitch + colb) = vr[e];
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char lds[C::kLds];

  // Workgroup -> (head, query block). Consecutive workgroup ids go to
  // consecutive XCDs; XCD x owns query blocks [x*per, (x+1)*per) of every head.
  const int64_t wid = blockIdx.x;
  const int64_t xcd = wid % kNumXcd;
  const int64_t it = wid / kNumXcd;
  const int64_t bh = it / p.per_xcd;
  const int64_t qb = xcd * p.per_xcd + (it - bh * p.per_xcd);
  if (qb >= p.n_qb) return;
  const int64_t b = bh / p.H, h = bh - (bh / p.H) * p.H;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n = lane & 31, g = lane >> 5;

  const uint16_t* qh = p.q + b * p.qs.b + h * p.qs.h;
  const uint16_t* kh = p.k + b * p.ks.b + h * p.ks.h;
  const uint16_t* vh = p.v + b * p.vs.b + h * p.vs.h;
  uint16_t* oh = p.o + b * p.os.b + h * p.os.h;

  const int64_t row_id = bh * p.n_qb + qb;
  int cnt;
  const int32_t* list = nullptr;
  if (p.kv_idx) {
    cnt = p.kv_cnt[row_id];
    cnt = cnt < 0 ? 0 : (cnt > p.ld_idx ? static_cast<int>(p.ld_idx) : cnt);
    list = p.kv_idx + row_id * p.ld_idx;
  } else {
    cnt = static_cast<int>(p.n_kb);
  }

  // Q^T operands: lane (n, g) holds query row qrow, columns 16s + 8g .. +7.
  const int64_t qrow = qb * kQBlock + wave * 32 + n;
  bf16x8 qreg[C::kSteps];
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) {
    uint4 raw = (qrow < p.N) ? load16(qh + qrow * p.qs.n + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    qreg[s] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 o[C::kDChunks];
#pragma unroll
  for (int cc = 0; cc < C::kDChunks; ++cc)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cc][i] = 0.f;
  float m = -INFINITY;
  float l = 0.f;

  const int sig = sigma(n);
  // transpose-read lane geometry for the V^T operand
  const int tr_key = 8 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (cnt > 0) {
    uint4 kr[C::kChunksPerThread], vr[C::kChunksPerThread];
    load_tile<D>(kh, vh, p.ks.n, p.vs.n, p.N, block_id(list, 0, p.n_kb), t, kr, vr);
    store_tile<D>(lds, t, kr, vr);
    __syncthreads();

    for (int tt = 0; tt < cnt; ++tt) {
      char* cur = lds + (tt & 1) * C::kStage;
      const bool has_next = tt + 1 < cnt;
      if (has_next) load_tile<D>(kh, vh, p.ks.n, p.vs.n, p.N, block_id(list, tt + 1, p.n_kb), t, kr, vr);
      const int64_t j = block_id(list, tt, p.n_kb);

      // S^T = K Q^T for keys [0, 32) and [32, 64) of the tile.
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
      const char* krow0 = cur + sig * C::kKPitch + 16 * g;
      const char* krow1 = krow0 + 32 * C::kKPitch;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow0 + 32 * s);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(krow1 + 32 * s);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[s], s1, 0, 0, 0);
      }

      // Keys past N in a ragged last block take no weight.
      if (j * kKBlock + kKBlock > p.N) {
        const int64_t lim = p.N - j * kKBlock;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = (i < 8) ? 8 * g + i : 16 + 8 * g + (i - 8);
          if (kl >= lim) s0[i] = -INFINITY;
          if (kl + 32 >= lim) s1[i] = -INFINITY;
        }
      }

      // Online softmax in base 2.
      float mx = s0[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx * p.c);
      // A fully masked first tile (possible only for invalid list entries) keeps
      // m at -inf; subtracting 0 instead then yields zero weights, not NaN.
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
      m = m_new;

      bf16x8 pb[4];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const __bf16 e0 = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s0[i], p.c, -m_ref)));
        const __bf16 e1 = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s1[i], p.c, -m_ref)));
        pb[i >> 3][i & 7] = e0;
        pb[2 + (i >> 3)][i & 7] = e1;
        rs += static_cast<float>(e0) + static_cast<float>(e1);
      }
      l = l * alpha + rs;
#pragma unroll
      for (int cc = 0; cc < C::kDChunks; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cc][i] *= alpha;

      // O^T += V^T P^T over four 16-key steps.
      const char* vt = cur + C::kKBytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const char* vrow = vt + (16 * u + tr_key) * C::kVPitch;
#pragma unroll
        for (int cc = 0; cc < C::kDChunks; ++cc) {
          const char* a_lo = vrow + (32 * cc + tr_col) * 2;
          const char* a_hi = a_lo + 4 * C::kVPitch;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) char*)(a_lo));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(__attribute__((address_space(3))) char*)(a_hi));
          const s16x4 lohi[2] = {lo, hi};
          const bf16x8 a = __builtin_bit_cast(bf16x8, lohi);
          o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[cc], 0, 0, 0);
        }
      }

      if (has_next) store_tile<D>(lds + ((tt + 1) & 1) * C::kStage, t, kr, vr);
      __syncthreads();
    }
  }

  // Normalise and store: lane (n, g) holds columns 32cc + 8a + 4g + {0..3} of row qrow.
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  if (qrow < p.N) {
    uint16_t* orow = oh + qrow * p.os.n;
#pragma unroll
    for (int cc = 0; cc < C::kDChunks; ++cc)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        __bf16 r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = static_cast<__bf16>(o[cc][4 * a + e] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * cc + 8 * a + 4 * g) = __builtin_bit_cast(uint2, r4);
      }
  }
}

template <int D>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  Params p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.kv_idx = a.kv_idx; p.kv_cnt = a.kv_cnt; p.ld_idx = a.ld_idx;
  p.H = a.H; p.N = a.N;
  p.n_qb = (a.N + kQBlock - 1) / kQBlock;
  p.n_kb = (a.N + kKBlock - 1) / kKBlock;
  p.per_xcd = (p.n_qb + kNumXcd - 1) / kNumXcd;
  p.qs = a.qs; p.ks = a.ks; p.vs = a.vs; p.os = a.os;
  p.c = a.scale * kLog2e;
  const int64_t grid = a.B * a.H * kNumXcd * p.per_xcd;
  void* args[] = {(void*)&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<D>),
                         dim3(static_cast<uint32_t>(grid)), dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  return a.D == 128 ? launch_t<128>(a, stream) : launch_t<64>(a, stream);
}

}  // namespace sparge
