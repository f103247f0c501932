// Block-sparse flash attention forward for gfx950 (MI355X).
//
// Softmax attention in which query block i (128 rows) visits only
// the 64-key blocks of its list (SpargeAttention Documentation,
// block_sparse_sage2_attn_cuda and "Mask Requirements": fixed 128x64 tiles).
// Skipped tiles are never loaded. With causal masking (the top-k API's
// is_causal flag) a row also ignores the keys after it. Online softmax keeps a
// running max m and sum l per query row and rescales the output accumulator in
// registers.
//
// Work decomposition
//   One workgroup = one query block of one head: 4 wavefronts x 32 query rows.
//   Per 64-key tile, each wavefront computes S^T = K_tile Q_w^T (64 x 32) with
//   v_mfma_f32_32x32x16_bf16, so every lane owns one query row (lane % 32) and
//   32 of the tile's 64 scores; row max and row sum need one exchange with the
//   partner lane (lane ^ 32). The probabilities, rounded to bf16, are already
//   laid out as the B operand of O^T += V^T P^T, so they never leave registers.
//   V^T operands come straight from the row-major V tile through the gfx950
//   transpose read ds_read_b64_tr_b16. K rows are read in a permuted order
//   (sigma below) so that the S^T accumulators hold consecutive keys, which is
//   the key order the PV operands need.
//
// Softmax
//   Base 2 with the scale folded into one FMA. The running max is only a
//   reference that keeps the weights in range, so no per-tile row max is taken:
//   weights are computed against the current reference, and only when they
//   grow too large (their per-lane sum passes 2^20) is the tile's exact max
//   taken, the reference raised, O and l rescaled and the tile's weights
//   recomputed; that happens on the first tile of a row and rarely after. Row
//   sums add the bf16-rounded weights with v_dot2_f32_bf16, so they match the
//   weights the PV product actually used.
//
// Memory
//   Q rows stay in registers for the whole walk. K and V tiles go global -> LDS
//   with buffer_load_dwordx4 ... lds (no data registers, no LDS write
//   instructions), double buffered with one barrier per tile. The loads of
//   tile t+1 are interleaved one by one with the QK MFMAs of tile t: issued as
//   a burst right after the barrier, the loads of all eight wavefronts of a CU
//   fill the vector-memory queue and stall instruction issue for hundreds of
//   cycles. Tiles are stored unpadded (64 KB of LDS per workgroup at
//   D=128, so two workgroups share a CU) with 16-byte chunks XOR-swizzled per
//   row: K so that the 16 rows one A-operand read touches hit distinct banks,
//   V so that the 4 rows of one transpose read do.
//   Workgroups are numbered so that each of the 8 XCDs (each with its own L2)
//   walks a contiguous range of query blocks of one head while all XCDs move
//   through the heads together: one head's K/V stays hot in the last-level
//   cache and neighbouring query blocks, whose lists overlap, share L2.
#include <type_traits>

#include "common.h"

namespace sparge {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSumLog2 = 20;            // per-lane weight sum that triggers a new reference max
constexpr float kSumLimit = static_cast<float>(1 << kSumLog2);
// Word 3 of a raw (untyped) buffer resource on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
// sched_barrier mask: VALU (0x2), SALU (0x4), LDS reads (0x100), transcendental (0x400).
constexpr int kSchedKeepLoads = 0x0506;

template <int D>
struct Cfg {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                     // 16-byte chunks per row
  static constexpr int kTile = kKBlock * kRowBytes;         // one K or V tile in LDS
  static constexpr int kStage = 2 * kTile;                  // K tile then V tile
  static constexpr int kLds = 2 * kStage;                   // double buffered
  static constexpr int kRowsPerInst = 64 / kChunks;         // rows one wavefront load fills
  static constexpr int kInstPerWave = kKBlock / (4 * kRowsPerInst);
  static constexpr int kSteps = D / 16;                     // k-steps of QK^T
  static constexpr int kDChunks = D / 32;                   // 32-column chunks of O
};

// Chunk swizzles (XOR on the 16-byte chunk index within a row).
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }

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
// the end of the sequence whose keys are all masked, so a corrupt list entry
// contributes nothing instead of reading out of bounds.
__device__ __forceinline__ int64_t sanitize_id(int64_t j, int64_t n_kb) {
  return (j >= 0 && j < n_kb) ? j : n_kb;
}
__device__ __forceinline__ int64_t block_id(const int32_t* list, int tt, int64_t n_kb) {
  return list ? sanitize_id(list[tt], n_kb) : tt;
}

// Value of x in the partner lane (lane ^ 32) combined with x: v_permlane32_swap
// hands lane l both x[l % 32] and x[l % 32 + 32].
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D, bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  // Four separate LDS objects (not one array) so that waits for the loads
  // filling one buffer are not imposed on reads of another.
  __shared__ __attribute__((aligned(1024))) char lds_k0[C::kTile];
  __shared__ __attribute__((aligned(1024))) char lds_k1[C::kTile];
  __shared__ __attribute__((aligned(1024))) char lds_v0[C::kTile];
  __shared__ __attribute__((aligned(1024))) char lds_v1[C::kTile];

  // Workgroup -> (head, query block). Consecutive workgroup ids go to
  // consecutive XCDs. Non-causal lists are about equally long: XCD x owns query
  // blocks [x*per, (x+1)*per) of every head, so neighbouring blocks, whose
  // lists overlap, share its L2. Causal lists grow with the block index: each
  // head's blocks are dispatched longest first and dealt round the XCDs, so
  // short lists fill in at the end instead of one XCD carrying the long ones.
  const int64_t wid = blockIdx.x;
  int64_t bh, qb;
  if constexpr (!kCausal) {
    const int64_t xcd = wid % kNumXcd;
    const int64_t it = wid / kNumXcd;
    bh = it / p.per_xcd;
    qb = xcd * p.per_xcd + (it - bh * p.per_xcd);
  } else {
    const int64_t per_head = kNumXcd * p.per_xcd;
    bh = wid / per_head;
    qb = p.n_qb - 1 - (wid - bh * per_head);
  }
  if (qb < 0 || qb >= p.n_qb) return;
  const int64_t b = bh / p.H, h = bh - (bh / p.H) * p.H;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // uniform copy for scalar addressing
  const int n = lane & 31, g = lane >> 5;

  const uint16_t* qh = p.q + b * p.qs.b + h * p.qs.h;
  const uint16_t* kh = p.k + b * p.ks.b + h * p.ks.h;
  const uint16_t* vh = p.v + b * p.vs.b + h * p.vs.h;
  uint16_t* oh = p.o + b * p.os.b + h * p.os.h;

  // The block list is read-only for the whole launch: read it through the
  // scalar cache (constant address space), a few tiles ahead of its use.
  typedef __attribute__((address_space(4))) const int32_t cint32;
  const int64_t row_id = bh * p.n_qb + qb;
  int cnt;
  const cint32* list = nullptr;
  if (p.kv_idx) {
    cnt = ((const cint32*)p.kv_cnt)[row_id];
    cnt = cnt < 0 ? 0 : (cnt > p.ld_idx ? static_cast<int>(p.ld_idx) : cnt);
    list = (const cint32*)(p.kv_idx + row_id * p.ld_idx);
  } else {
    cnt = static_cast<int>(p.n_kb);
  }
  auto raw_id = [&](int i) -> int64_t { return (i < cnt) ? (list ? list[i] : i) : 0; };

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

  // ---- per-lane LDS geometry (constant over the walk)
  // K A-operand: row sigma(n) (+32 for the second half), logical chunk 2s + g.
  const int krow = sigma(n);
  const int kx = swz_k<D>(krow);
  int koff[C::kSteps];
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) koff[s] = krow * C::kRowBytes + 16 * ((2 * s + g) ^ kx);
  // V transpose read: row 16u + 8g + 4r + (lane%16)/4, logical chunk 4cc + lcx, half (lane & 1).
  const int vrow = 8 * g + ((lane & 15) >> 2);
  const int vx = swz_v<D>(vrow);
  const int lcx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int voff[C::kDChunks];
#pragma unroll
  for (int cc = 0; cc < C::kDChunks; ++cc)
    voff[cc] = vrow * C::kRowBytes + 16 * ((4 * cc + lcx) ^ vx) + 8 * (lane & 1);

  // ---- global -> LDS: wavefront load e fills rows [r0, r0 + kRowsPerInst) of a tile.
  // Loads go through a buffer resource per tile (scalar base and byte bound) with
  // a fixed 32-bit per-lane offset; rows past N fall outside the bound and read
  // as zeros (their scores are masked), so ragged and invalid blocks need no
  // special path.
  uint32_t ld_koff[C::kInstPerWave], ld_voff[C::kInstPerWave];
#pragma unroll
  for (int e = 0; e < C::kInstPerWave; ++e) {
    const int inst = wave * C::kInstPerWave + e;
    const int r = inst * C::kRowsPerInst + lane / C::kChunks;
    const int pc = lane % C::kChunks;
    ld_koff[e] = static_cast<uint32_t>((r * p.ks.n + 8 * (pc ^ swz_k<D>(r))) * 2);
    ld_voff[e] = static_cast<uint32_t>((r * p.vs.n + 8 * (pc ^ swz_v<D>(r))) * 2);
  }
  // Tile j of an operand starts j * tile_bytes past its head; its bound is the
  // whole tile, the rows left at the sequence end, or nothing (j past the end).
  const int64_t n_full = p.N / kKBlock;
  const uint32_t k_tile = static_cast<uint32_t>(kKBlock * p.ks.n * 2);
  const uint32_t v_tile = static_cast<uint32_t>(kKBlock * p.vs.n * 2);
  const uint32_t k_tail = static_cast<uint32_t>((p.N - n_full * kKBlock) * p.ks.n * 2);
  const uint32_t v_tail = static_cast<uint32_t>((p.N - n_full * kKBlock) * p.vs.n * 2);
  auto tile_rsrc = [&](const uint16_t* base, int64_t j, uint32_t tile_bytes, uint32_t tail_bytes) {
    const uint32_t bound = j < n_full ? tile_bytes : (j == n_full ? tail_bytes : 0u);
    const char* ptr = reinterpret_cast<const char*>(base) +
                      static_cast<uint64_t>(static_cast<uint32_t>(j)) * tile_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(ptr), static_cast<short>(0),
                                             static_cast<int>(bound), kBufferFlags);
  };
  auto issue_one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, char* buf, int e) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + (wave_s * C::kInstPerWave + e) * 1024),
                                             16, static_cast<int>(off), 0, 0, 0);
  };
  // Pins a load between the MFMAs around it: VALU, SALU, transcendental and
  // LDS-read instructions may still move across, MFMAs and memory loads may not.
  auto pinned_issue = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, char* buf, int e) {
    __builtin_amdgcn_sched_barrier(kSchedKeepLoads);
    issue_one(rs, off, buf, e);
    __builtin_amdgcn_sched_barrier(kSchedKeepLoads);
  };
  auto issue = [&](int64_t j, char* kbuf, char* vbuf) {
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kh, j, k_tile, k_tail);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vh, j, v_tile, v_tail);
#pragma unroll
    for (int e = 0; e < C::kInstPerWave; ++e) {
      issue_one(kr, ld_koff[e], kbuf, e);
      issue_one(vr, ld_voff[e], vbuf, e);
    }
  };

  // S^T = K Q^T for keys [0, 32) and [32, 64) of a tile; hook(s) runs after k-step s.
  auto qk = [&](const char* kb, f32x16& s0, f32x16& s1, auto hook) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kb + koff[s]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kb + koff[s] + 32 * C::kRowBytes);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[s], s1, 0, 0, 0);
      hook(s);
    }
  };

  // Keys past N in a ragged (or invalid) block take no weight, and with causal
  // masking neither do keys after this lane's query row. Only tiles at the
  // sequence end or across the block's diagonal need the per-key test.
  auto mask_keys = [&](int64_t j, f32x16& s0, f32x16& s1) {
    const int64_t k0 = j * kKBlock;
    if (k0 + kKBlock > p.N || (kCausal && k0 + kKBlock - 1 > qb * kQBlock)) {
      // keys k0 + lim and later are masked; register i of this lane holds key
      // 8g + i (i < 8) or 8g + 16 + (i - 8)
      int64_t lim64 = p.N - k0;
      if (kCausal && qrow - k0 + 1 < lim64) lim64 = qrow - k0 + 1;
      const int lim = static_cast<int>(lim64 < 0 ? 0 : (lim64 > kKBlock ? kKBlock : lim64)) - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = (i < 8) ? i : 16 + (i - 8);
        if (kl >= lim) s0[i] = -INFINITY;
        if (kl + 32 >= lim) s1[i] = -INFINITY;
      }
    }
  };

  // Probabilities of a tile as bf16 PV operands, against reference mref (log2
  // units); returns this lane's sum of the rounded weights.
  auto probs = [&](const f32x16& s0, const f32x16& s1, float mref, bf16x8 (&pb)[4]) -> float {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const f32x2 e0 = {__builtin_amdgcn_exp2f(fmaf(s0[i], p.c, -mref)),
                        __builtin_amdgcn_exp2f(fmaf(s0[i + 1], p.c, -mref))};
      const f32x2 e1 = {__builtin_amdgcn_exp2f(fmaf(s1[i], p.c, -mref)),
                        __builtin_amdgcn_exp2f(fmaf(s1[i + 1], p.c, -mref))};
      const bf16x2 b0 = __builtin_convertvector(e0, bf16x2);
      const bf16x2 b1 = __builtin_convertvector(e1, bf16x2);
      pb[i >> 3][i & 7] = b0[0];
      pb[i >> 3][(i & 7) + 1] = b0[1];
      pb[2 + (i >> 3)][i & 7] = b1[0];
      pb[2 + (i >> 3)][(i & 7) + 1] = b1[1];
      lt = __builtin_amdgcn_fdot2_f32_bf16(b0, ones, lt, false);
      lt = __builtin_amdgcn_fdot2_f32_bf16(b1, ones, lt, false);
    }
    return lt;
  };

  // Softmax weights of a tile. The running max m only serves as a reference
  // that keeps the weights in range, so it is not recomputed per tile: the
  // weights are taken against the current m, and only when a lane's weights
  // sum past 2^kSumLog2 (a score far above m; or m still unset) is the tile's
  // exact row max taken, m raised to it, O and l rescaled, and the weights
  // recomputed. Weights up to 2^kSumLog2 are as exact in bf16 and fp32 as
  // weights below 1, and the accumulators have ample range for them.
  auto weights = [&](const f32x16& s0, const f32x16& s1, bf16x8 (&pb)[4]) {
    // m stays -inf only while every key seen so far was masked (invalid ids);
    // a reference of 0 then gives zero weights instead of NaN.
    float mref = (m == -INFINITY) ? 0.f : m;
    float lt = probs(s0, s1, mref, pb);
    if (__builtin_amdgcn_ballot_w64(!(lt <= kSumLimit) || (m == -INFINITY && lt > 0.f))) {
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      const float mt = max_with_partner(mx) * p.c;
      const float m_new = fmaxf(m, mt);
      // O and l are still 0 while m is unset
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int cc = 0; cc < C::kDChunks; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cc][i] *= alpha;
      m = m_new;
      mref = (m == -INFINITY) ? 0.f : m;
      lt = probs(s0, s1, mref, pb);
    }
    l += lt;
  };

  // O^T += V^T P^T over four 16-key steps.
  auto pv = [&](const char* vt, const bf16x8 (&pb)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int cc = 0; cc < C::kDChunks; ++cc) {
        const char* a_lo = vt + (16 * u) * C::kRowBytes + voff[cc];
        const char* a_hi = a_lo + 4 * C::kRowBytes;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(a_lo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) char*)(a_hi));
        const s16x4 lohi[2] = {lo, hi};
        const bf16x8 a = __builtin_bit_cast(bf16x8, lohi);
        o[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[cc], 0, 0, 0);
      }
    }
  };

  if (cnt > 0) {
    // Double buffering: step t computes tile t from buffers t%2 while the
    // loads of tile t+1 fill the other pair.
    int64_t j0 = sanitize_id(raw_id(0), p.n_kb);
    int64_t j1 = sanitize_id(raw_id(1), p.n_kb);
    issue(j0, lds_k0, lds_v0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // The next tile's loads are spread through this tile's QK MFMAs, one load
    // per k-step.
    auto step = [&](auto parity, int tt) {
      constexpr int P = decltype(parity)::value;
      char* k_cur = P ? lds_k1 : lds_k0;
      char* v_cur = P ? lds_v1 : lds_v0;
      char* k_fill = P ? lds_k0 : lds_k1;
      char* v_fill = P ? lds_v0 : lds_v1;
      const bool more = tt + 1 < cnt;
      // past the last tile the resources hold no bytes: the loads only write
      // zeros into the buffer that was just released
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kh, more ? j1 : p.n_kb, k_tile, k_tail);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vh, more ? j1 : p.n_kb, v_tile, v_tail);
      const int32_t raw2 = static_cast<int32_t>(raw_id(tt + 2));
      f32x16 sa, sb;
      // The QK phase (MFMAs and the tile loads) runs at raised wavefront
      // priority, so the SIMD's other wavefront fills in with its softmax.
      __builtin_amdgcn_s_setprio(2);
      qk(k_cur, sa, sb, [&](int st) {
        // load i of the 2 * kInstPerWave loads (K, then V) follows k-step
        // i * kSteps / (2 * kInstPerWave): all of tile t+1 is in flight before
        // the softmax of tile t starts, with PV still ahead to cover its latency
        constexpr int kLoads = 2 * C::kInstPerWave;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          if ((i * C::kSteps) / kLoads == st) {
            if (i < C::kInstPerWave) pinned_issue(kr, ld_koff[i], k_fill, i);
            else pinned_issue(vr, ld_voff[i - C::kInstPerWave], v_fill, i - C::kInstPerWave);
          }
        }
      });
      __builtin_amdgcn_s_setprio(0);
      mask_keys(j0, sa, sb);
      bf16x8 pb[4];
      weights(sa, sb, pb);
      pv(v_cur, pb);
      j0 = j1;
      j1 = sanitize_id(raw2, p.n_kb);
      if (more) {
        // This wavefront's loads of tile t+1 have landed; the barrier makes
        // every wavefront's loads visible and frees the buffers just read.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    };
    for (int tt = 0; tt < cnt; tt += 2) {
      step(std::integral_constant<int, 0>(), tt);
      if (tt + 1 < cnt) step(std::integral_constant<int, 1>(), tt + 1);
    }
    // no LDS write may still be in flight when the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // Normalise and store: lane (n, g) holds columns 32cc + 8a + 4g + {0..3} of row qrow.
  const float lt = sum_with_partner(l);
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
  const void* fn = a.causal ? reinterpret_cast<const void*>(&attn_fwd_kernel<D, true>)
                           : reinterpret_cast<const void*>(&attn_fwd_kernel<D, false>);
  return hipLaunchKernel(fn,
                         dim3(static_cast<uint32_t>(grid)), dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  return a.D == 128 ? launch_t<128>(a, stream) : launch_t<64>(a, stream);
}

}  // namespace sparge
