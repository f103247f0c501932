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
//   (sigma in attn_geometry.h) so that the S^T accumulators hold consecutive keys, which is
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
//   instructions), double buffered with one barrier per tile. The loads are
//   issued as inline assembly, invisible to the compiler's wait insertion: the
//   only wait for them is the explicit vmcnt(0) before the barrier that
//   publishes a stage, so reads of the current stage never wait on them.
//   MFMA operands are read from LDS ahead of their use (K two k-steps ahead,
//   V^T two MFMAs ahead), an order imposed on the scheduler with
//   sched_group_barrier: left to itself it reads each operand right before
//   its MFMA and the MFMA waits out the LDS latency. The loads of
//   tile t+1 are interleaved one by one with the QK MFMAs of tile t: issued as
//   a burst right after the barrier, the loads of all eight wavefronts of a CU
//   fill the vector-memory queue and stall instruction issue for hundreds of
//   cycles. Tiles are stored unpadded (64 KB of LDS per workgroup at
//   D=128, so two workgroups share a CU) with 16-byte chunks XOR-swizzled per
//   row: K so that the 16 rows one A-operand read touches hit distinct banks,
//   V so that the 4 rows of one transpose read do.
//   Workgroups are numbered so that each round of an XCD's resident
//   workgroups (each XCD has its own L2) takes consecutive query blocks of one
//   head while all XCDs move through the heads together: one head's K/V stays
//   hot in the last-level cache, and the workgroups sharing an L2 start
//   together on neighbouring query blocks, whose lists overlap.
#include <type_traits>

#include "attn_geometry.h"
#include "common.h"

namespace sparge {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSumLog2 = 20;            // per-lane weight sum that triggers a new reference max
constexpr float kSumLimit = static_cast<float>(1 << kSumLog2);
// Word 3 of a raw (untyped) buffer resource on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
// sched_group_barrier instruction classes: MFMA (0x8), LDS reads (0x100).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedLdsRead = 0x100;

// Consecutive work items dealt to an XCD at a time. At D=128 these are the
// workgroups an XCD (32 CUs) holds at once, two per CU (64 KB of LDS each).
// At D=64 an XCD holds 128, but its tiles are half the size and its L2 keeps
// most of them anyway, and smaller chunks spread the last, partial round over
// more XCDs: 32 measured best there.
template <int D>
constexpr int64_t kRound = D == 128 ? 64 : 32;
static_assert(geom::kXcdCount == kNumXcd, "one XCD count");

template <int D>
struct Cfg : geom::Tile<D> {
  static constexpr int kTile = geom::Tile<D>::kBytes;       // one K or V tile in LDS
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
  int64_t n_items;     // B * H * n_qb (head, query block) pairs
  Strides qs, ks, vs, os;
  float c;             // scale * log2(e)
};

// Key block of a list entry. An id outside [0, n_kb) maps to a block past the
// end of the sequence whose keys are all masked (its tile loads read nothing),
// so a corrupt list entry contributes nothing instead of reading out of bounds.
__device__ __forceinline__ int32_t sanitize_id(int32_t j, int32_t n_kb) {
  return (j >= 0 && j < n_kb) ? j : n_kb;
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

// One LDS-DMA load: 16 bytes per lane from buffer `rs` at byte offset `voff`
// into LDS at byte address `lds` + 16 * lane (m0 holds the LDS address; it is
// an input operand, so the compiler sets it and knows its value). Issued as
// inline assembly with no result registers, so the compiler does not see an
// LDS write: the one wait for these loads is the explicit vmcnt(0) before the
// barrier that publishes a stage.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D, bool kCausal, bool kSameKV>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(Params p) {
  using C = Cfg<D>;
  // Tile buffers: K stage 0, K stage 1, V stage 0, V stage 1.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::kTile];

  // Workgroup -> (head, query block) by geom::work_item: at D=128 the
  // workgroups resident on an XCD (kRound of them) run in rounds that start,
  // and walk their ascending lists, together, and each round takes consecutive
  // query blocks (lists that overlap) of one head, while all XCDs work on
  // about one head at a time. Causal lists grow with the block index, so each head's
  // blocks are taken longest first: the short lists fill in at the end.
  int64_t bh, qb;
  {
    int64_t item;
    if (!geom::work_item(blockIdx.x, p.n_items, kRound<D>, item)) return;
    bh = item / p.n_qb;
    qb = item - bh * p.n_qb;
    if constexpr (kCausal) qb = p.n_qb - 1 - qb;
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
  auto raw_id = [&](int i) -> int32_t { return (i < cnt) ? (list ? list[i] : i) : 0; };
  const int32_t n_kb32 = static_cast<int32_t>(p.n_kb);
  const int32_t n32 = static_cast<int32_t>(p.N);

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
  float mref = 0.f;        // m, or 0 while m is unset (m only changes on the exact path)
  bool all_ref = false;    // wavefront-uniform: every lane has a reference m
  float l = 0.f;

  // ---- per-lane LDS geometry (constant over the walk; see attn_geometry.h)
  int koff[C::kSteps];
#pragma unroll
  for (int s = 0; s < C::kSteps; ++s) koff[s] = geom::k_read<D>(n, g, s);
  int voff[C::kDChunks];
#pragma unroll
  for (int cc = 0; cc < C::kDChunks; ++cc) voff[cc] = geom::v_read<D>(lane, cc);

  // ---- global -> LDS: wavefront load e fills rows [r0, r0 + kRowsPerInst) of a tile.
  // Loads go through a buffer resource per tile (scalar base and byte bound) with
  // a fixed 32-bit per-lane offset; rows past N fall outside the bound and read
  // as zeros (their scores are masked), so ragged and invalid blocks need no
  // special path.
  uint32_t ld_koff[C::kInstPerWave], ld_voff[C::kInstPerWave];
#pragma unroll
  for (int e = 0; e < C::kInstPerWave; ++e) {
    ld_koff[e] = geom::load_offset<D, false>(wave, e, lane, p.ks.n);
    ld_voff[e] = geom::load_offset<D, true>(wave, e, lane, p.vs.n);
  }
  // Tile j of an operand starts j * tile_bytes past its head; its bound is the
  // whole tile, the rows left at the sequence end, or nothing (j past the end).
  const int32_t n_full = static_cast<int32_t>(p.N / kKBlock);
  const uint32_t k_tile = static_cast<uint32_t>(kKBlock * p.ks.n * 2);
  const uint32_t v_tile = static_cast<uint32_t>(kKBlock * p.vs.n * 2);
  const uint32_t k_tail = static_cast<uint32_t>((p.N - n_full * kKBlock) * p.ks.n * 2);
  const uint32_t v_tail = static_cast<uint32_t>((p.N - n_full * kKBlock) * p.vs.n * 2);
  auto tile_rsrc = [&](const uint16_t* base, int32_t j, uint32_t tile_bytes, uint32_t tail_bytes) {
    const uint32_t bound = geom::tile_bound(j, n_full, tile_bytes, tail_bytes);
    const uint64_t ptr = reinterpret_cast<uint64_t>(base) + static_cast<uint64_t>(static_cast<uint32_t>(j)) * tile_bytes;
    i32x4 r;
    r[0] = static_cast<int>(static_cast<uint32_t>(ptr));
    r[1] = static_cast<int>(static_cast<uint32_t>(ptr >> 32) & 0xffffu);
    r[2] = static_cast<int>(bound);
    r[3] = kBufferFlags;
    return r;
  };
  // LDS byte address of this wavefront's part of the tile buffers (load_lds is
  // linear: load_lds(wave, e) = load_lds(wave, 0) + load_lds(0, e)). It is made
  // opaque once per step, so the compiler forms each load's address with one
  // scalar add instead of keeping sixteen addresses live (and spilled to
  // vector lanes).
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds_wave = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem)) +
                            static_cast<uint32_t>(geom::load_lds<D>(wave_s, 0));
  auto issue_one = [&](i32x4 rs, uint32_t off, uint32_t lds_base, int buf, int e) {
    dma16(rs, off, lds_base + buf * C::kTile + geom::load_lds<D>(0, e));
  };
  auto issue = [&](int32_t j, int kbuf, int vbuf) {
    const i32x4 kr = tile_rsrc(kh, j, k_tile, k_tail);
    const i32x4 vr = tile_rsrc(vh, j, v_tile, v_tail);
#pragma unroll
    for (int e = 0; e < C::kInstPerWave; ++e) {
      issue_one(kr, ld_koff[e], lds_wave, kbuf, e);
      issue_one(vr, ld_voff[e], lds_wave, vbuf, e);
    }
  };

  // S^T = K Q^T for keys [0, 32) and [32, 64) of a tile; hook(s) runs after k-step s.
  auto qk = [&](const char* kb, f32x16& s0, f32x16& s1, auto hook) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
    // K fragments two k-steps ahead of their MFMAs
    bf16x8 ka[2][2];
    auto rd = [&](int s, bf16x8 (&d)[2]) {
      d[0] = *reinterpret_cast<const bf16x8*>(kb + koff[s]);
      d[1] = *reinterpret_cast<const bf16x8*>(kb + koff[s] + 32 * C::kRowBytes);
    };
    rd(0, ka[0]);
    if (C::kSteps > 1) rd(1, ka[1]);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      const bf16x8 a0 = ka[s & 1][0], a1 = ka[s & 1][1];
      if (s + 2 < C::kSteps) rd(s + 2, ka[s & 1]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[s], s1, 0, 0, 0);
      hook(s);
    }
    // issue order: the first two k-steps' K reads, then per k-step its two
    // MFMAs followed by the reads of the k-step two ahead
    __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 4, 0);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      if (s + 2 < C::kSteps) __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 2, 0);
    }
  };

  // Keys past N in a ragged (or invalid) block take no weight, and with causal
  // masking neither do keys after this lane's query row. Only tiles at the
  // sequence end or across the block's diagonal need the per-key test.
  auto mask_keys = [&](int32_t j, f32x16& s0, f32x16& s1) {
    const int32_t k0 = j * kKBlock;
    if (k0 + kKBlock > n32 || (kCausal && k0 + kKBlock - 1 > static_cast<int32_t>(qb) * kQBlock)) {
      // keys k0 + lim and later are masked; register i of this lane holds key
      // 8g + i (i < 8) or 8g + 16 + (i - 8)
      int32_t lim32 = n32 - k0;
      if (kCausal && static_cast<int32_t>(qrow) - k0 + 1 < lim32) lim32 = static_cast<int32_t>(qrow) - k0 + 1;
      const int lim = (lim32 < 0 ? 0 : (lim32 > kKBlock ? kKBlock : lim32)) - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = (i < 8) ? i : 16 + (i - 8);
        if (kl >= lim) s0[i] = -INFINITY;
        if (kl + 32 >= lim) s1[i] = -INFINITY;
      }
    }
  };

  // Probabilities of a tile as bf16 PV operands, against reference mref (log2
  // units); returns this lane's sum of the rounded weights (two independent
  // dot2 chains).
  auto probs = [&](const f32x16& s0, const f32x16& s1, float mref, bf16x8 (&pb)[4]) -> float {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float la = 0.f, lb = 0.f;
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
      la = __builtin_amdgcn_fdot2_f32_bf16(b0, ones, la, false);
      lb = __builtin_amdgcn_fdot2_f32_bf16(b1, ones, lb, false);
    }
    return la + lb;
  };

  // Softmax weights of a tile. The running max m only serves as a reference
  // that keeps the weights in range, so it is not recomputed per tile: the
  // weights are taken against the current m, and only when a lane's weights
  // sum past 2^kSumLog2 (a score far above m), or some lane of the wavefront
  // has no reference yet, is the tile's exact row max taken, m raised to it, O
  // and l rescaled, and the weights recomputed. Weights up to 2^kSumLog2 are
  // as exact in bf16 and fp32 as weights below 1, and the accumulators have
  // ample range for them. (A row without a reference takes the exact path
  // whatever its weights: against the placeholder reference 0 they may all
  // have underflowed to zero.)
  auto weights = [&](const f32x16& s0, const f32x16& s1, bf16x8 (&pb)[4]) {
    // m stays -inf only while every key seen so far was masked (invalid ids);
    // a reference of 0 then gives zero weights instead of NaN.
    float lt = probs(s0, s1, mref, pb);
    if (!all_ref || __builtin_amdgcn_ballot_w64(!(lt <= kSumLimit))) {
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
      all_ref = __builtin_amdgcn_ballot_w64(m == -INFINITY) == 0;
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
    // issue order: the first two MFMAs' V^T reads, then each MFMA followed by
    // the reads of the MFMA two ahead
    __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * C::kDChunks; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + 2 < 4 * C::kDChunks) __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 2, 0);
    }
  };

  if (cnt > 0) {
    // Double buffering: step t computes tile t from buffers t%2 while the
    // loads of tile t+1 fill the other pair.
    int32_t j0 = sanitize_id(raw_id(0), n_kb32);
    int32_t j1 = sanitize_id(raw_id(1), n_kb32);
    issue(j0, 0, 2);
    // Buffer resources of the loads a step issues (tile t+1 in step t), set
    // at the end of the previous step, where the wavefront goes on to wait at
    // the barrier: the scalar work is off the path into the next QK. Past the
    // last tile they hold no bytes, so those loads only write zeros into the
    // buffers just released. With equal K and V token strides one product
    // and one bound serve both.
    i32x4 kr, vr;
    kr[3] = kBufferFlags;
    vr[3] = kBufferFlags;
    const uint64_t kbase = reinterpret_cast<uint64_t>(kh), vbase = reinterpret_cast<uint64_t>(vh);
    auto set_next = [&](int32_t j) {
      const uint64_t kp = kbase + static_cast<uint64_t>(static_cast<uint32_t>(j)) * k_tile;
      const uint32_t kb = geom::tile_bound(j, n_full, k_tile, k_tail);
      kr[0] = static_cast<int>(static_cast<uint32_t>(kp));
      kr[1] = static_cast<int>(static_cast<uint32_t>(kp >> 32) & 0xffffu);
      kr[2] = static_cast<int>(kb);
      uint64_t vp;
      uint32_t vb;
      if constexpr (kSameKV) {
        vp = vbase + (kp - kbase);
        vb = kb;
      } else {
        vp = vbase + static_cast<uint64_t>(static_cast<uint32_t>(j)) * v_tile;
        vb = geom::tile_bound(j, n_full, v_tile, v_tail);
      }
      vr[0] = static_cast<int>(static_cast<uint32_t>(vp));
      vr[1] = static_cast<int>(static_cast<uint32_t>(vp >> 32) & 0xffffu);
      vr[2] = static_cast<int>(vb);
    };
    set_next(cnt > 1 ? j1 : n_kb32);
    // vmcnt(0) as a builtin, so that the compiler counts the Q loads as done too
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();

    // The next tile's loads are spread through this tile's QK MFMAs, one load
    // per k-step.
    auto step = [&](auto parity, int tt) {
      constexpr int P = decltype(parity)::value;
      const char* k_cur = smem + (P ? 1 : 0) * C::kTile;
      const char* v_cur = smem + (P ? 3 : 2) * C::kTile;
      constexpr int k_fill = P ? 0 : 1;
      constexpr int v_fill = P ? 2 : 3;
      uint32_t lds_base = lds_wave;
      asm volatile("" : "+s"(lds_base));
      const bool more = tt + 1 < cnt;
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
            if (i < C::kInstPerWave) issue_one(kr, ld_koff[i], lds_base, k_fill, i);
            else issue_one(vr, ld_voff[i - C::kInstPerWave], lds_base, v_fill, i - C::kInstPerWave);
          }
        }
      });
      __builtin_amdgcn_s_setprio(0);
      // The block id two tiles ahead is read here: the softmax has no LDS
      // reads for its scalar load to hold up (scalar and LDS loads share a
      // counter, and an outstanding scalar load forces full waits), and it has
      // landed by the time PV waits for its first operands.
      const int32_t raw2 = static_cast<int32_t>(raw_id(tt + 2));
      mask_keys(j0, sa, sb);
      bf16x8 pb[4];
      weights(sa, sb, pb);
      // the block id's scalar load has long landed; saying so here lets PV's
      // operand waits count LDS reads only
      __builtin_amdgcn_s_waitcnt(0xc07f);
      pv(v_cur, pb);
      j0 = j1;
      j1 = sanitize_id(raw2, n_kb32);
      if (more) {
        set_next(tt + 2 < cnt ? j1 : n_kb32);
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
  p.qs = a.qs; p.ks = a.ks; p.vs = a.vs; p.os = a.os;
  p.c = a.scale * kLog2e;
  p.n_items = a.B * a.H * p.n_qb;
  const int64_t grid = geom::work_grid(p.n_items, kRound<D>);
  void* args[] = {(void*)&p};
  const bool same = a.ks.n == a.vs.n;
  const void* fn = a.causal ? (same ? reinterpret_cast<const void*>(&attn_fwd_kernel<D, true, true>)
                                    : reinterpret_cast<const void*>(&attn_fwd_kernel<D, true, false>))
                            : (same ? reinterpret_cast<const void*>(&attn_fwd_kernel<D, false, true>)
                                    : reinterpret_cast<const void*>(&attn_fwd_kernel<D, false, false>));
  return hipLaunchKernel(fn,
                         dim3(static_cast<uint32_t>(grid)), dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  return a.D == 128 ? launch_t<128>(a, stream) : launch_t<64>(a, stream);
}

}  // namespace sparge
