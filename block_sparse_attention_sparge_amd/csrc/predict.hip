// Pooled-block scoring and per-row top-k selection.
//
// For every query block i of a head: s[i][j] = scale * qbar_i . kbar_j over the
// head's key blocks j (fp32 FMAs), then keep the k largest s, ties going to the
// lower j. Ranking s ranks the row's softmax identically (softmax is strictly
// increasing within a row), so no exponentials are needed. Outputs the 0/1
// mask row (mask_id of SpargeAttention Documentation, "Mask Requirements") and
// the ascending list of kept key blocks that the attention kernel walks.
//
// Causal variant (the top-k API's is_causal flag): query block i ranks only the
// key blocks 0 .. J(i) = (last row of the block) / 64, whose keys some of its
// rows may see, and keeps ceil(topk * (J(i) + 1)) of them (the host's rounding
// rule, evaluated here in double precision).
//
// CDF-threshold variant (the "cdfthreshd" mode of the inference scripts, only
// named on the pages): each row keeps its key blocks in decreasing softmax
// probability until their running sum reaches tau. The probabilities are taken
// in fp32 against the row max and turned into 31-bit fixed-point weights, whose
// integer sums are exact in any order; the cut is found by the same radix
// select with weight histograms instead of counts.
//
// One workgroup (8 wavefronts) takes R <= 8 query blocks of one head. Scores for
// all R rows live in LDS. Selection is an exact radix select on order-preserving
// 32-bit keys (4 passes of 8 bits, LDS histograms, wavefront prefix sums), one
// wavefront per row; the final pass emits the list in index order with ballots.
// No atomics touch global memory, so repeated runs give identical bytes.
#include "common.h"

namespace sparge {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

// Float -> uint32 whose unsigned order matches the float order (-0 folded to +0).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ceil(topk * n) in double, a product within 1e-9 of an integer counting as
// that integer, clamped to [1, n]: the host's k for a row of n candidates.
__device__ __forceinline__ int64_t topk_count_dev(int64_t n, double topk) {
  const double x = topk * static_cast<double>(n);
  const double r = __builtin_rint(x);
  int64_t k = (__builtin_fabs(x - r) <= 1e-9) ? static_cast<int64_t>(r) : static_cast<int64_t>(__builtin_ceil(x));
  return k < 1 ? 1 : (k > n ? n : k);
}

// Number of set bits of `m` in lanes below this lane.
__device__ __forceinline__ uint32_t count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Workgroup -> (head bh, group of query blocks). Consecutive workgroup ids go
// to consecutive XCDs. With `deal`, every group of a head runs on one XCD, so
// the head's pooled keys are fetched into one L2 instead of all eight; the
// grid then covers a multiple of 8 heads and ids past the last head get
// bh = BH (nothing to do).
__device__ __forceinline__ void work_item(int64_t n_groups, int64_t BH, int deal, int64_t& bh, int64_t& group) {
  const int64_t w = blockIdx.x;
  if (deal) {
    const int64_t it = w / kNumXcd;
    bh = (it / n_groups) * kNumXcd + (w - (w / kNumXcd) * kNumXcd);
    group = it - (it / n_groups) * n_groups;
    if (bh > BH) bh = BH;
  } else {
    bh = w / n_groups;
    group = w - bh * n_groups;
  }
}

// Writes the fp32 scores of the R pooled query rows of a group (rows past the
// last query block repeat it; their scores are never read) against every key
// block of the head to sc. The query rows are wavefront-uniform, so they are
// read through the scalar cache and feed the FMAs as scalar operands.
template <int D, int R>
__device__ __forceinline__ void pooled_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                              int64_t bh, int64_t row0, int64_t n_qb, int64_t n_kb,
                                              float scale, float* sc) {
  typedef float fv4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(4))) const fv4 cfloat4;
  const int t = threadIdx.x;
  cfloat4* qrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t qi = (row0 + r < n_qb) ? row0 + r : n_qb - 1;
    qrow[r] = (cfloat4*)(qbar + (bh * n_qb + qi) * D);
  }
  // thread t takes key blocks t, t + kThreads, ... and all R rows
  const float* kb_head = kbar + bh * n_kb * D;
  for (int j = t; j < n_kb; j += kThreads) {
    const float4* kr = reinterpret_cast<const float4*>(kb_head + static_cast<int64_t>(j) * D);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll 4
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 kv = kr[d4];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const fv4 qv = qrow[r][d4];
        acc[r] = fmaf(qv.x, kv.x, acc[r]);
        acc[r] = fmaf(qv.y, kv.y, acc[r]);
        acc[r] = fmaf(qv.z, kv.z, acc[r]);
        acc[r] = fmaf(qv.w, kv.w, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r * n_kb + j] = scale * acc[r];
  }
  __syncthreads();
}

// Candidate key blocks of query block qi: all of them, or with causal masking
// the blocks 0 .. (last row of the block) / 64.
__device__ __forceinline__ int64_t candidates(int causal, int64_t qi, int64_t N, int64_t n_kb) {
  if (!causal) return n_kb;
  const int64_t last_row = (qi + 1) * kQBlock < N ? (qi + 1) * kQBlock - 1 : N - 1;
  return last_row / kKBlock + 1;
}

template <int D, int R>
__global__ __launch_bounds__(kThreads) void predict_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int64_t N, int64_t n_qb,
    int64_t n_kb, int64_t n_groups, int64_t BH, int deal, int64_t k, double topk, int causal, float scale,
    uint8_t* __restrict__ mask, int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
  extern __shared__ float4 smem4[];
  float* sc = reinterpret_cast<float*>(smem4);             // [R][n_kb]
  uint32_t* hist = reinterpret_cast<uint32_t*>(sc + R * n_kb);   // [kWaves][256]

  int64_t bh, group;
  work_item(n_groups, BH, deal, bh, group);
  if (bh >= BH) return;
  const int64_t row0 = group * R;   // first query block of this group
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  pooled_scores<D, R>(qbar, kbar, bh, row0, n_qb, n_kb, scale, sc);

  // Selection: wavefront `wave` takes row `wave` of the group (R <= kWaves, so
  // one round; wavefronts past R or past the last query block only join the
  // barriers). Every wavefront runs the same rounds so the barriers stay uniform.
  uint32_t* h = hist + wave * 256;
  constexpr int kRounds = (R + kWaves - 1) / kWaves;
  for (int round = 0; round < kRounds; ++round) {
    const int r = wave + round * kWaves;
    const int64_t qi = row0 + r;
    const bool active = (r < R) && (qi < n_qb);
    const float* srow = sc + (r < R ? r : 0) * n_kb;
    // candidates [0, n_cand) and the number kept, k_row
    int64_t n_cand = n_kb, k_row = k;
    if (causal && active) {
      n_cand = candidates(causal, qi, N, n_kb);
      k_row = topk_count_dev(n_cand, topk);
    }

    uint32_t prefix = 0, prefix_mask = 0;
    int64_t kk = k_row;   // how many still to take among keys matching the prefix
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int q = 0; q < 4; ++q) h[lane * 4 + q] = 0u;
      __syncthreads();
      if (active) {
        for (int64_t j = lane; j < n_cand; j += 64) {
          const uint32_t u = order_key(srow[j]);
          if ((u & prefix_mask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      // Lane L owns bins 4L..4L+3. above(d) = number of candidates with a larger digit.
      const uint32_t c0 = h[lane * 4 + 0], c1 = h[lane * 4 + 1], c2 = h[lane * 4 + 2],
                     c3 = h[lane * 4 + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      // inclusive suffix sum over lanes (lanes above contribute larger digits)
      uint32_t suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += o;
      }
      const int64_t above3 = static_cast<int64_t>(suf - mine);
      const int64_t above2 = above3 + c3, above1 = above2 + c2, above0 = above1 + c1;
      int digit = -1;
      int64_t above = 0;
      if (above3 < kk && kk <= above3 + c3) { digit = lane * 4 + 3; above = above3; }
      else if (above2 < kk && kk <= above2 + c2) { digit = lane * 4 + 2; above = above2; }
      else if (above1 < kk && kk <= above1 + c1) { digit = lane * 4 + 1; above = above1; }
      else if (above0 < kk && kk <= above0 + c0) { digit = lane * 4 + 0; above = above0; }
      const uint64_t who = __ballot(digit >= 0);
      const int src = who ? (__builtin_ctzll(who)) : 0;
      digit = __shfl(digit, src, 64);
      const int64_t above_sel = __shfl(above, src, 64);
      prefix |= static_cast<uint32_t>(digit < 0 ? 0 : digit) << shift;
      prefix_mask |= 255u << shift;
      kk -= above_sel;
    }
    // prefix is now the k-th largest key; take every larger key and the first
    // kk keys equal to it in index order.
    if (active) {
      const uint32_t thr = prefix;
      const int64_t row = bh * n_qb + qi;
      int32_t* out_idx = kv_idx + row * k;
      uint8_t* out_mask = mask ? mask + row * n_kb : nullptr;
      int64_t base = 0, eq_seen = 0;
      for (int64_t j0 = 0; j0 < n_kb; j0 += 64) {
        const int64_t j = j0 + lane;
        const bool valid = j < n_cand;
        const uint32_t u = valid ? order_key(srow[j]) : 0u;
        const bool is_eq = valid && u == thr;
        const uint64_t eq_b = __ballot(is_eq);
        const int64_t eq_rank = eq_seen + count_below(eq_b);
        const bool sel = valid && (u > thr || (is_eq && eq_rank < kk));
        const uint64_t sel_b = __ballot(sel);
        const int64_t pos = base + count_below(sel_b);
        if (sel && pos < k_row) out_idx[pos] = static_cast<int32_t>(j);
        if (out_mask && j < n_kb) out_mask[j] = sel ? 1 : 0;
        base += __popcll(sel_b);
        eq_seen += __popcll(eq_b);
      }
      if (lane == 0) kv_cnt[row] = static_cast<int32_t>(k_row);
    }
  }
}

// Wavefront reductions and scans (every lane ends with the same result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return __shfl(x, 0, 64);
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return __shfl(x, 0, 64);   // lanes may round differently: take lane 0's
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// Sum of x over the lanes below this one.
__device__ __forceinline__ uint64_t wave_exclusive_u64(uint64_t x, int lane) {
  uint64_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  return incl - x;
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kFixedOne = 2147483648.0f;   // weights in units of 2^-31

template <int D, int R>
__global__ __launch_bounds__(kThreads) void predict_cdf_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int64_t N, int64_t n_qb,
    int64_t n_kb, int64_t n_groups, int64_t BH, int deal, double tau, int causal, float scale,
    uint8_t* __restrict__ mask, int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt) {
  extern __shared__ float4 smem4[];
  float* sc = reinterpret_cast<float*>(smem4);             // [R][n_kb]
  // [kWaves][256] 64-bit weight histograms, 8-byte aligned after the scores
  uint64_t* hist = reinterpret_cast<uint64_t*>(sc + ((R * n_kb + 1) & ~int64_t(1)));

  int64_t bh, group;
  work_item(n_groups, BH, deal, bh, group);
  if (bh >= BH) return;
  const int64_t row0 = group * R;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  pooled_scores<D, R>(qbar, kbar, bh, row0, n_qb, n_kb, scale, sc);

  uint64_t* h = hist + wave * 256;
  constexpr int kRounds = (R + kWaves - 1) / kWaves;
  for (int round = 0; round < kRounds; ++round) {
    const int r = wave + round * kWaves;
    const int64_t qi = row0 + r;
    const bool active = (r < R) && (qi < n_qb);
    const float* srow = sc + (r < R ? r : 0) * n_kb;
    const int64_t n_cand = active ? candidates(causal, qi, N, n_kb) : 0;

    // softmax over the candidates, as fixed-point weights
    float mx = -INFINITY;
    for (int64_t j = lane; j < n_cand; j += 64) mx = fmaxf(mx, srow[j]);
    mx = wave_max(mx);
    float z = 0.f;
    for (int64_t j = lane; j < n_cand; j += 64) z += __builtin_amdgcn_exp2f((srow[j] - mx) * kLog2eF);
    z = wave_sum(z);
    const float inv_z = (z > 0.f) ? 1.f / z : 0.f;
    auto weight = [&](int64_t j) -> uint64_t {
      const float pj = __builtin_amdgcn_exp2f((srow[j] - mx) * kLog2eF) * inv_z;
      const float f = fminf(pj * kFixedOne + 0.5f, kFixedOne);
      return static_cast<uint64_t>(f);
    };
    uint64_t w_all = 0;
    for (int64_t j = lane; j < n_cand; j += 64) w_all += weight(j);
    w_all = wave_sum_u64(w_all);
    const bool keep_all = tau >= 1.0;
    uint64_t rem = keep_all ? w_all : static_cast<uint64_t>(__builtin_ceil(tau * static_cast<double>(w_all)));
    if (rem < 1) rem = 1;

    uint32_t prefix = 0, prefix_mask = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int q = 0; q < 4; ++q) h[lane * 4 + q] = 0u;
      __syncthreads();
      if (!keep_all) {
        for (int64_t j = lane; j < n_cand; j += 64) {
          const uint32_t u = order_key(srow[j]);
          if ((u & prefix_mask) == prefix) atomicAdd(&h[(u >> shift) & 255u], weight(j));
        }
      }
      __syncthreads();
      // lane L owns bins 4L..4L+3; above(d) = weight of the candidates with a larger digit
      const uint64_t c0 = h[lane * 4 + 0], c1 = h[lane * 4 + 1], c2 = h[lane * 4 + 2], c3 = h[lane * 4 + 3];
      const uint64_t mine = c0 + c1 + c2 + c3;
      uint64_t suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint64_t o = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += o;
      }
      const uint64_t above3 = suf - mine;
      const uint64_t above2 = above3 + c3, above1 = above2 + c2, above0 = above1 + c1;
      int digit = -1;
      uint64_t above = 0;
      if (c3 && above3 < rem && rem <= above3 + c3) { digit = lane * 4 + 3; above = above3; }
      else if (c2 && above2 < rem && rem <= above2 + c2) { digit = lane * 4 + 2; above = above2; }
      else if (c1 && above1 < rem && rem <= above1 + c1) { digit = lane * 4 + 1; above = above1; }
      else if (c0 && above0 < rem && rem <= above0 + c0) { digit = lane * 4 + 0; above = above0; }
      const uint64_t who = __ballot(digit >= 0);
      const int src = who ? __builtin_ctzll(who) : 0;
      digit = __shfl(digit, src, 64);
      const uint64_t above_sel = __shfl(above, src, 64);
      prefix |= static_cast<uint32_t>(digit < 0 ? 0 : digit) << shift;
      prefix_mask |= 255u << shift;
      if (digit >= 0) rem -= above_sel;
    }

    // keep every key above the cut and, in index order, the keys equal to it
    // until their weight reaches what is still missing
    if (active) {
      const uint32_t thr = prefix;
      const int64_t row = bh * n_qb + qi;
      int32_t* out_idx = kv_idx + row * n_kb;
      uint8_t* out_mask = mask ? mask + row * n_kb : nullptr;
      int64_t base = 0;
      uint64_t eq_before = 0;
      for (int64_t j0 = 0; j0 < n_kb; j0 += 64) {
        const int64_t j = j0 + lane;
        const bool valid = j < n_cand;
        const uint32_t u = valid ? order_key(srow[j]) : 0u;
        const bool is_eq = valid && !keep_all && u == thr;
        const uint64_t w_eq = is_eq ? weight(j) : 0u;
        const uint64_t eq_cum = eq_before + wave_exclusive_u64(w_eq, lane);
        const bool sel = valid && (keep_all || u > thr || (is_eq && eq_cum < rem));
        const uint64_t sel_b = __ballot(sel);
        const int64_t pos = base + count_below(sel_b);
        if (sel) out_idx[pos] = static_cast<int32_t>(j);
        if (out_mask && j < n_kb) out_mask[j] = sel ? 1 : 0;
        base += __popcll(sel_b);
        eq_before += wave_sum_u64(w_eq);
      }
      if (lane == 0) kv_cnt[row] = static_cast<int32_t>(base);
    }
  }
}

// Heads are dealt whole to XCDs when that leaves the XCDs evenly loaded (at
// most one head in eight more on the busiest XCD than an even split).
int deal_heads(int64_t BH) {
  const int64_t per = (BH + kNumXcd - 1) / kNumXcd;
  return BH >= kNumXcd && (per * kNumXcd - BH) * 8 <= BH;
}
int64_t grid_size(int64_t BH, int64_t n_groups, int deal) {
  return deal ? kNumXcd * ((BH + kNumXcd - 1) / kNumXcd) * n_groups : BH * n_groups;
}

template <int D, int R>
hipError_t launch_predict_t(const float* qbar, const float* kbar, int64_t BH, int64_t N, int64_t n_qb,
                            int64_t n_kb, int64_t k, double topk, int causal, float scale,
                            uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream) {
  const int64_t n_groups = (n_qb + R - 1) / R;
  const size_t lds = sizeof(float) * R * n_kb + sizeof(uint32_t) * kWaves * 256;
  const int deal = deal_heads(BH);
  void* args[] = {(void*)&qbar, (void*)&kbar, (void*)&N, (void*)&n_qb, (void*)&n_kb,
                  (void*)&n_groups, (void*)&BH, (void*)&deal, (void*)&k, (void*)&topk, (void*)&causal,
                  (void*)&scale, (void*)&mask, (void*)&kv_idx, (void*)&kv_cnt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&predict_kernel<D, R>),
                         dim3(static_cast<uint32_t>(grid_size(BH, n_groups, deal))), dim3(kThreads), args, lds,
                         stream);
}

template <int D>
hipError_t launch_predict_d(const float* qbar, const float* kbar, int64_t BH, int64_t N, int64_t n_qb,
                            int64_t n_kb, int64_t k, double topk, int causal, float scale,
                            uint8_t* mask, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream) {
  if (n_kb <= 2304)
    return launch_predict_t<D, 8>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
  if (n_kb <= 4608)
    return launch_predict_t<D, 4>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
  if (n_kb <= 9216)
    return launch_predict_t<D, 2>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
  return launch_predict_t<D, 1>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
}

template <int D, int R>
hipError_t launch_cdf_t(const float* qbar, const float* kbar, int64_t BH, int64_t N, int64_t n_qb,
                        int64_t n_kb, double tau, int causal, float scale, uint8_t* mask,
                        int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream) {
  const int64_t n_groups = (n_qb + R - 1) / R;
  const size_t lds = sizeof(float) * ((R * n_kb + 1) & ~int64_t(1)) + sizeof(uint64_t) * kWaves * 256;
  const int deal = deal_heads(BH);
  void* args[] = {(void*)&qbar, (void*)&kbar, (void*)&N, (void*)&n_qb, (void*)&n_kb,
                  (void*)&n_groups, (void*)&BH, (void*)&deal, (void*)&tau, (void*)&causal, (void*)&scale,
                  (void*)&mask, (void*)&kv_idx, (void*)&kv_cnt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&predict_cdf_kernel<D, R>),
                         dim3(static_cast<uint32_t>(grid_size(BH, n_groups, deal))), dim3(kThreads), args, lds,
                         stream);
}

template <int D>
hipError_t launch_cdf_d(const float* qbar, const float* kbar, int64_t BH, int64_t N, int64_t n_qb,
                        int64_t n_kb, double tau, int causal, float scale, uint8_t* mask,
                        int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream) {
  if (n_kb <= 2304)
    return launch_cdf_t<D, 8>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
  if (n_kb <= 4608)
    return launch_cdf_t<D, 4>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
  if (n_kb <= 9216)
    return launch_cdf_t<D, 2>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
  return launch_cdf_t<D, 1>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
}

}  // namespace

hipError_t launch_predict_cdf(const float* qbar, const float* kbar, int64_t BH, int64_t N, int D,
                              double tau, int causal, float scale, uint8_t* mask, int32_t* kv_idx,
                              int32_t* kv_cnt, hipStream_t stream) {
  const int64_t n_qb = (N + kQBlock - 1) / kQBlock;
  const int64_t n_kb = (N + kKBlock - 1) / kKBlock;
  if (D == 128)
    return launch_cdf_d<128>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
  return launch_cdf_d<64>(qbar, kbar, BH, N, n_qb, n_kb, tau, causal, scale, mask, kv_idx, kv_cnt, stream);
}

hipError_t launch_predict(const float* qbar, const float* kbar, int64_t BH, int64_t N, int D,
                          int64_t k, double topk, int causal, float scale, uint8_t* mask,
                          int32_t* kv_idx, int32_t* kv_cnt, hipStream_t stream) {
  const int64_t n_qb = (N + kQBlock - 1) / kQBlock;
  const int64_t n_kb = (N + kKBlock - 1) / kKBlock;
  if (D == 128)
    return launch_predict_d<128>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
  return launch_predict_d<64>(qbar, kbar, BH, N, n_qb, n_kb, k, topk, causal, scale, mask, kv_idx, kv_cnt, stream);
}

}  // namespace sparge
