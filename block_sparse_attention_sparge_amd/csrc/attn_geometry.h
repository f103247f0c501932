// Addressing of the block-sparse attention kernel's K/V tiles: which bytes of
// global memory each lane loads, where they land in LDS, and which LDS bytes
// the MFMA operand reads take. The kernel (attn_fwd.hip) and the host-side
// address replay test use these same functions, so the test checks the code
// the GPU runs.
//
// A tile is 64 key rows of D bf16 (kRowBytes = 2D bytes) stored unpadded in
// LDS, row r at byte r * kRowBytes, with its 16-byte chunks XOR-swizzled: the
// chunk stored at physical position pc of row r is logical chunk pc ^ swz(r).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparge {
namespace geom {

constexpr int kTileRows = 64;        // keys per tile (one key block)

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kBytes = kTileRows * kRowBytes;         // one K or V tile in LDS
  static constexpr int kRowsPerInst = 64 / kChunks;            // rows one wavefront load fills (1 KiB)
  static constexpr int kInstPerWave = kTileRows / (4 * kRowsPerInst);   // loads per wavefront per tile
  static constexpr int kSteps = D / 16;                        // k-steps of QK^T
  static constexpr int kDChunks = D / 32;                      // 32-column chunks of O
};

// Chunk swizzles: K so that the 16 rows one A-operand read touches hit
// distinct banks, V so that the 4 rows of one transpose read do.
template <int D>
__host__ __device__ constexpr int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__host__ __device__ constexpr int swz_v(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }

// Row of the K tile that feeds A-operand row m, chosen so that accumulator
// register i of lane (n, g) holds key 8g + i (i < 8) or 16 + 8g + (i - 8).
__host__ __device__ constexpr int sigma(int m) {
  return 16 * ((m >> 3) >> 1) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Load e of wavefront `wave` (0..3): lane `lane` fills tile row load_row and
// physical chunk load_chunk, 16 bytes at LDS byte load_lds(wave, e) + 16 * lane
// of the tile buffer (= load_row * kRowBytes + 16 * load_chunk).
template <int D>
__host__ __device__ constexpr int load_row(int wave, int e, int lane) {
  return (wave * Tile<D>::kInstPerWave + e) * Tile<D>::kRowsPerInst + lane / Tile<D>::kChunks;
}
template <int D>
__host__ __device__ constexpr int load_chunk(int lane) { return lane % Tile<D>::kChunks; }
template <int D>
__host__ __device__ constexpr int load_lds(int wave, int e) { return (wave * Tile<D>::kInstPerWave + e) * 1024; }

// Byte offset, from the tile's first row in global memory, of the 16 bytes that
// lane loads: logical chunk load_chunk ^ swz(row) of row load_row, rows
// row_stride elements apart (a 32-bit offset: row strides are at most 2^24).
template <int D, bool kIsV>
__host__ __device__ inline uint32_t load_offset(int wave, int e, int lane, int64_t row_stride) {
  const int r = load_row<D>(wave, e, lane);
  const int pc = load_chunk<D>(lane);
  const int lc = pc ^ (kIsV ? swz_v<D>(r) : swz_k<D>(r));
  return static_cast<uint32_t>((r * row_stride + 8 * lc) * 2);
}

// Byte bound of tile j's buffer resource: the whole tile for the n_full full
// tiles, the rows left at the sequence end for tile n_full, nothing past it.
// Loads at offsets >= the bound read zeros and touch no memory.
__host__ __device__ inline uint32_t tile_bound(int32_t j, int32_t n_full, uint32_t tile_bytes,
                                               uint32_t tail_bytes) {
  return j < n_full ? tile_bytes : (j == n_full ? tail_bytes : 0u);
}

// LDS byte (in the K tile) of lane (n, g)'s A operand for k-step s: row
// sigma(n), logical chunk 2s + g; the keys 32..63 half adds 32 rows.
template <int D>
__host__ __device__ constexpr int k_read(int n, int g, int s) {
  return sigma(n) * Tile<D>::kRowBytes + 16 * ((2 * s + g) ^ swz_k<D>(sigma(n)));
}

// LDS byte (in the V tile) of a lane's transpose read for output chunk cc:
// row 8g + (lane % 16) / 4, logical chunk 4cc + 2((lane / 16) & 1) + (lane & 3) / 2,
// half lane & 1. Key step u adds 16u rows, the upper four rows of a read pair 4 rows.
template <int D>
__host__ __device__ constexpr int v_read(int lane, int cc) {
  return (8 * (lane >> 5) + ((lane & 15) >> 2)) * Tile<D>::kRowBytes +
         16 * ((4 * cc + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ swz_v<D>(8 * (lane >> 5) + ((lane & 15) >> 2))) +
         8 * (lane & 1);
}

// Workgroup -> work item of the attention launch. Items are the (head, query
// block) pairs in head-major order (item = bh * n_qb + qb). Consecutive
// workgroup ids go to consecutive XCDs, and an XCD starts its workgroups in id
// order, so the `round` workgroups resident on an XCD at once run in rounds.
// The items are cut into chunks of `round` and the chunks dealt round the XCDs,
// 0..7 in even rounds and 7..0 in odd ones: each round on an XCD takes
// consecutive items, and chunks of unequal work even out. The items left for
// a last, partial round are split over the XCDs in shares that differ by at
// most one, so that no XCD runs a whole extra chunk while the others idle. Returns false for the padding
// workgroups of the last round.
constexpr int kXcdCount = 8;
__host__ __device__ inline bool work_item(int64_t wid, int64_t n_items, int64_t round, int64_t& item) {
  const int64_t xcd = wid % kXcdCount;
  const int64_t it = wid / kXcdCount;
  const int64_t r = it / round, off = it - r * round;
  const int64_t full = n_items / (round * kXcdCount);   // rounds with a whole chunk per XCD
  if (r < full) {
    item = (r * kXcdCount + ((r & 1) ? kXcdCount - 1 - xcd : xcd)) * round + off;
  } else {
    const int64_t rest = n_items - full * round * kXcdCount;
    const int64_t per = rest / kXcdCount, extra = rest - per * kXcdCount;
    const int64_t count = per + (xcd < extra ? 1 : 0);
    const int64_t start = xcd * per + (xcd < extra ? xcd : extra);
    item = off < count ? full * round * kXcdCount + start + off : n_items;
  }
  return item < n_items;
}
// Workgroups of the launch: whole rounds of every XCD.
__host__ __device__ inline int64_t work_grid(int64_t n_items, int64_t round) {
  const int64_t per = round * kXcdCount;
  return (n_items + per - 1) / per * per;
}

}  // namespace geom
}  // namespace sparge
