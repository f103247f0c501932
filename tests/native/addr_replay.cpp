// Host replay of the block-sparse attention kernel's K/V tile addressing,
// using the kernel's own geometry functions (csrc/attn_geometry.h).
//
// For each head dimension, sequence length and token stride given, it checks:
//  - LDS writes: the 4 wavefronts x kInstPerWave loads x 64 lanes of a tile
//    fill every (row, physical chunk) of the tile buffer exactly once, inside it;
//  - global reads: for every key block j in [0, n_kb] (n_kb is where an
//    invalid list entry is sent), every lane load at an offset below the tile's
//    bound reads 16 bytes that lie inside a valid row (< N) of the head, within
//    its D columns, and holds exactly the logical chunk that the LDS position
//    expects (physical chunk ^ swizzle); loads at or past the bound touch no
//    memory; 32-bit offsets and bounds do not overflow; bounds and offsets are
//    multiples of 16 bytes, so a load is either wholly in or wholly out;
//  - LDS reads: every K A-operand read (both 32-key halves, every k-step) and
//    every V transpose read (every key step, both row quads, every output chunk)
//    lies inside the tile buffer, and the K reads fetch exactly the logical
//    chunk (2s + g) of row sigma(n) (+32) that the MFMA operand needs.
// With --map it checks instead the launch's workgroup -> work-item mapping
// (geom::work_item, geom::work_grid) for the item counts and round sizes
// given: every (head, query block) item is taken by exactly one workgroup,
// padding workgroups take none, each XCD's workgroups come in rounds of
// consecutive items, no XCD gets more than one chunk beyond another, and the
// last, partial round is split into XCD shares that differ by at most one.
// Exit status 0 when every check holds; failures are printed.
//
// usage: addr_replay [--plant tail|swizzle] D N row_stride [D N row_stride ...]
//        addr_replay --map [--plant deal] n_items round [n_items round ...]
// --plant replays a deliberately wrong variant (the tail tile bounded as a full
// tile, K loaded with V's swizzle, or the mapping without its in-round offset)
// to show the checks catch it.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../block_sparse_attention_sparge_amd/csrc/attn_geometry.h"

using namespace sparge::geom;

static long failures = 0;
static int plant = 0;   // 1: tail tile bounded as a full tile; 2: K loads with V's swizzle; 3: mapping bug
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      if (failures < 20) {                                \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);                \
        std::fprintf(stderr, "\n");                       \
      }                                                   \
      ++failures;                                         \
    }                                                     \
  } while (0)

template <int D>
static void replay(int64_t N, int64_t row_stride) {
  using T = Tile<D>;
  const int64_t n_kb = (N + 63) / 64;
  const int64_t n_full = N / 64;
  // bounds as the kernel computes them (32-bit)
  const uint64_t tile64 = 64ull * static_cast<uint64_t>(row_stride) * 2;
  const uint64_t tail64 = static_cast<uint64_t>(N - n_full * 64) * static_cast<uint64_t>(row_stride) * 2;
  CHECK(tile64 < (1ull << 32), "tile bytes %llu overflow 32 bits", (unsigned long long)tile64);
  const uint32_t tile_bytes = static_cast<uint32_t>(tile64), tail_bytes = static_cast<uint32_t>(tail64);
  CHECK(tile_bytes % 16 == 0 && tail_bytes % 16 == 0, "bounds not multiples of 16");
  // one head's valid bytes: rows 0..N-1, each D columns
  const uint64_t head_end = static_cast<uint64_t>(N - 1) * row_stride * 2 + 2 * D;

  // LDS writes: a bijection onto the tile
  std::vector<int> hits(T::kBytes / 16, 0);
  for (int wave = 0; wave < 4; ++wave)
    for (int e = 0; e < T::kInstPerWave; ++e)
      for (int lane = 0; lane < 64; ++lane) {
        const int dst = load_lds<D>(wave, e) + 16 * lane;
        const int r = load_row<D>(wave, e, lane), pc = load_chunk<D>(lane);
        CHECK(dst >= 0 && dst + 16 <= T::kBytes, "LDS write %d outside the %d-byte tile", dst, T::kBytes);
        CHECK(dst == r * T::kRowBytes + 16 * pc, "LDS write %d is not row %d chunk %d", dst, r, pc);
        if (dst >= 0 && dst + 16 <= T::kBytes) hits[dst / 16]++;
      }
  for (size_t i = 0; i < hits.size(); ++i) CHECK(hits[i] == 1, "tile chunk %zu written %d times", i, hits[i]);

  // global reads of every key block, the invalid-id block n_kb included
  for (int64_t j = 0; j <= n_kb; ++j) {
    const uint32_t bound = tile_bound(j, n_full, tile_bytes, plant == 1 ? tile_bytes : tail_bytes);
    const uint64_t base = static_cast<uint64_t>(j) * tile64;     // the kernel's 64-bit tile base
    for (int iv = 0; iv < 2; ++iv)
      for (int wave = 0; wave < 4; ++wave)
        for (int e = 0; e < T::kInstPerWave; ++e)
          for (int lane = 0; lane < 64; ++lane) {
            const int r = load_row<D>(wave, e, lane), pc = load_chunk<D>(lane);
            const uint64_t off64 = static_cast<uint64_t>(r) * row_stride * 2 +
                                   16ull * (pc ^ (iv ? swz_v<D>(r) : swz_k<D>(r)));
            const uint32_t off = (iv || plant == 2) ? load_offset<D, true>(wave, e, lane, row_stride)
                                                    : load_offset<D, false>(wave, e, lane, row_stride);
            CHECK(off64 < (1ull << 32) && off == off64, "load offset overflow (row %d, stride %lld)", r,
                  (long long)row_stride);
            CHECK(off % 16 == 0, "unaligned load offset");
            if (off >= bound) continue;                           // zero fill, no access
            const uint64_t addr = base + off;
            const int64_t key = j * 64 + r;
            CHECK(key < N, "block %lld row %d (key %lld >= N=%lld) is read", (long long)j, r, (long long)key,
                  (long long)N);
            CHECK(addr + 16 <= head_end, "read [%llu, +16) past the head's last byte %llu",
                  (unsigned long long)addr, (unsigned long long)head_end);
            const uint64_t col = addr - static_cast<uint64_t>(key) * row_stride * 2;
            CHECK(col + 16 <= static_cast<uint64_t>(2 * D), "read outside row %lld's D columns", (long long)key);
          }
  }

  // LDS reads of the MFMA operands
  for (int lane = 0; lane < 64; ++lane) {
    const int n = lane & 31, g = lane >> 5;
    for (int s = 0; s < T::kSteps; ++s)
      for (int half = 0; half < 2; ++half) {
        const int a = k_read<D>(n, g, s) + half * 32 * T::kRowBytes;
        CHECK(a >= 0 && a + 16 <= T::kBytes, "K read %d outside the tile", a);
        const int row = a / T::kRowBytes, pc = (a % T::kRowBytes) / 16;
        CHECK(a % 16 == 0 && row == sigma(n) + 32 * half && (pc ^ swz_k<D>(row)) == 2 * s + g,
              "K read of lane %d step %d takes row %d logical chunk %d", lane, s, row, pc ^ swz_k<D>(row));
      }
    for (int cc = 0; cc < T::kDChunks; ++cc)
      for (int u = 0; u < 4; ++u)
        for (int hi = 0; hi < 2; ++hi) {
          const int a = v_read<D>(lane, cc) + (16 * u + 4 * hi) * T::kRowBytes;
          CHECK(a >= 0 && a + 8 <= T::kBytes, "V read %d outside the tile", a);
          const int row = a / T::kRowBytes, pc = (a % T::kRowBytes) / 16;
          const int lc = pc ^ swz_v<D>(row);
          CHECK(row >= 16 * u && row < 16 * u + 16, "V read of key step %d in row %d", u, row);
          CHECK(lc / 4 == cc, "V read for output chunk %d takes logical chunk %d", cc, lc);
        }
  }
}

static void replay_map(int64_t n_items, int64_t round) {
  const int64_t grid = work_grid(n_items, round);
  CHECK(grid % (round * kXcdCount) == 0 && grid >= n_items && grid < n_items + round * kXcdCount,
        "grid %lld for %lld items", (long long)grid, (long long)n_items);
  std::vector<int> seen(static_cast<size_t>(n_items), 0);
  std::vector<int64_t> per_xcd(kXcdCount, 0);
  for (int64_t wid = 0; wid < grid; ++wid) {
    int64_t item;
    bool ok = work_item(wid, n_items, round, item);
    if (plant == 3) {   // the in-round offset dropped
      const int64_t it = wid / kXcdCount, r = it / round, x = wid % kXcdCount;
      item = (r * kXcdCount + ((r & 1) ? kXcdCount - 1 - x : x)) * round;
      ok = item < n_items;
    }
    if (!ok) {
      if (plant != 3)
        CHECK(item >= n_items, "workgroup %lld refused item %lld < %lld", (long long)wid, (long long)item,
              (long long)n_items);
      continue;
    }
    CHECK(item >= 0 && item < n_items, "workgroup %lld took item %lld", (long long)wid, (long long)item);
    if (item < 0 || item >= n_items) continue;
    ++seen[static_cast<size_t>(item)];
    ++per_xcd[static_cast<size_t>(wid % kXcdCount)];
    // the workgroups of one round on an XCD take consecutive items
    const int64_t it = wid / kXcdCount;
    if (it % round != 0) {
      int64_t first;
      work_item(wid - (it % round) * kXcdCount, n_items, round, first);
      CHECK(item - first == it % round, "round of XCD %lld not consecutive at workgroup %lld",
            (long long)(wid % kXcdCount), (long long)wid);
    }
  }
  for (int64_t i = 0; i < n_items; ++i)
    CHECK(seen[static_cast<size_t>(i)] == 1, "item %lld taken %d times", (long long)i, seen[static_cast<size_t>(i)]);
  int64_t lo = per_xcd[0], hi = per_xcd[0];
  for (int64_t c : per_xcd) { lo = c < lo ? c : lo; hi = c > hi ? c : hi; }
  CHECK(hi - lo <= round, "XCD loads %lld..%lld differ by more than a chunk", (long long)lo, (long long)hi);
  // the last, partial round is split evenly: its XCD shares differ by at most one
  const int64_t full = n_items / (round * kXcdCount);
  if (plant != 3 && n_items > full * round * kXcdCount) {
    std::vector<int64_t> last(kXcdCount, 0);
    for (int64_t wid = full * round * kXcdCount; wid < grid; ++wid) {
      int64_t item;
      if (work_item(wid, n_items, round, item)) ++last[static_cast<size_t>(wid % kXcdCount)];
    }
    int64_t l0 = last[0], l1 = last[0];
    for (int64_t c : last) { l0 = c < l0 ? c : l0; l1 = c > l1 ? c : l1; }
    CHECK(l1 - l0 <= 1, "last round split %lld..%lld", (long long)l0, (long long)l1);
  }
}

int main(int argc, char** argv) {
  if (argc > 1 && std::string(argv[1]) == "--map") {
    argv += 1;
    argc -= 1;
    if (argc > 2 && std::string(argv[1]) == "--plant" && std::string(argv[2]) == "deal") {
      plant = 3;
      argv += 2;
      argc -= 2;
    }
    if (argc < 3 || (argc - 1) % 2 != 0) {
      std::fprintf(stderr, "usage: addr_replay --map n_items round [...]\n");
      return 2;
    }
    int cases = 0;
    for (int i = 1; i + 1 < argc; i += 2) {
      replay_map(std::atoll(argv[i]), std::atoll(argv[i + 1]));
      ++cases;
    }
    std::printf("%d cases, %ld failures\n", cases, failures);
    return failures ? 1 : 0;
  }
  if (argc > 2 && std::string(argv[1]) == "--plant") {
    plant = std::string(argv[2]) == "tail" ? 1 : std::string(argv[2]) == "swizzle" ? 2 : 0;
    argv += 2;
    argc -= 2;
  }
  if (argc < 4 || (argc - 1) % 3 != 0) {
    std::fprintf(stderr, "usage: %s D N row_stride [...]\n", argv[0]);
    return 2;
  }
  int cases = 0;
  for (int i = 1; i + 2 < argc; i += 3) {
    const int D = std::atoi(argv[i]);
    const int64_t N = std::atoll(argv[i + 1]), st = std::atoll(argv[i + 2]);
    if (D == 128) replay<128>(N, st);
    else if (D == 64) replay<64>(N, st);
    else { std::fprintf(stderr, "bad D %d\n", D); return 2; }
    ++cases;
  }
  std::printf("%d cases, %ld failures\n", cases, failures);
  return failures ? 1 : 0;
}
