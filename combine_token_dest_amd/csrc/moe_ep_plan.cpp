// Host-side launch planning of the gfx950 dispatch/combine kernels: the
// workgroup tiles and, for dispatch, the choice and layout of the copy
// order.  Plain C++ (no device code), so it builds and is tested on the host.

#include <algorithm>
#include <cstdint>

#include "moe_ep.h"
#include "moe_ep_internal.h"

namespace moe_ep_detail {

namespace {

int round_block(int64_t threads, int max_block) {
  int64_t b = (threads + 63) / 64 * 64;
  if (b < 64) b = 64;
  if (b > max_block) b = max_block;
  return (int)b;
}

}  // namespace

// Multiply-shift constants for e / d with 0 <= e < 2^31 (Granlund &
// Montgomery 1994, Thm. 4.2 with N = 31): l = ceil(log2 d),
// magic = ceil(2^(31+l) / d), shift = 31 + l.
OwnerDiv make_owner_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
  const uint64_t magic = (uint64_t)((num + d - 1) / d);
  return OwnerDiv{magic, 31 + l};
}

// Tile of a dispatch workgroup over a row of nv vectors: 8 or 7 vectors per
// thread and up to kDispatchBlock threads, whichever leaves fewer idle lanes
// in the row's last chunk (8 on a tie).  A 14 KiB row is 896 16-byte
// vectors, 128 x 7 exactly; 128 x 8 left 1/8 of the lanes idle and measured
// ~2% slower.
LaunchShape row_tile(int64_t rows, int64_t nv) {
  LaunchShape best{(int)rows, 0, 0, 0};
  int64_t best_waste = -1;
  for (int u = 8; u >= 7; --u) {
    const int block = round_block(std::min<int64_t>(kDispatchBlock, (nv + u - 1) / u), kMaxBlock);
    const int64_t per = (int64_t)block * u;
    const int64_t chunks = std::max<int64_t>(1, (nv + per - 1) / per);
    const int64_t waste = chunks * per - nv;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best = LaunchShape{(int)rows, (int)std::min<int64_t>(kMaxGridY, chunks), block, u};
    }
  }
  return best;
}

// Source-row order.  Rows of up to 512 vectors (8 KiB of 16-byte vectors)
// take two-wave workgroups of 4 vectors per thread instead of one wave of 7
// or 8 when all of those workgroups are resident at once (MI355X: 256 CUs x
// 32 waves): 3% faster on a 16-rank round of 7 KiB rows and 2% on an
// 8-rank ragged one, but 6% slower on a 32-rank round of 8 KiB rows, whose
// 8192 rows would need two passes.
constexpr int64_t kResidentWaves = 256 * 32;

LaunchShape dispatch_shape(int64_t rows, int64_t hidden_bytes, int vec_bytes) {
  const int64_t nv = hidden_bytes / vec_bytes;
  if (nv > 256 && nv <= 512 && rows * 2 <= kResidentWaves) {
    const int block = round_block(std::min<int64_t>(kDispatchBlock, (nv + 3) / 4), kMaxBlock);
    return LaunchShape{(int)rows, 1, block, 4};
  }
  return row_tile(rows, nv);
}

// Combine: workgroups of up to kCombineBlock threads, one per (token slot,
// column chunk), in a 1-D grid whose workgroup i runs on XCD i % 8.  The
// grid holds the token slots in groups of 8 -- token 8q + x on XCD x -- and,
// within a group, chunk-major, so all chunks of a token run on one XCD back
// to back.  Past kMaxCombineGrid workgroups a workgroup loops over chunks.
// (A 2-D grid of (slots, chunks) keeps the XCD placement but sweeps chunk 0
// of every token first: 4% slower on the DeepSeek-V3 round, 11% on a
// 16-rank fp8 one.)
// Rows of at least kCombineCapChunks chunks run with at most 18 workgroups
// per CU (LDS reserved at launch, see kCombineCapLds) instead of 32: on
// 14 KiB rows (8 ranks x 128 tokens, and 16 ranks x 256 tokens of fp8
// dispatch) combine was 1.2-1.6% faster with 16-20 per CU, over three
// boxes; on a ragged 8-rank round of 8 KiB rows (2.8 ranks per token, so
// fewer row loads in flight per wave) 16-20 per CU were 3-5% slower and
// 22-24 even.
LaunchShape combine_shape(int64_t tokens, int64_t hidden, int vec_elems) {
  const int64_t nv = hidden / vec_elems;
  const int block = round_block(std::min<int64_t>(kCombineBlock, nv), kMaxCombineBlock);
  const int64_t chunks = std::max<int64_t>(1, (nv + block - 1) / block);
  const int64_t slots = (tokens + 7) / 8 * 8;
  if (slots <= 0) return LaunchShape{0, 0, block, kCombineU};
  const int64_t g = std::min<int64_t>(chunks, std::max<int64_t>(1, kMaxCombineGrid / slots));
  const int lds = (block == 64 && chunks >= kCombineCapChunks) ? kCombineCapLds : 0;
  return LaunchShape{(int)(slots * g), (int)g, block, kCombineU, lds};
}

// Do the non-NULL entries of p[0..n) lie at base + d * stride?  NULL
// entries (masked-off ranks, never read) are skipped.  On success sets base
// and stride (stride 0 with fewer than two entries); all NULL is a success.
bool common_stride(const uint8_t* const* p, int n, const uint8_t** base, int64_t* stride) {
  int d0 = -1, d1 = -1;
  for (int d = 0; d < n && d1 < 0; ++d) {
    if (!p[d]) continue;
    if (d0 < 0) d0 = d;
    else d1 = d;
  }
  *base = nullptr;
  *stride = 0;
  if (d0 < 0) return true;
  const intptr_t p0 = reinterpret_cast<intptr_t>(p[d0]);
  intptr_t st = 0;
  if (d1 >= 0) {
    const intptr_t diff = reinterpret_cast<intptr_t>(p[d1]) - p0;
    if (diff % (d1 - d0) != 0) return false;
    st = diff / (d1 - d0);
  }
  for (int d = d0; d < n; ++d)
    if (p[d] && reinterpret_cast<intptr_t>(p[d]) != p0 + (intptr_t)(d - d0) * st) return false;
  *base = reinterpret_cast<const uint8_t*>(p0 - (intptr_t)d0 * st);
  *stride = (int64_t)st;
  return true;
}

// Destination-major order: rows per XCD block such that a block's source
// rows (about 512 KiB) stay in the XCD's L2 while every destination re-reads
// them.  It launches one workgroup per (destination, row); AUTO takes it for
// groups of at most 16 ranks with ep * ep * tpr <= 16384 while the
// source-row grid alone (one workgroup per row) does not fill the chip, and
// the source-row order otherwise.  Measured before the residency cap below
// (µs per dispatch, source-row vs destination-major, one box):
//   14 KiB rows, 8 ranks: 1 token per rank 5.10 vs 4.34, 4: 5.58 vs 4.47,
//   16: 5.96 vs 5.09, 32: 7.18 vs 6.63, 64: 10.62 vs 10.44, 128: 18.58 vs
//   16.75, 256: 36.76 vs 36.04;  4 ranks: 16: 5.35 vs 4.51, 64: 6.19 vs
//   5.38, 256: 13.58 vs 12.48, 512: 26.76 vs 23.99, 1024 (4096 source rows
//   fill the chip): 53.56 vs 55.54;  16 ranks: 4: 6.16 vs 4.82, 16: 8.40 vs
//   7.66, 64: 23.01 vs 20.51;
//   8 KiB rows: 8 ranks x 32/64/128 and 16 x 32/64 tokens 2-10% faster,
//   4 x 256 even, 4 x 1024 (chip filled) 11% slower; 512-byte rows (4 and
//   8 ranks x 16 tokens) 9-13% faster.
// With 16 ranks and 256 tokens, 32 ranks, or 512-token ragged steps it was
// 1.2-2x slower (most of its workgroups copy nothing when a row reaches few
// of many ranks).  An earlier version of this kernel, whose workgroups
// waited on a longer chain of argument loads, also needed two resident
// generations of workgroups to win.
// Past those bounds, groups of at most 8 ranks whose rows are nearly all
// real tokens (at least kDmAutoMinFill of ep * tpr, host counts) also take
// the destination-major order: with the residency cap it won at nearly every
// such step measured (µs per dispatch, source-row vs destination-major; 14 KiB
// rows unless noted): 8 x 512 73.9 vs 72.4, 8 x 768 114.6 vs 107.0,
// 8 x 1024 154.1 vs 141.3, 8 x 2048 306.9 vs 276.5; 8 KiB rows 8 x 512
// 42.6 vs 33.0, 8 x 1024 86.3 vs 82.2; 16 KiB 8 x 1024 176.6 vs 154.4;
// 12 KiB 8 x 1024 129.7 vs 122.1; 6 x 512 48.3 vs 37.1, 6 x 1024 101.8 vs
// 93.7; 4 x 2048 105.6 vs 98.1 (8 KiB 60.5 vs 58.1); fp8 rows with scales
// 8 x 512 38.4 vs 31.0; except 4 x 1024 of 8 KiB rows (30.0 vs 30.8) and
// 2 x 2048 (32.0 vs 32.7).  With fewer real rows it loses: 8 x 1024 with
// each rank 60% full 93.8 vs 101.9 (75%: even, 90%: 140.8 vs 131.7), and
// ragged counts (U[0, cap], ~40% of the rows) 63.8 vs 74.3 at 8 x 1024 and
// 17.4 vs 20.8 at 8 x 512 of 8 KiB rows.  Device-count steps, whose counts
// the host does not know, keep the bounds above.
constexpr int64_t kDmBlockBytes = 512 * 1024;
constexpr int64_t kDmXcdRows = 4;            // the kernels' kXcdRows
constexpr int64_t kDmAutoMaxPairs = 16384;   // ep * ep * tpr
constexpr int kDmAutoMaxRanks = 16;
constexpr int kDmAutoFullMaxRanks = 8;
constexpr double kDmAutoMinFill = 0.8;

bool plan_dispatch(DispatchKArgs& a, int vec_bytes, int requested) {
  const int64_t rows = (int64_t)a.ep * a.tpr;
  const bool automatic = requested == MOE_EP_ORDER_AUTO;
  a.order = MOE_EP_ORDER_SOURCE_ROW;
  a.dm_items = 0;
  if (requested == MOE_EP_ORDER_SOURCE_ROW) return true;
  int64_t real_rows = 0;
  for (int s = 0; s < a.ep; ++s) real_rows += a.src[s].n;
  const bool full_small_group = a.dev_n == nullptr && a.ep <= kDmAutoFullMaxRanks && rows > 0 &&
                                (double)real_rows >= kDmAutoMinFill * (double)rows;
  if (automatic && !full_small_group && (a.ep > kDmAutoMaxRanks || rows * a.ep > kDmAutoMaxPairs)) return true;
  // Rows per XCD (the kernel hands rows to the XCDs in blocks of
  // kDmXcdRows), and rows per XCD block, a multiple of kDmXcdRows.
  const int64_t rmax = (rows + 8 * kDmXcdRows - 1) / (8 * kDmXcdRows) * kDmXcdRows;
  int64_t b = kDmBlockBytes / std::max<int64_t>(1, a.hidden_bytes);
  b = std::min<int64_t>(b, std::max<int64_t>(kDmXcdRows, rmax)) / kDmXcdRows * kDmXcdRows;
  b = std::max<int64_t>(kDmXcdRows, b);
  const int64_t nq = rmax > 0 ? (rmax + b - 1) / b : 0;
  const LaunchShape tile = row_tile(0, a.hidden_bytes / vec_bytes);
  const int64_t nv = a.hidden_bytes / vec_bytes;
  const int64_t chunks = std::max<int64_t>(1, (nv + (int64_t)tile.block * tile.u - 1) / ((int64_t)tile.block * tile.u));
  // the product is formed in double first: in int64 it can overflow
  const double est = 8.0 * (double)nq * a.ep * (double)b * (double)chunks;
  if (est + a.ep > 2147483647.0) return automatic;     // AUTO falls back to the source-row order
  const int64_t items = 8 * nq * a.ep * b * chunks;
  if (automatic && !full_small_group) {
    const LaunchShape src = dispatch_shape(rows, a.hidden_bytes, vec_bytes);
    if (rows >= kResidentWaves / ((src.block + 63) / 64)) return true;    // the source-row grid fills the chip
  }
  a.order = MOE_EP_ORDER_DESTINATION;
  a.dm_block_rows = (int32_t)b;
  a.dm_blocks = (int32_t)nq;
  a.dm_chunks = (int32_t)chunks;
  a.dm_items = items;
  a.dm_u = tile.u;
  a.dm_threads = tile.block;
  return true;
}

// Destination-major residency cap: 16 KiB of LDS per workgroup leaves room
// for 10 workgroups per CU (160 KiB) instead of 16.  In interleaved sweeps
// (µs per dispatch, uncapped vs capped) it made the lean kernel faster once
// its grid holds at least 8192 workgroups, two generations of the uncapped
// residency: 8 ranks x 128 tokens of 14 KiB rows 15.66-15.76 vs 15.44-15.49,
// of 8 KiB rows (one-wave workgroups) 10.56-10.61 vs 10.10-10.13, 16 x 64
// 19.35-19.51 vs 19.21-19.24, 4 x 512 1-2% faster; smaller grids were even
// or slower (16 x 16: 6.69-6.73 vs 6.88).  The kernel with scale rows or
// statistics rows was 18-25% slower capped (fp8 rows, 8 x 128), and so was
// the source-row kernel (5-25%), so neither is capped.
constexpr int64_t kDmCapItems = 8192;
constexpr int kDmCapLds = 16384;

int dispatch_dst_lds(int64_t items, bool lean) {
  return lean && items >= kDmCapItems ? kDmCapLds : 0;
}

}  // namespace moe_ep_detail
