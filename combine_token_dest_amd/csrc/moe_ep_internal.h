// Internal interface between the C-ABI host code (moe_ep_api.cpp) and the
// gfx950 kernels (moe_ep_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ep.h"

namespace moe_ep_detail {

constexpr int kMaxRanks = MOE_EP_MAX_RANKS;

// Byte offsets of one rank's partition of the workspace.  Partition d starts
// at d * part_stride; the per-token destination masks follow the last one.
struct Layout {
  int64_t off_hidden;    // [ep*cap, hidden_row_bytes]
  int64_t off_scale;     // [ep*cap, scale_row_bytes]
  int64_t off_ids;       // [ep*cap, top_k] int32
  int64_t off_weights;   // [ep*cap, top_k] float
  int64_t off_combine;   // [ep*cap, hidden_size * combine_max_elem_bytes]
  int64_t off_eplb;      // [ep, eplb_stats_bytes]
  int64_t part_stride;   // bytes per rank partition
  int64_t off_route;     // [ep, cap] uint64 destination masks
  int64_t off_tokens;    // [ep*cap] TokenRec, one per real token in source-rank order (host-count steps)
  int64_t off_counts;    // [ep] int32 token counts of the last dispatch (device-count steps)
  int64_t total;         // workspace bytes
};

// Exact division of expert ids by experts-per-rank with a multiply and a
// shift (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994, Thm. 4.2, with N = 31): for 0 <= e < 2^31,
// e / epr == (e * magic) >> shift.
struct OwnerDiv {
  uint64_t magic;
  uint32_t shift;
};

// What combine needs of real token b (source-rank order): its destination
// mask and where it sits.  Written by dispatch, read with one 16-byte load.
struct alignas(16) TokenRec {
  uint64_t mask;
  int32_t s;
  int32_t t;
};

// What the dispatch kernels read of one source rank: one 64-byte record, so
// a workgroup gets all of it with one scalar load (in separate per-field
// tables it took two dependent round trips to four cache lines).
struct SourceRank {
  const uint8_t* hidden;               // [n, hidden_row_bytes]
  const int32_t* ids;                  // [n, top_k]
  const float* weights;                // [n, top_k], or NULL
  const uint8_t* scale;                // [n, scale_row_bytes], or NULL
  const uint8_t* eplb;                 // its statistics row, or NULL
  int32_t n;                           // local_num_tokens
  int32_t token_start;                 // prefix sum of n over the ranks before (host counts only)
  int64_t pad[2];
};
static_assert(sizeof(SourceRank) == 64, "one cache line per source rank");

// Arguments of the dispatch kernels.  The launcher passes the item decode
// (the div_* constants, the plan values, ep and tpr) as leading scalar
// kernel arguments, preloaded into registers at wave launch, and a
// DispatchArgs<MR> by value after them.  Its scalars come first and
// contiguous, so a workgroup gets the rest of them in one batch of scalar
// loads, together with its source rank's record (spread over 3 KB of
// arguments, they had cost each workgroup a chain of dependent scalar-cache
// round trips before its first data load).
struct DispatchArgsHead {
  OwnerDiv div_chunks;                 // destination-major decode: / dm_chunks (set by the launcher)
  OwnerDiv div_block_rows;             //   / dm_block_rows
  OwnerDiv div_ep;                     //   / ep
  OwnerDiv div_tpr;                    // receive row r / tpr
  int32_t ep;
  int32_t tpr;
  int32_t top_k;
  int32_t num_experts;
  int32_t dm_chunks;                   // destination-major order: column chunks per row,
  int32_t dm_block_rows;               //   rows per block on one XCD,
  int32_t dm_blocks;                   //   blocks per XCD
  int32_t invalid_id;
  int32_t block;                       // threads per workgroup of the launch (blockDim.x; set by the launcher)
  int32_t grid_y;                      // source-row order: column chunks in the grid (gridDim.y; set by the launcher)
  uint64_t active;                     // active ranks & ((1 << ep) - 1)
  OwnerDiv owner;
  uint8_t* ws;                         // workspace base
  int64_t part_stride;
  int64_t off_hidden, off_scale, off_ids, off_weights;
  int64_t hidden_bytes;                // H
  int64_t scale_bytes;                 // S (0 when no scales are forwarded)
  uint64_t* route;                     // [ep, tpr] destination masks (inside ws)
  TokenRec* tokens;                    // [N] records of the real tokens (host counts only)
  const int32_t* dev_n;                // device token counts, or NULL to use n[]
  int32_t* counts;                     // [ep] counts the kernel used (read by combine)
  int32_t has_weights;
  int32_t scale_vec4;                  // scale rows copied as 4-byte words (else bytes)
  int32_t order;                       // MOE_EP_ORDER_SOURCE_ROW or MOE_EP_ORDER_DESTINATION
  int32_t dm_u;                        // vectors per thread (7 or 8) and threads per workgroup
  int32_t dm_threads;
  int32_t eplb_vec4;                   // statistics copied as 4-byte words (else bytes)
  int64_t dm_items;                    // (destination, row, chunk) items
  int64_t off_eplb;
  int64_t eplb_bytes;                  // 0 when no statistics are gathered
  int64_t pad1[6];                     // the per-rank records start on a 64-byte boundary
};
static_assert(sizeof(DispatchArgsHead) % 64 == 0, "per-rank records on 64-byte boundaries");

// The head and one record per source rank, for groups of up to MR ranks.
// The host builds the MR = kMaxRanks form; a group of at most kSmallGroup
// ranks launches with the kSmallGroup form (see kSmallGroup).
template <int MR>
struct DispatchArgs : DispatchArgsHead {
  SourceRank src[MR];                  // per source rank
};
using DispatchKArgs = DispatchArgs<kMaxRanks>;

// Arguments of the combine kernel.  The launcher passes the fields every
// workgroup needs before its first row load (chunk_div through eo_stride)
// as leading scalar kernel arguments, preloaded into registers, and a
// CombineArgs<MR> by value after them for the rest.
struct CombineArgsHead {
  OwnerDiv chunk_div;                       // workgroup index / 8 / chunks
  int32_t ntok;                             // token slots (slots past it store nothing)
  int32_t chunks;                           // column chunks of a row per token in the grid
  int32_t block;                            // threads per workgroup (blockDim.x)
  int32_t tpr;
  const TokenRec* tokens;                   // [token_start[ep]] (host-count steps)
  int64_t hidden;                           // elements per row
  // When every read rank's expert_output lies at eo_base + d * eo_stride (the
  // library's own combine buffers always do), row addresses are computed
  // from these instead of loaded from the per-rank table.
  const uint8_t* eo_base;
  int64_t eo_stride;
  const uint64_t* route;                    // [ep, tpr]
  const int32_t* dev_counts;                // counts written by dispatch (device-count steps), else NULL
  OwnerDiv tpr_div;                         // slot / tpr (device-count steps)
  int32_t ep;
};

template <int MR>
struct CombineArgs : CombineArgsHead {
  const uint8_t* expert_output[MR];         // per rank d: [ep*tpr, hidden]
  uint8_t* output[MR];                      // per source rank s: [n_s, hidden]
  int32_t token_start[MR + 1];              // prefix sums of n_s (host counts)
};
using CombineKArgs = CombineArgs<kMaxRanks>;

// Groups of at most kSmallGroup ranks launch with argument blocks sized for
// kSmallGroup ranks: 888 bytes of kernel arguments for dispatch and 328 for
// combine, instead of 4472 and 1448.  On this stack a kernel whose arguments
// fit in 1 KiB starts ~3 us sooner on an idle GPU (launch + synchronise
// 11.3-11.8 us against 13.0-14.9 us from 1088 bytes up) and costs the host
// ~0.5-1 us less per launch.  The kernels read no implicit arguments
// (blockDim and gridDim come in the argument block), which would add 256
// bytes.
constexpr int kSmallGroup = 8;
static_assert(sizeof(DispatchArgs<kSmallGroup>) + 64 <= 1024 && sizeof(CombineArgs<kSmallGroup>) + 64 <= 1024,
              "the small argument blocks (after at most 64 bytes of leading arguments) fit in 1 KiB");

// Launch configurations, chosen by timing variants on MI355X in the same
// alternation the bench uses (8 workspaces rotated so the 256 MB MALL holds
// none of the data between uses; 8 dispatches then 8 combines), mostly with
// the DeepSeek-V3-shaped round (ep 8, 128 tokens per rank, 14 KiB rows):
//  - dispatch: up to 128 threads with 7 or 8 vectors of 16 B each, whichever
//    leaves fewer idle lanes (a 14 KiB row is 128 x 7).  In the source-row
//    order all waves of a workgroup store a destination row before moving to
//    the next: interleaving the destinations per vector halved throughput,
//    and staggered orders, blocked lane maps or several rows per workgroup
//    were 2-10% slower.  Destination-major workgroups of one wave, 4 waves
//    or 7 waves were 7-58% slower than 2.
//  - combine: one column vector per thread, one-wave workgroups over
//    column chunks of a row, the chunks of one token on one XCD, all (up
//    to 8) destination rows loaded in one batch.  On the DeepSeek-V3 round
//    the XCD placement made the small tiles faster than a whole row per
//    896-thread workgroup; the same tiles placed round-robin over the XCDs
//    were no faster than it.  One wave beat two by 1% there and 2.4% on a
//    32-rank round of 8 KiB rows (0.4% behind on a 16-rank fp8 round).
//    One batch of 8 rows was 5% faster than 2 vectors x 4 rows per batch.
//  - nontemporal loads and stores in both (the cache policies are in the
//    kernels): cached combine loads were ~40% slower, and sc1 or default
//    dispatch stores ~45% slower.
//  Capping the grid below one workgroup per row (persistent loops) was
//  slower for both kernels, and a grid-stride loop alone cost combine 15%
//  (its route-mask load became a vector load).
constexpr int kMaxBlock = 512;           // dispatch workgroups (launch bound)
constexpr int kMaxCombineBlock = 64;     // combine workgroups (launch bound)
constexpr int64_t kMaxGridY = 65535;     // chunks beyond this are looped over inside a workgroup
constexpr int64_t kMaxCombineGrid = 1 << 24;     // combine workgroups; beyond, chunks loop
constexpr int kDispatchBlock = 128;      // dispatch threads per workgroup, at most
constexpr int kCombineU = 1;             // combine: vectors per thread
constexpr int kCombineDB = 8;            // combine: destination rows loaded per batch
constexpr int kCombineBlock = 64;        // combine threads per workgroup, at most
// Combine residency cap for long rows: LDS reserved per one-wave
// workgroup so that at most 18 share a CU (160 KiB of LDS each), taken when
// a token's row spans at least kCombineCapChunks column chunks.
constexpr int kCombineCapLds = 9088;
constexpr int64_t kCombineCapChunks = 12;

struct LaunchShape {
  int grid_x;   // dispatch: rows; combine: workgroups (token slots rounded up to 8, x chunks)
  int grid_y;   // column chunks of a row (combine: per token, in the 1-D grid)
  int block;    // threads per workgroup
  int u;        // vectors per thread
  int lds = 0;  // dynamic LDS bytes per workgroup, reserved only to cap residency (unused by the code)
};

// Fills a.order and the destination-major fields for a step: `requested` is
// the params' dispatch_order.  Returns false when the destination order was
// asked for but its grid would not fit.
bool plan_dispatch(DispatchKArgs& a, int vec_bytes, int requested);

// Dynamic LDS bytes to reserve per destination-major workgroup (never
// touched by the code): a residency cap for the lean instantiation on grids
// of at least two resident generations, else 0.
int dispatch_dst_lds(int64_t items, bool lean);

// Enqueue one dispatch kernel (after plan_dispatch).  vec_bytes in
// {16, 8, 4, 2, 1} must divide hidden_bytes and every hidden row pointer.
hipError_t launch_dispatch(const DispatchKArgs& a, int vec_bytes, hipStream_t stream);

// Enqueue one combine kernel over a.token_start[ep] tokens.  vec_elems must
// divide the hidden size and every row pointer's alignment in elements.
hipError_t launch_combine(const CombineKArgs& a, int dtype, int vec_elems, hipStream_t stream);

// Multiply-shift constants for x / d with 0 <= x < 2^31 (host code).
OwnerDiv make_owner_div(uint32_t d);

// Where moe_ep_dispatch_noalloc keeps the records its combine reads: the
// library's fixed device array on one GPU (MOE_EP_NOALLOC_MAX_ROWS rows).
struct NoallocArea {
  uint64_t* route;     // [MOE_EP_NOALLOC_MAX_ROWS] destination masks
  TokenRec* tokens;    // [MOE_EP_NOALLOC_MAX_ROWS] token records
  int32_t* counts;     // [MOE_EP_MAX_RANKS] counts of a device-count step
  int64_t bytes;       // size of the array
};

// The array's address on `device` (looked up once per device, with that
// device current; later calls return the kept address).  Host code.
hipError_t noalloc_scratch(int device, NoallocArea* out);

// Whether the non-NULL entries of p[0..n) lie at *base + d * *stride (host code).
bool common_stride(const uint8_t* const* p, int n, const uint8_t** base, int64_t* stride);

// Launch shapes the two launchers use (host code, moe_ep_plan.cpp).
LaunchShape row_tile(int64_t rows, int64_t nv);
LaunchShape dispatch_shape(int64_t rows, int64_t hidden_bytes, int vec_bytes);
LaunchShape combine_shape(int64_t tokens, int64_t hidden, int vec_elems);

}  // namespace moe_ep_detail
