// gfx950 kernels of rank-major MoE expert-parallel dispatch and combine.
//
// The whole EP group lives in one GPU: rank d's receive region and combine
// input region are partition d of one workspace.  Both operations are pure
// data movement (plus one float32 add per element and routed row in
// combine), so they are bound by HBM bandwidth; the kernels aim at 16-byte
// coalesced accesses, every input byte read once from HBM, and no workspace
// traffic beyond what the method moves.
//
// dispatch works out each token's destination ranks from its top_k expert
//   ids (contiguous ownership, masked by the active ranks), writes the top_k
//   ids/weights slot of its receive row r = s*tpr + t on every rank (the
//   token's own where routed, invalid_expert_id / 0.0 elsewhere) and copies
//   its hidden and scale rows to every destination.  Two kernels do this in
//   different orders (same bytes): dispatch_kernel, one workgroup per row r
//   that loads the row once and stores it to each destination in turn, and
//   dispatch_dst_kernel, one workgroup per (destination, row) with rows
//   pinned to XCDs so re-reads hit L2.  Both also write, for each real token,
//   the record combine starts from (mask and position).
//   Placement and invalid rows: flashinfer.moe_ep.NVLinkOneSidedAlltoAll,
//   class description; routing: flashinfer.moe_ep.MoEEpCommunication,
//   dispatch(); mask: NVLinkOneSidedAlltoAll, dispatch().
//
// combine: one one-wave workgroup per (real token (s, t < n_s), 1 KiB column
//   chunk).  It reads the token's record and loads its chunk of the token's
//   row from every destination rank (ascending), adds them in float32 in
//   that order starting from +0.0, rounds once and stores the output chunk.
//   Rows of ranks the token did not reach are never read.
//   flashinfer.moe_ep.MoEEpCommunication, combine().

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "moe_ep_internal.h"

namespace moe_ep_detail {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int B> struct Bytes;
template <> struct Bytes<16> { typedef u32x4 type; };
template <> struct Bytes<8> { typedef u32x2 type; };
template <> struct Bytes<4> { typedef uint32_t type; };
template <> struct Bytes<2> { typedef uint16_t type; };
template <> struct Bytes<1> { typedef uint8_t type; };


__device__ __forceinline__ int expert_owner(const OwnerDiv& od, uint32_t e) {
  return (int)(((uint64_t)e * od.magic) >> od.shift);
}

// Row accesses go through buffer resources: one resource per row (base
// address, byte size) lets the hardware discard any access past the row,
// lanes need only 32-bit offsets, and the instruction carries an explicit
// cache policy (CP):
//   0 = default, 2 = nt (nontemporal), 16 = sc1, 17 = sc0 sc1, 18 = sc1 nt.
enum : int { kCpDefault = 0, kCpNt = 2, kCpSc1 = 16, kCpSc0Sc1 = 17, kCpSc1Nt = 18 };

// Buffer resource word 3 for raw (unswizzled, stride 0) buffers on gfx9-class parts.
constexpr int kRawBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferFlags);
}

template <int VB, int CP>
__device__ __forceinline__ typename Bytes<VB>::type buf_load(__amdgpu_buffer_rsrc_t r, int off) {
  typedef typename Bytes<VB>::type V;
  if constexpr (VB == 16) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP));
  } else if constexpr (VB == 8) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP));
  } else if constexpr (VB == 4) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP));
  } else if constexpr (VB == 2) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP));
  } else {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, CP));
  }
}

// The same load through a plain global address (GL rows in combine).
template <int VB, int CP>
__device__ __forceinline__ typename Bytes<VB>::type glob_load(const uint8_t* p) {
  typedef typename Bytes<VB>::type V;
  if constexpr (CP == kCpNt) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}

template <int VB, int CP>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int off, const typename Bytes<VB>::type& v) {
  if constexpr (VB == 16) {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)) W;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(W, v), r, off, 0, CP);
  } else if constexpr (VB == 8) {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)) W;
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(W, v), r, off, 0, CP);
  } else if constexpr (VB == 4) {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0)) W;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(W, v), r, off, 0, CP);
  } else if constexpr (VB == 2) {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b16(r, 0, 0, 0)) W;
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(W, v), r, off, 0, CP);
  } else {
    typedef decltype(__builtin_amdgcn_raw_buffer_load_b8(r, 0, 0, 0)) W;
    __builtin_amdgcn_raw_buffer_store_b8(__builtin_bit_cast(W, v), r, off, 0, CP);
  }
}

// Cache policies of the row accesses (see the tuning notes with the launch
// constants in moe_ep_internal.h).
constexpr int kDispatchLP = kCpNt;
constexpr int kDispatchSP = kCpNt;
constexpr int kCombineLP = kCpNt;
constexpr int kCombineSP = kCpNt;

// ---------------------------------------------------------------------------
// dispatch
//
// Source-row order: one receive row r = s*tpr + t per workgroup (and
// column chunk).  Every workgroup works out the row's destination mask (one
// id load per lane); chunk 0 (blockIdx.y == 0) also writes the route mask,
// the token record, the ids/weights slot of row r on every rank and the
// scale row.  Each thread holds U vectors of VB bytes of its column chunk.
// ---------------------------------------------------------------------------
// Destination mask of token (s, t): lane j of every wave loads id j, the
// owner bits are OR-ed across the lanes (a single load for top_k <= 64), and
// the active-rank mask is applied.  Zero for padding rows.
template <class A>
__device__ __forceinline__ uint64_t route_token(const A& a, const int32_t* __restrict__ idr, const bool real) {
  if (!real) return 0;
  const int K = a.top_k;
  const int lane = threadIdx.x & 63;
  uint64_t m = 0;
  for (int j0 = 0; j0 < K; j0 += 64) {
    uint64_t bit = 0;
    if (j0 + lane < K) {
      const uint32_t e = (uint32_t)idr[j0 + lane];
      if (e < (uint32_t)a.num_experts) bit = 1ull << expert_owner(a.owner, e);
    }
    const int jn = K - j0 < 64 ? K - j0 : 64;
    for (int j = 0; j < jn; ++j) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bit, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bit >> 32), j);
      m |= ((uint64_t)hi << 32) | lo;
    }
  }
  return m & a.active;
}

// Slot j of receive row r on rank d: the token's id and weight when d
// receives it, else the invalid id and 0.0.  (Both branches are written out
// so the compiler does not merge the two sources into one flat load.)
template <class A>
__device__ __forceinline__ void write_slot(const A& a, uint8_t* part, const int r, const int j, const bool routed,
                                           const int32_t* __restrict__ idr, const float* __restrict__ wr) {
  const int64_t slot = (int64_t)r * a.top_k + j;
  int32_t* ids_out = reinterpret_cast<int32_t*>(part + a.off_ids) + slot;
  float* w_out = reinterpret_cast<float*>(part + a.off_weights) + slot;
  if (routed) {
    const int32_t id = idr[j];
    if (a.has_weights) *w_out = wr[j];
    *ids_out = id;
  } else {
    *ids_out = a.invalid_id;
    if (a.has_weights) *w_out = 0.0f;
  }
}

// What a dispatch workgroup needs to find its item (row, destination,
// chunk) and source rank.  These are the kernels' leading scalar arguments,
// preloaded into scalar registers at wave launch, so the first memory access
// of a workgroup is its source rank's argument record.  The four divisions
// are multiply-shift constants (Granlund-Montgomery, as make_owner_div), the
// four shift counts packed into one word so that all of it fits the
// preloadable registers.
struct DispatchHead {
  uint64_t m_chunks, m_block_rows, m_ep, m_tpr;
  uint32_t shifts;                     // bytes: chunks, block_rows, ep, tpr
  int32_t dm_chunks, dm_block_rows, ep, tpr;
};

// x / d for 0 <= x < 2^31 with the multiply-shift constant of d and the
// shift count in byte `which` of h.shifts.
__device__ __forceinline__ int hdiv(uint64_t magic, uint32_t shifts, int which, int x) {
  return (int)(((uint64_t)(uint32_t)x * magic) >> ((shifts >> (8 * which)) & 0xff));
}

// Token count of source rank s for this step.  DEVN: read from device memory
// when the kernel runs (clamped to the rows the buffers hold) and recorded
// for combine; else the host's count.  The two are separate instantiations:
// the run-time test alone cost ~2% on the DeepSeek-V3-shaped dispatch.
template <bool DEVN, class A>
__device__ __forceinline__ int step_count(const A& a, const int s, const bool first, const int tpr) {
  if (!DEVN) return a.src[s].n;
  const int c = a.dev_n[s];
  const int ns = c < 0 ? 0 : (c > tpr ? tpr : c);
  if (first && threadIdx.x == 0) a.counts[s] = ns;
  return ns;
}

template <int VB, int U, int LP, int SP, bool DEVN, class A>
__device__ __forceinline__ void dispatch_row(const A& a, const DispatchHead& h, const int r) {
  typedef typename Bytes<VB>::type V;
  const int s = hdiv(h.m_tpr, h.shifts, 3, r);
  const int t = r - s * h.tpr;
  const int K = a.top_k;
  const int ns = step_count<DEVN>(a, s, t == 0 && blockIdx.y == 0, h.tpr);
  const bool real = t < ns;
  const int32_t* __restrict__ idr = a.src[s].ids + (int64_t)t * K;
  const int64_t nv = a.hidden_bytes / VB;
  const int64_t per_block = (int64_t)a.block * U;
  // A padding row (t >= n_s) has no source row: its resource has size 0, so
  // the hardware discards its loads (they return 0 and touch no memory).
  const __amdgpu_buffer_rsrc_t src =
      row_rsrc(a.src[s].hidden + (int64_t)t * a.hidden_bytes, real ? a.hidden_bytes : 0);
  const int64_t c_first = (int64_t)blockIdx.y * per_block;

  // The first chunk of the token's hidden row is loaded before the routing
  // is known, so its latency overlaps that of the expert ids.  Lanes past
  // the end of the row load column 0 and store nothing.  The loads are
  // unconditional: behind a branch, the compiler waited for them at the
  // join before the ids load (5% slower on the ragged workload).
  int off[U];
  bool live[U];
  V v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c_first + threadIdx.x + (int64_t)u * a.block;
    live[u] = c < nv;
    off[u] = live[u] ? (int)(c * VB) : 0;
    v[u] = buf_load<VB, LP>(src, off[u]);
  }

  const uint64_t m = route_token(a, idr, real);

  if (blockIdx.y == 0) {
    if (threadIdx.x == 0) {
      a.route[r] = m;
      if (!DEVN && real) a.tokens[a.src[s].token_start + t] = TokenRec{m, s, t};
    }
    // ids / weights slot of row r on every rank.
    const float* __restrict__ wr = a.has_weights ? a.src[s].weights + (int64_t)t * K : nullptr;
    const int slots = a.ep * K;
    for (int i = threadIdx.x; i < slots; i += a.block) {
      const int d = i / K;
      write_slot(a, a.ws + (int64_t)d * a.part_stride, r, i - d * K, (m >> d) & 1, idr, wr);
    }
    // Scale row (a few hundred bytes), row-aligned with hidden.
    if (m && a.scale_bytes) {
      const int64_t S = a.scale_bytes;
      const int64_t dst_off = a.off_scale + (int64_t)r * S;
      if (a.scale_vec4) {
        const int64_t nw = S / 4;
        const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(a.src[s].scale + (int64_t)t * S);
        for (int64_t c = threadIdx.x; c < nw; c += a.block) {
          const uint32_t x = ssrc[c];
          uint64_t mm = m;
          while (mm) {
            const int d = __builtin_ctzll(mm);
            mm &= mm - 1;
            reinterpret_cast<uint32_t*>(a.ws + (int64_t)d * a.part_stride + dst_off)[c] = x;
          }
        }
      } else {
        const uint8_t* ssrc = a.src[s].scale + (int64_t)t * S;
        for (int64_t c = threadIdx.x; c < S; c += a.block) {
          const uint8_t x = ssrc[c];
          uint64_t mm = m;
          while (mm) {
            const int d = __builtin_ctzll(mm);
            mm &= mm - 1;
            (a.ws + (int64_t)d * a.part_stride + dst_off)[c] = x;
          }
        }
      }
    }
  }
  if (m == 0) return;

  // Store each chunk to every destination; further chunks (rows longer than
  // the grid's chunks) are loaded here.
  const int64_t dst_off = a.off_hidden + (int64_t)r * a.hidden_bytes;
  for (int64_t c0 = c_first; c0 < nv; c0 += (int64_t)a.grid_y * per_block) {
    if (c0 != c_first) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + threadIdx.x + (int64_t)u * a.block;
        live[u] = c < nv;
        off[u] = live[u] ? (int)(c * VB) : 0;
        v[u] = buf_load<VB, LP>(src, off[u]);
      }
    }
    uint64_t mm = m;
    while (mm) {
      const int d = __builtin_ctzll(mm);
      mm &= mm - 1;
      const __amdgpu_buffer_rsrc_t dst = row_rsrc(a.ws + (int64_t)d * a.part_stride + dst_off, a.hidden_bytes);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) buf_store<VB, SP>(dst, off[u], v[u]);
    }
  }
}

// Gathers source rank s's expert-load statistics into row s of the
// [ep, eplb_bytes] statistics region of every rank.
template <class A>
__device__ __forceinline__ void gather_stats_row(const A& a, const int s) {
  const int64_t B = a.eplb_bytes;
  const int64_t dst_off = a.off_eplb + (int64_t)s * B;
  if (a.eplb_vec4) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.src[s].eplb);
    for (int64_t c = threadIdx.x; c < B / 4; c += a.block) {
      const uint32_t x = src[c];
      for (int d = 0; d < a.ep; ++d)
        reinterpret_cast<uint32_t*>(a.ws + (int64_t)d * a.part_stride + dst_off)[c] = x;
    }
  } else {
    const uint8_t* src = a.src[s].eplb;
    for (int64_t c = threadIdx.x; c < B; c += a.block) {
      const uint8_t x = src[c];
      for (int d = 0; d < a.ep; ++d) (a.ws + (int64_t)d * a.part_stride + dst_off)[c] = x;
    }
  }
}

// Receive rows go to the XCDs in blocks of kXcdRows consecutive rows, so the
// ids / weights slots of those rows (32 bytes each for top_k = 8: a 128-byte
// line holds four) are written by one XCD's L2 as whole lines.  Handed out
// row by row, the four slots of a line came from four XCDs as partial lines:
// DeepSeek-V3-shaped dispatch 1-1.5% slower, a ragged one 2%.
constexpr int kXcdRows = 4;

// Row of source-row workgroup i (workgroup i runs on XCD i mod 8): within
// each full group of 8 * kXcdRows rows, XCD x takes rows
// kXcdRows * x .. kXcdRows * x + kXcdRows - 1; rows past the last full group
// (and the statistics rows after them) keep their index.
__device__ __forceinline__ int source_row_of(const int i, const int rows) {
  constexpr int G = 8 * kXcdRows;
  return i < (rows & ~(G - 1)) ? (i & ~(G - 1)) + kXcdRows * (i & 7) + ((i >> 3) & (kXcdRows - 1)) : i;
}

// Grid: x = receive row (source_row_of the workgroup index; r = s*tpr + t),
// then one statistics row per source rank when statistics are gathered;
// y = column chunk of the hidden row.
template <int VB, int U, int LP, int SP, bool DEVN, int MR>
__global__ void __launch_bounds__(kMaxBlock)
dispatch_kernel(const uint64_t m_chunks, const uint64_t m_block_rows, const uint64_t m_ep, const uint64_t m_tpr,
                const uint32_t shifts, const int32_t dm_chunks, const int32_t dm_block_rows, const int32_t ep,
                const int32_t tpr, const DispatchArgs<MR> a) {
  // One workgroup per item (no grid-stride loop: a store of one item could
  // then alias the next item's loads, which keeps the compiler from using
  // scalar loads for the uniform ones).
  const DispatchHead h{m_chunks, m_block_rows, m_ep, m_tpr, shifts, dm_chunks, dm_block_rows, ep, tpr};
  const int rows = ep * tpr;
  const int r = source_row_of(blockIdx.x, rows);
  if (r < rows) {
    dispatch_row<VB, U, LP, SP, DEVN>(a, h, r);
  } else if (blockIdx.y == 0) {
    gather_stats_row(a, r - rows);
  }
}

// ---------------------------------------------------------------------------
// dispatch, destination-major order
//
// One workgroup per (destination d, receive row r, column chunk).  Work-
// groups go to the 8 XCDs round-robin (workgroup i runs on XCD i mod 8), so
// item i is decoded as: XCD x = i mod 8 owns the rows in every kXcdRows-row
// block b with b = x (mod 8); on an XCD the rows come in blocks of
// dm_block_rows (a multiple of kXcdRows) and, within a block, in
// destination-major order.  All destinations of a row therefore read it on
// the same XCD within a short window: the first read comes from HBM, the
// others from that XCD's L2 (cached loads), while each destination's rows
// are written as one sequential sweep (nontemporal stores).
// LEAN: the common step shape -- top_k <= 64, no scale rows, no statistics
// rows -- without the loops and branches the general one needs; it took
// ~0.3 us (1.6%) off the DeepSeek-V3-shaped dispatch in interleaved runs.
// ---------------------------------------------------------------------------
template <int VB, int U, int SP, bool DEVN, bool LEAN, class A>
__device__ __forceinline__ void dispatch_dst_item(const A& a, const DispatchHead& h, const int i) {
  typedef typename Bytes<VB>::type V;
  // 32-bit decode: the host keeps the item count below 2^31.
  const int rows = h.ep * h.tpr;
  const int x = i & 7;
  int k = i >> 3;
  int k1 = hdiv(h.m_chunks, h.shifts, 0, k);
  const int chunk = k - k1 * h.dm_chunks;
  k = k1;
  k1 = hdiv(h.m_block_rows, h.shifts, 1, k);
  const int j = k - k1 * h.dm_block_rows;
  k = k1;
  const int q = hdiv(h.m_ep, h.shifts, 2, k);
  const int d = k - q * h.ep;
  const int xm = q * h.dm_block_rows + j;            // the XCD's xm-th row
  const int r = 8 * kXcdRows * (xm / kXcdRows) + kXcdRows * x + (xm % kXcdRows);
  if (r >= rows) return;
  const int s = hdiv(h.m_tpr, h.shifts, 3, r);
  const int t = r - s * h.tpr;
  const int K = a.top_k;
  const int ns = step_count<DEVN>(a, s, t == 0 && d == 0 && chunk == 0, h.tpr);
  const bool real = t < ns;
  const int32_t* __restrict__ idr = a.src[s].ids + (int64_t)t * K;

  const int64_t nv = a.hidden_bytes / VB;
  const int64_t c0 = (int64_t)chunk * a.block * U;
  const __amdgpu_buffer_rsrc_t src = row_rsrc(a.src[s].hidden + (int64_t)t * a.hidden_bytes, a.hidden_bytes);
  int off[U];
  bool live[U];
  V v[U];
  // Cached loads: the row's other destinations re-read it from L2.
  auto load_row = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + threadIdx.x + (int64_t)u * a.block;
      live[u] = c < nv;
      off[u] = live[u] ? (int)(c * VB) : 0;
      v[u] = buf_load<VB, kCpDefault>(src, off[u]);
    }
  };
  // Destination mask of the token (as route_token, written out here: this
  // form measured ~3% faster in this kernel).
  uint64_t m = 0;
  uint32_t e = 0xffffffffu;             // LEAN: lane j's expert id and weight
  float wv = 0.0f;
  if (LEAN) {
    // top_k <= 64: id and weight j in lane j, then the row right behind
    // them, so the row is in flight while the mask is worked out (the wait
    // for the ids does not wait for the row).  A padding row's resource has
    // size 0: its loads return 0 and touch no memory.  With this, the ids
    // and weights stored from registers: 1.8% faster on the DeepSeek-V3
    // round than loading the row after the metadata stores.
    const __amdgpu_buffer_rsrc_t src_row =
        row_rsrc(a.src[s].hidden + (int64_t)t * a.hidden_bytes, real ? a.hidden_bytes : 0);
    const int lane = threadIdx.x & 63;
    if (real && lane < K) {
      e = (uint32_t)idr[lane];
      if (a.has_weights) wv = a.src[s].weights[(int64_t)t * K + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + threadIdx.x + (int64_t)u * a.block;
      live[u] = c < nv;
      off[u] = live[u] ? (int)(c * VB) : 0;
      v[u] = buf_load<VB, kCpDefault>(src_row, off[u]);
    }
    uint64_t bit = 0;
    if (e < (uint32_t)a.num_experts) bit = 1ull << expert_owner(a.owner, e);
    for (int jj = 0; jj < K; ++jj) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bit, jj);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bit >> 32), jj);
      m |= ((uint64_t)hi << 32) | lo;
    }
    m &= a.active;
  } else if (real) {
    const int lane = threadIdx.x & 63;
    for (int j0 = 0; j0 < K; j0 += 64) {
      uint64_t bit = 0;
      if (j0 + lane < K) {
        const uint32_t e = (uint32_t)idr[j0 + lane];
        if (e < (uint32_t)a.num_experts) bit = 1ull << expert_owner(a.owner, e);
      }
      const int jn = K - j0 < 64 ? K - j0 : 64;
      for (int jj = 0; jj < jn; ++jj) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bit, jj);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bit >> 32), jj);
        m |= ((uint64_t)hi << 32) | lo;
      }
    }
    m &= a.active;
  }
  const bool routed = (m >> d) & 1;     // uniform over the workgroup
  uint8_t* part = a.ws + (int64_t)d * a.part_stride;

  if (chunk == 0) {
    if (d == 0 && threadIdx.x == 0) {
      a.route[r] = m;
      if (!DEVN && real) a.tokens[a.src[s].token_start + t] = TokenRec{m, s, t};
    }
    // This destination's ids / weights slot of row r.  LEAN: lane j of the
    // first wave stores slot j from its registers.  Otherwise written as
    // selects (the compiler turns the id select into one load from either
    // source): here that measured a few percent faster than write_slot's
    // branches, which the source-row kernel keeps.
    if (LEAN) {
      if (threadIdx.x < K) {
        const int64_t slot = (int64_t)r * K + threadIdx.x;
        reinterpret_cast<int32_t*>(part + a.off_ids)[slot] = routed ? (int32_t)e : a.invalid_id;
        if (a.has_weights) reinterpret_cast<float*>(part + a.off_weights)[slot] = routed ? wv : 0.0f;
      }
    } else {
      for (int jj = threadIdx.x; jj < K; jj += a.block) {
        const int64_t slot = (int64_t)r * K + jj;
        reinterpret_cast<int32_t*>(part + a.off_ids)[slot] = routed ? idr[jj] : a.invalid_id;
        if (a.has_weights)
          reinterpret_cast<float*>(part + a.off_weights)[slot] = routed ? a.src[s].weights[(int64_t)t * K + jj] : 0.0f;
      }
    }
    if (!LEAN && routed && a.scale_bytes) {
      const int64_t S = a.scale_bytes;
      uint8_t* dst = part + a.off_scale + (int64_t)r * S;
      if (a.scale_vec4) {
        const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(a.src[s].scale + (int64_t)t * S);
        for (int64_t c = threadIdx.x; c < S / 4; c += a.block) reinterpret_cast<uint32_t*>(dst)[c] = ssrc[c];
      } else {
        const uint8_t* ssrc = a.src[s].scale + (int64_t)t * S;
        for (int64_t c = threadIdx.x; c < S; c += a.block) dst[c] = ssrc[c];
      }
    }
  }
  // General shape: the row is loaded after the metadata stores (loading it
  // before the routing was known measured slower when the ids and weights
  // were loaded again for the stores).
  if (!routed) return;
  if (!LEAN) load_row();

  const __amdgpu_buffer_rsrc_t dst =
      row_rsrc(part + a.off_hidden + (int64_t)r * a.hidden_bytes, a.hidden_bytes);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (live[u]) buf_store<VB, SP>(dst, off[u], v[u]);
}

// Grid: x = destination-major item, then one statistics row per source rank
// when statistics are gathered.
template <int VB, int U, int SP, bool DEVN, bool LEAN, int MR>
__global__ void __launch_bounds__(kMaxBlock)
dispatch_dst_kernel(const uint64_t m_chunks, const uint64_t m_block_rows, const uint64_t m_ep, const uint64_t m_tpr,
                    const uint32_t shifts, const int32_t dm_chunks, const int32_t dm_block_rows, const int32_t ep,
                    const int32_t tpr, const DispatchArgs<MR> a) {
  const DispatchHead h{m_chunks, m_block_rows, m_ep, m_tpr, shifts, dm_chunks, dm_block_rows, ep, tpr};
  const int i = blockIdx.x;
  if (LEAN || i < a.dm_items) {
    dispatch_dst_item<VB, U, SP, DEVN, LEAN>(a, h, i);
  } else {
    gather_stats_row(a, i - (int)a.dm_items);
  }
}

// ---------------------------------------------------------------------------
// combine
//
// Grid (1-D): one workgroup per (token slot, column chunk), the chunks of a
// token on one XCD (see combine_kernel).  Each thread owns U column vectors
// of VE elements; it loads them from up to DB destination rows at a time
// (ascending rank) before adding, so one batch covers every destination
// when the token reached at most DB ranks.
// ---------------------------------------------------------------------------
// Raw storage of VE elements of a combine dtype.
template <int DT, int VE> struct CVec;
template <int VE> struct CVec<MOE_EP_F32, VE> { typedef typename Bytes<VE * 4>::type type; };
template <int VE> struct CVec<MOE_EP_BF16, VE> { typedef typename Bytes<VE * 2>::type type; };
template <int VE> struct CVec<MOE_EP_F16, VE> { typedef typename Bytes<VE * 2>::type type; };

// acc += v (widened to float32) when `use`, else acc += +0.0.  The
// accumulator starts at +0.0 and a round-to-nearest sum is -0.0 only when
// both operands are -0.0, so acc is never -0.0 and adding +0.0 leaves it
// bit-identical: the unused slots change nothing, and no branch stands
// between the loads and the adds.
template <int DT, int VE>
__device__ __forceinline__ void unpack_add(const typename CVec<DT, VE>::type& v, float (&acc)[VE], bool use) {
  if constexpr (DT == MOE_EP_F32) {
    uint32_t w[VE];
    __builtin_memcpy(w, &v, sizeof(w));
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = acc[i] + (use ? __uint_as_float(w[i]) : 0.0f);
  } else if constexpr (DT == MOE_EP_F16) {
    // binary16 -> float32 is exact (v_cvt_f32_f16).
    uint16_t h[VE];
    __builtin_memcpy(h, &v, sizeof(h));
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = acc[i] + (use ? (float)__builtin_bit_cast(_Float16, h[i]) : 0.0f);
  } else if constexpr (VE == 1) {
    acc[0] = acc[0] + (use ? __uint_as_float((uint32_t)v << 16) : 0.0f);
  } else {
    uint32_t w[VE / 2];
    __builtin_memcpy(w, &v, sizeof(w));
#pragma unroll
    for (int i = 0; i < VE / 2; ++i) {
      acc[2 * i] = acc[2 * i] + (use ? __uint_as_float(w[i] << 16) : 0.0f);
      acc[2 * i + 1] = acc[2 * i + 1] + (use ? __uint_as_float(w[i] & 0xffff0000u) : 0.0f);
    }
  }
}

template <int DT, int VE>
__device__ __forceinline__ typename CVec<DT, VE>::type pack(const float (&acc)[VE]) {
  typename CVec<DT, VE>::type v;
  if constexpr (DT == MOE_EP_F32) {
    uint32_t w[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) w[i] = __float_as_uint(acc[i]);
    __builtin_memcpy(&v, w, sizeof(w));
  } else if constexpr (DT == MOE_EP_F16) {
    // float32 -> binary16, round to nearest even (v_cvt_f16_f32 in the
    // default rounding mode; overflow gives infinity).
    uint16_t h[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) h[i] = __builtin_bit_cast(uint16_t, (_Float16)acc[i]);
    __builtin_memcpy(&v, h, sizeof(h));
  } else {
    // float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
    uint16_t h[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) h[i] = __builtin_bit_cast(uint16_t, (__bf16)acc[i]);
    __builtin_memcpy(&v, h, sizeof(h));
  }
  return v;
}

// The arguments a combine workgroup needs before its first row load.  They
// are the kernel's leading scalar arguments, which the dispatcher preloads
// into scalar registers at wave launch (built with
// -amdgpu-kernarg-preload-count), so the first memory access of a workgroup
// is its token record: 1.2% faster on the DeepSeek-V3 round's combine and
// 3.8% on a ragged one than loading them from the argument block.
struct CombineHead {
  const TokenRec* tokens;
  const uint8_t* eo_base;
  int64_t eo_stride;
  int64_t hidden;
  int32_t block;
  int32_t chunks;
};

// The argument set of the compact combine launch (the all-scalar combine_kernel):
// outputs at a constant stride instead of a per-rank table.
struct CompactCombine {
  int32_t tpr;
  uint8_t* out_base;
  int64_t out_stride;
};

// Output row base of source rank s.
template <class A>
__device__ __forceinline__ uint8_t* output_of(const A& a, const int s) {
  return a.output[s];
}
__device__ __forceinline__ uint8_t* output_of(const CompactCombine& a, const int s) {
  return a.out_base + (int64_t)s * a.out_stride;
}

// Expert-output base of rank d: from the base and stride, or the per-rank table.
template <bool STRIDED, class A>
__device__ __forceinline__ const uint8_t* expert_output_of(const A& a, const CombineHead& h, const int d) {
  if constexpr (STRIDED) return h.eo_base + (int64_t)d * h.eo_stride;
  else return a.expert_output[d];
}

template <int DT, int VE, int U, int DB, int LP, int SP, bool ONEPASS, bool STRIDED, bool DEVN, bool GL, class A>
__device__ __forceinline__ void combine_token(const A& a, const CombineHead& h, const int b,
                                              const int chunk, const bool store) {
  typedef typename CVec<DT, VE>::type V;
  int s;
  int t;
  uint64_t m;
  if constexpr (DEVN) {
    // Slots of every possible token (b = s*tpr + t); those past the count
    // dispatch used hold none.
    s = (int)(((uint64_t)b * a.tpr_div.magic) >> a.tpr_div.shift);
    t = b - s * a.tpr;
    if (t >= a.dev_counts[s]) return;
    m = a.route[b];
  } else {
    // Real token b's record, written by dispatch: one load instead of a
    // search over the per-source prefix followed by the mask load.
    const u32x4 rec = *reinterpret_cast<const u32x4*>(h.tokens + b);    // {mask lo, mask hi, s, t}
    m = ((uint64_t)rec.y << 32) | rec.x;
    s = (int)rec.z;
    t = (int)rec.w;
  }
  const int64_t r = (int64_t)s * a.tpr + t;
  const int64_t nv = h.hidden / VE;
  constexpr int esz = DT == MOE_EP_F32 ? 4 : 2;
  const int64_t row_bytes = h.hidden * esz;
  const int64_t per_block = (int64_t)h.block * U;
  constexpr int VB = VE * esz;
  const __amdgpu_buffer_rsrc_t out = row_rsrc(output_of(a, s) + (int64_t)t * row_bytes, row_bytes);

  auto pass = [&](const int64_t c0) {
    // Lanes past the end of the row read column 0 (in bounds) and store
    // nothing, so every load below is unconditional and they all issue
    // before the first add waits.
    int off[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + threadIdx.x + (int64_t)u * h.block;
      live[u] = c < nv;
      off[u] = live[u] ? (int)(c * VB) : 0;
    }
    float acc[U][VE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[u][i] = 0.0f;

    uint64_t mm = m;
    // One batch: the next DBX destination rows in ascending rank order;
    // slots past the last one repeat it (its loads are already in flight)
    // and add +0.0.
    auto batch = [&](auto dbx) {
      constexpr int DBX = decltype(dbx)::value;
      V v[DBX][U];
      int cnt = 0;
      if constexpr (GL) {
        // Plain global addresses.  A batch with no row left loads nothing
        // (the call sites never make one), so slot 0 is always a routed row
        // and every other slot is a routed row or a copy of the one before.
        if (mm == 0) return;
        auto row_of = [&](const int d) { return expert_output_of<STRIDED>(a, h, d) + r * row_bytes; };
        const uint8_t* rows[DBX];
        rows[0] = row_of(__builtin_ctzll(mm));
        mm &= mm - 1;
        cnt = 1;
#pragma unroll
        for (int k = 1; k < DBX; ++k) {
          if (mm) {
            rows[k] = row_of(__builtin_ctzll(mm));
            mm &= mm - 1;
            cnt = k + 1;
          } else {
            rows[k] = rows[k - 1];
          }
        }
#pragma unroll
        for (int k = 0; k < DBX; ++k)
#pragma unroll
          for (int u = 0; u < U; ++u) v[k][u] = glob_load<VB, LP>(rows[k] + off[u]);
      } else {
        // Every slot starts as a size-0 resource (its loads return 0 and
        // touch no memory), so no path can load through an unset one.
        __amdgpu_buffer_rsrc_t rows[DBX];
#pragma unroll
        for (int k = 0; k < DBX; ++k) rows[k] = row_rsrc(h.eo_base, 0);
#pragma unroll
        for (int k = 0; k < DBX; ++k) {
          if (mm) {
            const int d = __builtin_ctzll(mm);
            mm &= mm - 1;
            rows[k] = row_rsrc(expert_output_of<STRIDED>(a, h, d) + r * row_bytes, row_bytes);
            cnt = k + 1;
          } else if (k > 0) {
            rows[k] = rows[k - 1];
          }
        }
#pragma unroll
        for (int k = 0; k < DBX; ++k)
#pragma unroll
          for (int u = 0; u < U; ++u) v[k][u] = buf_load<VB, LP>(rows[k], off[u]);
      }
#pragma unroll
      for (int k = 0; k < DBX; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) unpack_add<DT, VE>(v[k][u], acc[u], k < cnt);
    };
    // A token that reached at most 2 (DB/2) ranks loads only 2 (DB/2) rows
    // (a uniform branch): on a ragged round of 8 KiB rows (2.8 ranks per
    // token) the 4-row batch made combine 20% faster and the 2-row one
    // another 1.6%; the other workloads are even.  (A 6-row batch for 5 or 6
    // ranks was slower on the 16- and 32-rank rounds.)
    // A batch needs at least one row: its first slot is the one every
    // unused slot repeats.  A token that reached no rank takes no batch.
    if (mm != 0 && __builtin_popcountll(mm) <= 2) {
      batch(std::integral_constant<int, 2>{});
    } else if (mm != 0 && __builtin_popcountll(mm) <= DB / 2) {
      batch(std::integral_constant<int, DB / 2>{});
    } else {
      while (mm) batch(std::integral_constant<int, DB>{});
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (store && live[u]) buf_store<VB, SP>(out, off[u], pack<DT, VE>(acc[u]));
  };
  if (ONEPASS) {
    // The grid covers the row: straight-line code, no loop test between the
    // argument loads and the row loads.
    pass((int64_t)chunk * per_block);
  } else {
    for (int64_t c0 = (int64_t)chunk * per_block; c0 < nv; c0 += (int64_t)h.chunks * per_block) pass(c0);
  }
}

// Grid (1-D): one workgroup per (token slot, column chunk).  Token slots are
// the real tokens (prefix over source ranks), or all ep*tpr slots after a
// dispatch that read device-resident counts.  Workgroup i runs on XCD i % 8,
// so i is decoded as: token 8q + x on XCD x = i % 8, and its chunks one after
// another on that XCD (q and the chunk from i / 8).  Placing all chunks of a
// token on one XCD made these small workgroups 5% faster on the
// DeepSeek-V3-shaped round than one 896-thread workgroup per token; placed
// round-robin they were no faster.
// One workgroup per item, no grid-stride loop: with stores ahead of it in
// the same workgroup the token-record load could not be a scalar load.
// Every test or argument load between the start and the first row load
// costs the workgroup another dependent round trip, hence: the leading
// arguments arrive preloaded, i / 8 / chunks is a multiply and a shift,
// DEVN (device-resident counts) and STRIDED are instantiations, and a slot
// past the last token (the grid holds whole groups of 8) repeats the last
// token's loads and stores nothing instead of returning.
// Row loads (GL): through plain global addresses for groups of up to
// kSmallGroup ranks, through one buffer resource per row above that.  In
// interleaved runs the global loads made the DeepSeek-V3 round's combine
// 1.1% faster (16.54 against 16.71-16.76 us, two boxes) and a ragged 8-rank
// one 0.6%, but a 32-rank round's 3% slower (95.1-95.4 against 92.4-93.0
// us); a 16-rank fp8 one was even.
template <int DT, int VE, int U, int DB, int LP, int SP, bool ONEPASS, bool STRIDED, bool DEVN, bool GL, class A>
__device__ __forceinline__ void combine_item(const A& a, const uint64_t chunk_magic, const uint32_t chunk_shift,
                                             const int32_t ntok, const CombineHead& h) {
  const int i = blockIdx.x;
  const int rest = i >> 3;
  const int q = (int)(((uint64_t)rest * chunk_magic) >> chunk_shift);
  const int chunk = rest - q * h.chunks;
  const int b = q * 8 + (i & 7);
  const bool real = b < ntok;
  combine_token<DT, VE, U, DB, LP, SP, ONEPASS, STRIDED, DEVN, GL>(a, h, real ? b : ntok - 1, chunk, real);
}

template <int DT, int VE, int U, int DB, int LP, int SP, bool ONEPASS, bool STRIDED, bool DEVN, int MR>
__global__ void __launch_bounds__(kMaxCombineBlock)
combine_kernel(const uint64_t chunk_magic, const uint32_t chunk_shift, const int32_t ntok, const int32_t chunks,
               const int32_t block, const TokenRec* tokens, const uint8_t* eo_base, const int64_t eo_stride,
               const int64_t hidden, const CombineArgs<MR> a) {
  const CombineHead h{tokens, eo_base, eo_stride, hidden, block, chunks};
  combine_item<DT, VE, U, DB, LP, SP, ONEPASS, STRIDED, DEVN, (MR <= kSmallGroup)>(a, chunk_magic, chunk_shift, ntok, h);
}

// The same combine for host-count steps whose expert outputs and outputs
// both lie at constant strides (an overload of the kernel template above):
// every argument is a scalar (80 bytes in all), and the HIP runtime on this
// stack enqueues a launch with at most ~96 bytes of arguments ~0.6 us
// faster than one with 128 or more (host time per call 2.6-2.7 against
// 3.2-3.4 us).
template <int DT, int VE, int U, int DB, int LP, int SP, bool ONEPASS, bool GL>
__global__ void __launch_bounds__(kMaxCombineBlock)
combine_kernel(const uint64_t chunk_magic, const uint32_t chunk_shift, const int32_t ntok,
                       const int32_t chunks, const int32_t block, const TokenRec* tokens, const uint8_t* eo_base,
                       const int64_t eo_stride, const int64_t hidden, uint8_t* out_base, const int64_t out_stride,
                       const int32_t tpr) {
  const CombineHead h{tokens, eo_base, eo_stride, hidden, block, chunks};
  const CompactCombine a{tpr, out_base, out_stride};
  combine_item<DT, VE, U, DB, LP, SP, ONEPASS, true, false, GL>(a, chunk_magic, chunk_shift, ntok, h);
}

template <int DT, int VE>
const void* pick_combine_compact(bool onepass, bool gl) {
#define MOE_EP_CC(OP, G) \
  reinterpret_cast<const void*>(&combine_kernel<DT, VE, kCombineU, kCombineDB, kCombineLP, kCombineSP, OP, G>)
  if (onepass) return gl ? MOE_EP_CC(true, true) : MOE_EP_CC(true, false);
  return gl ? MOE_EP_CC(false, true) : MOE_EP_CC(false, false);
#undef MOE_EP_CC
}

template <int DT, int VE, int MR>
const void* pick_combine(bool onepass, bool strided, bool devn) {
#define MOE_EP_CK(OP, ST, DV) \
  reinterpret_cast<const void*>(&combine_kernel<DT, VE, kCombineU, kCombineDB, kCombineLP, kCombineSP, OP, ST, DV, MR>)
  if (onepass) {
    if (strided) return devn ? MOE_EP_CK(true, true, true) : MOE_EP_CK(true, true, false);
    return devn ? MOE_EP_CK(true, false, true) : MOE_EP_CK(true, false, false);
  }
  if (strided) return devn ? MOE_EP_CK(false, true, true) : MOE_EP_CK(false, true, false);
  return devn ? MOE_EP_CK(false, false, true) : MOE_EP_CK(false, false, false);
#undef MOE_EP_CK
}


}  // namespace


// Kernel for a vector width, a tile width (4, 7 or 8 vectors per thread) and a
// count source, as a table: (VB, U, DEVN) are template arguments.
template <template <int, int, bool> class K>
const void* pick_kernel(int vec_bytes, int u, bool devn) {
#define MOE_EP_PICK(VB) \
  case VB: \
    if (u == 8) return devn ? K<VB, 8, true>::fn() : K<VB, 8, false>::fn(); \
    if (u == 4) return devn ? K<VB, 4, true>::fn() : K<VB, 4, false>::fn(); \
    return devn ? K<VB, 7, true>::fn() : K<VB, 7, false>::fn();
  switch (vec_bytes) {
    MOE_EP_PICK(16) MOE_EP_PICK(8) MOE_EP_PICK(4) MOE_EP_PICK(2) MOE_EP_PICK(1)
    default: return nullptr;
  }
#undef MOE_EP_PICK
}

// The dispatch kernels for argument blocks of MR ranks.
template <int MR> struct DispatchKernels {
  template <int VB, int U, bool DEVN> struct SourceRow {
    static const void* fn() {
      return reinterpret_cast<const void*>(&dispatch_kernel<VB, U, kDispatchLP, kDispatchSP, DEVN, MR>);
    }
  };
  template <int VB, int U, bool DEVN> struct Destination {
    static const void* fn() {
      return reinterpret_cast<const void*>(&dispatch_dst_kernel<VB, U, kDispatchSP, DEVN, false, MR>);
    }
  };
  template <int VB, int U, bool DEVN> struct DestinationLean {
    static const void* fn() {
      return reinterpret_cast<const void*>(&dispatch_dst_kernel<VB, U, kDispatchSP, DEVN, true, MR>);
    }
  };
};

// The argument block a group of at most kSmallGroup ranks launches with: the
// same head and the first kSmallGroup per-rank entries.
DispatchArgs<kSmallGroup> small_args(const DispatchKArgs& a) {
  DispatchArgs<kSmallGroup> o;
  static_cast<DispatchArgsHead&>(o) = a;
  for (int s = 0; s < kSmallGroup; ++s) o.src[s] = a.src[s];
  return o;
}

CombineArgs<kSmallGroup> small_args(const CombineKArgs& a) {
  CombineArgs<kSmallGroup> o;
  static_cast<CombineArgsHead&>(o) = a;
  for (int s = 0; s < kSmallGroup; ++s) {
    o.expert_output[s] = a.expert_output[s];
    o.output[s] = a.output[s];
    o.token_start[s] = a.token_start[s];
  }
  o.token_start[kSmallGroup] = a.token_start[kSmallGroup];
  return o;
}

hipError_t launch_dispatch(const DispatchKArgs& args, int vec_bytes, hipStream_t stream) {
  DispatchKArgs a = args;
  a.div_tpr = make_owner_div((uint32_t)std::max(1, a.tpr));
  a.div_chunks = make_owner_div((uint32_t)std::max(1, a.dm_chunks));
  a.div_block_rows = make_owner_div((uint32_t)std::max(1, a.dm_block_rows));
  a.div_ep = make_owner_div((uint32_t)std::max(1, a.ep));
  const int64_t extra = a.eplb_bytes ? a.ep : 0;
  const bool devn = a.dev_n != nullptr;
  const bool small = a.ep <= kSmallGroup;
  const void* fn;
  dim3 grid, block;
  size_t lds = 0;
  if (a.order == MOE_EP_ORDER_DESTINATION) {
    if (a.dm_items + extra <= 0) return hipSuccess;
    // top_k <= 64, no scale rows, no statistics rows: the lean instantiation
    const bool lean = a.top_k <= 64 && a.scale_bytes == 0 && extra == 0 && a.dm_threads >= 64;
    if (small)
      fn = lean ? pick_kernel<DispatchKernels<kSmallGroup>::DestinationLean>(vec_bytes, a.dm_u, devn)
                : pick_kernel<DispatchKernels<kSmallGroup>::Destination>(vec_bytes, a.dm_u, devn);
    else
      fn = lean ? pick_kernel<DispatchKernels<kMaxRanks>::DestinationLean>(vec_bytes, a.dm_u, devn)
                : pick_kernel<DispatchKernels<kMaxRanks>::Destination>(vec_bytes, a.dm_u, devn);
    grid = dim3((unsigned)(a.dm_items + extra));
    lds = (size_t)dispatch_dst_lds(a.dm_items, lean);
    block = dim3(a.dm_threads);
    a.block = a.dm_threads;
  } else {
    const LaunchShape sh = dispatch_shape((int64_t)a.ep * a.tpr + extra, a.hidden_bytes, vec_bytes);
    if (sh.grid_x <= 0) return hipSuccess;
    fn = small ? pick_kernel<DispatchKernels<kSmallGroup>::SourceRow>(vec_bytes, sh.u, devn)
               : pick_kernel<DispatchKernels<kMaxRanks>::SourceRow>(vec_bytes, sh.u, devn);
    grid = dim3(sh.grid_x, sh.grid_y);
    block = dim3(sh.block);
    a.block = sh.block;
    a.grid_y = sh.grid_y;
  }
  if (!fn) return hipErrorInvalidValue;
  // The leading arguments (preloaded into scalar registers), then the rest.
  uint64_t m_chunks = a.div_chunks.magic, m_block_rows = a.div_block_rows.magic;
  uint64_t m_ep = a.div_ep.magic, m_tpr = a.div_tpr.magic;
  uint32_t shifts = a.div_chunks.shift | a.div_block_rows.shift << 8 | a.div_ep.shift << 16 | a.div_tpr.shift << 24;
  DispatchArgs<kSmallGroup> sa;
  if (small) sa = small_args(a);
  void* kargs[] = {&m_chunks, &m_block_rows, &m_ep, &m_tpr, &shifts, &a.dm_chunks, &a.dm_block_rows, &a.ep, &a.tpr,
                   small ? static_cast<void*>(&sa) : static_cast<void*>(&a)};
  return hipLaunchKernel(fn, grid, block, kargs, lds, stream);
}

hipError_t launch_combine(const CombineKArgs& args, int dtype, int vec_elems, hipStream_t stream) {
  CombineKArgs a = args;
  a.ntok = a.dev_counts ? a.ep * a.tpr : a.token_start[a.ep];
  const LaunchShape sh = combine_shape(a.ntok, a.hidden, vec_elems);
  if (sh.grid_x <= 0) return hipSuccess;
  a.chunks = sh.grid_y;
  const void* fn = nullptr;
  const bool onepass = (int64_t)sh.grid_y * sh.block * kCombineU >= a.hidden / vec_elems;
  const bool strided = common_stride(a.expert_output, a.ep, &a.eo_base, &a.eo_stride);
  const bool devn = a.dev_counts != nullptr;
  const bool small = a.ep <= kSmallGroup;
  // Host-count steps with expert outputs and outputs at constant strides
  // take the compact launch (all-scalar arguments).
  const uint8_t* out_base = nullptr;
  int64_t out_stride = 0;
  const bool compact =
      !devn && strided && common_stride(const_cast<const uint8_t* const*>(a.output), a.ep, &out_base, &out_stride);
  a.block = sh.block;
  a.chunk_div = make_owner_div((uint32_t)a.chunks);
  if (devn) a.tpr_div = make_owner_div((uint32_t)a.tpr);
#define MOE_EP_C(DT, VE) \
    case VE: \
      fn = compact ? pick_combine_compact<DT, VE>(onepass, small) \
           : small ? pick_combine<DT, VE, kSmallGroup>(onepass, strided, devn) \
                   : pick_combine<DT, VE, kMaxRanks>(onepass, strided, devn); \
      break;
  if (dtype == MOE_EP_F32) {
    switch (vec_elems) {
      MOE_EP_C(MOE_EP_F32, 4) MOE_EP_C(MOE_EP_F32, 2) MOE_EP_C(MOE_EP_F32, 1)
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == MOE_EP_BF16) {
    switch (vec_elems) {
      MOE_EP_C(MOE_EP_BF16, 8) MOE_EP_C(MOE_EP_BF16, 4) MOE_EP_C(MOE_EP_BF16, 2) MOE_EP_C(MOE_EP_BF16, 1)
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == MOE_EP_F16) {
    switch (vec_elems) {
      MOE_EP_C(MOE_EP_F16, 8) MOE_EP_C(MOE_EP_F16, 4) MOE_EP_C(MOE_EP_F16, 2) MOE_EP_C(MOE_EP_F16, 1)
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef MOE_EP_C
  // The leading arguments (preloaded into scalar registers), then the rest.
  uint64_t magic = a.chunk_div.magic;
  uint32_t shift = a.chunk_div.shift;
  const TokenRec* tokens = a.tokens;
  const uint8_t* eo_base = a.eo_base;
  int64_t eo_stride = a.eo_stride;
  int64_t hidden = a.hidden;
  if (compact) {
    uint8_t* obase = const_cast<uint8_t*>(out_base);
    void* cargs[] = {&magic, &shift, &a.ntok, &a.chunks, &a.block, &tokens, &eo_base, &eo_stride, &hidden,
                     &obase, &out_stride, &a.tpr};
    return hipLaunchKernel(fn, dim3(sh.grid_x), dim3(sh.block), cargs, (size_t)sh.lds, stream);
  }
  CombineArgs<kSmallGroup> sa;
  if (small) sa = small_args(a);
  void* kargs[] = {&magic, &shift, &a.ntok, &a.chunks, &a.block, &tokens, &eo_base, &eo_stride, &hidden,
                   small ? static_cast<void*>(&sa) : static_cast<void*>(&a)};
  return hipLaunchKernel(fn, dim3(sh.grid_x), dim3(sh.block), kargs, (size_t)sh.lds, stream);
}

// ---------------------------------------------------------------------------
// Fixed record area of moe_ep_dispatch_noalloc
//
// The destination masks, token records and counts a dispatch leaves for its
// combine, kept in the library instead of the workspace: route masks
// [kNoallocRows] u64, then token records [kNoallocRows] TokenRec, then
// counts [kMaxRanks] int32.  Each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels get the address noalloc_scratch() looked
// up for the device.
// ---------------------------------------------------------------------------
constexpr int64_t kNoallocRows = MOE_EP_NOALLOC_MAX_ROWS;
constexpr int64_t kNoallocTokensOff = kNoallocRows * 8;
constexpr int64_t kNoallocCountsOff = kNoallocTokensOff + kNoallocRows * (int64_t)sizeof(TokenRec);
constexpr int64_t kNoallocBytes = kNoallocCountsOff + kMaxRanks * 4;
static_assert(kNoallocTokensOff % 16 == 0 && kNoallocCountsOff % 16 == 0, "aligned sub-arrays");

static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t noalloc_scratch(int device, NoallocArea* out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  uint8_t* p = g_scratch_ptr[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[device].load(std::memory_order_relaxed);
    if (!p) {
      // The symbol's address on `device`, looked up with that device current.
      int prev = -1;
      hipError_t e = hipGetDevice(&prev);
      if (e != hipSuccess) return e;
      if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (prev != device) {
        const hipError_t e2 = hipSetDevice(prev);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<uint8_t*>(addr);
      g_scratch_ptr[device].store(p, std::memory_order_release);
    }
  }
  out->route = reinterpret_cast<uint64_t*>(p);
  out->tokens = reinterpret_cast<TokenRec*>(p + kNoallocTokensOff);
  out->counts = reinterpret_cast<int32_t*>(p + kNoallocCountsOff);
  out->bytes = kNoallocBytes;
  return hipSuccess;
}

}  // namespace moe_ep_detail
