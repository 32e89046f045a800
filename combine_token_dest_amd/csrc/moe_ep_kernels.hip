// gfx950 kernels of rank-major MoE expert-parallel dispatch and combine.
//
// The whole EP group lives in one GPU: rank d's receive region and combine
// input region are partition d of one workspace.  Both operations are pure
// data movement (plus one float32 add per element and routed row in
// combine), so they are bound by HBM bandwidth; the kernels aim at 16-byte
// coalesced accesses, every input byte read once, and no workspace traffic
// beyond what the method moves.
//
// dispatch: one workgroup per receive row index r = s*tpr + t.  It works out
//   the token's destination ranks from its top_k expert ids (contiguous
//   ownership, masked by the active ranks), writes the top_k ids/weights slot
//   of row r on every rank (the token's own where routed, invalid_expert_id /
//   0.0 elsewhere), loads the token's hidden row once into registers and
//   stores it to every destination, then the scale row the same way.
//   Placement and invalid rows: flashinfer.moe_ep.NVLinkOneSidedAlltoAll,
//   class description; routing: flashinfer.moe_ep.MoEEpCommunication,
//   dispatch(); mask: NVLinkOneSidedAlltoAll, dispatch().
//
// combine: one workgroup per real token (s, t < n_s).  It reads the token's
//   destination mask and, for each 16-byte column chunk, loads the token's
//   row from every destination rank (ascending), adds them in float32 in
//   that order starting from +0.0, rounds once and stores the output row.
//   Rows of ranks the token did not reach are never read.
//   flashinfer.moe_ep.MoEEpCommunication, combine().

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kMaxBlock = 512;
constexpr int kDispatchUnroll = 4;   // 16-byte chunks per thread held in registers
constexpr int kCombineUnroll = 2;    // column vectors per thread per pass
constexpr int kCombineBatch = 4;     // destination rows loaded before they are added

__device__ __forceinline__ int expert_owner(const OwnerDiv& od, uint32_t e) {
  return (int)(((uint64_t)e * od.magic) >> od.shift);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int VB>
__global__ void __launch_bounds__(kMaxBlock)
dispatch_kernel(const DispatchKArgs a) {
  typedef typename Bytes<VB>::type V;
  const int r = blockIdx.x;               // receive row index s*tpr + t
  const int s = r / a.tpr;
  const int t = r - s * a.tpr;
  const int K = a.top_k;
  const bool real = t < a.n[s];
  const int32_t* __restrict__ idr = a.ids[s] + (int64_t)t * K;

  // Destination ranks of token (s, t); zero for padding rows.  Uniform.
  uint64_t m = 0;
  if (real) {
    for (int j = 0; j < K; ++j) {
      const uint32_t e = (uint32_t)idr[j];
      if (e < (uint32_t)a.num_experts) m |= 1ull << expert_owner(a.owner, e);
    }
    m &= a.active;
  }
  if (threadIdx.x == 0) a.route[r] = m;

  // ids / weights slot of row r on every rank.
  const int slots = a.ep * K;
  for (int i = threadIdx.x; i < slots; i += blockDim.x) {
    const int d = i / K;
    const int j = i - d * K;
    const bool routed = (m >> d) & 1;
    uint8_t* part = a.ws + (int64_t)d * a.part_stride;
    const int64_t slot = (int64_t)r * K + j;
    reinterpret_cast<int32_t*>(part + a.off_ids)[slot] = routed ? idr[j] : a.invalid_id;
    if (a.has_weights) {
      const float w = routed ? a.weights[s][(int64_t)t * K + j] : 0.0f;
      reinterpret_cast<float*>(part + a.off_weights)[slot] = w;
    }
  }
  if (m == 0) return;

  // Hidden row: read once, store to every destination.
  {
    const int64_t nv = a.hidden_bytes / VB;
    const V* __restrict__ src = reinterpret_cast<const V*>(a.hidden[s] + (int64_t)t * a.hidden_bytes);
    const int64_t dst_off = a.off_hidden + (int64_t)r * a.hidden_bytes;
    const int64_t step = (int64_t)blockDim.x * kDispatchUnroll;
    for (int64_t c0 = threadIdx.x; c0 < nv; c0 += step) {
      V v[kDispatchUnroll];
#pragma unroll
      for (int u = 0; u < kDispatchUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * blockDim.x;
        if (c < nv) v[u] = src[c];
      }
      uint64_t mm = m;
      while (mm) {
        const int d = __builtin_ctzll(mm);
        mm &= mm - 1;
        V* __restrict__ dst = reinterpret_cast<V*>(a.ws + (int64_t)d * a.part_stride + dst_off);
#pragma unroll
        for (int u = 0; u < kDispatchUnroll; ++u) {
          const int64_t c = c0 + (int64_t)u * blockDim.x;
          if (c < nv) dst[c] = v[u];
        }
      }
    }
  }

  // Scale row (small: a few hundred bytes), row-aligned with hidden.
  if (a.scale_bytes) {
    const int64_t S = a.scale_bytes;
    const int64_t dst_off = a.off_scale + (int64_t)r * S;
    if (a.scale_vec4) {
      const int64_t nw = S / 4;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.scale[s] + (int64_t)t * S);
      for (int64_t c = threadIdx.x; c < nw; c += blockDim.x) {
        const uint32_t v = src[c];
        uint64_t mm = m;
        while (mm) {
          const int d = __builtin_ctzll(mm);
          mm &= mm - 1;
          reinterpret_cast<uint32_t*>(a.ws + (int64_t)d * a.part_stride + dst_off)[c] = v;
        }
      }
    } else {
      const uint8_t* src = a.scale[s] + (int64_t)t * S;
      for (int64_t c = threadIdx.x; c < S; c += blockDim.x) {
        const uint8_t v = src[c];
        uint64_t mm = m;
        while (mm) {
          const int d = __builtin_ctzll(mm);
          mm &= mm - 1;
          (a.ws + (int64_t)d * a.part_stride + dst_off)[c] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------
// Raw storage of VE elements of a combine dtype.
template <int DT, int VE> struct CVec;
template <int VE> struct CVec<MOE_EP_F32, VE> { typedef typename Bytes<VE * 4>::type type; };
template <int VE> struct CVec<MOE_EP_BF16, VE> { typedef typename Bytes<VE * 2>::type type; };

template <int DT, int VE>
__device__ __forceinline__ void unpack_add(const typename CVec<DT, VE>::type& v, float (&acc)[VE]) {
  if constexpr (DT == MOE_EP_F32) {
    uint32_t w[VE];
    __builtin_memcpy(w, &v, sizeof(w));
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = acc[i] + __uint_as_float(w[i]);
  } else if constexpr (VE == 1) {
    acc[0] = acc[0] + __uint_as_float((uint32_t)v << 16);
  } else {
    uint32_t w[VE / 2];
    __builtin_memcpy(w, &v, sizeof(w));
#pragma unroll
    for (int i = 0; i < VE / 2; ++i) {
      acc[2 * i] = acc[2 * i] + __uint_as_float(w[i] << 16);
      acc[2 * i + 1] = acc[2 * i + 1] + __uint_as_float(w[i] & 0xffff0000u);
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
  } else {
    // float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
    uint16_t h[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) h[i] = __builtin_bit_cast(uint16_t, (__bf16)acc[i]);
    __builtin_memcpy(&v, h, sizeof(h));
  }
  return v;
}

template <int DT, int VE>
__global__ void __launch_bounds__(kMaxBlock)
combine_kernel(const CombineKArgs a) {
  typedef typename CVec<DT, VE>::type V;
  constexpr int U = kCombineUnroll;
  constexpr int DB = kCombineBatch;
  const int b = blockIdx.x;
  int s = 0;
  while (s + 1 < a.ep && b >= a.token_start[s + 1]) ++s;    // uniform scan, ep <= 64
  const int t = b - a.token_start[s];
  const int64_t r = (int64_t)s * a.tpr + t;
  const uint64_t m = a.route[r];
  const int64_t nv = a.hidden / VE;
  constexpr int esz = DT == MOE_EP_F32 ? 4 : 2;
  const int64_t row_bytes = a.hidden * esz;
  V* __restrict__ out = reinterpret_cast<V*>(a.output[s] + (int64_t)t * row_bytes);

  for (int64_t c0 = threadIdx.x; c0 < nv; c0 += (int64_t)blockDim.x * U) {
    float acc[U][VE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[u][i] = 0.0f;

    uint64_t mm = m;
    while (mm) {
      // Up to DB destination rows in flight, then added in ascending rank order.
      const V* rows[DB];
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < DB; ++k) {
        if (mm) {
          const int d = __builtin_ctzll(mm);
          mm &= mm - 1;
          rows[k] = reinterpret_cast<const V*>(a.expert_output[d] + r * row_bytes);
          cnt = k + 1;
        }
      }
      V v[DB][U];
#pragma unroll
      for (int k = 0; k < DB; ++k) {
        if (k < cnt) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * blockDim.x;
            if (c < nv) v[k][u] = rows[k][c];
          }
        }
      }
#pragma unroll
      for (int k = 0; k < DB; ++k) {
        if (k < cnt) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * blockDim.x;
            if (c < nv) unpack_add<DT, VE>(v[k][u], acc[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * blockDim.x;
      if (c < nv) out[c] = pack<DT, VE>(acc[u]);
    }
  }
}

int pick_block(int64_t work_items) {
  int64_t b = (work_items + 63) / 64 * 64;
  if (b < 64) b = 64;
  if (b > kMaxBlock) b = kMaxBlock;
  return (int)b;
}

}  // namespace

LaunchShape dispatch_shape(int64_t rows, int64_t hidden_bytes, int vec_bytes) {
  const int64_t nv = hidden_bytes / vec_bytes;
  return LaunchShape{(int)rows, pick_block((nv + kDispatchUnroll - 1) / kDispatchUnroll)};
}

LaunchShape combine_shape(int64_t tokens, int64_t hidden, int vec_elems) {
  const int64_t nv = hidden / vec_elems;
  return LaunchShape{(int)tokens, pick_block((nv + kCombineUnroll - 1) / kCombineUnroll)};
}

hipError_t launch_dispatch(const DispatchKArgs& a, int vec_bytes, hipStream_t stream) {
  const LaunchShape sh = dispatch_shape((int64_t)a.ep * a.tpr, a.hidden_bytes, vec_bytes);
  if (sh.grid <= 0) return hipSuccess;
  const void* fn;
  switch (vec_bytes) {
    case 16: fn = reinterpret_cast<const void*>(&dispatch_kernel<16>); break;
    case 8: fn = reinterpret_cast<const void*>(&dispatch_kernel<8>); break;
    case 4: fn = reinterpret_cast<const void*>(&dispatch_kernel<4>); break;
    case 2: fn = reinterpret_cast<const void*>(&dispatch_kernel<2>); break;
    case 1: fn = reinterpret_cast<const void*>(&dispatch_kernel<1>); break;
    default: return hipErrorInvalidValue;
  }
  void* args[] = {const_cast<DispatchKArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(sh.grid), dim3(sh.block), args, 0, stream);
}

hipError_t launch_combine(const CombineKArgs& a, int dtype, int vec_elems, hipStream_t stream) {
  const LaunchShape sh = combine_shape(a.token_start[a.ep], a.hidden, vec_elems);
  if (sh.grid <= 0) return hipSuccess;
  const void* fn = nullptr;
  if (dtype == MOE_EP_F32) {
    switch (vec_elems) {
      case 4: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_F32, 4>); break;
      case 2: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_F32, 2>); break;
      case 1: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_F32, 1>); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == MOE_EP_BF16) {
    switch (vec_elems) {
      case 8: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_BF16, 8>); break;
      case 4: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_BF16, 4>); break;
      case 2: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_BF16, 2>); break;
      case 1: fn = reinterpret_cast<const void*>(&combine_kernel<MOE_EP_BF16, 1>); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  void* args[] = {const_cast<CombineKArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(sh.grid), dim3(sh.block), args, 0, stream);
}

}  // namespace moe_ep_detail
