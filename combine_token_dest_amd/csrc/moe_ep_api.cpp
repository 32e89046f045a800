// C-ABI host side of the gfx950 rank-major MoE expert-parallel
// dispatch/combine library: argument validation, the dispatch -> combine
// call protocol, the workspace layout, and kernel launches.
//
// Everything here runs on the host before anything is enqueued, so a call
// that fails leaves no device work behind and the handle unchanged.

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>

#include "moe_ep.h"
#include "moe_ep_internal.h"

using namespace moe_ep_detail;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  return MOE_EP_OK;
}

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x, int64_t a) {
  return (x + a - 1) / a * a;
}

enum State { kIdle = 0, kDispatched = 1 };

// Bytes of a combine element type, 0 for an unknown one.
int dtype_bytes(int dtype) {
  switch (dtype) {
    case MOE_EP_F32: return 4;
    case MOE_EP_BF16: return 2;
    case MOE_EP_F16: return 2;
    default: return 0;
  }
}

uint64_t rank_bits(int ep) {
  return ep >= 64 ? ~0ull : ((1ull << ep) - 1);
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Largest power of two <= cap that divides x (x > 0).
int64_t pow2_divisor(uint64_t x, int64_t cap) {
  int64_t v = cap;
  while (v > 1 && (x % (uint64_t)v) != 0) v >>= 1;
  return v;
}

int validate_params(const moe_ep_params* p) {
  if (!p) return fail(MOE_EP_ERR_INVALID_ARG, "params is NULL");
  if (p->ep_size < 1 || p->ep_size > MOE_EP_MAX_RANKS)
    return fail(MOE_EP_ERR_INVALID_ARG, "ep_size %d outside [1, %d]", p->ep_size, MOE_EP_MAX_RANKS);
  if (p->num_experts < p->ep_size || p->num_experts % p->ep_size != 0)
    return fail(MOE_EP_ERR_INVALID_ARG, "num_experts %d is not a positive multiple of ep_size %d",
                p->num_experts, p->ep_size);
  if (p->top_k < 1) return fail(MOE_EP_ERR_INVALID_ARG, "top_k %d < 1", p->top_k);
  if (p->max_tokens_per_rank < 0)
    return fail(MOE_EP_ERR_INVALID_ARG, "max_tokens_per_rank %d < 0", p->max_tokens_per_rank);
  if (p->hidden_size < 1) return fail(MOE_EP_ERR_INVALID_ARG, "hidden_size %d < 1", p->hidden_size);
  if (p->combine_max_elem_bytes != 2 && p->combine_max_elem_bytes != 4)
    return fail(MOE_EP_ERR_INVALID_ARG, "combine_max_elem_bytes %d is not 2 or 4", p->combine_max_elem_bytes);
  if (p->hidden_row_bytes < 1)
    return fail(MOE_EP_ERR_INVALID_ARG, "hidden_row_bytes %lld < 1", (long long)p->hidden_row_bytes);
  if (p->scale_row_bytes < 0)
    return fail(MOE_EP_ERR_INVALID_ARG, "scale_row_bytes %lld < 0", (long long)p->scale_row_bytes);
  if (p->dispatch_order < MOE_EP_ORDER_AUTO || p->dispatch_order > MOE_EP_ORDER_DESTINATION)
    return fail(MOE_EP_ERR_INVALID_ARG, "dispatch_order %d unknown", p->dispatch_order);
  if (p->eplb_stats_bytes < 0 || p->eplb_stats_bytes > INT32_MAX)
    return fail(MOE_EP_ERR_INVALID_ARG, "eplb_stats_bytes %lld outside [0, 2^31)", (long long)p->eplb_stats_bytes);
  // Row and grid indices are 32-bit in the kernels; byte offsets are 64-bit.
  const int64_t rows = (int64_t)p->ep_size * p->max_tokens_per_rank;
  if (rows > (int64_t)1 << 30) return fail(MOE_EP_ERR_INVALID_ARG, "ep_size * capacity too large");
  // Rows are addressed with 32-bit byte offsets inside the kernels.
  if (p->hidden_row_bytes > INT32_MAX || p->scale_row_bytes > INT32_MAX || p->hidden_size > INT32_MAX / 4)
    return fail(MOE_EP_ERR_INVALID_ARG, "row bytes too large");
  return ok();
}

// Partition layout; returns false on overflow.
bool make_layout(const moe_ep_params* p, Layout* L) {
  const unsigned __int128 rows = (unsigned __int128)p->ep_size * (unsigned __int128)p->max_tokens_per_rank;
  const unsigned __int128 hid = rows * (unsigned __int128)p->hidden_row_bytes;
  const unsigned __int128 scl = rows * (unsigned __int128)p->scale_row_bytes;
  const unsigned __int128 ids = rows * (unsigned __int128)p->top_k * 4;
  const unsigned __int128 cmb = rows * (unsigned __int128)p->hidden_size * (unsigned __int128)p->combine_max_elem_bytes;
  const unsigned __int128 limit = (unsigned __int128)1 << 62;
  if (hid > limit || scl > limit || ids > limit || cmb > limit) return false;
  int64_t off = 0;
  L->off_hidden = off;
  off += align_up((int64_t)hid, kAlign);
  L->off_scale = off;
  off += align_up((int64_t)scl, kAlign);
  L->off_ids = off;
  off += align_up((int64_t)ids, kAlign);
  L->off_weights = off;
  off += align_up((int64_t)ids, kAlign);
  L->off_combine = off;
  off += align_up((int64_t)cmb, kAlign);
  L->off_eplb = off;
  off += align_up((int64_t)p->ep_size * p->eplb_stats_bytes, kAlign);
  L->part_stride = align_up(off, 4096);
  const unsigned __int128 parts = (unsigned __int128)L->part_stride * (unsigned __int128)p->ep_size;
  if (parts > limit) return false;
  L->off_route = (int64_t)parts;
  L->off_tokens = L->off_route + align_up((int64_t)(rows * 8), kAlign);
  L->off_counts = L->off_tokens + align_up((int64_t)(rows * sizeof(TokenRec)), kAlign);
  const unsigned __int128 total = (unsigned __int128)L->off_counts + kAlign;
  if (total > limit) return false;
  L->total = (int64_t)total;
  return true;
}

}  // namespace

// Workspace mapped by the library with HIP virtual memory management.
struct VmmWorkspace {
  bool enabled = false;   // handle made by moe_ep_create_vmm
  bool mapped = false;    // physical memory currently backs the range
  bool broken = false;    // a map/unmap failed part-way: the range cannot be reused
  int device = 0;
  void* va = nullptr;
  size_t size = 0;
  hipMemGenericAllocationHandle_t mem{};
};

struct moe_ep_handle_s {
  VmmWorkspace vmm;
  moe_ep_params p;
  Layout L;
  uint8_t* ws;
  int device;          // device holding the workspace, or -1 when HIP cannot tell
  void* checked_stream;  // last non-null stream found on `device`
  OwnerDiv owner;
  int state;
  // Remembered from the dispatch for its combine.
  uint64_t* route;     // where the dispatch left its destination masks,
  TokenRec* tokens;    //   token records
  int32_t* counts;     //   and device-step counts (workspace or fixed area)
  int32_t tpr;
  int32_t n[MOE_EP_MAX_RANKS];
  uint64_t mask;       // as passed (MOE_EP_ALL_RANKS = none)
  bool device_counts;  // the dispatch read its token counts from device memory
};

namespace {

hipMemAllocationProp vmm_prop(int device) {
  hipMemAllocationProp prop{};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Backs the reserved range with a new physical allocation.
int vmm_map(VmmWorkspace& v) {
  const hipMemAllocationProp prop = vmm_prop(v.device);
  hipError_t e = hipMemCreate(&v.mem, v.size, &prop, 0);
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "hipMemCreate: %s", hipGetErrorString(e));
  e = hipMemMap(v.va, v.size, 0, v.mem, 0);
  if (e != hipSuccess) {
    (void)hipMemRelease(v.mem);
    return fail(MOE_EP_ERR_HIP, "hipMemMap: %s", hipGetErrorString(e));
  }
  hipMemAccessDesc access{};
  access.location.type = hipMemLocationTypeDevice;
  access.location.id = v.device;
  access.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(v.va, v.size, &access, 1);
  if (e != hipSuccess) {
    (void)hipMemUnmap(v.va, v.size);
    (void)hipMemRelease(v.mem);
    return fail(MOE_EP_ERR_HIP, "hipMemSetAccess: %s", hipGetErrorString(e));
  }
  v.mapped = true;
  return MOE_EP_OK;
}

// Waits for the device, then unmaps and releases the physical allocation.
int vmm_unmap(VmmWorkspace& v) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
  e = hipMemUnmap(v.va, v.size);
  if (e != hipSuccess) {
    v.broken = true;
    return fail(MOE_EP_ERR_HIP, "hipMemUnmap: %s", hipGetErrorString(e));
  }
  v.mapped = false;
  e = hipMemRelease(v.mem);
  if (e != hipSuccess) {
    v.broken = true;
    return fail(MOE_EP_ERR_HIP, "hipMemRelease: %s", hipGetErrorString(e));
  }
  return MOE_EP_OK;
}

// Device of a workspace pointer, or -1 when HIP does not know the pointer.
int workspace_device(const void* ws) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, ws) != hipSuccess) {
    (void)hipGetLastError();          // leave no sticky error for the caller's next call
    return -1;
  }
  return attr.type == hipMemoryTypeDevice ? attr.device : -1;
}

// The launch would run on the device that holds the workspace: the stream's
// device, or the current device for the null stream.  A definite mismatch
// is refused before anything is enqueued (the kernels would touch another
// device's memory); when HIP cannot tell, the call goes ahead.
int check_launch_device(moe_ep_handle h, void* stream) {
  if (h->device < 0) return MOE_EP_OK;
  if (stream && stream == h->checked_stream) return MOE_EP_OK;   // a stream keeps its device
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EP_OK;
  }
  if (dev != h->device)
    return fail(MOE_EP_ERR_INVALID_ARG, "the stream runs on device %d but the workspace is on device %d", dev,
                h->device);
  if (stream) h->checked_stream = stream;
  return MOE_EP_OK;
}

// dispatch / combine / the combine buffer need a mapped, usable workspace.
int check_workspace_usable(const moe_ep_handle h) {
  if (h->vmm.broken) return fail(MOE_EP_ERR_STATE, "the workspace failed to map or unmap; destroy the handle");
  if (h->vmm.enabled && !h->vmm.mapped)
    return fail(MOE_EP_ERR_STATE, "the workspace is released for a checkpoint; call moe_ep_checkpoint_restore");
  return MOE_EP_OK;
}

}  // namespace

extern "C" {

const char* moe_ep_status_string(int status) {
  switch (status) {
    case MOE_EP_OK: return "MOE_EP_OK";
    case MOE_EP_ERR_INVALID_ARG: return "MOE_EP_ERR_INVALID_ARG";
    case MOE_EP_ERR_STATE: return "MOE_EP_ERR_STATE";
    case MOE_EP_ERR_CAPACITY: return "MOE_EP_ERR_CAPACITY";
    case MOE_EP_ERR_MASK: return "MOE_EP_ERR_MASK";
    case MOE_EP_ERR_ALIGN: return "MOE_EP_ERR_ALIGN";
    case MOE_EP_ERR_HIP: return "MOE_EP_ERR_HIP";
    case MOE_EP_ERR_UNSUPPORTED: return "MOE_EP_ERR_UNSUPPORTED";
    default: return "MOE_EP_ERR_UNKNOWN";
  }
}

const char* moe_ep_last_error(void) {
  return g_last_error.c_str();
}

int moe_ep_is_platform_supported(void) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

int moe_ep_workspace_bytes(const moe_ep_params* params, size_t* out_bytes) {
  if (!out_bytes) return fail(MOE_EP_ERR_INVALID_ARG, "out_bytes is NULL");
  const int st = validate_params(params);
  if (st != MOE_EP_OK) return st;
  Layout L;
  if (!make_layout(params, &L)) return fail(MOE_EP_ERR_INVALID_ARG, "workspace size overflows");
  *out_bytes = (size_t)L.total;
  return ok();
}

int moe_ep_create(const moe_ep_params* params, void* workspace, size_t workspace_bytes,
                  moe_ep_handle* out_handle) {
  if (!out_handle) return fail(MOE_EP_ERR_INVALID_ARG, "out_handle is NULL");
  const int st = validate_params(params);
  if (st != MOE_EP_OK) return st;
  Layout L;
  if (!make_layout(params, &L)) return fail(MOE_EP_ERR_INVALID_ARG, "workspace size overflows");
  if (!workspace) return fail(MOE_EP_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(MOE_EP_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (workspace_bytes < (size_t)L.total)
    return fail(MOE_EP_ERR_INVALID_ARG, "workspace has %zu bytes, needs %lld", workspace_bytes,
                (long long)L.total);
  moe_ep_handle h = new (std::nothrow) moe_ep_handle_s();
  if (!h) return fail(MOE_EP_ERR_INVALID_ARG, "out of host memory");
  h->p = *params;
  h->L = L;
  h->ws = static_cast<uint8_t*>(workspace);
  h->owner = make_owner_div((uint32_t)(params->num_experts / params->ep_size));
  h->device = workspace_device(workspace);
  if (h->device >= 0) {
    // Set-up of the fixed record area for moe_ep_dispatch_noalloc on this
    // device; a failure here is reported by that call, which looks again.
    NoallocArea area;
    if (noalloc_scratch(h->device, &area) != hipSuccess) (void)hipGetLastError();
  }
  h->checked_stream = nullptr;
  h->state = kIdle;
  h->tpr = 0;
  h->mask = MOE_EP_ALL_RANKS;
  *out_handle = h;
  return ok();
}

int moe_ep_destroy(moe_ep_handle handle) {
  if (!handle) return ok();
  int st = MOE_EP_OK;
  if (handle->vmm.enabled) {
    if (handle->vmm.mapped) st = vmm_unmap(handle->vmm);
    if (!handle->vmm.broken) {
      const hipError_t e = hipMemAddressFree(handle->vmm.va, handle->vmm.size);
      if (e != hipSuccess && st == MOE_EP_OK) st = fail(MOE_EP_ERR_HIP, "hipMemAddressFree: %s", hipGetErrorString(e));
    }
  }
  delete handle;
  return st;
}

int moe_ep_create_vmm(const moe_ep_params* params, moe_ep_handle* out_handle) {
  if (!out_handle) return fail(MOE_EP_ERR_INVALID_ARG, "out_handle is NULL");
  int st = validate_params(params);
  if (st != MOE_EP_OK) return st;
  Layout L;
  if (!make_layout(params, &L)) return fail(MOE_EP_ERR_INVALID_ARG, "workspace size overflows");
  VmmWorkspace v;
  hipError_t e = hipGetDevice(&v.device);
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int supported = 0;
  e = hipDeviceGetAttribute(&supported, hipDeviceAttributeVirtualMemoryManagementSupported, v.device);
  if (e != hipSuccess || !supported)
    return fail(MOE_EP_ERR_UNSUPPORTED, "device %d has no virtual memory management", v.device);
  const hipMemAllocationProp prop = vmm_prop(v.device);
  size_t gran = 0;
  e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityRecommended);
  if (e != hipSuccess || gran == 0)
    return fail(MOE_EP_ERR_HIP, "hipMemGetAllocationGranularity: %s", hipGetErrorString(e));
  v.size = (size_t)((L.total + (int64_t)gran - 1) / (int64_t)gran) * gran;
  e = hipMemAddressReserve(&v.va, v.size, gran, nullptr, 0);
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "hipMemAddressReserve: %s", hipGetErrorString(e));
  v.enabled = true;
  st = vmm_map(v);
  if (st != MOE_EP_OK) {
    (void)hipMemAddressFree(v.va, v.size);
    return st;
  }
  moe_ep_handle h = nullptr;
  st = moe_ep_create(params, v.va, v.size, &h);
  if (st != MOE_EP_OK) {
    (void)vmm_unmap(v);
    (void)hipMemAddressFree(v.va, v.size);
    return st;
  }
  h->vmm = v;
  h->device = v.device;
  *out_handle = h;
  return ok();
}

int moe_ep_workspace(moe_ep_handle h, void** out_ptr, size_t* out_bytes) {
  if (!h || !out_ptr || !out_bytes) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle or output");
  *out_ptr = h->ws;
  *out_bytes = h->vmm.enabled ? h->vmm.size : (size_t)h->L.total;
  return ok();
}

int moe_ep_checkpoint_prepare(moe_ep_handle h) {
  if (!h) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle");
  if (!h->vmm.enabled) return fail(MOE_EP_ERR_UNSUPPORTED, "the workspace is caller-owned; use moe_ep_create_vmm");
  if (h->vmm.broken) return fail(MOE_EP_ERR_STATE, "the workspace failed to map or unmap; destroy the handle");
  if (!h->vmm.mapped) return ok();                      // already released
  if (h->state != kIdle) return fail(MOE_EP_ERR_STATE, "checkpoint_prepare between a dispatch and its combine");
  return vmm_unmap(h->vmm);
}

int moe_ep_checkpoint_restore(moe_ep_handle h) {
  if (!h) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle");
  if (!h->vmm.enabled) return fail(MOE_EP_ERR_UNSUPPORTED, "the workspace is caller-owned; use moe_ep_create_vmm");
  if (h->vmm.broken) return fail(MOE_EP_ERR_STATE, "the workspace failed to map or unmap; destroy the handle");
  if (h->vmm.mapped) return ok();                       // nothing to restore
  const int st = vmm_map(h->vmm);
  if (st != MOE_EP_OK) h->vmm.broken = true;
  return st;
}

int moe_ep_active_rank_mask(const int32_t* ranks, int32_t n, uint64_t* out_mask) {
  if (!out_mask) return fail(MOE_EP_ERR_INVALID_ARG, "out_mask is NULL");
  if (n < 0 || (n > 0 && !ranks)) return fail(MOE_EP_ERR_INVALID_ARG, "bad rank list");
  uint64_t m = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (ranks[i] < 0 || ranks[i] >= MOE_EP_MAX_RANKS)
      return fail(MOE_EP_ERR_MASK, "rank %d outside [0, %d)", ranks[i], MOE_EP_MAX_RANKS);
    m |= 1ull << ranks[i];
  }
  *out_mask = m;
  return ok();
}

static int check_mask(const moe_ep_params& p, uint64_t mask) {
  if (mask == MOE_EP_ALL_RANKS) return MOE_EP_OK;
  if (!p.enable_rank_mask) return fail(MOE_EP_ERR_MASK, "active_rank_mask passed without enable_rank_mask");
  if (mask & ~rank_bits(p.ep_size))
    return fail(MOE_EP_ERR_MASK, "active_rank_mask 0x%llx has bits at or above ep_size %d",
                (unsigned long long)mask, p.ep_size);
  return MOE_EP_OK;
}

namespace {

int dispatch_impl(moe_ep_handle h, const moe_ep_dispatch_args* a, moe_ep_dispatch_result* results,
                  void* stream, bool noalloc) {
  if (!h || !a || !results) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle, args or results");
  const moe_ep_params& p = h->p;
  const int ep = p.ep_size;
  int ust = check_workspace_usable(h);
  if (ust != MOE_EP_OK) return ust;
  if (h->state != kIdle) return fail(MOE_EP_ERR_STATE, "dispatch called before the previous dispatch's combine");

  const bool dev_counts = a->local_num_tokens_device != nullptr;
  if (dev_counts && !aligned(a->local_num_tokens_device, 4))
    return fail(MOE_EP_ERR_ALIGN, "local_num_tokens_device not 4-byte aligned");
  const int32_t tpr = a->runtime_max_tokens_per_rank < 0 ? p.max_tokens_per_rank : a->runtime_max_tokens_per_rank;
  // With device counts every rank may hold up to tpr tokens when the kernel runs.
  int32_t host_n[MOE_EP_MAX_RANKS];
  int32_t largest = 0;
  for (int s = 0; s < ep; ++s) {
    const int32_t n = dev_counts ? tpr : a->local_num_tokens[s];
    if (n < 0) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: local_num_tokens %d < 0", s, n);
    if (n > p.max_tokens_per_rank)
      return fail(MOE_EP_ERR_CAPACITY, "rank %d: local_num_tokens %d > capacity %d", s, n,
                  p.max_tokens_per_rank);
    host_n[s] = n;
    if (n > largest) largest = n;
  }
  if (tpr > p.max_tokens_per_rank)
    return fail(MOE_EP_ERR_CAPACITY, "runtime_max_tokens_per_rank %d > capacity %d", tpr, p.max_tokens_per_rank);
  if (tpr < largest)
    return fail(MOE_EP_ERR_CAPACITY, "runtime_max_tokens_per_rank %d < largest local_num_tokens %d", tpr,
                largest);
  int st = check_mask(p, a->active_rank_mask);
  if (st != MOE_EP_OK) return st;

  const uint64_t all = rank_bits(ep);
  const uint64_t wp = a->weights_present & all;
  const uint64_t sp = a->scales_present & all;
  if (wp != 0 && wp != all)
    return fail(MOE_EP_ERR_INVALID_ARG, "topk_weights passed by some ranks only (mask 0x%llx)",
                (unsigned long long)wp);
  if (sp != 0 && sp != all)
    return fail(MOE_EP_ERR_INVALID_ARG, "hidden_states_scale passed by some ranks only (mask 0x%llx)",
                (unsigned long long)sp);
  const bool has_w = wp != 0;
  const bool has_s = sp != 0;
  if (has_s && p.scale_row_bytes == 0)
    return fail(MOE_EP_ERR_INVALID_ARG, "hidden_states_scale passed but scale_row_bytes is 0");
  const uint64_t ep_present = a->eplb_present & all;
  if (ep_present != 0 && ep_present != all)
    return fail(MOE_EP_ERR_INVALID_ARG, "eplb_local_stats passed by some ranks only (mask 0x%llx)",
                (unsigned long long)ep_present);
  const bool has_e = ep_present != 0;
  if (has_e && p.eplb_stats_bytes == 0)
    return fail(MOE_EP_ERR_INVALID_ARG, "eplb_local_stats passed but eplb_stats_bytes is 0");

  DispatchKArgs k;
  std::memset(&k, 0, sizeof(k));
  uint64_t hidden_align_or = (uint64_t)p.hidden_row_bytes;
  uint64_t scale_align_or = has_s ? (uint64_t)p.scale_row_bytes : 0;
  for (int s = 0; s < ep; ++s) {
    const int32_t n = host_n[s];
    k.src[s].n = n;
    if (n == 0) continue;
    if (!a->hidden[s] || !a->topk_ids[s])
      return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: NULL hidden or topk_ids with %d tokens", s, n);
    if (!aligned(a->topk_ids[s], 4)) return fail(MOE_EP_ERR_ALIGN, "rank %d: topk_ids not 4-byte aligned", s);
    if (has_w) {
      if (!a->topk_weights[s]) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: NULL topk_weights", s);
      if (!aligned(a->topk_weights[s], 4))
        return fail(MOE_EP_ERR_ALIGN, "rank %d: topk_weights not 4-byte aligned", s);
    }
    if (has_s) {
      if (!a->hidden_scale[s]) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: NULL hidden_states_scale", s);
      scale_align_or |= reinterpret_cast<uintptr_t>(a->hidden_scale[s]);
    }
    hidden_align_or |= reinterpret_cast<uintptr_t>(a->hidden[s]);
    k.src[s].hidden = static_cast<const uint8_t*>(a->hidden[s]);
    k.src[s].ids = a->topk_ids[s];
    k.src[s].weights = has_w ? a->topk_weights[s] : nullptr;
    k.src[s].scale = has_s ? static_cast<const uint8_t*>(a->hidden_scale[s]) : nullptr;
  }
  const int vec_bytes = (int)pow2_divisor(hidden_align_or, 16);
  uint64_t eplb_align_or = (uint64_t)p.eplb_stats_bytes;
  if (has_e) {
    for (int s = 0; s < ep; ++s) {
      if (!a->eplb_local_stats[s]) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: NULL eplb_local_stats", s);
      eplb_align_or |= reinterpret_cast<uintptr_t>(a->eplb_local_stats[s]);
      k.src[s].eplb = static_cast<const uint8_t*>(a->eplb_local_stats[s]);
    }
  }
  k.dev_n = a->local_num_tokens_device;
  if (noalloc) {
    // The records go to the library's fixed array on the workspace's device.
    if ((int64_t)ep * tpr > MOE_EP_NOALLOC_MAX_ROWS)
      return fail(MOE_EP_ERR_CAPACITY, "ep_size * tokens_per_rank = %lld exceeds the %d rows of the fixed record area",
                  (long long)ep * tpr, MOE_EP_NOALLOC_MAX_ROWS);
    // The device the kernels will run on: the workspace's, else the
    // stream's (the current device's for the null stream).
    int dev = h->device;
    if (dev < 0) {
      const hipError_t e =
          stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_EP_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
      }
    }
    NoallocArea area;
    const hipError_t e = noalloc_scratch(dev, &area);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MOE_EP_ERR_HIP, "fixed record area on device %d: %s", dev, hipGetErrorString(e));
    }
    k.counts = area.counts;
    k.tokens = area.tokens;
    k.route = area.route;
  } else {
    k.counts = reinterpret_cast<int32_t*>(h->ws + h->L.off_counts);
    k.tokens = reinterpret_cast<TokenRec*>(h->ws + h->L.off_tokens);
    k.route = reinterpret_cast<uint64_t*>(h->ws + h->L.off_route);
  }
  for (int s = 0, start = 0; s < ep; ++s) {
    k.src[s].token_start = start;
    start += host_n[s];
  }
  k.off_eplb = h->L.off_eplb;
  k.eplb_bytes = has_e ? p.eplb_stats_bytes : 0;
  k.eplb_vec4 = has_e && (eplb_align_or % 4 == 0);

  k.ws = h->ws;
  k.part_stride = h->L.part_stride;
  k.off_hidden = h->L.off_hidden;
  k.off_scale = h->L.off_scale;
  k.off_ids = h->L.off_ids;
  k.off_weights = h->L.off_weights;
  k.hidden_bytes = p.hidden_row_bytes;
  k.scale_bytes = has_s ? p.scale_row_bytes : 0;
  k.scale_vec4 = has_s && (scale_align_or % 4 == 0);
  k.active = (a->active_rank_mask == MOE_EP_ALL_RANKS ? ~0ull : a->active_rank_mask) & all;
  k.owner = h->owner;
  k.num_experts = p.num_experts;
  k.top_k = p.top_k;
  k.ep = ep;
  k.tpr = tpr;
  k.invalid_id = p.invalid_expert_id;
  k.has_weights = has_w ? 1 : 0;

  if (!plan_dispatch(k, vec_bytes, p.dispatch_order))
    return fail(MOE_EP_ERR_INVALID_ARG, "destination-order dispatch grid too large for this step");
  st = check_launch_device(h, stream);
  if (st != MOE_EP_OK) return st;
  const hipError_t e = launch_dispatch(k, vec_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "dispatch launch failed: %s", hipGetErrorString(e));

  h->state = kDispatched;
  h->route = k.route;
  h->tokens = k.tokens;
  h->counts = k.counts;
  h->tpr = tpr;
  for (int s = 0; s < MOE_EP_MAX_RANKS; ++s) h->n[s] = s < ep ? host_n[s] : 0;
  h->mask = a->active_rank_mask;
  h->device_counts = dev_counts;
  for (int d = 0; d < ep; ++d) {
    uint8_t* part = h->ws + (int64_t)d * h->L.part_stride;
    results[d].hidden = part + h->L.off_hidden;
    results[d].hidden_scale = has_s ? part + h->L.off_scale : nullptr;
    results[d].topk_ids = reinterpret_cast<int32_t*>(part + h->L.off_ids);
    results[d].topk_weights = has_w ? reinterpret_cast<float*>(part + h->L.off_weights) : nullptr;
    results[d].tokens_per_rank = tpr;
    results[d].num_rows = ep * tpr;
    results[d].eplb_global_stats = has_e ? part + h->L.off_eplb : nullptr;
    results[d].dispatch_order = k.order;
  }
  return ok();
}

}  // namespace

int moe_ep_dispatch(moe_ep_handle h, const moe_ep_dispatch_args* a, moe_ep_dispatch_result* results,
                    void* stream) {
  return dispatch_impl(h, a, results, stream, false);
}

int moe_ep_dispatch_noalloc(moe_ep_handle h, const moe_ep_dispatch_args* a, moe_ep_dispatch_result* results,
                            void* stream) {
  return dispatch_impl(h, a, results, stream, true);
}

int moe_ep_get_combine_input_buffer(moe_ep_handle h, int32_t rank, int32_t dtype, void** out_ptr) {
  if (!h || !out_ptr) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle or out_ptr");
  int ust = check_workspace_usable(h);
  if (ust != MOE_EP_OK) return ust;
  if (h->state != kDispatched)
    return fail(MOE_EP_ERR_STATE, "the combine input buffer is valid only between dispatch and combine");
  if (rank < 0 || rank >= h->p.ep_size) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, h->p.ep_size);
  const int esz = dtype_bytes(dtype);
  if (esz == 0) return fail(MOE_EP_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (esz > h->p.combine_max_elem_bytes)
    return fail(MOE_EP_ERR_INVALID_ARG, "dtype of %d bytes exceeds combine_max_elem_bytes %d", esz,
                h->p.combine_max_elem_bytes);
  *out_ptr = h->ws + (int64_t)rank * h->L.part_stride + h->L.off_combine;
  return ok();
}

int moe_ep_combine(moe_ep_handle h, const moe_ep_combine_args* a, void* stream) {
  if (!h || !a) return fail(MOE_EP_ERR_INVALID_ARG, "NULL handle or args");
  const moe_ep_params& p = h->p;
  const int ep = p.ep_size;
  int ust = check_workspace_usable(h);
  if (ust != MOE_EP_OK) return ust;
  if (h->state != kDispatched) return fail(MOE_EP_ERR_STATE, "combine called without a preceding dispatch");
  int st = check_mask(p, a->active_rank_mask);
  if (st != MOE_EP_OK) return st;
  if (a->active_rank_mask != h->mask)
    return fail(MOE_EP_ERR_MASK, "combine active_rank_mask 0x%llx differs from dispatch's 0x%llx",
                (unsigned long long)a->active_rank_mask, (unsigned long long)h->mask);
  const int esz = dtype_bytes(a->dtype);
  if (esz == 0) return fail(MOE_EP_ERR_INVALID_ARG, "unknown dtype %d", a->dtype);

  const uint64_t active = (h->mask == MOE_EP_ALL_RANKS ? ~0ull : h->mask) & rank_bits(ep);
  CombineKArgs k;
  std::memset(&k, 0, sizeof(k));
  uint64_t align_or = (uint64_t)p.hidden_size * esz;
  for (int d = 0; d < ep; ++d) {
    const uint8_t* src = static_cast<const uint8_t*>(a->expert_output[d]);
    if (!((active >> d) & 1)) {      // masked-off ranks are never read
      k.expert_output[d] = nullptr;
      continue;
    }
    if (!src) {
      if (esz > p.combine_max_elem_bytes)
        return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: the combine input buffer holds %d-byte elements at most",
                    d, p.combine_max_elem_bytes);
      src = h->ws + (int64_t)d * h->L.part_stride + h->L.off_combine;
    }
    if (!aligned(src, esz)) return fail(MOE_EP_ERR_ALIGN, "rank %d: expert_output not element-aligned", d);
    align_or |= reinterpret_cast<uintptr_t>(src);
    k.expert_output[d] = src;
  }
  int32_t total = 0;
  for (int s = 0; s < ep; ++s) {
    k.token_start[s] = total;
    const int32_t n = h->n[s];
    total += n;
    if (n == 0) continue;
    if (!a->output[s]) return fail(MOE_EP_ERR_INVALID_ARG, "rank %d: NULL output with %d tokens", s, n);
    if (!aligned(a->output[s], esz)) return fail(MOE_EP_ERR_ALIGN, "rank %d: output not element-aligned", s);
    align_or |= reinterpret_cast<uintptr_t>(a->output[s]);
    k.output[s] = static_cast<uint8_t*>(a->output[s]);
  }
  k.token_start[ep] = total;
  // After a device-count dispatch, h->n holds tpr for every rank (the most
  // any rank can have); the kernel reads the counts that dispatch used.
  k.dev_counts = h->device_counts ? h->counts : nullptr;
  const int vec_elems = (int)(pow2_divisor(align_or, 16) / esz);
  k.route = h->route;
  k.tokens = h->tokens;
  k.hidden = p.hidden_size;
  k.tpr = h->tpr;
  k.ep = ep;
  st = check_launch_device(h, stream);
  if (st != MOE_EP_OK) return st;

  const hipError_t e = launch_combine(k, a->dtype, vec_elems < 1 ? 1 : vec_elems, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EP_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  h->state = kIdle;
  return ok();
}

}  // extern "C"
