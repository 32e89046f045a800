// Host-only driver of the C ABI's validation and planning paths, built with
// the address and undefined-behaviour sanitizers by tests/test_host_sanitized.py.
// No call here reaches the GPU: every dispatch/combine below is rejected by
// the host checks before anything is enqueued, so the two kernel launchers
// are stubs that must never run.

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "moe_ep.h"
#include "moe_ep_internal.h"

namespace moe_ep_detail {
hipError_t launch_dispatch(const DispatchKArgs&, int, hipStream_t) {
  std::printf("launch_dispatch reached\n");
  return hipErrorInvalidValue;
}
hipError_t launch_combine(const CombineKArgs&, int, int, hipStream_t) {
  std::printf("launch_combine reached\n");
  return hipErrorInvalidValue;
}
hipError_t noalloc_scratch(int, NoallocArea*) {
  std::printf("noalloc_scratch reached\n");
  return hipErrorInvalidValue;
}
}  // namespace moe_ep_detail

namespace {

void* const kFakeWorkspace = reinterpret_cast<void*>(uintptr_t(1) << 40);
int g_fails = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s (%s)\n", what, moe_ep_last_error());
    ++g_fails;
  }
}

moe_ep_params base() {
  moe_ep_params p;
  std::memset(&p, 0, sizeof(p));
  p.ep_size = 4;
  p.num_experts = 8;
  p.top_k = 2;
  p.max_tokens_per_rank = 16;
  p.hidden_size = 128;
  p.combine_max_elem_bytes = 4;
  p.hidden_row_bytes = 512;
  p.invalid_expert_id = -1;
  return p;
}

}  // namespace

int main() {
  size_t n = 0;
  // Sizes at and beyond every limit: the layout arithmetic must not overflow.
  for (int ep : {-1, 0, 1, 3, 8, 64, 65})
    for (int cap : {-5, 0, 1, 1 << 20, 1 << 25, 1 << 30})
      for (long long hb : {1LL, 7LL, 14336LL, (1LL << 31) - 1, 1LL << 31})
        for (int order : {-1, 0, 1, 2, 3}) {
          moe_ep_params p = base();
          p.ep_size = ep;
          p.num_experts = ep > 0 ? 2 * ep : 2;
          p.max_tokens_per_rank = cap;
          p.hidden_row_bytes = hb;
          p.scale_row_bytes = hb / 3;
          p.eplb_stats_bytes = hb / 5;
          p.dispatch_order = order;
          (void)moe_ep_workspace_bytes(&p, &n);
        }

  // Launch shapes over many row sizes: every tile covers its row.
  using moe_ep_detail::LaunchShape;
  for (int64_t nv = 1; nv <= 70000; nv = nv < 64 ? nv + 1 : nv * 3 / 2) {
    const LaunchShape t = moe_ep_detail::row_tile(7, nv);
    expect(t.u == 7 || t.u == 8, "tile u");
    expect(t.block % 64 == 0 && t.block <= moe_ep_detail::kDispatchBlock, "tile block");
    expect((int64_t)t.grid_y * t.block * t.u >= nv || t.grid_y == moe_ep_detail::kMaxGridY, "tile covers the row");
    for (int64_t rows : {1, 4096, 8192}) {
      const LaunchShape d = moe_ep_detail::dispatch_shape(rows, nv * 16, 16);
      expect(d.u == 4 || d.u == 7 || d.u == 8, "dispatch tile u");
      expect((int64_t)d.grid_y * d.block * d.u >= nv || d.grid_y == moe_ep_detail::kMaxGridY, "dispatch covers the row");
    }
    const LaunchShape c = moe_ep_detail::combine_shape(5, nv, 1);
    expect((int64_t)c.grid_y * c.block * c.u >= nv || c.grid_y == moe_ep_detail::kMaxGridY, "combine covers the row");
    expect(c.lds == ((nv + 63) / 64 >= moe_ep_detail::kCombineCapChunks ? moe_ep_detail::kCombineCapLds : 0),
           "combine residency cap only on rows of many chunks");
  }

  // The copy order AUTO picks: destination-major for groups of at most 16
  // ranks with ep * ep * tpr <= 16384 while the source rows alone do not
  // fill the chip; else source-row.
  // fill: percent of each rank's tpr rows that are real tokens (host counts);
  // devn: counts come from device memory.
  struct OrderCase { int ep, tpr; int64_t row_bytes; int requested, expect; int fill = 0; bool devn = false; };
  const OrderCase order_cases[] = {
      {8, 128, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},    // DeepSeek-V3 decode round
      {8, 256, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {8, 64, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {8, 32, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {8, 1, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {8, 512, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},     // ep * ep * tpr > 16384
      {8, 128, 8192, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {4, 512, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {4, 256, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {4, 1024, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},    // 4096 source rows fill the chip
      {4, 1024, 8192, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},     // 4096 two-wave source rows too
      {2, 2048, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},
      {16, 32, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {16, 64, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {16, 16, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {16, 256, 7168, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},     // 16-rank fp8 round
      {32, 256, 8192, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW},     // more than 16 ranks
      {4, 16, 512, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION},
      {4, 16, 512, MOE_EP_ORDER_DESTINATION, MOE_EP_ORDER_DESTINATION},
      {8, 0, 14336, MOE_EP_ORDER_DESTINATION, MOE_EP_ORDER_DESTINATION},
      {8, 128, 14336, MOE_EP_ORDER_SOURCE_ROW, MOE_EP_ORDER_SOURCE_ROW},
      // groups of at most 8 ranks with at least 80% real rows: destination-major past the bounds
      {8, 512, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION, 100},
      {8, 2048, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION, 100},
      {8, 1024, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION, 81},
      {8, 1024, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW, 75},
      {8, 1024, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW, 100, true},   // device counts
      {4, 1024, 14336, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION, 100},
      {8, 512, 7168, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_DESTINATION, 100},
      {16, 256, 7168, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW, 100},          // more than 8 ranks
      {8, 445, 8192, MOE_EP_ORDER_AUTO, MOE_EP_ORDER_SOURCE_ROW, 42},            // the ragged step's fill
  };
  for (const OrderCase& oc : order_cases) {
    moe_ep_detail::DispatchKArgs k;
    std::memset(&k, 0, sizeof(k));
    k.ep = oc.ep;
    k.tpr = oc.tpr;
    k.hidden_bytes = oc.row_bytes;
    for (int s = 0; s < oc.ep; ++s) k.src[s].n = (int32_t)((int64_t)oc.tpr * oc.fill / 100);
    static const int32_t dev_counts_stand_in = 0;
    if (oc.devn) k.dev_n = &dev_counts_stand_in;
    expect(moe_ep_detail::plan_dispatch(k, 16, oc.requested), "plan_dispatch");
    expect(k.order == oc.expect, "dispatch order");
    if (k.order == MOE_EP_ORDER_DESTINATION) {
      // every (destination, row, chunk) item of the decode exists
      expect(k.dm_items == 8LL * k.dm_blocks * k.ep * k.dm_block_rows * k.dm_chunks, "item count");
      expect(8LL * k.dm_blocks * k.dm_block_rows >= (int64_t)k.ep * k.tpr, "blocks cover the rows");
      expect((int64_t)k.dm_chunks * k.dm_threads * k.dm_u * 16 >= oc.row_bytes, "chunks cover the row");
    } else {
      expect(k.dm_items == 0, "no destination-major items");
    }
  }

  // Multiply-shift division (item decodes): exact for 0 <= x < 2^31.
  for (uint32_t dv : {1u, 2u, 3u, 5u, 7u, 8u, 14u, 16u, 36u, 64u, 127u, 128u, 1000u, 65535u, 65536u,
                      (1u << 30) + 7u, 0x7fffffffu}) {
    const moe_ep_detail::OwnerDiv od = moe_ep_detail::make_owner_div(dv);
    for (uint64_t x : {(uint64_t)0, (uint64_t)1, (uint64_t)dv - 1, (uint64_t)dv, (uint64_t)dv + 1,
                       (uint64_t)12345, (uint64_t)1 << 20, ((uint64_t)1 << 31) - 2, ((uint64_t)1 << 31) - 1}) {
      if (x >= ((uint64_t)1 << 31)) continue;
      expect(((x * od.magic) >> od.shift) == x / dv, "multiply-shift division");
    }
  }

  // Destination-major residency cap: lean kernel, grids of 8192+ workgroups.
  expect(moe_ep_detail::dispatch_dst_lds(8192, true) == 16384 && 163840 / 16384 == 10, "dispatch cap on large grids");
  expect(moe_ep_detail::dispatch_dst_lds(8191, true) == 0, "no dispatch cap below two generations");
  expect(moe_ep_detail::dispatch_dst_lds(16384, false) == 0, "no dispatch cap on the full kernel");

  // Combine grid: every (token slot, chunk) once, token 8q + x on XCD x.
  for (int64_t tokens : {1, 7, 8, 9, 1000, 1024}) {
    const LaunchShape c = moe_ep_detail::combine_shape(tokens, 7168, 8);
    const int64_t slots = (tokens + 7) / 8 * 8;
    expect(c.grid_x == slots * c.grid_y && c.block == moe_ep_detail::kCombineBlock, "combine grid");
    expect(c.lds == moe_ep_detail::kCombineCapLds && 163840 / c.lds == 18, "combine residency cap on 14 KiB rows");
    expect((int64_t)c.grid_y * c.block >= 7168 / 8, "combine chunks cover the row");
    const moe_ep_detail::OwnerDiv od = moe_ep_detail::make_owner_div((uint32_t)c.grid_y);
    std::vector<int> seen((size_t)slots * c.grid_y, 0);
    for (int64_t i = 0; i < c.grid_x; ++i) {
      const int64_t rest = i >> 3;
      const int64_t q = (int64_t)(((uint64_t)rest * od.magic) >> od.shift);
      const int64_t chunk = rest - q * c.grid_y;
      const int64_t b = q * 8 + (i & 7);
      expect(b % 8 == i % 8 && chunk >= 0 && chunk < c.grid_y && b < slots, "combine decode");
      if (b < slots && chunk >= 0 && chunk < c.grid_y) ++seen[(size_t)(b * c.grid_y + chunk)];
    }
    for (int v : seen) expect(v == 1, "combine decode covers every item once");
  }

  // Constant-stride detection of the combine inputs (NULL = masked rank).
  {
    using moe_ep_detail::common_stride;
    const uint8_t* base = nullptr;
    int64_t stride = -1;
    uint8_t* const b0 = reinterpret_cast<uint8_t*>(uintptr_t(1) << 36);
    const uint8_t* p4[4] = {b0, b0 + 1000, b0 + 2000, b0 + 3000};
    expect(common_stride(p4, 4, &base, &stride) && base == b0 && stride == 1000, "stride forward");
    const uint8_t* r4[4] = {b0 + 3000, b0 + 2000, b0 + 1000, b0};
    expect(common_stride(r4, 4, &base, &stride) && base == b0 + 3000 && stride == -1000, "stride reverse");
    const uint8_t* g4[4] = {nullptr, b0 + 1000, nullptr, b0 + 3000};
    expect(common_stride(g4, 4, &base, &stride) && base == b0 && stride == 1000, "stride with masked ranks");
    const uint8_t* u4[4] = {b0, b0 + 1000, b0 + 2001, b0 + 3000};
    expect(!common_stride(u4, 4, &base, &stride), "uneven");
    const uint8_t* h4[4] = {nullptr, b0 + 1000, nullptr, b0 + 2001};
    expect(!common_stride(h4, 4, &base, &stride), "stride not a whole multiple across a gap");
    const uint8_t* one[3] = {nullptr, b0 + 77, nullptr};
    expect(common_stride(one, 3, &base, &stride) && base == b0 + 77 && stride == 0, "one rank");
    const uint8_t* none[2] = {nullptr, nullptr};
    expect(common_stride(none, 2, &base, &stride) && base == nullptr && stride == 0, "no rank");
    const uint8_t* same[3] = {b0, b0, b0};
    expect(common_stride(same, 3, &base, &stride) && base == b0 && stride == 0, "one buffer for every rank");
  }

  // Validation paths of one handle over a fake workspace.
  moe_ep_params p = base();
  expect(moe_ep_workspace_bytes(&p, &n) == MOE_EP_OK, "workspace_bytes");
  moe_ep_handle h = nullptr;
  expect(moe_ep_create(&p, kFakeWorkspace, n, &h) == MOE_EP_OK, "create");
  moe_ep_dispatch_args a;
  std::memset(&a, 0, sizeof(a));
  a.runtime_max_tokens_per_rank = -1;
  a.active_rank_mask = MOE_EP_ALL_RANKS;
  moe_ep_dispatch_result res[MOE_EP_MAX_RANKS];
  a.local_num_tokens[0] = 17;
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_CAPACITY, "capacity");
  a.local_num_tokens[0] = 5;
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_INVALID_ARG, "NULL rows");
  a.hidden[0] = kFakeWorkspace;
  a.topk_ids[0] = reinterpret_cast<const int32_t*>(static_cast<char*>(kFakeWorkspace) + 2);
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_ALIGN, "misaligned ids");
  a.topk_ids[0] = static_cast<const int32_t*>(kFakeWorkspace);
  a.active_rank_mask = 0x3;
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_MASK, "mask without enable");
  a.active_rank_mask = MOE_EP_ALL_RANKS;
  a.weights_present = 0x1;
  a.topk_weights[0] = static_cast<const float*>(kFakeWorkspace);
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_INVALID_ARG, "weights from some ranks");
  moe_ep_combine_args c;
  std::memset(&c, 0, sizeof(c));
  c.active_rank_mask = MOE_EP_ALL_RANKS;
  expect(moe_ep_combine(h, &c, nullptr) == MOE_EP_ERR_STATE, "combine before dispatch");
  void* buf = nullptr;
  expect(moe_ep_get_combine_input_buffer(h, 0, MOE_EP_F32, &buf) == MOE_EP_ERR_STATE, "buffer before dispatch");
  expect(moe_ep_checkpoint_prepare(h) == MOE_EP_ERR_UNSUPPORTED, "checkpoint on a caller workspace");
  expect(moe_ep_destroy(h) == MOE_EP_OK, "destroy");
  expect(moe_ep_destroy(nullptr) == MOE_EP_OK, "destroy NULL");

  // An explicit destination-major request whose grid passes 2^31 - 1.
  p = base();
  p.ep_size = 64;
  p.num_experts = 64;
  p.top_k = 1;
  p.max_tokens_per_rank = 1 << 19;
  p.hidden_size = 8;
  p.combine_max_elem_bytes = 2;
  p.hidden_row_bytes = 16;
  p.dispatch_order = MOE_EP_ORDER_DESTINATION;
  expect(moe_ep_workspace_bytes(&p, &n) == MOE_EP_OK, "workspace_bytes 2");
  expect(moe_ep_create(&p, kFakeWorkspace, n, &h) == MOE_EP_OK, "create 2");
  std::memset(&a, 0, sizeof(a));
  a.runtime_max_tokens_per_rank = 1 << 19;
  a.active_rank_mask = MOE_EP_ALL_RANKS;
  expect(moe_ep_dispatch(h, &a, res, nullptr) == MOE_EP_ERR_INVALID_ARG, "grid limit");
  // The same step is past the fixed record area of the noalloc dispatch.
  expect(moe_ep_dispatch_noalloc(h, &a, res, nullptr) == MOE_EP_ERR_CAPACITY, "noalloc area");
  a.runtime_max_tokens_per_rank = MOE_EP_NOALLOC_MAX_ROWS / 64 + 1;
  expect(moe_ep_dispatch_noalloc(h, &a, res, nullptr) == MOE_EP_ERR_CAPACITY, "noalloc area + 1 token");
  expect(moe_ep_destroy(h) == MOE_EP_OK, "destroy 2");

  int32_t ranks[] = {0, 5, 63};
  uint64_t m = 0;
  expect(moe_ep_active_rank_mask(ranks, 3, &m) == MOE_EP_OK && m == ((1ull << 63) | (1ull << 5) | 1ull), "mask helper");
  int32_t bad[] = {64};
  expect(moe_ep_active_rank_mask(bad, 1, &m) == MOE_EP_ERR_MASK, "mask helper range");
  for (int s = -9; s <= 2; ++s) expect(moe_ep_status_string(s) != nullptr, "status string");

  std::printf("fails %d\n", g_fails);
  return g_fails == 0 ? 0 : 1;
}
