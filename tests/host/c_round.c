/* One dispatch + combine round through the C ABI alone (no Python, no
 * torch): device memory from hipMalloc, a HIP stream, and checks that need
 * no reference implementation.
 *
 *  - Placement (NVLinkOneSidedAlltoAll, class description): on rank d, row
 *    s*tpr + t holds token (s, t) -- its hidden bytes, ids and weights --
 *    when d owns one of its experts (experts [2d, 2d+2) here); every other
 *    row carries the invalid id in all top_k slots and weight 0.
 *  - Combine (MoEEpCommunication, combine()): with rank d's expert rows all
 *    equal to 2^d (and NaN in rows no token was sent to), token (s, t)'s
 *    output is the sum of 2^d over the ranks it reached: its destination
 *    mask as a float, exact in float32.
 *
 * Runs both dispatch entry points (moe_ep_dispatch, moe_ep_dispatch_noalloc).
 * Prints "c_round ok" and exits 0 on success, exits 1 on the first mismatch.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

#define EP 4
#define E 8
#define K 2
#define CAP 16
#define HID 64                         /* float32 elements per row */
#define HB (HID * 4)                   /* hidden row bytes */

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
#define CHECK_EP(x) do { int st_ = (x); if (st_ != MOE_EP_OK) { \
  printf("moe_ep error %s (%s) at line %d\n", moe_ep_status_string(st_), moe_ep_last_error(), __LINE__); return 1; } } while (0)
#define FAIL(...) do { printf(__VA_ARGS__); printf("\n"); return 1; } while (0)

static const int n_tok[EP] = {16, 5, 0, 9};

/* the two experts of token (s, t): distinct, in [0, E) */
static void experts(int s, int t, int out[K]) {
  out[0] = (s + t) % E;
  out[1] = (s + 3 * t + 1) % E;
  if (out[1] == out[0]) out[1] = (out[0] + 1) % E;
}

static int round_trip(moe_ep_handle h, void* stream, int noalloc, float* d_hidden[EP], int32_t* d_ids[EP],
                      float* d_w[EP], float* d_out[EP]) {
  moe_ep_dispatch_args a;
  memset(&a, 0, sizeof(a));
  for (int s = 0; s < EP; ++s) {
    a.hidden[s] = d_hidden[s];
    a.topk_ids[s] = d_ids[s];
    a.topk_weights[s] = d_w[s];
    a.local_num_tokens[s] = n_tok[s];
  }
  a.weights_present = (1u << EP) - 1;
  a.runtime_max_tokens_per_rank = -1;
  a.active_rank_mask = MOE_EP_ALL_RANKS;
  moe_ep_dispatch_result res[EP];
  CHECK_EP(noalloc ? moe_ep_dispatch_noalloc(h, &a, res, stream) : moe_ep_dispatch(h, &a, res, stream));
  CHECK_HIP(hipStreamSynchronize((hipStream_t)stream));

  const int tpr = res[0].tokens_per_rank;
  if (tpr != CAP) FAIL("tokens_per_rank %d, expected %d", tpr, CAP);
  static int32_t ids[EP * CAP * K];
  static float w[EP * CAP * K];
  static float hid[EP * CAP * HID];
  for (int d = 0; d < EP; ++d) {
    CHECK_HIP(hipMemcpy(ids, res[d].topk_ids, sizeof(ids), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(w, res[d].topk_weights, sizeof(w), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hid, res[d].hidden, sizeof(hid), hipMemcpyDeviceToHost));
    for (int s = 0; s < EP; ++s) {
      for (int t = 0; t < tpr; ++t) {
        const int r = s * tpr + t;
        int ex[K];
        experts(s, t, ex);
        const int routed = t < n_tok[s] && (ex[0] / 2 == d || ex[1] / 2 == d);
        for (int j = 0; j < K; ++j) {
          const int32_t want_id = routed ? ex[j] : -1;
          const float want_w = routed ? (float)(j + 1) : 0.0f;
          if (ids[r * K + j] != want_id) FAIL("rank %d row %d slot %d: id %d, expected %d", d, r, j, ids[r * K + j], want_id);
          if (w[r * K + j] != want_w) FAIL("rank %d row %d slot %d: weight %g, expected %g", d, r, j, w[r * K + j], want_w);
        }
        if (routed)
          for (int c = 0; c < HID; ++c)
            if (hid[r * HID + c] != (float)(s * 1000 + t * 10 + c % 7))
              FAIL("rank %d row %d element %d: %g", d, r, c, hid[r * HID + c]);
      }
    }
  }

  /* expert outputs: 2^d on routed rows, NaN elsewhere */
  for (int d = 0; d < EP; ++d) {
    void* buf = NULL;
    CHECK_EP(moe_ep_get_combine_input_buffer(h, d, MOE_EP_F32, &buf));
    static float eo[EP * CAP * HID];
    CHECK_HIP(hipMemcpy(ids, res[d].topk_ids, sizeof(ids), hipMemcpyDeviceToHost));
    for (int r = 0; r < EP * tpr; ++r)
      for (int c = 0; c < HID; ++c) eo[r * HID + c] = ids[r * K] != -1 ? ldexpf(1.0f, d) : NAN;
    CHECK_HIP(hipMemcpy(buf, eo, sizeof(eo), hipMemcpyHostToDevice));
  }
  moe_ep_combine_args c;
  memset(&c, 0, sizeof(c));
  for (int s = 0; s < EP; ++s) c.output[s] = d_out[s];
  c.dtype = MOE_EP_F32;
  c.active_rank_mask = MOE_EP_ALL_RANKS;
  CHECK_EP(moe_ep_combine(h, &c, stream));
  CHECK_HIP(hipStreamSynchronize((hipStream_t)stream));
  for (int s = 0; s < EP; ++s) {
    static float out[CAP * HID];
    if (!n_tok[s]) continue;
    CHECK_HIP(hipMemcpy(out, d_out[s], (size_t)n_tok[s] * HB, hipMemcpyDeviceToHost));
    for (int t = 0; t < n_tok[s]; ++t) {
      int ex[K];
      experts(s, t, ex);
      const float want = (float)((1 << (ex[0] / 2)) | (1 << (ex[1] / 2)));
      for (int cc = 0; cc < HID; ++cc)
        if (out[t * HID + cc] != want) FAIL("token (%d, %d) element %d: %g, expected %g", s, t, cc, out[t * HID + cc], want);
    }
  }
  return 0;
}

int main(void) {
  if (!moe_ep_is_platform_supported()) FAIL("not a gfx950 device");
  moe_ep_params p;
  memset(&p, 0, sizeof(p));
  p.ep_size = EP; p.num_experts = E; p.top_k = K; p.max_tokens_per_rank = CAP; p.hidden_size = HID;
  p.combine_max_elem_bytes = 4; p.hidden_row_bytes = HB; p.invalid_expert_id = -1;
  size_t bytes = 0;
  CHECK_EP(moe_ep_workspace_bytes(&p, &bytes));
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, bytes));
  moe_ep_handle h = NULL;
  CHECK_EP(moe_ep_create(&p, ws, bytes, &h));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  float* d_hidden[EP]; int32_t* d_ids[EP]; float* d_w[EP]; float* d_out[EP];
  for (int s = 0; s < EP; ++s) {
    const int n = n_tok[s] ? n_tok[s] : 1;
    float hb[CAP * HID]; int32_t ib[CAP * K]; float wb[CAP * K];
    for (int t = 0; t < n_tok[s]; ++t) {
      int ex[K];
      experts(s, t, ex);
      for (int j = 0; j < K; ++j) { ib[t * K + j] = ex[j]; wb[t * K + j] = (float)(j + 1); }
      for (int c = 0; c < HID; ++c) hb[t * HID + c] = (float)(s * 1000 + t * 10 + c % 7);
    }
    CHECK_HIP(hipMalloc((void**)&d_hidden[s], (size_t)n * HB));
    CHECK_HIP(hipMalloc((void**)&d_ids[s], (size_t)n * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_w[s], (size_t)n * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_out[s], (size_t)n * HB));
    if (n_tok[s]) {
      CHECK_HIP(hipMemcpy(d_hidden[s], hb, (size_t)n_tok[s] * HB, hipMemcpyHostToDevice));
      CHECK_HIP(hipMemcpy(d_ids[s], ib, (size_t)n_tok[s] * K * 4, hipMemcpyHostToDevice));
      CHECK_HIP(hipMemcpy(d_w[s], wb, (size_t)n_tok[s] * K * 4, hipMemcpyHostToDevice));
    }
  }
  for (int noalloc = 0; noalloc < 2; ++noalloc) {
    if (round_trip(h, stream, noalloc, d_hidden, d_ids, d_w, d_out)) {
      printf("c_round failed (%s)\n", noalloc ? "moe_ep_dispatch_noalloc" : "moe_ep_dispatch");
      return 1;
    }
  }
  CHECK_EP(moe_ep_destroy(h));
  CHECK_EP(moe_ep_destroy(NULL));
  for (int s = 0; s < EP; ++s) {
    CHECK_HIP(hipFree(d_hidden[s])); CHECK_HIP(hipFree(d_ids[s])); CHECK_HIP(hipFree(d_w[s])); CHECK_HIP(hipFree(d_out[s]));
  }
  CHECK_HIP(hipStreamDestroy(stream));
  CHECK_HIP(hipFree(ws));
  printf("c_round ok\n");
  return 0;
}
