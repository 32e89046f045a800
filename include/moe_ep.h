/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) rank-major MoE expert-parallel
 * dispatch/combine library (libmoe_ep.so).
 *
 * One process holds a whole expert-parallel (EP) group of ep_size logical
 * ranks.  Each rank's receive region and combine input region is a partition
 * of one caller-owned device workspace, so dispatch and combine are on-device
 * scatter / gather-reduce kernels on one GPU.  Every per-rank argument of the
 * FlashInfer API becomes an array indexed by rank.
 *
 * Sources of the contract (FlashInfer API pages for flashinfer.moe_ep):
 *   MoEEpCommunication       class description, is_platform_supported(),
 *                            dispatch(), combine(), get_combine_input_buffer(),
 *                            destroy()
 *   NVLinkOneSidedAlltoAll   class description (rank-major placement and
 *                            invalid rows), active_rank_mask(), dispatch()
 *                            (mask and weights rules), combine() (mask rule),
 *                            get_combine_input_buffer()
 *   CakeAlltoAll             class description (rows beyond a source's count)
 *
 * Conventions for every entry point:
 *   - Pointers named "device" point to GPU memory of the current HIP device;
 *     all other pointers are host memory and are read only during the call.
 *   - Validation happens on the host before anything is enqueued.  On any
 *     error no device work is queued and the handle's state is unchanged.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream of the current device) and is asynchronous: inputs must stay
 *     valid, and outputs must not be read, until the stream has passed the
 *     call.  No entry point synchronizes the device or allocates device
 *     memory.  A stream on another device than the workspace's makes
 *     dispatch and combine fail with MOE_EP_ERR_INVALID_ARG.
 *   - A handle serves one in-flight dispatch/combine pair and is not
 *     thread-safe.
 *   - Every entry point returns a moe_ep_status (0 = success) unless stated.
 *     moe_ep_last_error() describes the most recent failure of this thread.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the library's only exports. */
#define MOE_EP_API __attribute__((visibility("default")))

/* A uint64 bitmask names the active ranks, so a group has at most 64 ranks
 * (NVLinkOneSidedAlltoAll, active_rank_mask()). */
#define MOE_EP_MAX_RANKS 64
/* active_rank_mask value meaning "no mask passed": every rank is active. */
#define MOE_EP_ALL_RANKS (~(uint64_t)0)

typedef enum moe_ep_status {
  MOE_EP_OK = 0,
  MOE_EP_ERR_INVALID_ARG = -1,  /* bad pointer, size, dtype, or weights/scales passed by some ranks only */
  MOE_EP_ERR_STATE = -2,        /* call out of the dispatch -> combine -> dispatch order */
  MOE_EP_ERR_CAPACITY = -3,     /* tokens_per_rank outside [largest local count, capacity] */
  MOE_EP_ERR_MASK = -4,         /* mask without enable_rank_mask, bits >= ep_size, or combine mask != dispatch mask */
  MOE_EP_ERR_ALIGN = -5,        /* an int32/float/workspace pointer not aligned to its element */
  MOE_EP_ERR_HIP = -6,          /* a HIP runtime call failed (launch or device query) */
  MOE_EP_ERR_UNSUPPORTED = -7   /* no virtual memory management on the device, or a checkpoint
                                   call on a handle whose workspace the caller owns */
} moe_ep_status;

/* Order in which dispatch writes the receive rows (moe_ep_params.dispatch_order).
 * Both write the same bytes; they differ only in speed:
 *  SOURCE_ROW:  a workgroup reads one token row once and writes it to every
 *               destination in turn (best for large groups and fan-out).
 *  DESTINATION: a workgroup writes one (destination, row) pair; rows are
 *               pinned to XCDs so the other destinations' re-reads of a row
 *               hit that XCD's L2, and each destination's region is written
 *               as one sequential sweep (best for groups of a few ranks
 *               whose rows are mostly real tokens).
 *  AUTO:        DESTINATION when ep_size <= 16, ep_size^2 * tokens_per_rank
 *               <= 16384 and the ep_size * tokens_per_rank source rows do
 *               not fill the chip on their own (MI355X runs 256 CUs x 32
 *               waves at once); also when ep_size <= 8 and at least 80% of
 *               the ep_size * tokens_per_rank rows are real tokens (host
 *               counts only: a step with device-resident counts uses the
 *               first rule); else SOURCE_ROW.
 * An explicit DESTINATION request whose grid would pass 2^31 - 1 workgroups
 * makes moe_ep_dispatch fail with MOE_EP_ERR_INVALID_ARG (nothing launched);
 * AUTO then takes SOURCE_ROW instead. */
typedef enum moe_ep_dispatch_order {
  MOE_EP_ORDER_AUTO = 0,
  MOE_EP_ORDER_SOURCE_ROW = 1,
  MOE_EP_ORDER_DESTINATION = 2
} moe_ep_dispatch_order;

/* Element type of combine's input and output rows (both use the same one;
 * MoEEpCommunication, get_combine_input_buffer() takes any torch dtype).
 * Combine widens every element exactly to float32, adds in float32, and
 * rounds the sum once to the type, to nearest even. */
typedef enum moe_ep_dtype {
  MOE_EP_F32 = 0,
  MOE_EP_BF16 = 1,
  MOE_EP_F16 = 2                  /* IEEE binary16 */
} moe_ep_dtype;

/* Static sizes of one EP group (the pages' MoEEpCommParams plus the
 * enable_rank_mask switch of the backend config). */
typedef struct moe_ep_params {
  int32_t ep_size;                /* ranks in the group, 1..64 */
  int32_t num_experts;            /* global experts, a multiple of ep_size; rank d owns
                                     experts [d*E/ep, (d+1)*E/ep) (contiguous blocks) */
  int32_t top_k;                  /* experts per token, >= 1 */
  int32_t max_tokens_per_rank;    /* capacity: the largest local_num_tokens of any rank */
  int32_t hidden_size;            /* elements of a combine row */
  int32_t combine_max_elem_bytes; /* element size the combine input buffer is sized for: 2 (bf16,
                                     f16) or 4 (also f32) */
  int64_t hidden_row_bytes;       /* bytes of one dispatched hidden_states row (opaque) */
  int64_t scale_row_bytes;        /* bytes of one hidden_states_scale row; 0 = no scales */
  int32_t invalid_expert_id;      /* written into every top_k slot of an invalid receive row */
  int32_t enable_rank_mask;       /* nonzero: dispatch/combine accept an active_rank_mask */
  int64_t eplb_stats_bytes;       /* bytes of one rank's expert-load statistics row, gathered
                                     by dispatch (MoEEpCommunication, dispatch(),
                                     eplb_local_stats); 0 = not supported */
  int32_t dispatch_order;         /* moe_ep_dispatch_order; 0 = AUTO */
} moe_ep_params;

/* Inputs of one dispatch, per SOURCE rank s < ep_size
 * (MoEEpCommunication, dispatch()).  Entries at s >= ep_size are ignored. */
typedef struct moe_ep_dispatch_args {
  const void*    hidden[MOE_EP_MAX_RANKS];        /* device [n_s, hidden_row_bytes], rows contiguous */
  const void*    hidden_scale[MOE_EP_MAX_RANKS];  /* device [n_s, scale_row_bytes] or NULL */
  const int32_t* topk_ids[MOE_EP_MAX_RANKS];      /* device [n_s, top_k] global expert ids */
  const float*   topk_weights[MOE_EP_MAX_RANKS];  /* device [n_s, top_k] or NULL */
  int32_t        local_num_tokens[MOE_EP_MAX_RANKS]; /* n_s, 0..capacity */
  uint64_t       weights_present;  /* bit s: rank s passed topk_weights (an empty [0, top_k]
                                      tensor counts).  Must be none or all ranks. */
  uint64_t       scales_present;   /* bit s: rank s passed hidden_states_scale.  None or all. */
  int32_t        runtime_max_tokens_per_rank; /* < 0 = None = capacity; else in [max n_s, capacity] */
  uint64_t       active_rank_mask; /* MOE_EP_ALL_RANKS = no mask; else needs enable_rank_mask
                                      and only bits < ep_size */
  const void*    eplb_local_stats[MOE_EP_MAX_RANKS]; /* device [eplb_stats_bytes] per rank, or NULL */
  uint64_t       eplb_present;     /* bit s: rank s passed eplb_local_stats.  None or all; needs
                                      eplb_stats_bytes > 0 */
  const int32_t* local_num_tokens_device; /* optional device int32 [ep_size]: the token counts,
                                      read by the kernels when they run (so a captured graph
                                      replays ragged steps).  When set, local_num_tokens is
                                      ignored, each count is clamped to [0, tokens_per_rank],
                                      every rank's hidden / ids / weights / scale buffers must
                                      hold tokens_per_rank rows, and so must every combine
                                      output buffer.  NULL = use local_num_tokens. */
} moe_ep_dispatch_args;

/* What destination rank d received: views into its workspace partition,
 * valid until the next moe_ep_dispatch on the handle. */
typedef struct moe_ep_dispatch_result {
  void*    hidden;          /* device [num_rows, hidden_row_bytes] */
  void*    hidden_scale;    /* device [num_rows, scale_row_bytes], NULL when no scales passed */
  int32_t* topk_ids;        /* device [num_rows, top_k] */
  float*   topk_weights;    /* device [num_rows, top_k], NULL when no weights passed */
  int32_t  tokens_per_rank; /* tpr of this step */
  int32_t  num_rows;        /* ep_size * tokens_per_rank */
  void*    eplb_global_stats; /* device [ep_size, eplb_stats_bytes]: row s holds rank s's
                                 eplb_local_stats; NULL when none were passed */
  int32_t  dispatch_order;  /* order the kernel ran in: MOE_EP_ORDER_SOURCE_ROW or
                               MOE_EP_ORDER_DESTINATION (AUTO resolved), same for every rank */
} moe_ep_dispatch_result;

/* Inputs of one combine (MoEEpCommunication, combine()). */
typedef struct moe_ep_combine_args {
  const void* expert_output[MOE_EP_MAX_RANKS]; /* per rank d: device [ep*tpr, hidden_size] (the same
                                                  memory as [ep, tpr, hidden_size]); NULL = rank d's
                                                  combine input buffer */
  void*       output[MOE_EP_MAX_RANKS];        /* per source rank s: device [n_s, hidden_size] */
  int32_t     dtype;                           /* moe_ep_dtype of expert_output and output */
  uint64_t    active_rank_mask;                /* must equal the dispatch's mask */
} moe_ep_combine_args;

typedef struct moe_ep_handle_s* moe_ep_handle;

/* 1 when the current HIP device is a gfx950 (MI355X-class) GPU, else 0.
 * Needs no handle and does no device work
 * (MoEEpCommunication, is_platform_supported()). */
MOE_EP_API int moe_ep_is_platform_supported(void);

/* Bytes of device workspace a group with these params needs (receive
 * regions, combine input regions, and the per-token destination masks and
 * records that dispatch leaves for combine, for capacity-sized steps).
 * *out_bytes is set on success. */
MOE_EP_API int moe_ep_workspace_bytes(const moe_ep_params* params, size_t* out_bytes);

/* Creates a handle over a caller-owned device workspace of at least
 * moe_ep_workspace_bytes() bytes, aligned to 256 bytes.  The workspace is
 * borrowed until moe_ep_destroy and needs no initialisation.  Host-only: no
 * device work (it asks HIP which device holds the workspace, so dispatch
 * and combine can refuse a stream on another device). */
MOE_EP_API int moe_ep_create(const moe_ep_params* params, void* workspace, size_t workspace_bytes,
                  moe_ep_handle* out_handle);

/* Sends every token to the ranks that own its selected experts
 * (MoEEpCommunication, dispatch()) with rank-major placement
 * (NVLinkOneSidedAlltoAll, class description): on destination d, row
 * s*tpr + t holds token t of source s -- its hidden row, scale row, topk_ids
 * and topk_weights, verbatim -- when d owns one of its experts and d is
 * active.  Every other row (token not routed to d, d masked off, or
 * t >= n_s) gets invalid_expert_id in all top_k slots and weight 0.0; its
 * hidden and scale bytes are left unspecified.  tpr is
 * runtime_max_tokens_per_rank, or the capacity when it is < 0.
 * When every rank passes eplb_local_stats, each rank's statistics row is
 * also gathered into row s of a [ep_size, eplb_stats_bytes] region on every
 * rank (MoEEpCommunication, dispatch(), eplb_local_stats), in the same launch.
 * Fills results[0 .. ep_size-1] (host array) with views into the workspace.
 * Needs the IDLE state; leaves the handle DISPATCHED.  One kernel launch. */
MOE_EP_API int moe_ep_dispatch(moe_ep_handle handle, const moe_ep_dispatch_args* args,
                    moe_ep_dispatch_result* results, void* stream);

/* Rank `rank`'s combine input buffer: device [ep_size*tpr, hidden_size] of
 * `dtype`, in its workspace partition, for the expert computation to write
 * into (MoEEpCommunication and NVLinkOneSidedAlltoAll,
 * get_combine_input_buffer()).  Valid only between dispatch and combine
 * (ERR_STATE otherwise); dtype's size must not exceed
 * combine_max_elem_bytes. */
MOE_EP_API int moe_ep_get_combine_input_buffer(moe_ep_handle handle, int32_t rank, int32_t dtype,
                                    void** out_ptr);

/* For every source rank s and token t < n_s: output[s][t] = sum, over the
 * ranks d that token was dispatched to in ascending d, of
 * expert_output[d][s*tpr + t], accumulated in float32 from +0.0 and rounded
 * once to dtype (bfloat16, float16: round to nearest even).  A token that reached no
 * rank gets zeros.  Rows of tokens not dispatched to d are never read, nor is
 * any row of a masked-off rank (MoEEpCommunication, combine();
 * NVLinkOneSidedAlltoAll, combine() mask rule).  Needs the DISPATCHED state;
 * leaves the handle IDLE.  One kernel launch.  After a host-count dispatch,
 * when the read ranks' expert_output rows and the non-empty outputs each lie
 * at one constant stride (the combine input buffers do; so do outputs sliced
 * from one [ep_size, n, hidden_size] allocation), the launch carries only
 * scalar arguments, which the HIP runtime enqueues ~0.6 us faster. */
MOE_EP_API int moe_ep_combine(moe_ep_handle handle, const moe_ep_combine_args* args, void* stream);

/* Releases the handle's host state; a workspace passed to moe_ep_create
 * stays the caller's, one made by moe_ep_create_vmm is unmapped and freed
 * (after waiting for the device).  NULL is a no-op.  Device work already
 * enqueued with the handle must have finished before a caller-owned
 * workspace is reused (MoEEpCommunication, destroy()). */
MOE_EP_API int moe_ep_destroy(moe_ep_handle handle);

/* Creates a handle whose workspace the library maps itself with HIP virtual
 * memory management on the current device: a reserved virtual address range
 * backed by one physical allocation.  Only such a handle can release its
 * physical memory for a process checkpoint while its addresses stay put
 * (NVLinkOneSidedAlltoAll and CakeAlltoAll, checkpoint_prepare() and
 * checkpoint_restore()).  ERR_UNSUPPORTED when the device lacks virtual
 * memory management; ERR_HIP when a mapping call fails (nothing is left
 * allocated). */
MOE_EP_API int moe_ep_create_vmm(const moe_ep_params* params, moe_ep_handle* out_handle);

/* Device address and size of the handle's workspace.  For a handle from
 * moe_ep_create_vmm the address is the same for the handle's whole life,
 * across checkpoints, but must not be touched while the memory is released. */
MOE_EP_API int moe_ep_workspace(moe_ep_handle handle, void** out_ptr, size_t* out_bytes);

/* Before a process checkpoint: waits for the device, then unmaps and
 * releases the workspace's physical memory, keeping its virtual addresses
 * reserved so that HIP graphs captured on the workspace replay once
 * moe_ep_checkpoint_restore has backed it again.  Only between rounds
 * (ERR_STATE after a dispatch without its combine).  A second call does
 * nothing.  Until the restore, dispatch, combine and
 * get_combine_input_buffer return ERR_STATE.  ERR_UNSUPPORTED for handles
 * from moe_ep_create.  If unmapping fails part-way the handle is unusable
 * (every later call but destroy returns ERR_STATE). */
MOE_EP_API int moe_ep_checkpoint_prepare(moe_ep_handle handle);

/* After the checkpoint: backs the reserved addresses with new physical
 * memory (contents undefined; the workspace needs no initialisation).  Does
 * nothing when the workspace is mapped.  If mapping fails part-way the
 * handle is unusable, as above. */
MOE_EP_API int moe_ep_checkpoint_restore(moe_ep_handle handle);

/* Receive rows (ep_size * tokens_per_rank) of the largest step
 * moe_ep_dispatch_noalloc takes: the size of the library's fixed record area
 * (24 bytes per row plus 256, 1.5 MiB, held on each GPU the library runs on
 * until the process ends). */
#define MOE_EP_NOALLOC_MAX_ROWS 65536

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * dispatch as moe_ep_dispatch -- same arguments, results, state change and
 * errors -- except that the per-token routing records dispatch leaves for
 * combine (destination masks, token positions, token counts) go to a fixed
 * device array inside the library instead of the workspace.  The handle's
 * next moe_ep_combine reads them from there.  Nothing is allocated or freed:
 * the array's device address is looked up once per device (at moe_ep_create
 * when the workspace's device is known, else at the first call on a device).
 * ERR_CAPACITY when ep_size * tokens_per_rank exceeds MOE_EP_NOALLOC_MAX_ROWS
 * (nothing enqueued); ERR_HIP when the lookup fails.
 * Every handle on a GPU shares that GPU's one array, and it keeps only the
 * last noalloc dispatch's records: a noalloc dispatch must not run between
 * another handle's noalloc dispatch and that handle's combine on the same
 * GPU (in stream order), and calls that overlap on one GPU, from several
 * streams or threads, race. */
MOE_EP_API int moe_ep_dispatch_noalloc(moe_ep_handle handle, const moe_ep_dispatch_args* args,
                                       moe_ep_dispatch_result* results, void* stream);

/* Bitmask with bit r set for each of the n listed ranks, all in [0, 64)
 * (NVLinkOneSidedAlltoAll, active_rank_mask()).  ERR_MASK for a rank out of
 * range. */
MOE_EP_API int moe_ep_active_rank_mask(const int32_t* ranks, int32_t n, uint64_t* out_mask);

/* Static text for a status code. */
MOE_EP_API const char* moe_ep_status_string(int status);

/* Description of this thread's most recent failed call ("" if none). */
MOE_EP_API const char* moe_ep_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
