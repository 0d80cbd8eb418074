/*
 * spkv.h -- C ABI of the streaming two-stream paged-KV attention library
 * (libspkv.so, MI355X / gfx950).
 *
 * The operations follow the KV-cache manager that these pages describe:
 *   [LB-KV]   "How LingBot-Map Implements the KV Cache Mechanism for Streaming
 *             Inference with FlashInfer Integration" (instagit.com)
 *   [LB-PERF] "How to Improve Streaming Inference Performance with FlashInfer
 *             KV Cache Backend" (instagit.com)
 *   [LB-SLOT] "LingBot-Map KV缓存机制深度揭秘：scale frames与keyframes如何占用slot"
 *             (mhpq.cn)
 *
 * Model.  Every transformer block owns one pool of pages
 *   pool[max_num_pages][2][page_size][num_heads][head_dim]   bf16, 0 = K, 1 = V
 * ([LB-KV] "Physical Page Layout and Indexing").  Pages 0..M-1, with
 * M = scale_frames + sliding_window + headroom, are recyclable patch pages
 * holding one frame's patch tokens each; pages M.. are the append-only special
 * stream, which packs floor(page_size / num_special_tokens) frames per page
 * ([LB-SLOT] sections on the two-stream layout and the special-token stream).
 * A frame's tokens are ordered [special..., patch...] (6 specials: camera,
 * 4 registers, scale).  Per block the library keeps, on the host, the scale
 * page list (the first scale_frames frames, never evicted), the live-window
 * deque and the free list; a manager-wide flag defers eviction.
 *
 * Conventions of all calls.
 *   - Return 0 (SPKV_OK) or a negative SPKV_ERR_* code; no exception crosses
 *     the ABI.  On any error the handle's state is unchanged.
 *   - Device pointers must be 16-byte aligned and point to memory of the
 *     device that was current when the handle was created.
 *   - `hip_stream` is a hipStream_t (NULL = the null stream).  append_frame,
 *     plan and run only enqueue work on it and return; plan and run of one
 *     frame step must use one stream (or the caller orders them).  All other
 *     calls are synchronous host operations.
 *   - A handle is not thread-safe: one host thread drives it at a time.
 *   - Only bf16 K/V/Q/O and head_dim == 64 are supported by the attention
 *     kernel; create() reports SPKV_ERR_UNSUPPORTED otherwise.
 *
 * Host-only handles.  create() with pool_ptrs == NULL and workspace == NULL
 * builds a handle that runs the page-pool bookkeeping only (no device memory,
 * no kernels): append_frame then takes k == v == NULL, plan builds the table
 * on the host, and run validates its arguments and the plan and then returns
 * SPKV_ERR_UNSUPPORTED.  It needs no GPU.
 */
#ifndef SPKV_H
#define SPKV_H

#include <stdint.h>

#if defined(__GNUC__)
#define SPKV_API __attribute__((visibility("default")))
#else
#define SPKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum spkv_status {
  SPKV_OK = 0,
  SPKV_ERR_INVALID_ARG = -1,         /* bad argument value, size or pointer */
  SPKV_ERR_BAD_BLOCK = -2,           /* block index out of range */
  SPKV_ERR_POOL_EXHAUSTED = -3,      /* no free patch page */
  SPKV_ERR_SPECIAL_OVERFLOW = -4,    /* special stream full */
  SPKV_ERR_NOTHING_TO_ROLLBACK = -5, /* no append to undo, or pages moved since */
  SPKV_ERR_EMPTY = -6,               /* plan with no frame in block 0 */
  SPKV_ERR_NOT_PLANNED = -7,         /* run before any plan (or after reset) */
  SPKV_ERR_STALE_PLAN = -8,          /* block state differs from the plan's */
  SPKV_ERR_UNSUPPORTED = -9,         /* valid request this library does not do */
  SPKV_ERR_HIP = -10,                /* a HIP runtime call or launch failed */
  SPKV_ERR_WORKSPACE = -11           /* workspace smaller than required */
};

typedef struct spkv_handle spkv_handle;

/* Manager parameters ([LB-PERF] "Minimal Streaming Inference Setup"; patch
 * pool size from [LB-KV] "How is memory bounded in streaming mode?"). */
typedef struct spkv_config {
  int32_t num_blocks;         /* transformer blocks, one pool each (>= 1) */
  int32_t num_heads;          /* H: query heads == K/V heads (>= 1) */
  int32_t head_dim;           /* D: must be 64 */
  int32_t page_size;          /* tokens per page (>= num_special_tokens) */
  int32_t patch_tokens;       /* P: patch tokens per frame, 1..page_size */
  int32_t num_special_tokens; /* specials per frame, first in the frame (6) */
  int32_t scale_frames;       /* S: frames kept forever as scale anchors (>= 0) */
  int32_t sliding_window;     /* W: live patch pages kept (>= 1) */
  int32_t headroom;           /* R: spare patch pages (>= 0) */
  int32_t max_total_frames;   /* frames the special stream is sized for (>= 1) */
} spkv_config;

/* get_cache_stats ([LB-SLOT] "动手验证：查看你的 KV 缓存占用"). */
typedef struct spkv_stats {
  int64_t frame_count;    /* frames whose specials are in the stream */
  int32_t scale_pages;
  int32_t live_pages;
  int32_t free_pages;
  int32_t reserved;       /* always 0 */
  int64_t special_tokens; /* num_special_tokens * frame_count */
} spkv_stats;

/* Sizes a caller needs before create():
 *   max_num_pages        = M + ceil(max_total_frames / floor(page_size / ns))
 *   pool_bytes_per_block = max_num_pages * 2 * page_size * H * D * 2
 *   min_workspace_bytes  = the least device workspace create() accepts: the
 *                          double-buffered device page table and its two
 *                          per-token expansions (4 bytes per page slot, the
 *                          second one frame longer, for run_own).
 *                          run() then processes each (query tile, head) in
 *                          one pass.
 * Any output pointer may be NULL.  INVALID_ARG for an invalid config,
 * UNSUPPORTED for head_dim != 64. */
SPKV_API int spkv_query_sizes(const spkv_config* cfg, int64_t* max_num_pages,
                              int64_t* pool_bytes_per_block,
                              int64_t* min_workspace_bytes);

/* Workspace that lets run() split the key range of nq query rows across
 * num_splits workgroups: min_workspace_bytes plus num_splits partial
 * results of nq * H * (2 * D + 8) bytes (each split's output normalised by
 * its row sum in bf16, and its fp32 running maximum and sum).
 * run() uses up to 32 splits, and fewer when the workspace holds fewer.
 * [LB-PERF] "Persistent Workspace Pre-allocation" pre-allocates 128 MiB; at
 * 1005 query rows x 16 heads that holds more than the 32 splits run() uses.  This call is an addition
 * of this library (the pages size no workspace by formula).  1 <= nq <=
 * 2^20, 1 <= num_splits <= 32, else INVALID_ARG. */
SPKV_API int spkv_query_workspace(const spkv_config* cfg, int32_t nq, int32_t num_splits,
                                  int64_t* workspace_bytes);

/* Create a manager.  pool_ptrs: num_blocks device pointers, each to
 * pool_bytes_per_block bytes laid out as above; the library only writes the
 * pages it appends to and reads what it attends to, so the caller should zero
 * them once (e.g. torch.zeros) if it wants every byte defined.  workspace:
 * device scratch of workspace_bytes >= min_workspace_bytes.  Both are
 * borrowed until destroy().  The handle owns host state and pinned staging
 * only; it allocates no device memory.  Both NULL: host-only handle. */
SPKV_API int spkv_create(const spkv_config* cfg, void* const* pool_ptrs,
                         void* workspace, int64_t workspace_bytes,
                         spkv_handle** out);

/* Waits for the handle's pending plan copies, then frees it.  NULL is OK. */
SPKV_API int spkv_destroy(spkv_handle* h);

/* append_frame(block_idx, K, V) ([LB-KV] "Append and Evict API";
 * [LB-SLOT] "scale frames：永不驱逐的前 8 个 slot", "特殊 token 流").
 * k, v: device [num_special_tokens + patch_tokens][H][D] bf16, contiguous.
 * Takes the head of the free list; the page joins the scale list while it
 * holds fewer than scale_frames pages, else the live window.  Enqueues one
 * kernel that copies the frame's patch tokens to that page and its special
 * tokens to the next slot of the special stream.  POOL_EXHAUSTED when no page
 * is free, SPECIAL_OVERFLOW when every special slot is taken. */
SPKV_API int spkv_append_frame(spkv_handle* h, int32_t block, const void* k,
                               const void* v, void* hip_stream);

/* append_frame with its copy folded into the block's next run() ([LB-KV]
 * "Append and Evict API" for the admission; the pages' streaming loop
 * appends, evicts, plans on block 0 and runs each block in turn, "Streaming
 * Forward Pass").  Admits the frame exactly like spkv_append_frame (same
 * state change, same errors) but enqueues nothing: the next spkv_run of this
 * block copies the frame into its pages inside the attention launch and
 * reads the frame's own tokens from k and v, so a keyframe costs no separate
 * copy launch.  If another call needs the bytes first -- the block's next
 * append, its rollback, run_own, run_noalloc, a run_batch holding the block,
 * a run that cannot fold the copy (a pool over 2 GiB, or a plan that is not
 * the one of this frame), reset or destroy -- the library enqueues the plain
 * copy on hip_stream first.  k and v must therefore stay valid and unchanged
 * until that copy has run, and hip_stream until it has been enqueued (the
 * pool's bytes end up the same either way). */
SPKV_API int spkv_append_frame_in_run(spkv_handle* h, int32_t block, const void* k,
                                      const void* v, void* hip_stream);

/* evict_frames(block_idx, scale_frames, sliding_window, cross_frame_special,
 * camera_only) ([LB-KV] "Append and Evict API", "Streaming Forward Pass").
 * While the live window holds more than sliding_window pages, its oldest page
 * returns to the tail of the free list.  Moves nothing while eviction is
 * deferred.  scale_frames must equal the config's; 1 <= sliding_window <=
 * M - S; each flag is 0 or 1 (else INVALID_ARG).
 * The flags say what of an evicted frame's special tokens stays visible
 * ([LB-KV] "Append and Evict API": specials are optionally preserved;
 * [LB-SLOT] "特殊 token 流": preserved specials, camera tokens above all,
 * carry context across frames): cross_frame_special = 1 keeps all of them
 * (camera_only = 0, the default) or only the camera token, the first of the
 * frame's specials (camera_only = 1); cross_frame_special = 0 keeps none.
 * Frames whose patch page is held (scale pages, live window) show all their
 * specials.  The special stream's bytes never change.  The block records the
 * flags: they also govern the pages its next execute_deferred_eviction
 * moves.  Special pages left with no visible token drop out of the plan's
 * table; spkv_get_plan_specials describes the visible special tokens. */
SPKV_API int spkv_evict_frames(spkv_handle* h, int32_t block,
                               int32_t scale_frames, int32_t sliding_window,
                               int32_t cross_frame_special,
                               int32_t camera_only);

/* _set_defer_eviction(enable) ([LB-PERF] "Deferred Eviction Strategy";
 * [LB-SLOT] "进阶：光流关键帧与回滚机制").  Manager-wide; enable is 0 or 1. */
SPKV_API int spkv_set_defer_eviction(spkv_handle* h, int32_t enable);

/* execute_deferred_eviction(block_idx, scale_frames, sliding_window): the
 * eviction loop of evict_frames, run whatever the defer flag says, with the
 * special-token flags of the block's last evict_frames call (the defaults
 * 1, 0 before any since create or reset). */
SPKV_API int spkv_execute_deferred_eviction(spkv_handle* h, int32_t block,
                                            int32_t scale_frames,
                                            int32_t sliding_window);

/* rollback_last_frame(block_idx) ([LB-SLOT] "进阶：光流关键帧与回滚机制"):
 * undo the block's last append exactly -- its patch page goes back to the
 * head of the free list and the frame and special counts drop by one.  Legal
 * once per append, and only while no page has moved since (else
 * NOTHING_TO_ROLLBACK).  Pool bytes are not touched. */
SPKV_API int spkv_rollback_last_frame(spkv_handle* h, int32_t block);

/* clean_kv_cache() ([LB-SLOT] "窗口模式：window_size 数的是 slot 不是帧"):
 * every block back to its initial state, deferral off, plan dropped.  Pool
 * bytes are not touched. */
SPKV_API int spkv_reset(spkv_handle* h);

/* plan() once per frame step, from block 0 ([LB-KV] "Kernel-Level Execution
 * Flow"; [LB-PERF] "One-Time Planning Pattern"): visible page table scale ->
 * live window -> special pages and last_page_len, the valid tokens of the last
 * special page ([LB-KV] "Physical Page Layout and Indexing").  Enqueues on
 * hip_stream one small host-to-device copy of the table and one kernel that
 * expands it into the pool row of every visible token, which run() reads.
 * EMPTY if block 0 holds no frame. */
SPKV_API int spkv_plan(spkv_handle* h, void* hip_stream);

/* run(block) ([LB-KV] "Kernel-Level Execution Flow"): for every query row i
 * and head h,  out[i,h,:] = sum_j softmax_j(sm_scale * q[i,h,:].k[j,h,:]) v[j,h,:]
 * over the visible tokens j of `block` in plan order (non-causal, no
 * positional encoding).  q, out: device [nq][H][D] bf16, contiguous, not
 * overlapping; sm_scale finite and > 0.  nq is one frame's tokens
 * (num_special_tokens + patch_tokens) or fewer rows of it, or the rows of
 * several frames at once: the batch mode of the first frames ([LB-KV]
 * "FlashInferAttention Layer Implementation", Phase 1; [LB-SLOT] scale-frame
 * section: the first frames attend to one another bidirectionally) is their
 * appends, one plan and one run with all their queries.  1 <= nq <= 2^20 and
 * nq * H * D / 4 < 2^31.  The split of the key range is limited by the
 * workspace: fewer splits for more query rows.  NOT_PLANNED before a plan, STALE_PLAN when the block's scale,
 * live and special state differ from block 0's at plan time.  UNSUPPORTED
 * when a block's pool exceeds 4 GiB (pool rows are addressed by 32-bit byte
 * offsets).  Enqueues the attention kernel (and, when the key range is split,
 * a merge kernel) and nothing else -- except that a frame admitted to this
 * block by spkv_append_frame_in_run is copied into its pages by that same
 * attention launch (or, when the launch cannot fold it, by a plain copy
 * enqueued first) -- so a run of a planned frame may be
 * captured into a HIP graph; plan() may not, since it copies the host
 * allocator's state of the moment.  A captured run binds the device row map
 * of the plan that was current at capture (plans alternate between two
 * slots), its visible-token count and its split: a replay is valid only
 * while that plan is still the current one, i.e. until the next plan() or
 * reset().  Replayed after that, it attends over whatever the slot then
 * holds.  A captured run that folds a frame's copy (append_frame_in_run)
 * copies it at every replay, not at capture; the same bytes land in the same
 * pages each time, which stays harmless while the plan is current. */
SPKV_API int spkv_run(spkv_handle* h, int32_t block, const void* q, void* out,
                      int32_t nq, float sm_scale, void* hip_stream);

/* run() for callers that cannot allocate device memory or size a workspace
 * for it (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same attention, with the key-range split's partial
 * results kept in device memory that the library itself holds, a 48 MiB
 * array per GPU (allocated when the library's code is loaded on that GPU and
 * held until the process ends), instead of in the handle's workspace.  So a
 * handle created with only min_workspace_bytes still gets run()'s split.
 * The call allocates nothing.  Limit: nq <= 48 MiB / (2 * H * (2 * D + 8))
 * rounded down (two splits of partials; 11565 rows at H = 16), else
 * SPKV_ERR_WORKSPACE and nothing is enqueued.  Every call on one GPU shares
 * that GPU's array, whatever the handle: two calls whose kernels overlap in
 * time on one GPU (different streams, no ordering between them) race on it
 * and give wrong results; calls ordered on one stream are safe.  Arguments,
 * other errors and the plan contract are run()'s. */
SPKV_API int spkv_run_noalloc(spkv_handle* h, int32_t block, const void* q, void* out,
                              int32_t nq, float sm_scale, void* hip_stream);

/* run(block) for a frame that attends to the cache without joining it: the
 * non-keyframe case of [LB-SLOT] "进阶：光流关键帧与回滚机制" (it attends to
 * the cache plus its own K/V, and its K/V are not stored) and the
 * configuration's "skip append".  The visible tokens are the plan's, as for
 * run(), followed by every row of the caller's frame own_k / own_v (device
 * [num_special_tokens + patch_tokens][H][D] bf16, contiguous, the layout
 * append_frame takes).  Neither the pool nor any state changes, so there is
 * nothing to roll back.  Arguments and errors as for run(); own_k and own_v
 * must not overlap out.  UNSUPPORTED when a block's pool exceeds 2 GiB (run()
 * itself takes pools up to 4 GiB).  Enqueues kernels only, as run() does, and
 * a captured run_own is valid only while its plan is current, as for run().
 * Host-only handles pass NULL own_k and own_v and get run()'s checks and
 * result. */
SPKV_API int spkv_run_own(spkv_handle* h, int32_t block, const void* q, void* out,
                          int32_t nq, float sm_scale, const void* own_k,
                          const void* own_v, void* hip_stream);

/* One request of run_batch(): a run() (own_k == own_v == NULL) or a
 * run_own() of one stream's handle, with that call's arguments. */
typedef struct {
  spkv_handle* handle;
  int32_t block;
  int32_t nq;
  const void* q;       /* device [nq][H][D] bf16 */
  void* out;           /* device [nq][H][D] bf16 */
  const void* own_k;   /* NULL, or the caller's frame as for run_own() */
  const void* own_v;
  float sm_scale;
} spkv_request;

#define SPKV_MAX_BATCH 16

/* Several independent streams in one launch.  The pages' attention is a
 * batched prefill over paged K/V whose plan takes per-request query and page
 * offsets (qo_indptr, paged_kv_indptr) so that one launch serves every
 * request ([LB-KV] "Kernel-Level Execution Flow"; the pages run one request
 * per manager), and they advise batching plans where latency allows
 * ([LB-PERF] "Practical Performance Tuning").  Here each stream keeps its own
 * handle and plan, and this call runs one request of each.  Each request is
 * what run() -- or run_own() when own_k and own_v are set -- of its handle
 * would compute, with the same checks and errors, on its handle's current
 * plan; results equal those calls' up to the order of floating-point
 * additions (the key range may be split differently).
 * 1 <= n <= SPKV_MAX_BATCH; every handle at most once (its workspace holds
 * its request's split partials); all handles of one device and all host-only
 * or none; no request's out may overlap another request's q, out, own_k or
 * own_v.  The key ranges are split so that the work items of all requests
 * are about equally long and fill the CUs once.  Nothing is enqueued unless
 * every check passes: first the checks across requests (INVALID_ARG), then
 * run()'s checks request by request, the first failure's code being
 * returned (host-only handles: UNSUPPORTED once all pass).  Enqueues one
 * attention kernel and, if any range is split, one merge kernel, and nothing
 * else: like run() and run_own(), it may be captured into a HIP graph, whose
 * replays are valid only while every request's plan is still current. */
SPKV_API int spkv_run_batch(const spkv_request* reqs, int32_t n, void* hip_stream);

/* Split of the key range across workgroups used by run(): 0 = automatic
 * (default), else a fixed count (clamped to what the workspace and the number
 * of key tiles allow).  For tests and tuning. */
SPKV_API int spkv_set_num_splits(spkv_handle* h, int32_t num_splits);

/* get_cache_stats(block_idx). */
SPKV_API int spkv_get_cache_stats(const spkv_handle* h, int32_t block,
                                  spkv_stats* out);

/* The current plan: table (cap entries available), its length, the number
 * of patch pages at its head and last_page_len.  NOT_PLANNED if none;
 * INVALID_ARG if cap is too small. */
SPKV_API int spkv_get_plan(const spkv_handle* h, int32_t* table, int32_t cap,
                           int32_t* n_pages, int32_t* n_patch_pages,
                           int32_t* last_page_len);

/* The special tokens the current plan shows, as runs (3 int32 each: first
 * frame of the special stream, number of frames, visible tokens per frame --
 * the first that many of each frame's specials), in stream order, equal
 * neighbours merged and runs with none left out; cap runs available.  The
 * run() token order is the patch pages' tokens, then these.  NOT_PLANNED if
 * there is no plan; INVALID_ARG if cap is too small. */
SPKV_API int spkv_get_plan_specials(const spkv_handle* h, int32_t* runs, int32_t cap,
                                    int32_t* n_runs);

/* The same runs for block `block`'s current state (what a plan built from it
 * would show), for inspection. */
SPKV_API int spkv_get_block_specials(const spkv_handle* h, int32_t block, int32_t* runs,
                                     int32_t cap, int32_t* n_runs);

/* A block's allocator state, for inspection: scale list, live window (oldest
 * first), free list (head first), each into an array of cap entries, and
 * the number of special frames. */
SPKV_API int spkv_get_block_state(const spkv_handle* h, int32_t block,
                                  int32_t* scale, int32_t* live,
                                  int32_t* free_list, int32_t cap,
                                  int32_t* n_scale, int32_t* n_live,
                                  int32_t* n_free, int64_t* n_special_frames);

/* Static string naming a status code. */
SPKV_API const char* spkv_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPKV_H */
