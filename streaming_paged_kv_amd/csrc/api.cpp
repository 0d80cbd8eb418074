// C ABI of libspkv.so: argument checks, the host allocator, the plan's
// host-to-device copy and the kernel launches.  See include/spkv.h for the
// contract of every call.
#include "../../include/spkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <vector>

#include "kernels.h"
#include "pool.h"

namespace {

constexpr int kMaxSplits = 32;
// Query rows of one run: a frame, or several frames at once (the batch mode
// of the first frames); bounded so that rows * H and the row offsets stay in
// 32 bits inside the kernels.
constexpr int32_t kMaxQueryRows = 1 << 20;
constexpr int64_t kAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool to_geometry(const spkv_config* c, spkv::Geometry* g) {
  if (!c) return false;
  *g = spkv::Geometry{};
  g->num_blocks = c->num_blocks;
  g->num_heads = c->num_heads;
  g->head_dim = c->head_dim;
  g->page_size = c->page_size;
  g->patch_tokens = c->patch_tokens;
  g->num_special = c->num_special_tokens;
  g->scale_frames = c->scale_frames;
  g->sliding_window = c->sliding_window;
  g->headroom = c->headroom;
  g->max_total_frames = c->max_total_frames;
  if (!g->derive()) return false;
  // Element offsets are computed in 64 bits, but a page's token count times
  // H*D and the visible token count must stay in int32 inside the kernels.
  const int64_t hd = int64_t(g->num_heads) * g->head_dim;
  if (hd > (1 << 20) || int64_t(g->page_size) * hd > (int64_t(1) << 31))
    return false;
  if (int64_t(g->max_num_pages) * g->page_size > (int64_t(1) << 30))
    return false;
  return true;
}

struct Sizes {
  int64_t max_num_pages, pool_bytes, table_bytes, segs_offset, rowmap_entries,
      rowmap_bytes, rowmap_own_bytes, min_ws;
};

// Split partials of nq query rows: each split's O normalised by its row sum
// (bf16) and its fp32 (m, l) per (query, head) row and split.
int64_t partial_bytes(const spkv::Geometry& g, int64_t nq, int64_t splits) {
  const int64_t rows = nq * g.num_heads;
  return round_up(rows * g.head_dim * 2 * splits, kAlign) + round_up(rows * 8 * splits, kAlign);
}

Sizes sizes_of(const spkv::Geometry& g) {
  Sizes s;
  s.max_num_pages = g.max_num_pages;
  s.pool_bytes = int64_t(g.max_num_pages) * 2 * g.page_size * g.num_heads *
                 g.head_dim * 2;
  // A plan's device table: the page ids, then (16-byte aligned) the runs of
  // visible special tokens, at most one per evicted run plus two.
  s.segs_offset = round_up(int64_t(g.max_num_pages) * 4, 16);
  s.table_bytes = round_up(s.segs_offset + (g.special_capacity + 2) *
                                               int64_t(sizeof(spkv::SpecialSeg)),
                           kAlign);
  // Row map: at most every slot of every page is visible; rounded up to a
  // key tile and padded.
  s.rowmap_entries = round_up(int64_t(g.max_num_pages) * g.page_size,
                              spkv::kAttnKeyTile) + spkv::kRowmapPad;
  s.rowmap_bytes = round_up(s.rowmap_entries * 4, kAlign);
  // The same plus one frame of the caller's own rows (run_own).
  s.rowmap_own_bytes =
      round_up((round_up(int64_t(g.max_num_pages) * g.page_size + g.tokens_per_frame,
                         spkv::kAttnKeyTile) + spkv::kRowmapPad) * 4, kAlign);
  // run()'s map, run_own()'s map and the map of a run that copies the newest
  // frame (append_frame_in_run), each double-buffered.
  s.min_ws = 2 * s.table_bytes + 4 * s.rowmap_bytes + 2 * s.rowmap_own_bytes;
  return s;
}

int status(spkv::Status s) { return static_cast<int>(s); }

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Makes the handle's device current for the duration of a call.
class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev_) == hipSuccess && prev_ != dev)
      switched_ = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (switched_) (void)hipSetDevice(prev_);
  }

 private:
  int prev_ = 0;
  bool switched_ = false;
};

}  // namespace

struct spkv_handle {
  spkv::Geometry g{};
  Sizes sz{};
  std::unique_ptr<spkv::PagePool> pool;
  bool host_only = true;
  int device = 0;
  std::vector<void*> pools;
  char* ws = nullptr;
  int64_t ws_bytes = 0;
  int32_t* dev_table[2] = {nullptr, nullptr};
  uint32_t* dev_rowmap[2] = {nullptr, nullptr};
  uint32_t* dev_rowmap_own[2] = {nullptr, nullptr};
  uint32_t* dev_rowmap_new[2] = {nullptr, nullptr};
  // A frame admitted by append_frame_in_run whose copy into the pool has not
  // been enqueued yet (at most one per block: it is the block's newest frame).
  struct Pending {
    bool set = false;
    spkv::AppendArgs copy{};
    int32_t patch_page = -1;
    hipStream_t stream = nullptr;
  };
  std::vector<Pending> pending;
  char* stage = nullptr;             // pinned, 2 x table_bytes
  hipEvent_t copied[2] = {nullptr, nullptr};
  bool copy_pending[2] = {false, false};
  int plan_slot = 0;                 // slot holding the current plan
  int next_slot = 0;
  char* partials = nullptr;
  char* scratch = nullptr;           // this device's library-held partials
  int forced_splits = 0;
  int num_cus = 256;
};

namespace {

// The copy of an admitted frame into its pages.
spkv::AppendArgs append_args(const spkv_handle* h, int32_t block, const void* k,
                             const void* v, const spkv::AppendResult& r) {
  const spkv::Geometry& g = h->g;
  const int64_t hd = int64_t(g.num_heads) * g.head_dim;
  const int64_t page = int64_t(g.page_size) * hd;
  spkv::AppendArgs a;
  a.k = k;
  a.v = v;
  a.pool = h->pools[block];
  a.patch_k_off = (int64_t(r.patch_page) * 2 + 0) * page;
  a.patch_v_off = (int64_t(r.patch_page) * 2 + 1) * page;
  a.special_k_off = (int64_t(r.special_page) * 2 + 0) * page + int64_t(r.special_slot) * hd;
  a.special_v_off = (int64_t(r.special_page) * 2 + 1) * page + int64_t(r.special_slot) * hd;
  a.patch_elems = int64_t(g.patch_tokens) * hd;
  a.special_elems = int64_t(g.num_special) * hd;
  return a;
}

// Enqueues block's pending copy (append_frame_in_run), if any, on the stream
// that call named.
int flush_pending(spkv_handle* h, int32_t block) {
  spkv_handle::Pending& p = h->pending[block];
  if (!p.set) return SPKV_OK;
  DeviceGuard guard(h->device);
  if (spkv::launch_append(p.copy, p.stream) != hipSuccess) return SPKV_ERR_HIP;
  p.set = false;
  return SPKV_OK;
}

int flush_all(spkv_handle* h) {
  for (int32_t b = 0; b < static_cast<int32_t>(h->pending.size()); ++b) {
    const int rc = flush_pending(h, b);
    if (rc != SPKV_OK) return rc;
  }
  return SPKV_OK;
}

}  // namespace

extern "C" {

SPKV_API const char* spkv_error_string(int code) {
  switch (code) {
    case SPKV_OK: return "ok";
    case SPKV_ERR_INVALID_ARG: return "invalid argument";
    case SPKV_ERR_BAD_BLOCK: return "block index out of range";
    case SPKV_ERR_POOL_EXHAUSTED: return "no free patch page";
    case SPKV_ERR_SPECIAL_OVERFLOW: return "special stream full";
    case SPKV_ERR_NOTHING_TO_ROLLBACK: return "nothing to roll back";
    case SPKV_ERR_EMPTY: return "no frame to plan";
    case SPKV_ERR_NOT_PLANNED: return "run before plan";
    case SPKV_ERR_STALE_PLAN: return "block state differs from the plan";
    case SPKV_ERR_UNSUPPORTED: return "unsupported";
    case SPKV_ERR_HIP: return "HIP runtime error";
    case SPKV_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

SPKV_API int spkv_query_sizes(const spkv_config* cfg, int64_t* max_num_pages,
                              int64_t* pool_bytes_per_block,
                              int64_t* min_workspace_bytes) {
  spkv::Geometry g;
  if (!to_geometry(cfg, &g)) return SPKV_ERR_INVALID_ARG;
  if (g.head_dim != 64) return SPKV_ERR_UNSUPPORTED;
  const Sizes s = sizes_of(g);
  if (max_num_pages) *max_num_pages = s.max_num_pages;
  if (pool_bytes_per_block) *pool_bytes_per_block = s.pool_bytes;
  if (min_workspace_bytes) *min_workspace_bytes = s.min_ws;
  return SPKV_OK;
}

SPKV_API int spkv_query_workspace(const spkv_config* cfg, int32_t nq, int32_t num_splits,
                                  int64_t* workspace_bytes) {
  spkv::Geometry g;
  if (!to_geometry(cfg, &g)) return SPKV_ERR_INVALID_ARG;
  if (g.head_dim != 64) return SPKV_ERR_UNSUPPORTED;
  if (nq < 1 || nq > kMaxQueryRows || num_splits < 1 || num_splits > kMaxSplits)
    return SPKV_ERR_INVALID_ARG;
  if (workspace_bytes)
    *workspace_bytes = sizes_of(g).min_ws + partial_bytes(g, nq, num_splits);
  return SPKV_OK;
}

SPKV_API int spkv_create(const spkv_config* cfg, void* const* pool_ptrs,
                         void* workspace, int64_t workspace_bytes,
                         spkv_handle** out) {
  if (!out) return SPKV_ERR_INVALID_ARG;
  *out = nullptr;
  spkv::Geometry g;
  if (!to_geometry(cfg, &g)) return SPKV_ERR_INVALID_ARG;
  if (g.head_dim != 64) return SPKV_ERR_UNSUPPORTED;
  const bool host_only = pool_ptrs == nullptr;
  if (host_only != (workspace == nullptr)) return SPKV_ERR_INVALID_ARG;
  const Sizes sz = sizes_of(g);
  if (!host_only) {
    for (int b = 0; b < g.num_blocks; ++b)
      if (!pool_ptrs[b] || !aligned16(pool_ptrs[b])) return SPKV_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return SPKV_ERR_INVALID_ARG;
    if (workspace_bytes < sz.min_ws) return SPKV_ERR_WORKSPACE;
  }

  std::unique_ptr<spkv_handle> h(new (std::nothrow) spkv_handle());
  if (!h) return SPKV_ERR_INVALID_ARG;
  h->g = g;
  h->sz = sz;
  h->host_only = host_only;
  try {
    h->pool.reset(new spkv::PagePool(g));
  } catch (...) {
    return SPKV_ERR_INVALID_ARG;
  }
  if (host_only) {
    *out = h.release();
    return SPKV_OK;
  }

  if (hipGetDevice(&h->device) != hipSuccess) return SPKV_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) == hipSuccess)
    h->num_cus = prop.multiProcessorCount;
  h->pools.assign(pool_ptrs, pool_ptrs + g.num_blocks);
  h->ws = static_cast<char*>(workspace);
  h->ws_bytes = workspace_bytes;
  h->dev_table[0] = reinterpret_cast<int32_t*>(h->ws);
  h->dev_table[1] = reinterpret_cast<int32_t*>(h->ws + sz.table_bytes);
  h->dev_rowmap[0] = reinterpret_cast<uint32_t*>(h->ws + 2 * sz.table_bytes);
  h->dev_rowmap[1] = reinterpret_cast<uint32_t*>(h->ws + 2 * sz.table_bytes +
                                                 sz.rowmap_bytes);
  h->dev_rowmap_own[0] = reinterpret_cast<uint32_t*>(h->ws + 2 * sz.table_bytes +
                                                     2 * sz.rowmap_bytes);
  h->dev_rowmap_own[1] = reinterpret_cast<uint32_t*>(
      h->ws + 2 * sz.table_bytes + 2 * sz.rowmap_bytes + sz.rowmap_own_bytes);
  for (int i = 0; i < 2; ++i)
    h->dev_rowmap_new[i] = reinterpret_cast<uint32_t*>(
        h->ws + 2 * sz.table_bytes + (2 + i) * sz.rowmap_bytes + 2 * sz.rowmap_own_bytes);
  h->pending.assign(g.num_blocks, spkv_handle::Pending{});
  h->partials = h->ws + sz.min_ws;
  // The device address of run_noalloc()'s scratch, looked up once per device
  // with that device current.
  void* scratch = nullptr;
  if (spkv::scratch_address(&scratch) != hipSuccess) return SPKV_ERR_HIP;
  h->scratch = static_cast<char*>(scratch);
  if (hipHostMalloc(reinterpret_cast<void**>(&h->stage), size_t(2 * sz.table_bytes),
                    hipHostMallocDefault) != hipSuccess) {
    h->stage = nullptr;
    return SPKV_ERR_HIP;
  }
  for (int i = 0; i < 2; ++i) {
    if (hipEventCreateWithFlags(&h->copied[i], hipEventDisableTiming) !=
        hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(h->copied[j]);
      (void)hipHostFree(h->stage);
      return SPKV_ERR_HIP;
    }
  }
  *out = h.release();
  return SPKV_OK;
}

SPKV_API int spkv_destroy(spkv_handle* h) {
  if (!h) return SPKV_OK;
  int rc = SPKV_OK;
  if (!h->host_only) {
    DeviceGuard guard(h->device);
    rc = flush_all(h);
    for (int i = 0; i < 2; ++i) {
      if (h->copy_pending[i] && hipEventSynchronize(h->copied[i]) != hipSuccess)
        rc = SPKV_ERR_HIP;
      if (h->copied[i]) (void)hipEventDestroy(h->copied[i]);
    }
    if (h->stage) (void)hipHostFree(h->stage);
  }
  delete h;
  return rc;
}

SPKV_API int spkv_append_frame(spkv_handle* h, int32_t block, const void* k,
                               const void* v, void* hip_stream) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (block < 0 || block >= h->g.num_blocks) return SPKV_ERR_BAD_BLOCK;
  if (h->host_only) {
    if (k || v) return SPKV_ERR_INVALID_ARG;
  } else {
    if (!k || !v || !aligned16(k) || !aligned16(v)) return SPKV_ERR_INVALID_ARG;
    const int f = flush_pending(h, block);
    if (f != SPKV_OK) return f;
  }
  spkv::AppendResult r;
  const spkv::Status s = h->pool->append(block, &r);
  if (s != spkv::Status::ok) return status(s);
  if (h->host_only) return SPKV_OK;

  DeviceGuard guard(h->device);
  if (spkv::launch_append(append_args(h, block, k, v, r),
                          static_cast<hipStream_t>(hip_stream)) != hipSuccess) {
    h->pool->undo_append(block, r);
    return SPKV_ERR_HIP;
  }
  return SPKV_OK;
}

SPKV_API int spkv_append_frame_in_run(spkv_handle* h, int32_t block, const void* k,
                                      const void* v, void* hip_stream) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (block < 0 || block >= h->g.num_blocks) return SPKV_ERR_BAD_BLOCK;
  if (h->host_only) {
    if (k || v) return SPKV_ERR_INVALID_ARG;
  } else {
    if (!k || !v || !aligned16(k) || !aligned16(v)) return SPKV_ERR_INVALID_ARG;
    const int f = flush_pending(h, block);
    if (f != SPKV_OK) return f;
  }
  spkv::AppendResult r;
  const spkv::Status s = h->pool->append(block, &r);
  if (s != spkv::Status::ok) return status(s);
  if (h->host_only) return SPKV_OK;
  spkv_handle::Pending& p = h->pending[block];
  p.copy = append_args(h, block, k, v, r);
  p.patch_page = r.patch_page;
  p.stream = static_cast<hipStream_t>(hip_stream);
  p.set = true;
  return SPKV_OK;
}

SPKV_API int spkv_evict_frames(spkv_handle* h, int32_t block,
                               int32_t scale_frames, int32_t sliding_window,
                               int32_t cross_frame_special,
                               int32_t camera_only) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  return status(h->pool->evict(block, scale_frames, sliding_window,
                               cross_frame_special, camera_only, nullptr));
}

SPKV_API int spkv_set_defer_eviction(spkv_handle* h, int32_t enable) {
  if (!h || (enable != 0 && enable != 1)) return SPKV_ERR_INVALID_ARG;
  h->pool->set_defer(enable == 1);
  return SPKV_OK;
}

SPKV_API int spkv_execute_deferred_eviction(spkv_handle* h, int32_t block,
                                            int32_t scale_frames,
                                            int32_t sliding_window) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  return status(
      h->pool->execute_deferred(block, scale_frames, sliding_window, nullptr));
}

SPKV_API int spkv_rollback_last_frame(spkv_handle* h, int32_t block) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  // the frame's bytes are written whether it stays or not
  if (!h->host_only && block >= 0 && block < h->g.num_blocks) {
    const int f = flush_pending(h, block);
    if (f != SPKV_OK) return f;
  }
  return status(h->pool->rollback(block));
}

SPKV_API int spkv_reset(spkv_handle* h) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (!h->host_only) {
    const int f = flush_all(h);
    if (f != SPKV_OK) return f;
  }
  h->pool->reset();
  return SPKV_OK;
}

SPKV_API int spkv_plan(spkv_handle* h, void* hip_stream) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (h->host_only) return status(h->pool->plan());
  DeviceGuard guard(h->device);
  // The staging slot is reused every other plan: its previous copy must have
  // left the host buffer before it is overwritten.
  const int slot = h->next_slot;
  if (h->copy_pending[slot]) {
    if (hipEventSynchronize(h->copied[slot]) != hipSuccess) return SPKV_ERR_HIP;
    h->copy_pending[slot] = false;
  }
  const spkv::Status s = h->pool->build_plan();
  if (s != spkv::Status::ok) return status(s);
  const spkv::PlanView pv = h->pool->pending_view();
  const Sizes& sz = h->sz;
  char* host = h->stage + slot * sz.table_bytes;
  std::memcpy(host, pv.table, size_t(pv.n_pages) * sizeof(int32_t));
  spkv::SpecialSeg* segs = reinterpret_cast<spkv::SpecialSeg*>(host + sz.segs_offset);
  int32_t offset = 0;
  for (int32_t i = 0; i < pv.n_segs; ++i) {
    const spkv::SpecialRun& r = pv.segs[i];
    segs[i] = spkv::SpecialSeg{r.first, r.count, r.kept, offset};
    offset += r.count * r.kept;
  }
  const size_t bytes = size_t(sz.segs_offset) + size_t(pv.n_segs) * sizeof(spkv::SpecialSeg);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const spkv::Geometry& g = h->g;
  char* dev = reinterpret_cast<char*>(h->dev_table[slot]);
  spkv::PlanArgs pa;
  pa.table = h->dev_table[slot];
  pa.segs = reinterpret_cast<const spkv::SpecialSeg*>(dev + sz.segs_offset);
  pa.rowmap = h->dev_rowmap[slot];
  pa.n_patch = pv.n_patch;
  pa.n_segs = pv.n_segs;
  pa.patch_len = g.patch_tokens;
  pa.num_special = g.num_special;
  pa.frames_per_spage = g.frames_per_spage;
  pa.first_spage = g.num_patch_pages;
  pa.page_size = g.page_size;
  pa.nk = static_cast<int32_t>(pv.visible_tokens);
  pa.n_out = static_cast<int32_t>(
      round_up(pv.visible_tokens, spkv::kAttnKeyTile) + spkv::kRowmapPad);
  pa.rowmap_own = h->dev_rowmap_own[slot];
  pa.rowmap_new = h->dev_rowmap_new[slot];
  pa.new_patch_begin = (pv.n_patch - 1) * g.patch_tokens;
  pa.n_own = g.tokens_per_frame;
  pa.n_out_own = static_cast<int32_t>(
      round_up(pv.visible_tokens + g.tokens_per_frame, spkv::kAttnKeyTile) +
      spkv::kRowmapPad);
  if (hipMemcpyAsync(dev, host, bytes, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipEventRecord(h->copied[slot], st) != hipSuccess ||
      spkv::launch_expand(pa, st) != hipSuccess) {
    return SPKV_ERR_HIP;  // the pending plan is simply not committed
  }
  h->pool->commit_plan();
  h->copy_pending[slot] = true;
  h->plan_slot = slot;
  h->next_slot = slot ^ 1;
  return SPKV_OK;
}

SPKV_API int spkv_set_num_splits(spkv_handle* h, int32_t num_splits) {
  if (!h || num_splits < 0) return SPKV_ERR_INVALID_ARG;
  h->forced_splits = num_splits;
  return SPKV_OK;
}

}  // extern "C"

namespace {

bool overlaps(const void* a, const void* b, size_t bytes_a, size_t bytes_b) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + bytes_b && y < x + bytes_a;
}

// Key tiles of a request after its checks.
struct RunShape {
  int64_t nk, n_ktiles, units;  // units = query tiles x heads
};

// Checks of run() and run_own() (own_k == own_v == nullptr for the planned
// pages alone) that need no split decision; fills *shape.
int check_run(spkv_handle* h, int32_t block, const void* q, void* out, int32_t nq,
              float sm_scale, const void* own_k, const void* own_v, RunShape* shape) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  const bool own = own_k != nullptr || own_v != nullptr;
  if (block < 0 || block >= h->g.num_blocks) return SPKV_ERR_BAD_BLOCK;
  const spkv::Geometry& g = h->g;
  if (nq < 1 || nq > kMaxQueryRows || !std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return SPKV_ERR_INVALID_ARG;
  // the merge runs one thread per (query, head, 4 dims)
  if (int64_t(nq) * g.num_heads * (g.head_dim / 4) >= (int64_t(1) << 31))
    return SPKV_ERR_INVALID_ARG;
  if (h->host_only) {
    if (q || out || own) return SPKV_ERR_INVALID_ARG;
  } else {
    if (!q || !out || !aligned16(q) || !aligned16(out)) return SPKV_ERR_INVALID_ARG;
    const size_t bytes = size_t(nq) * g.num_heads * g.head_dim * 2;
    if (overlaps(q, out, bytes, bytes)) return SPKV_ERR_INVALID_ARG;
    if (own) {
      if (!own_k || !own_v || !aligned16(own_k) || !aligned16(own_v))
        return SPKV_ERR_INVALID_ARG;
      const size_t fb = size_t(g.tokens_per_frame) * g.num_heads * g.head_dim * 2;
      if (overlaps(out, own_k, bytes, fb) || overlaps(out, own_v, bytes, fb))
        return SPKV_ERR_INVALID_ARG;
    }
  }
  const spkv::Status s = h->pool->check_run(block);
  if (s != spkv::Status::ok) return status(s);
  if (h->host_only) return SPKV_ERR_UNSUPPORTED;

  // The kernel addresses pool rows by 32-bit byte offsets, whose top bit
  // marks the caller's own rows in run_own's map.
  if (h->sz.pool_bytes > (int64_t(1) << (own ? 31 : 32))) return SPKV_ERR_UNSUPPORTED;
  const spkv::PlanView pv = h->pool->plan_view();
  shape->nk = pv.visible_tokens + (own ? g.tokens_per_frame : 0);
  shape->n_ktiles = (shape->nk + spkv::kAttnKeyTile - 1) / spkv::kAttnKeyTile;
  shape->units = (nq + spkv::kAttnQueryTile - 1) / spkv::kAttnQueryTile * g.num_heads;
  return SPKV_OK;
}

// Where a run's split partials go: the workspace after the plan's buffers,
// or the library's scratch (run_noalloc).
struct Partials {
  char* base;
  int64_t bytes;
};

Partials workspace_partials(const spkv_handle* h) {
  return Partials{h->partials, h->ws_bytes - h->sz.min_ws};
}

// Kernel arguments of a checked request with `want` splits of its key range
// (before the limits of the partials' buffer and of the key tiles).
spkv::AttnArgs make_run(spkv_handle* h, int32_t block, const void* q, void* out,
                        int32_t nq, float sm_scale, const void* own_k, const void* own_v,
                        const RunShape& shape, int64_t want, Partials part) {
  const spkv::Geometry& g = h->g;
  int64_t splits = h->forced_splits > 0 ? h->forced_splits : want;
  // Split partials: fp32 O and (m, l) per (query, head) row and split.
  const int64_t rows = int64_t(nq) * g.num_heads;
  int64_t cap = kMaxSplits;
  while (cap > 1 && partial_bytes(g, nq, cap) > part.bytes) --cap;
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, cap));
  splits = std::min<int64_t>(splits, shape.n_ktiles);
  const int64_t tiles_per_split = (shape.n_ktiles + splits - 1) / splits;
  splits = (shape.n_ktiles + tiles_per_split - 1) / tiles_per_split;  // none empty

  const bool own = own_k != nullptr;
  spkv::AttnArgs a;
  a.copy = spkv::FrameCopy{};
  a.pool = static_cast<const uint16_t*>(h->pools[block]);
  a.own_k = static_cast<const uint16_t*>(own_k);
  a.own_v = static_cast<const uint16_t*>(own_v);
  a.rowmap = own ? h->dev_rowmap_own[h->plan_slot] : h->dev_rowmap[h->plan_slot];
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.part_o = reinterpret_cast<uint16_t*>(part.base);
  a.part_ml = reinterpret_cast<float*>(
      part.base + round_up(rows * g.head_dim * 2 * splits, kAlign));
  a.nq = nq;
  a.num_heads = g.num_heads;
  a.page_size = g.page_size;
  a.nk = static_cast<int32_t>(shape.nk);
  a.n_cached = static_cast<int32_t>(shape.nk - (own ? g.tokens_per_frame : 0));
  a.splits = static_cast<int32_t>(splits);
  a.tokens_per_split = static_cast<int32_t>(tiles_per_split * spkv::kAttnKeyTile);
  a.sm_scale = sm_scale;
  return a;
}

// Query rows run_noalloc() takes: the library's scratch must hold two
// splits of their partials.
int64_t noalloc_max_rows(const spkv::Geometry& g) {
  int64_t n = spkv::kScratchBytes / (2 * int64_t(g.num_heads) * (g.head_dim * 2 + 8));
  while (n > 0 && partial_bytes(g, n, 2) > spkv::kScratchBytes) --n;
  return n;
}

int run_impl(spkv_handle* h, int32_t block, const void* q, void* out, int32_t nq,
             float sm_scale, const void* own_k, const void* own_v, void* hip_stream,
             bool noalloc = false) {
  RunShape shape;
  const int rc = check_run(h, block, q, out, nq, sm_scale, own_k, own_v, &shape);
  if (rc != SPKV_OK) return rc;
  if (noalloc && nq > noalloc_max_rows(h->g)) return SPKV_ERR_WORKSPACE;
  // A frame admitted by append_frame_in_run is copied by this launch when the
  // run reads the plan's pages alone and the plan's newest frame is it; its
  // rows are then read from the caller's buffers (the own-row mark needs a
  // pool of at most 2 GiB).  Otherwise its copy is enqueued first.
  const spkv::PlanView pv = h->pool->plan_view();
  spkv_handle::Pending& pend = h->pending[block];
  const bool fuse = pend.set && !own_k && !noalloc &&
                    h->sz.pool_bytes <= (int64_t(1) << 31) &&
                    pv.table[pv.n_patch - 1] == pend.patch_page;
  if (pend.set && !fuse) {
    const int f = flush_pending(h, block);
    if (f != SPKV_OK) return f;
  }
  // One resident workgroup per CU; each split keeps >= 4 key tiles.
  int64_t want = (int64_t(h->num_cus) + shape.units - 1) / shape.units;
  want = std::min<int64_t>(want, std::max<int64_t>(1, shape.n_ktiles / 4));
  const Partials part = noalloc ? Partials{h->scratch, spkv::kScratchBytes}
                                : workspace_partials(h);
  spkv::AttnArgs a =
      make_run(h, block, q, out, nq, sm_scale, own_k, own_v, shape, want, part);
  if (fuse) {
    const spkv::AppendArgs& c = pend.copy;
    a.own_k = static_cast<const uint16_t*>(c.k);
    a.own_v = static_cast<const uint16_t*>(c.v);
    a.rowmap = h->dev_rowmap_new[h->plan_slot];
    a.n_cached = (pv.n_patch - 1) * h->g.patch_tokens;  // first row read from k, v
    a.copy = spkv::FrameCopy{a.own_k, a.own_v, static_cast<uint16_t*>(c.pool),
                             c.patch_k_off / 8, c.patch_v_off / 8, c.special_k_off / 8,
                             c.special_v_off / 8, static_cast<int32_t>(c.patch_elems / 8),
                             static_cast<int32_t>(c.special_elems / 8)};
  }
  DeviceGuard guard(h->device);
  if (spkv::launch_attention(a, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return SPKV_ERR_HIP;
  if (fuse) pend.set = false;
  return SPKV_OK;
}

// Bytes a request reads (q, and own_k / own_v when set) and writes (out).
struct Extent {
  const void* p;
  size_t bytes;
};

}  // namespace

extern "C" {

SPKV_API int spkv_run(spkv_handle* h, int32_t block, const void* q, void* out,
                      int32_t nq, float sm_scale, void* hip_stream) {
  return run_impl(h, block, q, out, nq, sm_scale, nullptr, nullptr, hip_stream);
}

SPKV_API int spkv_run_noalloc(spkv_handle* h, int32_t block, const void* q, void* out,
                              int32_t nq, float sm_scale, void* hip_stream) {
  return run_impl(h, block, q, out, nq, sm_scale, nullptr, nullptr, hip_stream, true);
}

SPKV_API int spkv_run_own(spkv_handle* h, int32_t block, const void* q, void* out,
                          int32_t nq, float sm_scale, const void* own_k,
                          const void* own_v, void* hip_stream) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (!h->host_only && (!own_k || !own_v)) return SPKV_ERR_INVALID_ARG;
  return run_impl(h, block, q, out, nq, sm_scale, own_k, own_v, hip_stream);
}

SPKV_API int spkv_run_batch(const spkv_request* reqs, int32_t n, void* hip_stream) {
  if (!reqs || n < 1 || n > SPKV_MAX_BATCH) return SPKV_ERR_INVALID_ARG;
  static_assert(SPKV_MAX_BATCH <= spkv::kMaxBatchRuns, "batch capacity");
  for (int32_t i = 0; i < n; ++i) {
    const spkv_request& r = reqs[i];
    if (!r.handle) return SPKV_ERR_INVALID_ARG;
    if ((r.own_k == nullptr) != (r.own_v == nullptr) && !r.handle->host_only)
      return SPKV_ERR_INVALID_ARG;
    // Each stream's split partials live in its own workspace: one request
    // per handle.  All handles drive one device and kind.
    for (int32_t j = 0; j < i; ++j)
      if (reqs[j].handle == r.handle) return SPKV_ERR_INVALID_ARG;
    if (r.handle->host_only != reqs[0].handle->host_only ||
        r.handle->device != reqs[0].handle->device)
      return SPKV_ERR_INVALID_ARG;
  }
  // No request may write what another one reads or writes.
  if (!reqs[0].handle->host_only) {
    for (int32_t i = 0; i < n; ++i) {
      const spkv::Geometry& gi = reqs[i].handle->g;
      const size_t out_bytes = size_t(reqs[i].nq > 0 ? reqs[i].nq : 0) * gi.num_heads *
                               gi.head_dim * 2;
      for (int32_t j = 0; j < n; ++j) {
        if (j == i) continue;
        const spkv::Geometry& gj = reqs[j].handle->g;
        const size_t qb = size_t(reqs[j].nq > 0 ? reqs[j].nq : 0) * gj.num_heads *
                          gj.head_dim * 2;
        const size_t fb = size_t(gj.tokens_per_frame) * gj.num_heads * gj.head_dim * 2;
        const Extent ext[4] = {{reqs[j].q, qb}, {reqs[j].out, qb},
                               {reqs[j].own_k, fb}, {reqs[j].own_v, fb}};
        for (const Extent& e : ext)
          if (reqs[i].out && e.p && overlaps(reqs[i].out, e.p, out_bytes, e.bytes))
            return SPKV_ERR_INVALID_ARG;
      }
    }
  }
  RunShape shape[SPKV_MAX_BATCH];
  const bool host_only = reqs[0].handle->host_only;
  for (int32_t i = 0; i < n; ++i) {
    const spkv_request& r = reqs[i];
    const int rc = check_run(r.handle, r.block, r.q, r.out, r.nq, r.sm_scale, r.own_k,
                             r.own_v, &shape[i]);
    // a host-only handle passes every check and then reports UNSUPPORTED
    if (rc != SPKV_OK && !(host_only && rc == SPKV_ERR_UNSUPPORTED)) return rc;
  }
  if (host_only) return SPKV_ERR_UNSUPPORTED;
  // Frames admitted by append_frame_in_run are copied before the batch.
  for (int32_t i = 0; i < n; ++i) {
    const int f = flush_pending(reqs[i].handle, reqs[i].block);
    if (f != SPKV_OK) return f;
  }
  // Batch plan: split each request's key range so that every work item
  // (query tile x head x split) covers at most per_item key tiles, with the
  // smallest per_item (>= 4) whose items still fit the CUs once.
  const int64_t cus = reqs[0].handle->num_cus;
  int64_t work = 0, max_tiles = 0;
  for (int32_t i = 0; i < n; ++i) {
    work += shape[i].units * shape[i].n_ktiles;
    max_tiles = std::max(max_tiles, shape[i].n_ktiles);
  }
  auto items_at = [&](int64_t per) {
    int64_t items = 0;
    for (int32_t i = 0; i < n; ++i) items += shape[i].units * ((shape[i].n_ktiles + per - 1) / per);
    return items;
  };
  int64_t per_item = std::max<int64_t>(4, (work + cus - 1) / cus);
  while (per_item < max_tiles && items_at(per_item) > cus) ++per_item;
  spkv::AttnArgs runs[SPKV_MAX_BATCH];
  for (int32_t i = 0; i < n; ++i) {
    const spkv_request& r = reqs[i];
    const int64_t want = (shape[i].n_ktiles + per_item - 1) / per_item;
    runs[i] = make_run(r.handle, r.block, r.q, r.out, r.nq, r.sm_scale, r.own_k, r.own_v,
                       shape[i], want, workspace_partials(r.handle));
  }
  DeviceGuard guard(reqs[0].handle->device);
  if (spkv::launch_attention_batch(runs, n, static_cast<hipStream_t>(hip_stream)) !=
      hipSuccess)
    return SPKV_ERR_HIP;
  return SPKV_OK;
}

SPKV_API int spkv_get_cache_stats(const spkv_handle* h, int32_t block,
                                  spkv_stats* out) {
  if (!h || !out) return SPKV_ERR_INVALID_ARG;
  spkv::PagePool::Stats s;
  const spkv::Status st = h->pool->stats(block, &s);
  if (st != spkv::Status::ok) return status(st);
  out->frame_count = s.frames;
  out->scale_pages = s.scale;
  out->live_pages = s.live;
  out->free_pages = s.free_pages;
  out->reserved = 0;
  out->special_tokens = s.special_tokens;
  return SPKV_OK;
}

SPKV_API int spkv_get_plan(const spkv_handle* h, int32_t* table, int32_t cap,
                           int32_t* n_pages, int32_t* n_patch_pages,
                           int32_t* last_page_len) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (!h->pool->planned()) return SPKV_ERR_NOT_PLANNED;
  const spkv::PlanView pv = h->pool->plan_view();
  if (table) {
    if (cap < pv.n_pages) return SPKV_ERR_INVALID_ARG;
    std::memcpy(table, pv.table, size_t(pv.n_pages) * sizeof(int32_t));
  }
  if (n_pages) *n_pages = pv.n_pages;
  if (n_patch_pages) *n_patch_pages = pv.n_patch;
  if (last_page_len) *last_page_len = pv.last_page_len;
  return SPKV_OK;
}

namespace {

int copy_specials(const spkv::SpecialRun* runs, int32_t n, int32_t* out, int32_t cap,
                  int32_t* n_runs) {
  if (out) {
    if (cap < n) return SPKV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
      out[3 * i + 0] = runs[i].first;
      out[3 * i + 1] = runs[i].count;
      out[3 * i + 2] = runs[i].kept;
    }
  }
  if (n_runs) *n_runs = n;
  return SPKV_OK;
}

}  // namespace

SPKV_API int spkv_get_plan_specials(const spkv_handle* h, int32_t* runs, int32_t cap,
                                    int32_t* n_runs) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  if (!h->pool->planned()) return SPKV_ERR_NOT_PLANNED;
  const spkv::PlanView pv = h->pool->plan_view();
  return copy_specials(pv.segs, pv.n_segs, runs, cap, n_runs);
}

SPKV_API int spkv_get_block_specials(const spkv_handle* h, int32_t block, int32_t* runs,
                                     int32_t cap, int32_t* n_runs) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  int32_t n = 0;
  spkv::Status s = h->pool->block_specials(block, nullptr, 0, &n);
  if (s != spkv::Status::ok) return status(s);
  std::vector<spkv::SpecialRun> tmp(n);   // inspection only
  s = h->pool->block_specials(block, tmp.data(), n, &n);
  if (s != spkv::Status::ok) return status(s);
  return copy_specials(tmp.data(), n, runs, cap, n_runs);
}

SPKV_API int spkv_get_block_state(const spkv_handle* h, int32_t block,
                                  int32_t* scale, int32_t* live,
                                  int32_t* free_list, int32_t cap,
                                  int32_t* n_scale, int32_t* n_live,
                                  int32_t* n_free, int64_t* n_special_frames) {
  if (!h) return SPKV_ERR_INVALID_ARG;
  return status(h->pool->block_state(block, scale, live, free_list, cap, n_scale,
                                     n_live, n_free, n_special_frames));
}

}  // extern "C"
