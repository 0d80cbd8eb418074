// Host page-pool allocator: the rules of the two-stream paged KV cache.
//
// Pages cited by title and section:
//   [LB-KV]   "How LingBot-Map Implements the KV Cache Mechanism for Streaming
//             Inference with FlashInfer Integration"
//   [LB-PERF] "How to Improve Streaming Inference Performance with FlashInfer
//             KV Cache Backend"
//   [LB-SLOT] "LingBot-Map KV缓存机制深度揭秘：scale frames与keyframes如何占用slot"
#include "pool.h"

#include <algorithm>
#include <utility>

namespace spkv {

bool Geometry::derive() {
  if (num_blocks < 1 || num_heads < 1 || head_dim < 1 || num_special < 1 ||
      page_size < num_special || patch_tokens < 1 ||
      patch_tokens > page_size || scale_frames < 0 || sliding_window < 1 ||
      headroom < 0 || max_total_frames < 1)
    return false;
  const int64_t m = int64_t(scale_frames) + sliding_window + headroom;
  if (m > (1 << 24)) return false;
  num_patch_pages = static_cast<int32_t>(m);
  // [LB-SLOT] special-token stream: floor(page_size / 6) whole frames a page.
  frames_per_spage = page_size / num_special;
  const int64_t ns =
      (int64_t(max_total_frames) + frames_per_spage - 1) / frames_per_spage;
  if (m + ns > (1 << 24)) return false;
  num_special_pages = static_cast<int32_t>(ns);
  max_num_pages = static_cast<int32_t>(m + ns);
  special_capacity = ns * frames_per_spage;
  tokens_per_frame = num_special + patch_tokens;
  return true;
}

PagePool::PagePool(const Geometry& g) : g_(g) {
  blocks_.resize(g_.num_blocks);
  for (auto& b : blocks_) init_block(b);
  init_plan(cur_);
  init_plan(next_);
}

void PagePool::init_plan(PlanData& p) const {
  p.table.assign(g_.max_num_pages, 0);
  p.scale.reserve(g_.scale_frames);
  p.live.reserve(g_.num_patch_pages);
}

void PagePool::init_block(Block& b) {
  // Free list starts as 0..M-1 (allocation takes the head).
  b.free_list.init(g_.num_patch_pages);
  for (int32_t p = 0; p < g_.num_patch_pages; ++p) b.free_list.push_back(p);
  b.scale.clear();
  b.scale.reserve(g_.scale_frames);
  b.live.init(g_.num_patch_pages);
  b.nsf = 0;
  b.last_page = -1;
  b.last_in_scale = false;
}

// [LB-KV] "Append and Evict API"; [LB-SLOT] "scale frames：永不驱逐的前 8 个
// slot" (route to the scale pages while fewer than scale_frames are held) and
// "特殊 token 流" (append-only special stream).
Status PagePool::append(int32_t block, AppendResult* out) {
  if (!valid_block(block)) return Status::bad_block;
  Block& b = blocks_[block];
  if (b.free_list.empty()) return Status::pool_exhausted;
  if (b.nsf >= g_.special_capacity) return Status::special_overflow;
  out->prev_last_page = b.last_page;
  out->prev_last_in_scale = b.last_in_scale;
  const int32_t p = b.free_list.pop_front();
  if (static_cast<int32_t>(b.scale.size()) < g_.scale_frames) {
    b.scale.push_back(p);
    b.last_in_scale = true;
  } else {
    b.live.push_back(p);
    b.last_in_scale = false;
  }
  out->patch_page = p;
  out->special_page =
      g_.num_patch_pages + static_cast<int32_t>(b.nsf / g_.frames_per_spage);
  out->special_slot =
      g_.num_special * static_cast<int32_t>(b.nsf % g_.frames_per_spage);
  b.nsf += 1;
  b.last_page = p;
  return Status::ok;
}

// Exact inverse of the append that produced `r`, used when the copy kernel
// cannot be enqueued, so that a failed append leaves no trace.
void PagePool::undo_append(int32_t block, const AppendResult& r) {
  Block& b = blocks_[block];
  if (b.last_in_scale)
    b.scale.pop_back();
  else
    b.live.pop_back();
  b.free_list.push_front(r.patch_page);
  b.nsf -= 1;
  b.last_page = r.prev_last_page;
  b.last_in_scale = r.prev_last_in_scale;
}

Status PagePool::check_evict_args(int32_t scale_frames, int32_t window) const {
  if (scale_frames != g_.scale_frames) return Status::invalid_arg;
  if (window < 1 || window > g_.num_patch_pages - g_.scale_frames)
    return Status::invalid_arg;
  return Status::ok;
}

// [LB-SLOT] "keyframes：滑动窗口 slot 的进出规则": when the window is over its
// limit the oldest page goes back to the free list for reuse.
int32_t PagePool::evict_to(Block& b, int32_t window) {
  int32_t moved = 0;
  while (b.live.size() > window) {
    b.free_list.push_back(b.live.pop_front());
    ++moved;
  }
  if (moved) b.last_page = -1;  // the last append can no longer be undone
  return moved;
}

Status PagePool::evict(int32_t block, int32_t scale_frames, int32_t window,
                       int32_t cross_frame_special, int32_t camera_only,
                       int32_t* moved) {
  if (!valid_block(block)) return Status::bad_block;
  if (cross_frame_special != 1 || camera_only != 0) return Status::unsupported;
  Status s = check_evict_args(scale_frames, window);
  if (s != Status::ok) return s;
  int32_t m = 0;
  // [LB-PERF] "Deferred Eviction Strategy": paused while deferred.
  if (!defer_) m = evict_to(blocks_[block], window);
  if (moved) *moved = m;
  return Status::ok;
}

// [LB-SLOT] "进阶：光流关键帧与回滚机制": perform the backlogged eviction.
Status PagePool::execute_deferred(int32_t block, int32_t scale_frames,
                                  int32_t window, int32_t* moved) {
  if (!valid_block(block)) return Status::bad_block;
  Status s = check_evict_args(scale_frames, window);
  if (s != Status::ok) return s;
  int32_t m = evict_to(blocks_[block], window);
  if (moved) *moved = m;
  return Status::ok;
}

// [LB-SLOT] "进阶：光流关键帧与回滚机制": the patch page returns to the free
// list, the special count and frame count drop by one.
Status PagePool::rollback(int32_t block) {
  if (!valid_block(block)) return Status::bad_block;
  Block& b = blocks_[block];
  if (b.last_page < 0) return Status::nothing_to_rollback;
  if (b.last_in_scale)
    b.scale.pop_back();
  else
    b.live.pop_back();
  b.free_list.push_front(b.last_page);
  b.nsf -= 1;
  b.last_page = -1;
  return Status::ok;
}

// [LB-SLOT] "窗口模式": clean_kv_cache() at the start of each window.
void PagePool::reset() {
  for (auto& b : blocks_) init_block(b);
  defer_ = false;
  planned_ = false;
}

// [LB-KV] "Patch Pages vs. Special Pages" (scale -> live -> special) and
// "Physical Page Layout and Indexing" (last_page_len); [LB-PERF] "One-Time
// Planning Pattern" (block 0 only).
Status PagePool::build_plan() {
  const Block& b = blocks_[0];
  if (b.nsf == 0) return Status::empty;
  PlanData& p = next_;
  const int32_t fpp = g_.frames_per_spage;
  const int32_t n_sp = static_cast<int32_t>((b.nsf + fpp - 1) / fpp);
  int32_t n = 0;
  for (int32_t x : b.scale) p.table[n++] = x;
  for (int32_t i = 0; i < b.live.size(); ++i) p.table[n++] = b.live[i];
  p.n_patch = n;
  for (int32_t i = 0; i < n_sp; ++i) p.table[n++] = g_.num_patch_pages + i;
  p.n_pages = n;
  p.last_page_len =
      g_.num_special * static_cast<int32_t>(b.nsf - int64_t(fpp) * (n_sp - 1));
  p.visible_tokens = int64_t(p.n_patch) * g_.patch_tokens +
                     int64_t(n_sp - 1) * g_.num_special * fpp + p.last_page_len;
  p.scale.assign(b.scale.begin(), b.scale.end());
  p.live.clear();
  for (int32_t i = 0; i < b.live.size(); ++i) p.live.push_back(b.live[i]);
  p.nsf = b.nsf;
  return Status::ok;
}

void PagePool::commit_plan() {
  std::swap(cur_, next_);
  planned_ = true;
}

Status PagePool::plan() {
  const Status s = build_plan();
  if (s == Status::ok) commit_plan();
  return s;
}

// The plan is shared by all blocks; it is only valid for a block whose page
// state is the one the plan was built from.
Status PagePool::check_run(int32_t block) const {
  if (!valid_block(block)) return Status::bad_block;
  if (!planned_) return Status::not_planned;
  const Block& b = blocks_[block];
  if (b.nsf != cur_.nsf || b.scale.size() != cur_.scale.size() ||
      b.live.size() != static_cast<int32_t>(cur_.live.size()))
    return Status::stale_plan;
  if (!std::equal(b.scale.begin(), b.scale.end(), cur_.scale.begin()))
    return Status::stale_plan;
  for (int32_t i = 0; i < b.live.size(); ++i)
    if (b.live[i] != cur_.live[i]) return Status::stale_plan;
  return Status::ok;
}

// [LB-SLOT] "动手验证：查看你的 KV 缓存占用": frame_count, scale_pages,
// live_pages, free_pages, special_tokens.
Status PagePool::stats(int32_t block, Stats* s) const {
  if (!valid_block(block)) return Status::bad_block;
  const Block& b = blocks_[block];
  s->frames = b.nsf;
  s->scale = static_cast<int32_t>(b.scale.size());
  s->live = b.live.size();
  s->free_pages = b.free_list.size();
  s->special_tokens = b.nsf * g_.num_special;
  return Status::ok;
}

Status PagePool::block_state(int32_t block, int32_t* scale, int32_t* live,
                             int32_t* free_list, int32_t cap, int32_t* n_scale,
                             int32_t* n_live, int32_t* n_free,
                             int64_t* nsf) const {
  if (!valid_block(block)) return Status::bad_block;
  const Block& b = blocks_[block];
  const int32_t ns = static_cast<int32_t>(b.scale.size());
  if ((scale && cap < ns) || (live && cap < b.live.size()) ||
      (free_list && cap < b.free_list.size()))
    return Status::invalid_arg;
  if (scale) std::copy(b.scale.begin(), b.scale.end(), scale);
  if (live)
    for (int32_t i = 0; i < b.live.size(); ++i) live[i] = b.live[i];
  if (free_list)
    for (int32_t i = 0; i < b.free_list.size(); ++i)
      free_list[i] = b.free_list[i];
  if (n_scale) *n_scale = ns;
  if (n_live) *n_live = b.live.size();
  if (n_free) *n_free = b.free_list.size();
  if (nsf) *nsf = b.nsf;
  return Status::ok;
}

}  // namespace spkv
