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
  p.segs.assign(max_special_segments(), SpecialRun{0, 0, 0});
  p.scale.reserve(g_.scale_frames);
  p.live.reserve(g_.num_patch_pages);
  p.evicted.reserve(g_.special_capacity);
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
  b.evicted.clear();
  b.evicted.reserve(g_.special_capacity);
  b.kept_on_evict = g_.num_special;  // the pages' default flags (1, 0)
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
// limit the oldest page goes back to the free list for reuse.  The frame it
// held keeps kept_on_evict of its special tokens in view; their bytes stay.
int32_t PagePool::evict_to(Block& b, int32_t window) {
  int32_t moved = 0;
  while (b.live.size() > window) {
    // The live window holds frames nsf - live .. nsf - 1; the oldest leaves.
    const int32_t f = static_cast<int32_t>(b.nsf) - b.live.size();
    b.free_list.push_back(b.live.pop_front());
    SpecialRun* last = b.evicted.empty() ? nullptr : &b.evicted.back();
    if (last && last->kept == b.kept_on_evict && last->first + last->count == f)
      ++last->count;
    else
      b.evicted.push_back(SpecialRun{f, 1, b.kept_on_evict});
    ++moved;
  }
  if (moved) b.last_page = -1;  // the last append can no longer be undone
  return moved;
}

// [LB-KV] "Append and Evict API": eviction recycles the oldest patch pages,
// optionally preserving special tokens; [LB-SLOT] "特殊 token 流": preserved
// specials carry context across frames, the camera tokens in particular.
// cross_frame_special = 1 keeps an evicted frame's specials in view (only
// its camera token, the first, with camera_only = 1); 0 keeps none.  The
// flags apply to the pages this call moves and, under deferral, to those the
// block's next execute_deferred_eviction moves.
Status PagePool::evict(int32_t block, int32_t scale_frames, int32_t window,
                       int32_t cross_frame_special, int32_t camera_only,
                       int32_t* moved) {
  if (!valid_block(block)) return Status::bad_block;
  if ((cross_frame_special != 0 && cross_frame_special != 1) ||
      (camera_only != 0 && camera_only != 1))
    return Status::invalid_arg;
  Status s = check_evict_args(scale_frames, window);
  if (s != Status::ok) return s;
  Block& b = blocks_[block];
  b.kept_on_evict = cross_frame_special ? (camera_only ? 1 : g_.num_special) : 0;
  int32_t m = 0;
  // [LB-PERF] "Deferred Eviction Strategy": paused while deferred.
  if (!defer_) m = evict_to(b, window);
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
// Frames 0 .. S-1 (the scale pages) and the live window's frames show all of
// their specials; the evicted frames between them show their runs' counts.
int32_t PagePool::special_segments(const Block& b, SpecialRun* out) const {
  int32_t n = 0;
  auto add = [&](int32_t first, int32_t count, int32_t kept) {
    if (count <= 0 || kept <= 0) return;
    if (n > 0 && out[n - 1].kept == kept && out[n - 1].first + out[n - 1].count == first)
      out[n - 1].count += count;
    else
      out[n++] = SpecialRun{first, count, kept};
  };
  const int32_t nsf = static_cast<int32_t>(b.nsf);
  const int32_t held_from = nsf - b.live.size();  // first frame of the window
  int32_t f = 0;
  if (!b.evicted.empty()) {
    add(0, b.evicted.front().first, g_.num_special);
    for (const SpecialRun& r : b.evicted) add(r.first, r.count, r.kept);
    f = b.evicted.back().first + b.evicted.back().count;
  }
  add(f, held_from - f, g_.num_special);      // scale frames (no eviction yet)
  add(held_from, nsf - held_from, g_.num_special);
  return n;
}

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
  p.n_segs = special_segments(b, p.segs.data());
  // Special pages that hold at least one visible token, in stream order.
  int64_t special_tokens = 0;
  int32_t last_sp = -1;
  for (int32_t i = 0; i < p.n_segs; ++i) {
    const SpecialRun& r = p.segs[i];
    special_tokens += int64_t(r.count) * r.kept;
    for (int32_t k = std::max(last_sp + 1, r.first / fpp);
         k <= (r.first + r.count - 1) / fpp; ++k)
      p.table[n++] = g_.num_patch_pages + k;
    last_sp = (r.first + r.count - 1) / fpp;
  }
  p.n_pages = n;
  // The newest frame is always held, so the stream's last special page, the
  // one last_page_len describes, is always the table's last entry.
  p.last_page_len =
      g_.num_special * static_cast<int32_t>(b.nsf - int64_t(fpp) * (n_sp - 1));
  p.visible_tokens = int64_t(p.n_patch) * g_.patch_tokens + special_tokens;
  p.scale.assign(b.scale.begin(), b.scale.end());
  p.live.clear();
  for (int32_t i = 0; i < b.live.size(); ++i) p.live.push_back(b.live[i]);
  p.evicted.assign(b.evicted.begin(), b.evicted.end());
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
  if (b.evicted.size() != cur_.evicted.size() ||
      !std::equal(b.evicted.begin(), b.evicted.end(), cur_.evicted.begin()))
    return Status::stale_plan;
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

Status PagePool::block_specials(int32_t block, SpecialRun* out, int32_t cap,
                                int32_t* n) const {
  if (!valid_block(block)) return Status::bad_block;
  const Block& b = blocks_[block];
  // At most one segment per evicted run plus the two held ranges.
  std::vector<SpecialRun> segs(b.evicted.size() + 2);  // inspection, not the hot path
  const int32_t k = special_segments(b, segs.data());
  if (out && cap < k) return Status::invalid_arg;
  if (out) std::copy(segs.begin(), segs.begin() + k, out);
  if (n) *n = k;
  return Status::ok;
}

}  // namespace spkv
