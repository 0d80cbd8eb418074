// Host page-pool allocator of the streaming two-stream paged KV cache.
//
// Pure C++17, no HIP: the bookkeeping that the pages describe as moving page
// ids between deques ("How to Improve Streaming Inference Performance with
// FlashInfer KV Cache Backend", section "Two-Stream Page Pool Architecture").
// Every container has a fixed capacity set at construction, so no operation
// after construction allocates, and each one is O(1) except plan (O(table)).
//
// Ids are int32 page indices into the block's pool; patch pages are
// 0..M-1 and special pages M..M+NS-1.
#pragma once

#include <cstdint>
#include <vector>

namespace spkv {

// Fixed-capacity double-ended queue over a ring buffer.
class Ring {
 public:
  void init(int32_t cap) {
    buf_.assign(cap > 0 ? cap : 1, 0);
    head_ = 0;
    size_ = 0;
  }
  int32_t size() const { return size_; }
  bool empty() const { return size_ == 0; }
  int32_t operator[](int32_t i) const { return buf_[wrap(head_ + i)]; }
  int32_t front() const { return buf_[head_]; }
  int32_t back() const { return buf_[wrap(head_ + size_ - 1)]; }
  void push_back(int32_t x) {
    buf_[wrap(head_ + size_)] = x;
    ++size_;
  }
  void push_front(int32_t x) {
    head_ = wrap(head_ + cap() - 1);
    buf_[head_] = x;
    ++size_;
  }
  int32_t pop_front() {
    int32_t x = buf_[head_];
    head_ = wrap(head_ + 1);
    --size_;
    return x;
  }
  int32_t pop_back() {
    --size_;
    return buf_[wrap(head_ + size_)];
  }
  void clear() {
    head_ = 0;
    size_ = 0;
  }

 private:
  int32_t cap() const { return static_cast<int32_t>(buf_.size()); }
  int32_t wrap(int32_t i) const { return i >= cap() ? i - cap() : i; }
  std::vector<int32_t> buf_;
  int32_t head_ = 0;
  int32_t size_ = 0;
};

struct Geometry {
  int32_t num_blocks, num_heads, head_dim, page_size, patch_tokens,
      num_special, scale_frames, sliding_window, headroom, max_total_frames;
  // derived
  int32_t num_patch_pages;   // M = S + W + R
  int32_t frames_per_spage;  // floor(page_size / num_special)
  int32_t num_special_pages; // ceil(max_total_frames / frames_per_spage)
  int32_t max_num_pages;     // M + NS
  int64_t special_capacity;  // NS * frames_per_spage (physical slots)
  int32_t tokens_per_frame;  // num_special + patch_tokens

  // Fills the derived fields; false if the parameters are invalid.
  bool derive();
};

enum class Status : int {
  ok = 0,
  invalid_arg = -1,
  bad_block = -2,
  pool_exhausted = -3,
  special_overflow = -4,
  nothing_to_rollback = -5,
  empty = -6,
  not_planned = -7,
  stale_plan = -8,
  unsupported = -9,
};

// What an append did, for the kernel launch and for undoing it.
struct AppendResult {
  int32_t patch_page;
  int32_t special_page;
  int32_t special_slot;
  int32_t prev_last_page;      // rollback target before this append
  bool prev_last_in_scale;
};

// Frames [first, first + count) of the special stream, each showing its
// first `kept` special tokens to attention.
struct SpecialRun {
  int32_t first, count, kept;
  bool operator==(const SpecialRun& o) const {
    return first == o.first && count == o.count && kept == o.kept;
  }
};

struct PlanView {
  const int32_t* table;
  int32_t n_pages;
  int32_t n_patch;
  int32_t last_page_len;
  int64_t visible_tokens;
  const SpecialRun* segs;   // visible special tokens, in stream order
  int32_t n_segs;
};

class PagePool {
 public:
  explicit PagePool(const Geometry& g);

  const Geometry& geometry() const { return g_; }

  Status append(int32_t block, AppendResult* out);
  void undo_append(int32_t block, const AppendResult& r);  // exact inverse
  Status evict(int32_t block, int32_t scale_frames, int32_t window,
               int32_t cross_frame_special, int32_t camera_only,
               int32_t* moved);
  Status execute_deferred(int32_t block, int32_t scale_frames, int32_t window,
                          int32_t* moved);
  Status rollback(int32_t block);
  void set_defer(bool on) { defer_ = on; }
  bool defer() const { return defer_; }
  void reset();

  // plan() in two phases so that a caller can stage the table elsewhere
  // before it becomes the plan: build_plan() fills a pending plan from
  // block 0, commit_plan() makes it current.  plan() does both.
  Status build_plan();
  PlanView pending_view() const { return view_of(next_); }
  void commit_plan();
  Status plan();
  Status check_run(int32_t block) const;
  bool planned() const { return planned_; }
  PlanView plan_view() const { return view_of(cur_); }

  struct Stats {
    int64_t frames;
    int32_t scale, live, free_pages;
    int64_t special_tokens;
  };
  Status stats(int32_t block, Stats* s) const;
  Status block_state(int32_t block, int32_t* scale, int32_t* live,
                     int32_t* free_list, int32_t cap, int32_t* n_scale,
                     int32_t* n_live, int32_t* n_free, int64_t* nsf) const;
  // The special tokens block `block` shows, as coalesced runs (the segments
  // its plan would carry); *n gets the count, out (cap runs) the runs.
  Status block_specials(int32_t block, SpecialRun* out, int32_t cap,
                        int32_t* n) const;
  // Runs a plan or a block can hold at most.
  int32_t max_special_segments() const {
    return static_cast<int32_t>(g_.special_capacity) + 2;
  }

 private:
  struct Block {
    Ring free_list;
    std::vector<int32_t> scale;  // reserved to S, never reallocates
    Ring live;
    int64_t nsf = 0;
    int32_t last_page = -1;      // -1: nothing to roll back
    bool last_in_scale = false;
    // Evicted frames (a contiguous range starting at frame S, as eviction
    // is first in, first out) as runs of equal kept counts; reserved to the
    // special stream's capacity, never reallocates.
    std::vector<SpecialRun> evicted;
    int32_t kept_on_evict = 0;   // special tokens an evicted frame keeps
  };
  void init_block(Block& b);
  bool valid_block(int32_t b) const { return b >= 0 && b < g_.num_blocks; }
  Status check_evict_args(int32_t scale_frames, int32_t window) const;
  int32_t evict_to(Block& b, int32_t window);
  // Visible special tokens of a block as coalesced runs (kept > 0 only).
  int32_t special_segments(const Block& b, SpecialRun* out) const;

  Geometry g_;
  std::vector<Block> blocks_;
  bool defer_ = false;

  // A plan built from block 0, plus the state snapshot it was built from.
  struct PlanData {
    std::vector<int32_t> table;
    int32_t n_pages = 0, n_patch = 0, last_page_len = 0;
    int64_t visible_tokens = 0;
    std::vector<SpecialRun> segs;  // capacity max_special_segments()
    int32_t n_segs = 0;
    std::vector<int32_t> scale, live;
    std::vector<SpecialRun> evicted;
    int64_t nsf = 0;
  };
  void init_plan(PlanData& p) const;
  static PlanView view_of(const PlanData& p) {
    return PlanView{p.table.data(), p.n_pages, p.n_patch, p.last_page_len,
                    p.visible_tokens, p.segs.data(), p.n_segs};
  }
  bool planned_ = false;
  PlanData cur_, next_;
};

}  // namespace spkv
