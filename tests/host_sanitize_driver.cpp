// Host sanitizer driver for the page-pool allocator (csrc/pool.cpp).
//
// Runs seeded random operation sequences over several geometries and checks,
// after every operation, the invariants of the two-stream page pool:
//   * per block, the scale list, the live window and the free list hold each
//     patch page id 0..M-1 exactly once, and the scale list holds <= S pages;
//   * the special stream never exceeds its physical capacity, and an append
//     writes its specials at page M + f/fpp, slot 6*(f%fpp) for its frame f;
//   * a call that returns an error leaves every block's state unchanged;
//   * a plan lists scale, then live pages of block 0, then its special pages
//     that hold a visible token, with last_page_len = 6*(f - fpp*(n_sp-1)),
//     the runs of visible special tokens and the visible token count that
//     these imply; check_run accepts exactly the blocks in that state;
//   * the visible special tokens follow a model kept here: every frame shows
//     its 6 specials until its page is evicted, then as many as the block's
//     last eviction flags keep (6, the camera token only, or none).
// tests/test_host_sanitizers.py builds it with g++ -fsanitize=address,
// undefined (no GPU, no HIP) and runs it; any finding or broken invariant
// ends the process with a non-zero status.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pool.h"

using spkv::AppendResult;
using spkv::Geometry;
using spkv::PagePool;
using spkv::Status;

namespace {

uint64_t g_state = 0;

// How often each outcome was reached, so the caller can tell that every error
// path of the allocator ran under the sanitizers.
enum Outcome { kAppendOk, kExhausted, kOverflow, kUndo, kEvictMoved, kEvictDeferred,
               kBadBlock, kSpecialsThinned, kInvalid, kRollbackOk, kNothingToRollback,
               kPlanOk, kPlanEmpty, kRunOk, kStale, kNotPlanned, kSmallCap, kNumOutcomes };
const char* const kOutcomeName[kNumOutcomes] = {
    "append_ok", "pool_exhausted", "special_overflow", "undo_append", "evict_moved",
    "evict_deferred", "bad_block", "specials_thinned", "invalid_arg", "rollback_ok",
    "nothing_to_rollback", "plan_ok", "plan_empty", "run_ok", "stale_plan", "not_planned",
    "block_state_small_cap"};
long g_count[kNumOutcomes] = {};

// splitmix64 (Steele, Lea, Flood 2014).
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int rnd(int n) { return static_cast<int>(next_u64() % static_cast<uint64_t>(n)); }

#define REQUIRE(c)                                                               \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c);   \
      std::exit(2);                                                              \
    }                                                                            \
  } while (0)

struct BlockSnap {
  std::vector<int32_t> scale, live, free_list;
  int64_t nsf = 0;
  std::vector<spkv::SpecialRun> specials;
  bool operator==(const BlockSnap& o) const {
    return scale == o.scale && live == o.live && free_list == o.free_list && nsf == o.nsf &&
           specials == o.specials;
  }
};

// The driver's own model of which special tokens each block shows: per frame
// of the special stream, how many of its specials are visible, and the count
// the block's last eviction flags keep.
struct Model {
  std::vector<std::vector<int32_t>> vis;
  std::vector<int32_t> kept;
};

// Runs of equal counts of a per-frame list, zero counts left out.
std::vector<spkv::SpecialRun> runs_of(const std::vector<int32_t>& vis) {
  std::vector<spkv::SpecialRun> out;
  for (int32_t f = 0; f < static_cast<int32_t>(vis.size()); ++f) {
    if (!out.empty() && out.back().kept == vis[f] && out.back().first + out.back().count == f)
      ++out.back().count;
    else if (vis[f] > 0)
      out.push_back(spkv::SpecialRun{f, 1, vis[f]});
  }
  return out;
}

BlockSnap snap(const PagePool& p, int b) {
  const int32_t m = p.geometry().num_patch_pages;
  BlockSnap s;
  std::vector<int32_t> sc(m), lv(m), fr(m);
  int32_t ns = -1, nl = -1, nf = -1;
  int64_t nsf = -1;
  REQUIRE(p.block_state(b, sc.data(), lv.data(), fr.data(), m, &ns, &nl, &nf, &nsf) ==
          Status::ok);
  s.scale.assign(sc.begin(), sc.begin() + ns);
  s.live.assign(lv.begin(), lv.begin() + nl);
  s.free_list.assign(fr.begin(), fr.begin() + nf);
  s.nsf = nsf;
  int32_t n = -1;
  REQUIRE(p.block_specials(b, nullptr, 0, &n) == Status::ok && n >= 0);
  s.specials.resize(n);
  if (n > 0) {
    REQUIRE(p.block_specials(b, s.specials.data(), n - 1, &n) == Status::invalid_arg);
    REQUIRE(p.block_specials(b, s.specials.data(), n, &n) == Status::ok);
  }
  return s;
}

std::vector<BlockSnap> snap_all(const PagePool& p) {
  std::vector<BlockSnap> v;
  for (int b = 0; b < p.geometry().num_blocks; ++b) v.push_back(snap(p, b));
  return v;
}

void check_block(const PagePool& p, const Model& md, int b) {
  const Geometry& g = p.geometry();
  const BlockSnap s = snap(p, b);
  REQUIRE(static_cast<int64_t>(md.vis[b].size()) == s.nsf);
  REQUIRE(s.specials == runs_of(md.vis[b]));
  std::vector<int> seen(g.num_patch_pages, 0);
  for (const auto* list : {&s.scale, &s.live, &s.free_list})
    for (int32_t x : *list) {
      REQUIRE(x >= 0 && x < g.num_patch_pages);
      seen[x] += 1;
    }
  for (int c : seen) REQUIRE(c == 1);
  REQUIRE(static_cast<int32_t>(s.scale.size()) <= g.scale_frames);
  REQUIRE(s.nsf >= 0 && s.nsf <= g.special_capacity);
  PagePool::Stats st{};
  REQUIRE(p.stats(b, &st) == Status::ok);
  REQUIRE(st.frames == s.nsf);
  REQUIRE(st.scale == static_cast<int32_t>(s.scale.size()));
  REQUIRE(st.live == static_cast<int32_t>(s.live.size()));
  REQUIRE(st.free_pages == static_cast<int32_t>(s.free_list.size()));
  REQUIRE(st.special_tokens == s.nsf * g.num_special);
}

void check_all(const PagePool& p, const Model& md) {
  for (int b = 0; b < p.geometry().num_blocks; ++b) check_block(p, md, b);
}

// The committed plan against block 0's state when it was built (`at`, and
// the model's visible specials `vis` then).
void check_plan(const PagePool& p, const BlockSnap& at, const std::vector<int32_t>& vis) {
  const Geometry& g = p.geometry();
  const spkv::PlanView v = p.plan_view();
  const int32_t fpp = g.frames_per_spage;
  const int32_t n_sp = static_cast<int32_t>((at.nsf + fpp - 1) / fpp);
  REQUIRE(v.n_patch == static_cast<int32_t>(at.scale.size() + at.live.size()));
  REQUIRE(v.n_pages <= v.n_patch + n_sp);
  REQUIRE(v.n_pages <= g.max_num_pages);
  int32_t i = 0;
  for (int32_t x : at.scale) REQUIRE(v.table[i++] == x);
  for (int32_t x : at.live) REQUIRE(v.table[i++] == x);
  int64_t special_tokens = 0;
  for (int32_t k = 0; k < n_sp; ++k) {
    int32_t shown = 0;
    for (int32_t f = k * fpp; f < std::min<int64_t>((k + 1) * fpp, at.nsf); ++f) shown += vis[f];
    special_tokens += shown;
    if (shown > 0) REQUIRE(v.table[i++] == g.num_patch_pages + k);
  }
  REQUIRE(i == v.n_pages);
  REQUIRE(v.table[v.n_pages - 1] == g.num_patch_pages + n_sp - 1);
  REQUIRE(v.last_page_len == g.num_special * (at.nsf - int64_t(fpp) * (n_sp - 1)));
  REQUIRE(v.last_page_len >= g.num_special && v.last_page_len <= g.num_special * fpp);
  REQUIRE(v.visible_tokens == int64_t(v.n_patch) * g.patch_tokens + special_tokens);
  const std::vector<spkv::SpecialRun> want = runs_of(vis);
  REQUIRE(v.n_segs == static_cast<int32_t>(want.size()));
  REQUIRE(std::equal(want.begin(), want.end(), v.segs));
}

// Expects an error status and no state change.
void expect_error(const PagePool& p, const std::vector<BlockSnap>& before, Status s,
                  Status want) {
  REQUIRE(s == want);
  REQUIRE(snap_all(p) == before);
}

uint64_t run_sequence(const Geometry& g, int n_ops) {
  PagePool p(g);
  Model md;
  md.vis.assign(g.num_blocks, {});
  md.kept.assign(g.num_blocks, g.num_special);
  check_all(p, md);
  const int32_t S = g.scale_frames, M = g.num_patch_pages;
  const int32_t wmax = M - S;
  // The model's side of an eviction that moved `moved` pages of block b.
  auto evicted = [&](int b, const BlockSnap& sb, int32_t moved) {
    const int64_t oldest = sb.nsf - static_cast<int64_t>(sb.live.size());
    for (int32_t i = 0; i < moved; ++i) md.vis[b][oldest + i] = md.kept[b];
    if (moved > 0 && md.kept[b] < g.num_special) ++g_count[kSpecialsThinned];
  };
  BlockSnap planned_at;
  std::vector<int32_t> planned_vis;
  bool have_plan = false;
  uint64_t digest = 1469598103934665603ull;
  auto mix = [&](uint64_t x) { digest = (digest ^ x) * 1099511628211ull; };
  for (int op = 0; op < n_ops; ++op) {
    const int b = rnd(g.num_blocks);
    const int kind = rnd(100);
    const auto before = snap_all(p);
    if (kind < 30) {  // append, sometimes undone as after a failed copy launch
      AppendResult r{};
      const BlockSnap sb = before[b];
      const Status s = p.append(b, &r);
      if (sb.free_list.empty()) {
        expect_error(p, before, s, Status::pool_exhausted);
        ++g_count[kExhausted];
      } else if (sb.nsf >= g.special_capacity) {
        expect_error(p, before, s, Status::special_overflow);
        ++g_count[kOverflow];
      } else {
        ++g_count[kAppendOk];
        REQUIRE(s == Status::ok);
        REQUIRE(r.patch_page == sb.free_list.front());
        REQUIRE(r.special_page == M + static_cast<int32_t>(sb.nsf / g.frames_per_spage));
        REQUIRE(r.special_slot ==
                g.num_special * static_cast<int32_t>(sb.nsf % g.frames_per_spage));
        REQUIRE(r.special_page < g.max_num_pages);
        REQUIRE(r.special_slot + g.num_special <= g.page_size);
        mix(uint64_t(r.patch_page) << 32 | uint32_t(r.special_slot));
        md.vis[b].push_back(g.num_special);
        if (rnd(8) == 0) {
          p.undo_append(b, r);
          md.vis[b].pop_back();
          REQUIRE(snap_all(p) == before);
          ++g_count[kUndo];
        }
      }
    } else if (kind < 48) {  // evict, mostly with valid arguments
      int32_t w = 1 + rnd(std::max(1, wmax));
      int32_t s_arg = S;
      // the flags: mostly the defaults, else any valid pair
      int32_t cfs = rnd(3) ? 1 : rnd(2), cam = rnd(3) ? 0 : rnd(2);
      int bb = b;
      const int bad = rnd(12);
      if (bad == 0) s_arg = S + 1;
      if (bad == 1) w = rnd(2) ? 0 : wmax + 1;
      if (bad == 2) cfs = rnd(2) ? -1 : 2;
      if (bad == 3) cam = rnd(2) ? -1 : 2;
      if (bad == 4) bb = rnd(2) ? -1 : g.num_blocks;
      int32_t moved = -1;
      const Status s = p.evict(bb, s_arg, w, cfs, cam, &moved);
      if (bad == 4) {
        expect_error(p, before, s, Status::bad_block);
        ++g_count[kBadBlock];
      } else if (bad <= 3) {
        expect_error(p, before, s, Status::invalid_arg);
        ++g_count[kInvalid];
      } else {
        REQUIRE(s == Status::ok);
        md.kept[b] = cfs ? (cam ? 1 : g.num_special) : 0;
        const int32_t live = static_cast<int32_t>(before[b].live.size());
        REQUIRE(moved == (p.defer() ? 0 : std::max(0, live - w)));
        if (p.defer() && live > w) ++g_count[kEvictDeferred];
        if (moved > 0) ++g_count[kEvictMoved];
        evicted(b, before[b], moved);
        mix(uint64_t(moved));
      }
    } else if (kind < 56) {  // deferred eviction carried out
      const int32_t w = 1 + rnd(std::max(1, wmax));
      int32_t moved = -1;
      REQUIRE(p.execute_deferred(b, S, w, &moved) == Status::ok);
      REQUIRE(moved == std::max(0, static_cast<int32_t>(before[b].live.size()) - w));
      evicted(b, before[b], moved);
    } else if (kind < 70) {  // rollback
      const Status s = p.rollback(b);
      if (s != Status::ok) {
        expect_error(p, before, s, Status::nothing_to_rollback);
        ++g_count[kNothingToRollback];
      } else {
        ++g_count[kRollbackOk];
        md.vis[b].pop_back();
        const BlockSnap after = snap(p, b);
        REQUIRE(after.nsf == before[b].nsf - 1);
        REQUIRE(after.free_list.size() == before[b].free_list.size() + 1);
        REQUIRE(p.rollback(b) == Status::nothing_to_rollback);  // once per append
      }
    } else if (kind < 76) {
      p.set_defer(rnd(2) == 1);
    } else if (kind < 78) {
      p.reset();
      md.vis.assign(g.num_blocks, {});
      md.kept.assign(g.num_blocks, g.num_special);
      have_plan = false;
      for (int k = 0; k < g.num_blocks; ++k) {
        const BlockSnap s = snap(p, k);
        REQUIRE(s.scale.empty() && s.live.empty() && s.nsf == 0);
        for (int32_t i = 0; i < M; ++i) REQUIRE(s.free_list[i] == i);
      }
      REQUIRE(!p.defer());
    } else if (kind < 90) {  // plan, sometimes built but not committed
      const bool commit = rnd(4) != 0;
      const Status s = commit ? p.plan() : p.build_plan();
      if (before[0].nsf == 0) {
        expect_error(p, before, s, Status::empty);
        ++g_count[kPlanEmpty];
      } else {
        REQUIRE(s == Status::ok);
        ++g_count[kPlanOk];
        if (commit) {
          planned_at = before[0];
          planned_vis = md.vis[0];
          have_plan = true;
          check_plan(p, planned_at, planned_vis);
          mix(uint64_t(p.plan_view().visible_tokens));
        }
      }
    } else if (kind < 96) {  // check_run against the committed plan
      const Status s = p.check_run(b);
      if (!have_plan) {
        REQUIRE(s == Status::not_planned);
        ++g_count[kNotPlanned];
      } else {
        const BlockSnap sb = before[b];
        const bool same = sb.nsf == planned_at.nsf && sb.scale == planned_at.scale &&
                          sb.live == planned_at.live && md.vis[b] == planned_vis;
        REQUIRE(s == (same ? Status::ok : Status::stale_plan));
        ++g_count[same ? kRunOk : kStale];
      }
      REQUIRE(p.check_run(-1) == Status::bad_block);
    } else {  // block_state with a too-small output capacity
      const int32_t m = M;
      std::vector<int32_t> buf(m);
      int32_t ns, nl, nf;
      int64_t nsf;
      const int32_t cap = rnd(m + 1);
      const Status s = p.block_state(b, buf.data(), buf.data(), buf.data(), cap, &ns, &nl, &nf, &nsf);
      const bool fits = cap >= static_cast<int32_t>(before[b].scale.size()) &&
                        cap >= static_cast<int32_t>(before[b].live.size()) &&
                        cap >= static_cast<int32_t>(before[b].free_list.size());
      REQUIRE(s == (fits ? Status::ok : Status::invalid_arg));
      if (!fits) ++g_count[kSmallCap];
    }
    check_all(p, md);
  }
  return digest;
}

Geometry geometry(int blocks, int ps, int patch, int S, int W, int R, int mtf) {
  Geometry g{};
  g.num_blocks = blocks;
  g.num_heads = 4;
  g.head_dim = 64;
  g.page_size = ps;
  g.patch_tokens = patch;
  g.num_special = 6;
  g.scale_frames = S;
  g.sliding_window = W;
  g.headroom = R;
  g.max_total_frames = mtf;
  REQUIRE(g.derive());
  return g;
}

}  // namespace

int main(int argc, char** argv) {
  const int n_seq = argc > 1 ? std::atoi(argv[1]) : 40;
  const int n_ops = argc > 2 ? std::atoi(argv[2]) : 400;
  // Invalid geometries are refused.
  {
    Geometry g{};
    g.num_blocks = 1, g.num_heads = 1, g.head_dim = 64, g.page_size = 5, g.patch_tokens = 4;
    g.num_special = 6, g.scale_frames = 1, g.sliding_window = 1, g.headroom = 0;
    g.max_total_frames = 4;
    REQUIRE(!g.derive());  // page smaller than a frame's specials
    g.page_size = 16, g.patch_tokens = 17;
    REQUIRE(!g.derive());  // patches do not fit a page
  }
  const std::vector<Geometry> geoms = {
      geometry(1, 16, 16, 2, 4, 2, 32),      // the tiny stream
      geometry(3, 13, 11, 3, 5, 1, 9),       // odd page size, 2 frames per special page
      geometry(2, 8, 8, 0, 3, 0, 7),         // no scale frames, no headroom, 1 frame per page
      geometry(2, 6, 5, 1, 1, 0, 5),         // window of one page, exhaustion reachable
      geometry(3, 999, 999, 8, 64, 16, 2048),  // the 518x378 stream's pool
      geometry(2, 1024, 999, 8, 120, 16, 40),  // padded pages, window mode, small stream
  };
  uint64_t total = 0;
  for (size_t gi = 0; gi < geoms.size(); ++gi)
    for (int s = 0; s < n_seq; ++s) {
      g_state = 0x5eed0000ull + gi * 1000003ull + uint64_t(s);
      total ^= run_sequence(geoms[gi], n_ops) + gi;
    }
  for (int i = 0; i < kNumOutcomes; ++i) std::printf("%s %ld\n", kOutcomeName[i], g_count[i]);
  std::printf("ok %zu geometries x %d sequences x %d ops, digest %016llx\n", geoms.size(),
              n_seq, n_ops, static_cast<unsigned long long>(total));
  return 0;
}
