// Launch wrappers of the gfx950 kernels (internal to libspkv.so).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace spkv {

// Work of one append: four contiguous runs of 16-byte chunks.
struct AppendArgs {
  const void* k;          // [tokens_per_frame][H][D] bf16
  const void* v;
  void* pool;             // block's pool base
  int64_t patch_k_off;    // element offsets into the pool
  int64_t patch_v_off;
  int64_t special_k_off;
  int64_t special_v_off;
  int64_t patch_elems;    // patch_tokens * H * D
  int64_t special_elems;  // num_special * H * D
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// The same copy done by the workgroups of an attention launch (a keyframe's
// append folded into the block's run): four contiguous runs of 16-byte
// chunks, [0, n_patch) K patch, [n_patch, 2 n_patch) V patch, then n_spec K
// and n_spec V special chunks.  n_patch == 0: no copy.
struct FrameCopy {
  const uint16_t* k;      // caller's frame [tokens_per_frame][H][D]
  const uint16_t* v;
  uint16_t* pool;         // block's pool base
  int64_t pk, pv, sk, sv; // destination offsets in 16-byte chunks
  int32_t n_patch, n_spec;
};

// Expansion of a plan's page table into a per-token row map: for visible
// token t, the pool row (page * 2 * page_size + offset) of its K; its V is
// page_size rows further.  Entries past the last token repeat the last
// token's row, so a tile that runs past the end reads valid memory.
//
// The second map serves runs that also attend to the caller's own frame
// (run_own): its first nk entries are the same, the next n_own entries are
// kOwnRow | r for row r of the caller's frame buffers, and entries past them
// repeat the last of these.
constexpr uint32_t kOwnRow = 0x80000000u;

// A run of frames of the special stream whose first `kept` special tokens
// are visible; `offset` counts the visible special tokens before it.
struct SpecialSeg {
  int32_t first, count, kept, offset;
};

struct PlanArgs {
  const int32_t* table;     // device page table, n_patch patch entries used
  const SpecialSeg* segs;   // device, n_segs runs in stream order
  uint32_t* rowmap;         // out: n_out entries
  uint32_t* rowmap_own;     // out: n_out_own entries
  int32_t n_own;            // rows of a frame (specials + patches)
  int32_t n_out_own;        // entries written to rowmap_own
  int32_t n_patch, n_segs;
  int32_t patch_len;        // valid tokens of a patch page
  int32_t num_special;      // special tokens of a frame
  int32_t frames_per_spage; // frames of a special page
  int32_t first_spage;      // page id of the special stream's first page
  int32_t page_size;
  int32_t nk;               // visible tokens
  int32_t n_out;            // entries written (nk rounded up, plus padding)
  // The third map serves a run that also copies the newest frame into the
  // pool (append_frame_in_run): like the first, but the newest frame's
  // tokens -- patch tokens from new_patch_begin, and the last num_special
  // visible tokens -- are kOwnRow | their row in the caller's frame.
  uint32_t* rowmap_new;     // out: n_out entries
  int32_t new_patch_begin;  // first token of the newest frame's patch page
};

// Tiles the kernel uses; run() sizes the split from them.  One workgroup
// (512 threads, 128 KiB of LDS) is resident per CU.
constexpr int kAttnKeyTile = 64;
constexpr int kAttnQueryTile = 512;
// Tokens of a split whose row map the kernel stages in LDS at a time.
constexpr int kAttnRowmapChunk = 16384;
// Row-map entries written past the visible tokens.
constexpr int kRowmapPad = 2 * kAttnKeyTile;

hipError_t launch_expand(const PlanArgs& p, hipStream_t stream);

// One attention run over a planned row map.
struct AttnArgs {
  const uint16_t* pool;     // block's pool (bf16 bits)
  const uint16_t* own_k;    // caller's frame [n_own][H][D] for kOwnRow rows,
  const uint16_t* own_v;    //   or null when the map has none
  const uint32_t* rowmap;   // token -> K row of the pool (see PlanArgs)
  const uint16_t* q;        // [nq][H][D]
  uint16_t* out;            // [nq][H][D]
  uint16_t* part_o;         // [splits][nq][H][D] bf16, each split's O / l (splits > 1)
  float* part_ml;           // [splits][nq][H][2]     (m, l)         (splits > 1)
  int32_t nq, num_heads, page_size;
  int32_t nk;               // visible tokens
  int32_t n_cached;         // tokens before the caller's own rows (nk without them)
  int32_t splits, tokens_per_split;
  float sm_scale;
  FrameCopy copy;           // a keyframe's append done by this launch
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// Device memory the library itself holds for run_noalloc(): the split
// partials of one run, in a file-scope array of attn.hip (one copy per GPU,
// held until the process ends).  scratch_address() returns the calling
// thread's current device's copy; it looks the address up once per device
// and caches it.
constexpr int64_t kScratchBytes = int64_t(48) << 20;
hipError_t scratch_address(void** out);

// Several runs (independent streams, each with its own pool, row map and
// partials) in one attention launch and at most one merge launch.  Runs are
// validated by the caller; n <= kMaxBatchRuns.
constexpr int kMaxBatchRuns = 16;
hipError_t launch_attention_batch(const AttnArgs* runs, int n, hipStream_t stream);

}  // namespace spkv
