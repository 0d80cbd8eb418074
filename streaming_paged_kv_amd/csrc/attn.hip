// plan()'s device half and run(): paged prefill attention over the planned
// pages (gfx950).
//
// What it computes ("How LingBot-Map Implements the KV Cache Mechanism ...",
// section "Kernel-Level Execution Flow"): for every query row i and head h of
// the frame,
//     O[i,h,:] = sum_j softmax_j(s * Q[i,h,:] . K[j,h,:]) V[j,h,:]
// over the visible tokens j, in the table's order (scale pages, live window,
// special pages), non-causal and without positional encoding, with as many
// query heads as K/V heads.  Each table entry contributes its valid tokens
// only: patch_len for patch pages, special_len for full special pages and
// last_len for the last one ("Physical Page Layout and Indexing": the last
// special page's fill is described by last_page_len, so no mask is needed).
//
// Design (gfx950 / CDNA4):
//  * plan() expands the page table once per frame step into a row map (pool
//    row of every visible token) with a small kernel, so the attention loop
//    never divides or looks up pages: pages of any length (999, 996-token
//    special pages, a partly filled last page) are walked as one token
//    sequence, without padding.
//  * One workgroup = 8 waves = 512 query rows of one head; each wave owns 64
//    rows as two 32-row column tiles of v_mfma_f32_32x32x16_bf16.
//  * Scores are computed transposed, S^T = K Q^T: a lane then holds one query
//    column and 16 keys per 32x32 tile, so the softmax reductions are
//    in-lane plus one exchange with lane ^ 32.  The same lane layout is the B
//    operand of the second product O^T = V^T P^T, so P never leaves
//    registers.  V^T fragments are read from the natural [key][d] V tile
//    with the transposing LDS read (ds_read_b64_tr_b16).
//  * Ping-pong: waves w and w+4 share a SIMD.  The two groups of four waves
//    alternate between an MFMA phase (PV of the previous tile, scores of the
//    current one) and a softmax phase (VALU), one workgroup barrier per
//    phase, so each SIMD's matrix core and vector ALU work at the same time.
//  * K/V tiles of 64 tokens come in with direct-to-LDS loads
//    (global_load_lds_dwordx4) into a 4-stage ring, issued three phases
//    before their first use; they cost no registers and the wave never
//    waits for them inside a phase.  LDS rows are 128 B, unpadded, with the
//    16-byte chunks of row r at slot chunk ^ swz(r & 7): the permutation is
//    applied on the global side (each lane picks which chunk it fetches), so
//    both the K reads and the transposing V reads are free of bank
//    conflicts.  The split's row map is staged in LDS as byte offsets.
//  * Online softmax in fp32, base 2, with s*log2(e) and the running
//    reference m folded into one FMA per score.  The reference only moves on
//    a wave-uniform slow path (first tile, or a tile whose p would exceed
//    2^16), so most tiles neither take a maximum nor rescale.  Row sums are
//    fp32 sums of the p values; P is rounded to bf16 for the second product;
//    O is rounded to bf16 once.  (v_dot2 sums of the rounded values would
//    share the matrix pipe and stall behind the other wave's MFMAs.)
//  * The key range is split across workgroups when query tiles x heads
//    alone cannot fill the CUs; partial (O, m, l) go to the workspace and a
//    merge kernel combines them.  Work items are mapped so that the query
//    tiles sharing one (head, key split) land on the same XCD (workgroups are
//    dealt to the 8 XCDs round-robin), where they share that XCD's L2.
#include "kernels.h"

#include <mutex>

namespace spkv {
namespace {

// run_noalloc()'s split partials.  In host code `scratch` names a host-side
// stand-in: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[kScratchBytes];

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int kD = 64;
constexpr int kBN = kAttnKeyTile;       // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;   // 512
constexpr int kBM = kAttnQueryTile;     // query rows per workgroup (8 x 64)
static_assert(kBM == kWaves * 64, "one 64-row slice per wave");
constexpr int kRowB = 128;              // LDS bytes of one key row (64 bf16)
constexpr int kTileB = kBN * kRowB;     // one K or V tile: 8 KiB
constexpr int kStageB = 2 * kTileB;     // K tile, then V tile
constexpr int kStages = 4;
constexpr int kRmMax = kAttnRowmapChunk;  // row-map entries staged in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSumLimit = 65536.0f;   // bound on a lane's partial row sum

// ------------------------------------------------------------- plan expand
// Pool row of visible token t (0 <= t < nk) of a plan: the patch pages'
// tokens in table order, then the visible special tokens run by run (frame f
// of the special stream sits in page first_spage + f / frames_per_spage at
// slot num_special * (f % frames_per_spage)).
__device__ __forceinline__ uint32_t plan_row(const PlanArgs& p, int t) {
  const int patch_tokens = p.n_patch * p.patch_len;
  if (t < patch_tokens) {
    const int e = t / p.patch_len;
    return static_cast<uint32_t>(p.table[e]) * 2u * static_cast<uint32_t>(p.page_size) +
           static_cast<uint32_t>(t - e * p.patch_len);
  }
  const int u = t - patch_tokens;
  int lo = 0, hi = p.n_segs - 1;   // last run with offset <= u
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.segs[mid].offset <= u) lo = mid;
    else hi = mid - 1;
  }
  const SpecialSeg s = p.segs[lo];
  const int r = u - s.offset;
  const int f = s.first + r / s.kept;
  const int page = p.first_spage + f / p.frames_per_spage;
  const int slot = p.num_special * (f % p.frames_per_spage) + r % s.kept;
  return static_cast<uint32_t>(page) * 2u * static_cast<uint32_t>(p.page_size) +
         static_cast<uint32_t>(slot);
}

__global__ __launch_bounds__(256) void expand_kernel(PlanArgs p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < p.n_out) {
    const uint32_t row = plan_row(p, min(t, p.nk - 1));
    p.rowmap[t] = row;
    // The newest frame: its patch page is the last patch page of the table
    // and its specials are the last visible tokens (it is always held).
    const int d_patch = t - p.new_patch_begin;
    const int d_spec = t - (p.nk - p.num_special);
    uint32_t nrow = row;
    if (d_patch >= 0 && d_patch < p.patch_len)
      nrow = kOwnRow | uint32_t(p.num_special + d_patch);
    else if (d_spec >= 0 && t < p.nk)
      nrow = kOwnRow | uint32_t(d_spec);
    p.rowmap_new[t] = nrow;
  }
  if (t < p.n_out_own)
    p.rowmap_own[t] = t < p.nk ? plan_row(p, t) : kOwnRow | uint32_t(min(t - p.nk, p.n_own - 1));
}

// ---------------------------------------------------------------- attention
// LDS slot permutation of the eight 16-byte chunks of a key row r: chunk c
// sits at slot c ^ swz(r & 7).  For eight consecutive rows a chunk lands on
// eight distinct slots (K fragment reads, 8 lanes x 16 B per LDS cycle), and
// for keys 4a..4a+3 the chunk pair {2b, 2b+1} lands on four disjoint slot
// pairs (transposing V reads, 16 lanes x 8 B).
__device__ __forceinline__ int swz(int x) { return ((x & 3) << 1) | ((x >> 2) & 1); }

// 16 bytes per lane from base + voff into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

// 16 bytes per lane from the 64-bit address addr into LDS at lds_addr + 16 * lane.
__device__ __forceinline__ void dma16_at(const char* addr, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(addr), "{m0}"(lds_addr) : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
// The direct-to-LDS loads are not known to the compiler, so their waits are
// explicit; loads complete in order, so the count is exact.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Transposing LDS read: within each 16-lane group, lane j receives element
// j % 4 of the 8-byte chunks addressed by lanes 4i + j/4, i = 0..3.
__device__ __forceinline__ v4i16 lds_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(
          (__attribute__((address_space(3))) char*)(char*)p));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char*)(const char*)p));
}

// Per-lane LDS byte offsets of the MFMA operands inside a tile.
struct Frag {
  uint32_t kofs[4];   // K: key row col (+32 per m-tile), dims 16s + 8*half..+7
  uint32_t vofs[2];   // V: rows 4g + j/4 (+16 per k-step, +8), dims 32dt + ...
};

// A wave's share of every tile's loads: waves 0-3 fetch K, waves 4-7 V;
// wave w&3 fetches keys 16*(w&3) .. +15 in two loads of 8 keys x 128 B.
struct Dma {
  const char* base;   // pool + head slice (+ page_size rows for V), uniform
  const char* own;    // caller's frame + head slice (K or V buffer), uniform
  int own_tile;       // first tile of the chunk that may hold the caller's rows
  uint32_t dst;       // wave's destination inside a stage, uniform
  uint32_t rm_off;    // lane's key inside a tile
  uint32_t coff;      // lane's source chunk (bytes), chosen by the swizzle
};

// Loads of one tile into a stage.  The staged row map holds byte offsets of
// pool rows (multiples of 128), so the chunk offset is or-ed in.
// OWN: the row map ends with rows of the caller's frame (kOwnRow set), which
// are fetched from its buffers; tiles before d.own_tile hold pool rows only.
template <bool OWN>
__device__ __forceinline__ void issue_tile(const Dma& d, const uint32_t* rm_lds,
                                           uint32_t stage_addr, int tile) {
  const uint32_t o0 = rm_lds[tile * kBN + d.rm_off] | d.coff;
  const uint32_t o1 = rm_lds[tile * kBN + d.rm_off + 8] | d.coff;
  if (!OWN || tile < d.own_tile) {
    dma16(d.base, o0, stage_addr + d.dst);
    dma16(d.base, o1, stage_addr + d.dst + 1024u);
  } else {
    dma16_at(((o0 & kOwnRow) ? d.own : d.base) + (o0 & ~kOwnRow), stage_addr + d.dst);
    dma16_at(((o1 & kOwnRow) ? d.own : d.base) + (o1 & ~kOwnRow), stage_addr + d.dst + 1024u);
  }
}

// MFMA phase: O^T += V^T P^T for the previous tile, then S^T = K Q^T for
// the current one.  All V fragments are requested up front and the K
// fragments after the first half of the PV products, so the wave waits for
// LDS once per phase.
template <int NT, bool PV, bool SC>
__device__ __forceinline__ void mfma_phase(const char* vtile, const char* ktile,
                                           const Frag& f, const bf16x8 (&qf)[2][4],
                                           const bf16x8 (&pf)[2][4],
                                           f32x16 (&o_acc)[2][2], f32x16 (&sc)[2][2]) {
  bf16x8 vf[2][4];
  bf16x8 kf[2][4];
  if (PV) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const char* p = vtile + f.vofs[dt] + 16 * k2 * kRowB;
        const v4i16 lo = lds_tr(p);
        const v4i16 hi = lds_tr(p + 8 * kRowB);
        vf[dt][k2] = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  } else if (SC) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[mt][s] = *reinterpret_cast<const bf16x8*>(ktile + f.kofs[s] + 32 * mt * kRowB);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (PV) {
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o_acc[nt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0][k2], pf[nt][k2],
                                                               o_acc[nt][0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (SC) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          kf[mt][s] = *reinterpret_cast<const bf16x8*>(ktile + f.kofs[s] + 32 * mt * kRowB);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o_acc[nt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1][k2], pf[nt][k2],
                                                               o_acc[nt][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (SC) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][s], qf[nt][s], acc, 0, 0, 0);
        sc[nt][mt] = acc;
      }
  }
}

// p = 2^(s*c - m) of one column tile into bf16 B-operand order (keys
// 8*(lane/32)+j of each 16-key step); returns the lane's partial row sum.
__device__ __forceinline__ float exp_pack(const f32x16 (&x)[2], float c, float mneg,
                                          bf16x8 (&pf)[4]) {
  // The two sums start at the first two p values (not at 0: 0 + p is not
  // folded away, since the compiler cannot know that p is never -0).
  float s0, s1;
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
    const int mt = k2 >> 1, r0 = (k2 & 1) * 8;
    bf16x8 v;
#pragma unroll
    for (int jj = 0; jj < 8; jj += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(x[mt][r0 + jj], c, mneg));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(x[mt][r0 + jj + 1], c, mneg));
      s0 = k2 == 0 && jj == 0 ? p0 : s0 + p0;
      s1 = k2 == 0 && jj == 0 ? p1 : s1 + p1;
      v[jj] = (__bf16)p0;
      v[jj + 1] = (__bf16)p1;
    }
    pf[k2] = v;
  }
  return s0 + s1;
}

// Softmax phase for one tile (c = sm_scale * log2 e, m the column's running
// reference).  Fast path: p = 2^(s*c - m) without taking the tile maximum.
// While every p stays <= 2^16 the reference may lag the true maximum, and a
// lane's partial row sum bounds its p, so a sum above the bound (or inf /
// NaN, as on a column's first tile, where m is -inf) sends that column tile
// down the slow path: take the tile maximum, move the reference there,
// rescale O and l, redo p.
template <int NT>
__device__ __forceinline__ void softmax_tile(f32x16 (&sc)[2][2], int half, int valid,
                                             float c, f32x16 (&o_acc)[2][2],
                                             float (&m_run)[2], float (&l_run)[2],
                                             bf16x8 (&pf)[2][4]) {
  if (valid < kBN) {
    // Keys past the end of the range: register r of m-tile mt holds key
    // 32*mt + (r/4)*8 + 4*half + r%4.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * mt + (r >> 2) * 8 + half * 4 + (r & 3);
          if (key >= valid) sc[nt][mt][r] = -INFINITY;
        }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lsum = exp_pack(sc[nt], c, -m_run[nt], pf[nt]);
    if (__any(!(lsum <= kSumLimit))) {
      float mx = sc[nt][0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[nt][mt][r]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[nt], mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      m_run[nt] = m_new;
      l_run[nt] *= alpha;
      o_acc[nt][0] *= alpha;
      o_acc[nt][1] *= alpha;
      lsum = exp_pack(sc[nt], c, -m_new, pf[nt]);
    }
    l_run[nt] += lsum;
  }
}

// The phases of one wave over the T tiles of a chunk whose row map is staged
// in LDS and whose tiles 0..S-3 are in flight.  Iteration k covers phases 2k and 2k+1, each ended by
// a workgroup barrier.  Group 0 (waves 0-3): [MFMA: PV of tile k-1, scores
// of tile k][softmax of tile k]; group 1 one phase later: [softmax of tile
// k-1][MFMA: PV of tile k-1, scores of tile k].  Tile k occupies its stage
// from phase 2k to 2k+3.  At phase 2k every wave issues its share of tile
// k+S-2 into the stage that tile k-2 left, and before the barrier that ends
// phase 2k+1 it waits for its share of tile k+1.  The first and last
// iterations are peeled so that the loop body has one MFMA shape.
template <int NT, int GROUP, bool OWN>
__device__ __forceinline__ void chunk_phases(
    const Dma& d, const uint32_t* rm_lds, const char* lds, uint32_t lds_addr, int T,
    int last_valid, const Frag& f, int half, float c, const bf16x8 (&qf)[2][4],
    f32x16 (&o_acc)[2][2], float (&m_run)[2], float (&l_run)[2]) {
  f32x16 sc[2][2];
  bf16x8 pf[2][4];
  auto kt = [&](int k) { return lds + (k % kStages) * kStageB; };
  auto vt = [&](int k) { return lds + (k % kStages) * kStageB + kTileB; };
  auto issue = [&](int k) {
    const int nxt = k + kStages - 2;
    if (nxt < T) issue_tile<OWN>(d, rm_lds, lds_addr + (nxt % kStages) * kStageB, nxt);
  };
  auto wait = [&](int k) {
    if (k + kStages - 2 < T) wait_vm<2 * (kStages - 3)>();
    else wait_vm<0>();
  };
  // k = 0
  issue(0);
  if (NT > 0 && GROUP == 0) {
    __builtin_amdgcn_s_setprio(1);
    mfma_phase<NT, false, true>(vt(0), kt(0), f, qf, pf, o_acc, sc);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  if (NT > 0) {
    if (GROUP == 0) {
      softmax_tile<NT>(sc, half, T == 1 ? last_valid : kBN, c, o_acc, m_run, l_run, pf);
    } else {
      __builtin_amdgcn_s_setprio(1);
      mfma_phase<NT, false, true>(vt(0), kt(0), f, qf, pf, o_acc, sc);
      __builtin_amdgcn_s_setprio(0);
    }
  }
  wait(0);
  __syncthreads();
  for (int k = 1; k < T; ++k) {
    issue(k);
    if (NT > 0) {
      if (GROUP == 0) {
        __builtin_amdgcn_s_setprio(1);
        mfma_phase<NT, true, true>(vt(k - 1), kt(k), f, qf, pf, o_acc, sc);
        __builtin_amdgcn_s_setprio(0);
      } else {
        softmax_tile<NT>(sc, half, kBN, c, o_acc, m_run, l_run, pf);
      }
    }
    __syncthreads();
    if (NT > 0) {
      if (GROUP == 0) {
        softmax_tile<NT>(sc, half, k == T - 1 ? last_valid : kBN, c, o_acc, m_run, l_run,
                         pf);
      } else {
        __builtin_amdgcn_s_setprio(1);
        mfma_phase<NT, true, true>(vt(k - 1), kt(k), f, qf, pf, o_acc, sc);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait(k);
    __syncthreads();
  }
  // k = T
  if (NT > 0) {
    if (GROUP == 0) {
      __builtin_amdgcn_s_setprio(1);
      mfma_phase<NT, true, false>(vt(T - 1), kt(T), f, qf, pf, o_acc, sc);
      __builtin_amdgcn_s_setprio(0);
    } else {
      softmax_tile<NT>(sc, half, last_valid, c, o_acc, m_run, l_run, pf);
    }
  }
  __syncthreads();
  if (NT > 0 && GROUP == 1) {
    __builtin_amdgcn_s_setprio(1);
    mfma_phase<NT, true, false>(vt(T - 1), kt(T), f, qf, pf, o_acc, sc);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
}

// A wave's whole key range [t_begin, t_end): in chunks whose row map fits in
// LDS (one chunk unless the workspace limits the split count); the pipeline
// drains between chunks, the softmax state carries over.
template <int NT, int GROUP, bool OWN>
__device__ __forceinline__ void run_phases(
    const Dma& d, const uint32_t* rowmap, uint32_t* rm_lds, const char* lds,
    uint32_t lds_addr, int t_begin, int t_end, uint32_t row_bytes, const Frag& f,
    int half, float c, const bf16x8 (&qf)[2][4], f32x16 (&o_acc)[2][2], float (&m_run)[2],
    float (&l_run)[2], int n_cached) {
  for (int c0 = t_begin; c0 < t_end; c0 += kRmMax) {
    Dma dc = d;
    dc.own_tile = n_cached > c0 ? (n_cached - c0) / kBN : 0;
    const int c1 = min(t_end, c0 + kRmMax);
    const int T = (c1 - c0 + kBN - 1) / kBN;
    const int last_valid = c1 - (c0 + (T - 1) * kBN);
    // Row map -> byte offsets (the kOwnRow mark kept); the map is padded
    // past the last token, so reading whole tiles stays inside it.
    const uint32_t* rm = rowmap + c0;
    auto ofs = [&](uint32_t e) { return ((e & ~kOwnRow) * row_bytes) | (e & kOwnRow); };
    for (int i = threadIdx.x * 4; i < T * kBN; i += kThreads * 4) {
      const uint4 r = *reinterpret_cast<const uint4*>(rm + i);
      *reinterpret_cast<uint4*>(rm_lds + i) = make_uint4(ofs(r.x), ofs(r.y), ofs(r.z), ofs(r.w));
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStages - 2; ++u)
      if (u < T) issue_tile<OWN>(dc, rm_lds, lds_addr + u * kStageB, u);
    wait_vm<0>();
    __syncthreads();
    chunk_phases<NT, GROUP, OWN>(dc, rm_lds, lds, lds_addr, T, last_valid, f, half, c, qf,
                            o_acc, m_run, l_run);
  }
}

// The runs of one launch (several only when independent streams are batched):
// run r owns work items [item_end[r-1], item_end[r]); entries past the last
// run repeat the total.
template <int NB>
struct Runs {
  int32_t n_items;
  int32_t item_end[NB];
  int32_t n_qtiles[NB];
  AttnArgs a[NB];
};

// This workgroup's share of a frame copy (see FrameCopy): the chunks
// [part * n / parts, (part + 1) * n / parts), four 16-byte chunks per thread
// in flight, every load of a round issued before its stores.  Nothing in the
// launch reads the destination rows: its row map sends the newest frame's
// tokens to the caller's buffers.
__device__ __forceinline__ void copy_share(const FrameCopy& c, int part, int parts) {
  const int64_t n = 2 * (int64_t(c.n_patch) + c.n_spec);
  const int64_t lo = n * part / parts, hi = n * (part + 1) / parts;
  const uint4* k = reinterpret_cast<const uint4*>(c.k);
  const uint4* v = reinterpret_cast<const uint4*>(c.v);
  uint4* pool = reinterpret_cast<uint4*>(c.pool);
  constexpr int kU = 4;
  for (int64_t base = lo + threadIdx.x; base < hi; base += int64_t(kU) * kThreads) {
    uint4 buf[kU];
    uint4* dst[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      int64_t i = base + int64_t(u) * kThreads;
      i = i < hi ? i : hi - 1;   // past the share: re-read its last chunk, store nothing
      const uint4* src;
      if (i < c.n_patch) {
        src = k + c.n_spec + i;
        dst[u] = pool + c.pk + i;
      } else if (i < 2 * int64_t(c.n_patch)) {
        src = v + c.n_spec + (i - c.n_patch);
        dst[u] = pool + c.pv + (i - c.n_patch);
      } else if (i < 2 * int64_t(c.n_patch) + c.n_spec) {
        src = k + (i - 2 * int64_t(c.n_patch));
        dst[u] = pool + c.sk + (i - 2 * int64_t(c.n_patch));
      } else {
        const int64_t j = i - 2 * int64_t(c.n_patch) - c.n_spec;
        src = v + j;
        dst[u] = pool + c.sv + j;
      }
      buf[u] = *src;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      asm volatile("" : "+v"(buf[u].x), "+v"(buf[u].y), "+v"(buf[u].z), "+v"(buf[u].w));
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (base + int64_t(u) * kThreads < hi) *dst[u] = buf[u];
  }
}

template <bool OWN, int NB>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(const Runs<NB> runs) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageB];
  __shared__ __attribute__((aligned(16))) uint32_t rm_lds[kRmMax];
  // Work item: query tiles of one (head, split) are consecutive items, and a
  // contiguous range of items goes to one XCD.
  const int per_xcd = gridDim.x >> 3;
  int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= runs.n_items) return;
  int ri = 0;
#pragma unroll
  for (int r = 0; r < NB - 1; ++r) ri += item >= runs.item_end[r];
  if (NB > 1 && ri > 0) item -= runs.item_end[ri - 1];
  const AttnArgs& a = runs.a[ri];
  const int n_qtiles = runs.n_qtiles[ri];
  const int qt = item % n_qtiles;
  const int unit = item / n_qtiles;
  const int h = unit % a.num_heads;
  const int split = unit / a.num_heads;
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(a.nk, t_begin + a.tokens_per_split);
  if (t_begin >= t_end) return;  // the launch never makes an empty split
  if (NB == 1 && a.copy.n_patch > 0) copy_share(a.copy, item, runs.n_items);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const size_t hd = size_t(a.num_heads) * kD;
  const uint32_t row_bytes = uint32_t(hd) * 2u;

  Frag f;
  {
    // K: lane (col, half) reads row col, chunk 2s + half.
    const int fk = swz(col & 7);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f.kofs[s] = uint32_t(col * kRowB + (((2 * s + half) ^ fk) * 16));
    // V: in 16-lane group q16, lane j addresses key 4*(q16/2) + j/4 (+16
    // per k-step, +8 for the upper half) and dims 16*(q16&1) + 4*(j&3) of
    // the 32-dim tile dt, i.e. chunk 4dt + 2*(q16&1) + (j>>1 & 1), byte 8*(j&1).
    const int q16 = lane >> 4, j = lane & 15;
    const int r = 4 * (q16 >> 1) + (j >> 2);
    const int fv = swz(r);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      f.vofs[dt] = uint32_t(r * kRowB +
                            (((4 * dt + 2 * (q16 & 1) + ((j >> 1) & 1)) ^ fv) * 16) +
                            (j & 1) * 8);
  }
  Dma d;
  {
    const int kv = wave >> 2, wq = wave & 3;
    d.base = reinterpret_cast<const char*>(a.pool) + size_t(h) * kD * 2 +
             (kv ? size_t(a.page_size) * row_bytes : 0);
    d.own = OWN && a.own_k
                ? reinterpret_cast<const char*>(kv ? a.own_v : a.own_k) + size_t(h) * kD * 2
                : d.base;
    d.own_tile = 0;
    d.dst = uint32_t(kv * kTileB + 16 * wq * kRowB);
    const int r = lane >> 3;
    d.rm_off = uint32_t(16 * wq + r);
    d.coff = uint32_t(((lane & 7) ^ swz(r)) * 16);
  }
  const uint32_t lds_addr = lds_u32(lds);

  // Queries of this wave: rows q0 .. q0+63 of the frame, as Q^T fragments
  // (B operands).
  const int q0 = qt * kBM + wave * 64;
  const int n_active = (q0 < a.nq) + (q0 + 32 < a.nq);
  const float c = a.sm_scale * kLog2e;
  bf16x8 qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = q0 + nt * 32 + col;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[nt][s] = qi < a.nq ? *reinterpret_cast<const bf16x8*>(
                                  a.q + size_t(qi) * hd + size_t(h) * kD + 16 * s + 8 * half)
                            : bf16x8{};
    }
  }
  f32x16 o_acc[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) o_acc[nt][0] = o_acc[nt][1] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  // A run without own rows (a plain run() batched beside a run_own()) never
  // takes the own-row branch: its byte offsets may use the top bit.
  const int n_cached = OWN && a.own_k ? a.n_cached : INT_MAX;
#define SPKV_RUN(NT, G)                                                                \
  run_phases<NT, G, OWN>(d, a.rowmap, rm_lds, lds, lds_addr, t_begin, t_end, row_bytes, f, \
                         half, c, qf, o_acc, m_run, l_run, n_cached)
  if (wave < 4) {
    if (n_active == 2) SPKV_RUN(2, 0);
    else if (n_active == 1) SPKV_RUN(1, 0);
    else SPKV_RUN(0, 0);
  } else {
    if (n_active == 2) SPKV_RUN(2, 1);
    else if (n_active == 1) SPKV_RUN(1, 1);
    else SPKV_RUN(0, 1);
  }
#undef SPKV_RUN

  // Epilogue.  Lane (col, half) holds, for d tile dt and register r,
  // d = 32*dt + (r/4)*8 + half*4 + r%4 of query q0 + 32*nt + col.
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (nt >= n_active) continue;
    const int qi = q0 + nt * 32 + col;
    const float l_tot = l_run[nt] + xor32(l_run[nt]);
    if (qi >= a.nq) continue;
    if (a.splits == 1) {
      const float inv = 1.0f / l_tot;
      uint16_t* dst = a.out + size_t(qi) * hd + size_t(h) * kD;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * dt + rr * 8 + half * 4;
          const __bf16 b0 = (__bf16)(o_acc[nt][dt][4 * rr + 0] * inv);
          const __bf16 b1 = (__bf16)(o_acc[nt][dt][4 * rr + 1] * inv);
          const __bf16 b2 = (__bf16)(o_acc[nt][dt][4 * rr + 2] * inv);
          const __bf16 b3 = (__bf16)(o_acc[nt][dt][4 * rr + 3] * inv);
          uint2 wv;
          wv.x = uint32_t(__builtin_bit_cast(uint16_t, b0)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, b1)) << 16);
          wv.y = uint32_t(__builtin_bit_cast(uint16_t, b2)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, b3)) << 16);
          *reinterpret_cast<uint2*>(dst + d0) = wv;
        }
    } else {
      // This split's O normalised by its own row sum, in bf16, beside its
      // (m, l) in fp32: the merge weighs each split by 2^(m_s - M) l_s.
      const size_t row = (size_t(split) * a.nq + qi) * a.num_heads + h;
      const float inv = 1.0f / l_tot;
      uint16_t* dst = a.part_o + row * kD;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * dt + rr * 8 + half * 4;
          const __bf16 b0 = (__bf16)(o_acc[nt][dt][4 * rr + 0] * inv);
          const __bf16 b1 = (__bf16)(o_acc[nt][dt][4 * rr + 1] * inv);
          const __bf16 b2 = (__bf16)(o_acc[nt][dt][4 * rr + 2] * inv);
          const __bf16 b3 = (__bf16)(o_acc[nt][dt][4 * rr + 3] * inv);
          uint2 wv;
          wv.x = uint32_t(__builtin_bit_cast(uint16_t, b0)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, b1)) << 16);
          wv.y = uint32_t(__builtin_bit_cast(uint16_t, b2)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, b3)) << 16);
          *reinterpret_cast<uint2*>(dst + d0) = wv;
        }
      if (half == 0)
        *reinterpret_cast<float2*>(a.part_ml + row * 2) = make_float2(m_run[nt], l_tot);
    }
  }
}

// Combine the splits of each (query, head): with m the reference (base 2),
// l the sum and O_s / l_s the normalised output of each split,
// O = sum_s 2^(m_s - M) l_s (O_s / l_s) / sum_s 2^(m_s - M) l_s.
// One thread per (query, head, 4 dims).  Splits are read eight at a time with
// all their loads in flight together (this kernel is latency-bound); splits
// past the count re-read the last one and get weight 0.
constexpr int kMergeGroup = 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void merge_row(const uint16_t* __restrict__ part_o,
                                         const float* __restrict__ part_ml,
                                         uint16_t* __restrict__ out, int rows, int splits,
                                         int gid) {
  const int row = gid >> 4;   // (query, head) flattened
  const int d0 = (gid & 15) * 4;
  if (row >= rows) return;
  // One pass: each group's (m, l) and O are loaded together and folded into
  // a running reference, so a row costs one memory round trip per group of
  // splits (one in all launches of up to kMergeGroup splits).
  float mmax = -INFINITY;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kMergeGroup) {
    float2 ml[kMergeGroup];
    uint2 ov[kMergeGroup];
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) {
      const size_t r = size_t(min(s0 + j, splits - 1)) * rows + row;
      ml[j] = *reinterpret_cast<const float2*>(part_ml + r * 2);
      ov[j] = *reinterpret_cast<const uint2*>(part_o + r * kD + d0);
    }
    float gmax = mmax;
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) gmax = fmaxf(gmax, ml[j].x);
    // Every split saw at least one key, so gmax is finite; the first group
    // scales the empty accumulators by 2^-inf = 0.
    const float rescale = __builtin_amdgcn_exp2f(mmax - gmax);
    acc.x *= rescale;
    acc.y *= rescale;
    acc.z *= rescale;
    acc.w *= rescale;
    lsum *= rescale;
    mmax = gmax;
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) {
      const float w =
          s0 + j < splits ? __builtin_amdgcn_exp2f(ml[j].x - mmax) * ml[j].y : 0.f;
      acc.x += w * bf16_lo(ov[j].x);
      acc.y += w * bf16_hi(ov[j].x);
      acc.z += w * bf16_lo(ov[j].y);
      acc.w += w * bf16_hi(ov[j].y);
      lsum += w;
    }
  }
  const float inv = 1.0f / lsum;
  const __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv);
  const __bf16 b2 = (__bf16)(acc.z * inv), b3 = (__bf16)(acc.w * inv);
  uint2 w;
  w.x = uint32_t(__builtin_bit_cast(uint16_t, b0)) |
        (uint32_t(__builtin_bit_cast(uint16_t, b1)) << 16);
  w.y = uint32_t(__builtin_bit_cast(uint16_t, b2)) |
        (uint32_t(__builtin_bit_cast(uint16_t, b3)) << 16);
  *reinterpret_cast<uint2*>(out + size_t(row) * kD + d0) = w;
}

__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    uint16_t* __restrict__ out,
                                                    int rows, int splits) {
  merge_row(part_o, part_ml, out, rows, splits, blockIdx.x * 256 + threadIdx.x);
}

// The split runs of a batched launch: run r owns merge blocks
// [end_block[r-1], end_block[r]); entries past the last run repeat the total.
template <int NB>
struct Merges {
  int32_t end_block[NB];
  int32_t rows[NB], splits[NB];
  const uint16_t* part_o[NB];
  const float* part_ml[NB];
  uint16_t* out[NB];
};

template <int NB>
__global__ __launch_bounds__(256) void merge_batch_kernel(const Merges<NB> m) {
  const int blk = blockIdx.x;
  int r = 0;
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) r += blk >= m.end_block[i];
  const int b0 = r > 0 ? m.end_block[r - 1] : 0;
  merge_row(m.part_o[r], m.part_ml[r], m.out[r], m.rows[r], m.splits[r],
            (blk - b0) * 256 + int(threadIdx.x));
}

}  // namespace

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_expand(const PlanArgs& p, hipStream_t stream) {
  const int n = max(p.n_out, p.n_out_own);
  hipLaunchKernelGGL(expand_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  if (a.tokens_per_split <= 0 || a.tokens_per_split % kBN) return hipErrorInvalidValue;
  Runs<1> r;
  r.n_qtiles[0] = (a.nq + kBM - 1) / kBM;
  r.n_items = r.item_end[0] = r.n_qtiles[0] * a.num_heads * a.splits;
  r.a[0] = a;
  const int grid = (r.n_items + 7) / 8 * 8;
  if (a.own_k)
    hipLaunchKernelGGL((attn_kernel<true, 1>), dim3(grid), dim3(kThreads), 0, stream, r);
  else
    hipLaunchKernelGGL((attn_kernel<false, 1>), dim3(grid), dim3(kThreads), 0, stream, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.splits == 1) return err;
  const int rows = a.nq * a.num_heads;
  const int threads = rows * 16;
  hipLaunchKernelGGL(merge_kernel, dim3((threads + 255) / 256), dim3(256), 0,
                     stream, a.part_o, a.part_ml, a.out, rows, a.splits);
  return hipGetLastError();
}

hipError_t launch_attention_batch(const AttnArgs* runs, int n, hipStream_t stream) {
  if (n < 1 || n > kMaxBatchRuns) return hipErrorInvalidValue;
  if (n == 1) return launch_attention(runs[0], stream);
  constexpr int NB = kMaxBatchRuns;
  Runs<NB> r{};
  Merges<NB> m{};
  bool own = false;
  int items = 0, blocks = 0, n_merge = 0;
  for (int i = 0; i < n; ++i) {
    const AttnArgs& a = runs[i];
    if (a.tokens_per_split <= 0 || a.tokens_per_split % kBN) return hipErrorInvalidValue;
    r.n_qtiles[i] = (a.nq + kBM - 1) / kBM;
    items += r.n_qtiles[i] * a.num_heads * a.splits;
    r.item_end[i] = items;
    r.a[i] = a;
    own = own || a.own_k != nullptr;
    if (a.splits > 1) {
      const int rows = a.nq * a.num_heads;
      blocks += (rows * 16 + 255) / 256;
      m.end_block[n_merge] = blocks;
      m.rows[n_merge] = rows;
      m.splits[n_merge] = a.splits;
      m.part_o[n_merge] = a.part_o;
      m.part_ml[n_merge] = a.part_ml;
      m.out[n_merge] = a.out;
      ++n_merge;
    }
  }
  for (int i = n; i < NB; ++i) {
    r.item_end[i] = items;
    r.n_qtiles[i] = 1;
  }
  for (int i = n_merge; i < NB; ++i) m.end_block[i] = blocks;
  r.n_items = items;
  const int grid = (items + 7) / 8 * 8;
  if (own)
    hipLaunchKernelGGL((attn_kernel<true, NB>), dim3(grid), dim3(kThreads), 0, stream, r);
  else
    hipLaunchKernelGGL((attn_kernel<false, NB>), dim3(grid), dim3(kThreads), 0, stream, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_merge == 0) return err;
  hipLaunchKernelGGL((merge_batch_kernel<NB>), dim3(blocks), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace spkv
