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
//  * One workgroup = 4 waves = 256 query rows of one head; each wave owns 64
//    rows as two 32-row column tiles of v_mfma_f32_32x32x16_bf16.
//  * Scores are computed transposed, S^T = K Q^T: a lane then holds one query
//    column and 16 keys per 32x32 tile, so the softmax row max and row sum are
//    in-lane reductions plus one exchange with lane ^ 32.  The same lane
//    layout is exactly the B operand of the second product O^T = V^T P^T, so
//    P never leaves registers; the key order inside each 16-key step is the
//    MFMA output order, and V^T is stored in LDS in that order.
//  * Online softmax in fp32, in base 2 with s*log2(e) folded into one FMA;
//    the running maximum is only raised (and O, l rescaled) when a tile's
//    maximum exceeds it by more than 2^8, a wave-uniform decision, so most
//    tiles skip the rescale.  P is rounded to bf16 for the second product and
//    the row sums are taken from the same rounded values with
//    v_dot2_f32_bf16 (two per instruction); O is rounded to bf16 once.
//  * K/V tiles of 64 tokens are double-buffered in LDS; the next tile's K/V
//    loads and the row ids of the tile after it are in flight while the
//    current tile is computed.
//  * The key range is split across workgroups when the query tiles x heads
//    alone cannot fill 256 CUs; partial (O, m, l) go to the workspace and a
//    merge kernel combines them.  Work items are mapped so that the query
//    tiles sharing one (head, key split) land on the same XCD (workgroups are
//    dealt to the 8 XCDs round-robin), where they share that XCD's L2.
#include "kernels.h"

namespace spkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kBN = kAttnKeyTile;      // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kAttnQueryTile;    // query rows per workgroup
constexpr int kRow = 72;               // LDS row pitch in bf16 (144 B)
constexpr int kTile = kBN * kRow;      // one K or V^T tile in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 headroom before rescaling

// ------------------------------------------------------------- plan expand
__global__ __launch_bounds__(256) void expand_kernel(PlanArgs p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.n_out) return;
  const int tt = min(t, p.nk - 1);
  const int patch_tokens = p.n_patch * p.patch_len;
  int e, o;
  if (tt < patch_tokens) {
    e = tt / p.patch_len;
    o = tt - e * p.patch_len;
  } else {
    const int u = tt - patch_tokens;
    const int k = u / p.special_len;
    e = p.n_patch + k;
    o = u - k * p.special_len;
  }
  p.rowmap[t] = static_cast<uint32_t>(p.table[e]) * 2u *
                    static_cast<uint32_t>(p.page_size) +
                static_cast<uint32_t>(o);
}

// ---------------------------------------------------------------- attention
// Swap bits 2 and 3 of a key index: the order in which one 16-key step of
// the MFMA output holds its keys (see the file comment).
__device__ __forceinline__ int key_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

struct TileRegs {
  uint2 k[4];
  uint2 v[4];
};

// Each thread fetches 4 consecutive tokens x 4 dims (8 bytes) of K and of V.
// A wave covers 16 tokens x 128 B per load: full 128-byte rows.  Offsets are
// 32-bit byte offsets from uniform bases (a block's pool is below 4 GiB).
__device__ __forceinline__ void load_tile(const char* __restrict__ kbase,
                                          const char* __restrict__ vbase,
                                          uint4 rid, uint32_t row_bytes,
                                          uint32_t col_bytes, TileRegs& r) {
  const uint32_t ids[4] = {rid.x, rid.y, rid.z, rid.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = ids[i] * row_bytes + col_bytes;
    r.k[i] = *reinterpret_cast<const uint2*>(kbase + off);
    r.v[i] = *reinterpret_cast<const uint2*>(vbase + off);
  }
}

// K rows as they are; V transposed to V^T[d][key_pos(key)] so that one lane's
// 8 keys of an MFMA step are one 16-byte LDS read.
__device__ __forceinline__ void store_tile(uint16_t* ks, uint16_t* vt, int q4,
                                           int c, const TileRegs& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint2*>(ks + (4 * q4 + i) * kRow + 4 * c) = r.k[i];
  // 4x4 transpose of 16-bit values: column j of the 4 rows.
  const int pos = key_pos(4 * q4);
  const uint32_t lo0 = r.v[0].x, lo1 = r.v[1].x, lo2 = r.v[2].x, lo3 = r.v[3].x;
  const uint32_t hi0 = r.v[0].y, hi1 = r.v[1].y, hi2 = r.v[2].y, hi3 = r.v[3].y;
  uint2 col[4];
  col[0] = make_uint2(__builtin_amdgcn_perm(lo1, lo0, 0x05040100u),
                      __builtin_amdgcn_perm(lo3, lo2, 0x05040100u));
  col[1] = make_uint2(__builtin_amdgcn_perm(lo1, lo0, 0x07060302u),
                      __builtin_amdgcn_perm(lo3, lo2, 0x07060302u));
  col[2] = make_uint2(__builtin_amdgcn_perm(hi1, hi0, 0x05040100u),
                      __builtin_amdgcn_perm(hi3, hi2, 0x05040100u));
  col[3] = make_uint2(__builtin_amdgcn_perm(hi1, hi0, 0x07060302u),
                      __builtin_amdgcn_perm(hi3, hi2, 0x07060302u));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(vt + (4 * c + j) * kRow + pos) = col[j];
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// One 64-key tile for the wave's NT active 32-query column tiles.
template <int NT>
__device__ __forceinline__ void compute_tile(
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vt,
    const bf16x8 (&qf)[2][4], f32x16 (&o_acc)[2][2], float (&m_run)[2],
    float (&l_run)[2], int valid, float c2, int col, int half) {
  // S^T = K Q^T for the tile's two 32-key m-tiles.
  bf16x8 kf[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kf[mt][s] = lds_frag(ks + (32 * mt + col) * kRow + 16 * s + 8 * half);
  f32x16 sc[NT][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][s], qf[nt][s], acc,
                                                      0, 0, 0);
      sc[nt][mt] = acc;
    }

  if (valid < kBN) {
    // Keys past the end of the range: lane holds key
    // 32*mt + (r/4)*8 + half*4 + r%4 in register r.
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

  bf16x8 pf[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mx = sc[nt][0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[nt][mt][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_tile = mx * c2;
    // Raise the running maximum only when this tile would overflow the
    // slack; the decision is per wave so the branch is uniform.
    if (__any(m_tile > m_run[nt] + kRescaleSlack)) {
      const float m_new = fmaxf(m_run[nt], m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      m_run[nt] = m_new;
      l_run[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) o_acc[nt][dt] *= alpha;
    }
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const float mneg = -m_run[nt];
    float lsum = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int mt = k2 >> 1, r0 = (k2 & 1) * 8;
      bf16x8 v;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[nt][mt][r0 + j], c2, mneg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[nt][mt][r0 + j + 1], c2, mneg));
        bf16x2 pk;
        pk[0] = (__bf16)p0;
        pk[1] = (__bf16)p1;
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, lsum, false);
        v[j] = pk[0];
        v[j + 1] = pk[1];
      }
      pf[nt][k2] = v;
    }
    l_run[nt] += lsum;
  }

  // O^T += V^T P^T.
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    bf16x8 vf[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
      vf[k2] = lds_frag(vt + (32 * dt + col) * kRow + 16 * k2 + 8 * half);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o_acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vf[k2], pf[nt][k2], o_acc[nt][dt], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a,
                                                           int n_qtiles,
                                                           int n_items) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kTile];

  // Work item: query tiles of one (head, split) are consecutive items, and a
  // contiguous range of items goes to one XCD.
  const int per_xcd = gridDim.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= n_items) return;
  const int qt = item % n_qtiles;
  const int unit = item / n_qtiles;
  const int h = unit % a.num_heads;
  const int split = unit / a.num_heads;

  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(a.nk, t_begin + a.tokens_per_split);
  const int n_tiles = (t_end - t_begin + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column inside a 32-wide tile
  const int half = lane >> 5;  // which 8-element k group / 4-row group

  // Loader role: tokens 4*q4..4*q4+3 of each tile, dims 4*c..4*c+3.
  const int q4 = tid >> 4;
  const int c = tid & 15;
  const size_t hd = size_t(a.num_heads) * kD;
  const uint32_t row_bytes = uint32_t(hd) * 2u;
  const uint32_t col_bytes = uint32_t(c) * 8u;
  const char* kbase = reinterpret_cast<const char*>(a.pool) + size_t(h) * kD * 2;
  const char* vbase = kbase + size_t(a.page_size) * row_bytes;
  const uint32_t* rm = a.rowmap + t_begin + 4 * q4;

  // Queries of this wave; Q^T fragments as MFMA B operands.
  const int q0 = qt * kBM + wave * 64;
  const int n_active = (q0 < a.nq) + (q0 + 32 < a.nq);
  bf16x8 qf[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = q0 + nt * 32 + col;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (qi < a.nq) {
        qf[nt][s] = *reinterpret_cast<const bf16x8*>(
            a.q + size_t(qi) * hd + size_t(h) * kD + 16 * s + 8 * half);
      } else {
        qf[nt][s] = bf16x8{};
      }
    }
  }

  f32x16 o_acc[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) o_acc[nt][dt] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float c2 = a.sm_scale * kLog2e;

  // Prologue: tile 0 into LDS, row ids of tile 1 in registers.  The row map
  // is padded past the last token, so these reads stay inside it.
  TileRegs regs;
  uint4 rid = *reinterpret_cast<const uint4*>(rm);
  load_tile(kbase, vbase, rid, row_bytes, col_bytes, regs);
  rid = *reinterpret_cast<const uint4*>(rm + kBN);
  store_tile(lds, lds + kTile, q4, c, regs);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const uint16_t* ks = lds + buf * 2 * kTile;
    const uint16_t* vt = ks + kTile;
    const bool more = it + 1 < n_tiles;
    if (more) {
      load_tile(kbase, vbase, rid, row_bytes, col_bytes, regs);
      rid = *reinterpret_cast<const uint4*>(rm + (it + 2) * kBN);
    }

    const int valid = t_end - (t_begin + it * kBN);  // < kBN on the last tile
    if (n_active == 2) {
      compute_tile<2>(ks, vt, qf, o_acc, m_run, l_run, valid, c2, col, half);
    } else if (n_active == 1) {
      compute_tile<1>(ks, vt, qf, o_acc, m_run, l_run, valid, c2, col, half);
    }

    if (more) {
      uint16_t* nks = lds + (buf ^ 1) * 2 * kTile;
      store_tile(nks, nks + kTile, q4, c, regs);
    }
    __syncthreads();
  }

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
          __bf16 b0 = (__bf16)(o_acc[nt][dt][4 * rr + 0] * inv);
          __bf16 b1 = (__bf16)(o_acc[nt][dt][4 * rr + 1] * inv);
          __bf16 b2 = (__bf16)(o_acc[nt][dt][4 * rr + 2] * inv);
          __bf16 b3 = (__bf16)(o_acc[nt][dt][4 * rr + 3] * inv);
          uint2 w;
          w.x = uint32_t(__builtin_bit_cast(uint16_t, b0)) |
                (uint32_t(__builtin_bit_cast(uint16_t, b1)) << 16);
          w.y = uint32_t(__builtin_bit_cast(uint16_t, b2)) |
                (uint32_t(__builtin_bit_cast(uint16_t, b3)) << 16);
          *reinterpret_cast<uint2*>(dst + d0) = w;
        }
    } else {
      const size_t row = (size_t(split) * a.nq + qi) * a.num_heads + h;
      float* dst = a.part_o + row * kD;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * dt + rr * 8 + half * 4;
          *reinterpret_cast<float4*>(dst + d0) =
              make_float4(o_acc[nt][dt][4 * rr + 0], o_acc[nt][dt][4 * rr + 1],
                          o_acc[nt][dt][4 * rr + 2], o_acc[nt][dt][4 * rr + 3]);
        }
      if (half == 0)
        *reinterpret_cast<float2*>(a.part_ml + row * 2) =
            make_float2(m_run[nt], l_tot);
    }
  }
}

// Combine the splits of each (query, head): with m the running maxima (base
// 2) and l the sums of each split, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (query, head, 4 dims).
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    uint16_t* __restrict__ out,
                                                    int rows, int splits) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid >> 4;   // (query, head) flattened
  const int d0 = (gid & 15) * 4;
  if (row >= rows) return;
  float mmax = -INFINITY;
  for (int s = 0; s < splits; ++s)
    mmax = fmaxf(mmax, part_ml[(size_t(s) * rows + row) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const size_t r = size_t(s) * rows + row;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + r * 2);
    const float w = __builtin_amdgcn_exp2f(ml.x - mmax);
    const float4 ov = *reinterpret_cast<const float4*>(part_o + r * kD + d0);
    acc.x += w * ov.x;
    acc.y += w * ov.y;
    acc.z += w * ov.z;
    acc.w += w * ov.w;
    lsum += w * ml.y;
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

}  // namespace

hipError_t launch_expand(const PlanArgs& p, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kernel, dim3((p.n_out + 255) / 256), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.nq + kBM - 1) / kBM;
  const int n_items = n_qtiles * a.num_heads * a.splits;
  const int grid = (n_items + 7) / 8 * 8;
  hipLaunchKernelGGL(attn_kernel, dim3(grid), dim3(kThreads), 0, stream, a,
                     n_qtiles, n_items);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.splits == 1) return err;
  const int rows = a.nq * a.num_heads;
  const int threads = rows * 16;
  hipLaunchKernelGGL(merge_kernel, dim3((threads + 255) / 256), dim3(256), 0,
                     stream, a.part_o, a.part_ml, a.out, rows, a.splits);
  return hipGetLastError();
}

}  // namespace spkv
