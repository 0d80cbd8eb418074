// append_frame's device half: scatter one frame's K and V into the block's
// pages (gfx950).
//
// "How LingBot-Map Implements the KV Cache Mechanism ...", section "Physical
// Page Layout and Indexing": the pool is [pages][2][page_size][H][D] with
// K at index 0 and V at index 1.  One frame is [specials..., patches...] x H
// x D.  Its patch rows are one contiguous run of the source and land as one
// contiguous run at the start of the patch page; its special rows likewise
// land at the frame's slot of the special page.  So the whole append is four
// contiguous copies (K patch, V patch, K special, V special), done by one
// launch with 16-byte loads and stores spread over the whole chip, every
// load of a thread issued before its stores.
#include "kernels.h"

namespace spkv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerThread = 4;  // 64 B in flight per thread

struct alignas(16) Chunk {
  uint32_t w[4];
};

// Source and destination of chunk i of the append's index space:
// [0, n_patch) K patch, [n_patch, 2 n_patch) V patch, then n_spec K special
// chunks and n_spec V special chunks.
__device__ __forceinline__ void locate(int64_t i, const Chunk* k, const Chunk* v, Chunk* pool,
                                       int64_t pk, int64_t pv, int64_t sk, int64_t sv,
                                       int64_t n_patch, int64_t n_spec, const Chunk*& src,
                                       Chunk*& dst) {
  if (i < n_patch) {
    src = k + n_spec + i;
    dst = pool + pk + i;
  } else if (i < 2 * n_patch) {
    const int64_t j = i - n_patch;
    src = v + n_spec + j;
    dst = pool + pv + j;
  } else if (i < 2 * n_patch + n_spec) {
    const int64_t j = i - 2 * n_patch;
    src = k + j;
    dst = pool + sk + j;
  } else {
    const int64_t j = i - 2 * n_patch - n_spec;
    src = v + j;
    dst = pool + sv + j;
  }
}

// A block copies kThreads * kChunksPerThread consecutive chunks; a thread
// issues all of its loads before its first store, so that every load of the
// launch is in flight at once (a frame is a few MB: the copy is bound by
// memory latency, not by bandwidth, unless the loads overlap).
__global__ __launch_bounds__(kThreads) void append_kernel(
    const Chunk* __restrict__ k, const Chunk* __restrict__ v,
    Chunk* __restrict__ pool, int64_t pk, int64_t pv, int64_t sk, int64_t sv,
    int64_t n_patch, int64_t n_spec) {
  const int64_t total = 2 * (n_patch + n_spec);
  const int64_t base = int64_t(blockIdx.x) * (kThreads * kChunksPerThread) + threadIdx.x;
  Chunk buf[kChunksPerThread];
  Chunk* dst[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int64_t i = base + int64_t(u) * kThreads;
    const Chunk* src;
    // Chunks past the end re-read the last one and store nothing.
    locate(i < total ? i : total - 1, k, v, pool, pk, pv, sk, sv, n_patch, n_spec, src,
           dst[u]);
    buf[u] = *src;
  }
  // Keep the loads ahead of the stores: without this the compiler sinks each
  // load into its store's branch, one round trip per chunk.
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u)
    asm volatile("" : "+v"(buf[u].w[0]), "+v"(buf[u].w[1]), "+v"(buf[u].w[2]),
                 "+v"(buf[u].w[3]));
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u)
    if (base + int64_t(u) * kThreads < total) *dst[u] = buf[u];
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  // 8 bf16 per 16-byte chunk; run lengths are multiples of H*D, and
  // H*D % 8 == 0 is checked at create().
  const int64_t n_patch = a.patch_elems / 8;
  const int64_t n_spec = a.special_elems / 8;
  const int64_t total = 2 * (n_patch + n_spec);
  const int64_t per_block = int64_t(kThreads) * kChunksPerThread;
  const int64_t blocks = (total + per_block - 1) / per_block;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream,
                     static_cast<const Chunk*>(a.k),
                     static_cast<const Chunk*>(a.v),
                     static_cast<Chunk*>(a.pool), a.patch_k_off / 8,
                     a.patch_v_off / 8, a.special_k_off / 8,
                     a.special_v_off / 8, n_patch, n_spec);
  return hipGetLastError();
}

}  // namespace spkv
