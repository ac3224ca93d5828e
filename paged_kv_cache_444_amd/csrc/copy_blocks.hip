// Whole-block copy for copy-on-write (gfx950).
//
// Sequences that share a prompt reference the same physical blocks; a sequence gets a block of
// its own only where it diverges from the others ("Inference optimization" lesson, Paged
// attention section; vLLM-on-H100 article, PagedAttention section).  Before such a sequence
// writes into a block that others still reference, the caller gives it a fresh block and this
// kernel copies the shared block's K and V there.  The block is copied as raw bytes, every KV
// head at once, so the copy does not depend on the layout inside the block.
//
// A work item is one 16 KB piece of one pool's block in one pair: item i covers piece i % pieces
// of the K block (even i / pieces) or the V block (odd).  Each thread of the workgroup loads four
// 16-byte vectors, all in flight together, then stores them, so every byte of a call is
// requested in one round trip whenever the grid holds all the items.  A pair whose ids fall
// outside the pool is skipped.

#include "copy_blocks.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kPiece = (int64_t)kThreads * kUnroll;  // 16-byte vectors per work item

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksParams p) {
  const int64_t n = p.block_vec16;
  const int64_t pieces = (n + kPiece - 1) / kPiece;
  const int64_t items = 2 * (int64_t)p.num_pairs * pieces;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t half = it / pieces;  // 2*pair + (0: K, 1: V)
    const int64_t base = (it % pieces) * kPiece;
    const int64_t pair = half >> 1;
    const int64_t src = p.mapping[2 * pair];
    const int64_t dst = p.mapping[2 * pair + 1];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) continue;
    uint16_t* pool = (half & 1) ? p.vpool : p.kpool;
    const uint4* from = reinterpret_cast<const uint4*>(pool) + src * n;
    uint4* to = reinterpret_cast<uint4*>(pool) + dst * n;
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = base + u * kThreads + threadIdx.x;
      if (j < n) v[u] = from[j];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = base + u * kThreads + threadIdx.x;
      if (j < n) to[j] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const int64_t pieces = (p.block_vec16 + kPiece - 1) / kPiece;
  const int64_t items = 2 * (int64_t)p.num_pairs * pieces;
  const int grid = (int)(items < 65536 ? items : 65536);
  TraceScope t("copy_blocks", stream);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
