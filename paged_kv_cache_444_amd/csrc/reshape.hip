// Scatter of new tokens' K/V rows into their cache slots (gfx950).
//
// Blocks fill as tokens arrive ("Serving engine internals" lesson, PagedAttention section): the
// caller resolves each new token's logical position through its block table into a slot
// (physical block * block_size + offset) and this kernel copies the rows there, bit for bit.
//
// One thread moves 8 consecutive head-dim values (16 bytes) of one (token, head).  In the K
// layout those 8 values are contiguous (they sit inside one 32-wide slice), so K is written with
// one 16-byte store; in the V layout consecutive head-dim values are 16 tokens apart, so V is
// written as eight 2-byte stores.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeParams p) {
  const int D = p.head_dim;
  const int chunks = D / 8;
  const int64_t per_token = (int64_t)p.num_kv_heads * chunks;
  const int64_t total = per_token * p.num_tokens;
  const int64_t pool_slots = p.num_blocks * p.block_size;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_token);
    const int rem = (int)(i % per_token);
    const int h = rem / chunks;
    const int c = rem % chunks;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= pool_slots) continue;
    const int64_t blk = slot / p.block_size;
    const int off = (int)(slot % p.block_size);
    const int sb = off / kSub, tt = off % kSub;
    const int64_t src = (int64_t)t * p.token_stride + (int64_t)h * D + 8 * c;
    const uint4 kv = *(const uint4*)(p.key + src);
    const uint4 vv = *(const uint4*)(p.value + src);
    const int64_t tile = ((blk * p.num_kv_heads + h) * p.block_size + (int64_t)sb * kSub) * D;
    const int d0 = 8 * c;
    // K: slice d0/32, token tt, columns d0%32 .. +7
    *(uint4*)(p.kpool + tile + (d0 / kSlice) * (kSub * kSlice) + tt * kSlice + d0 % kSlice) = kv;
    // V: rows d0 .. d0+7, column tt
    uint16_t* vdst = p.vpool + tile + (int64_t)d0 * kSub + tt;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vdst[(2 * e) * kSub] = (uint16_t)(w[e] & 0xFFFFu);
      vdst[(2 * e + 1) * kSub] = (uint16_t)(w[e] >> 16);
    }
  }
}

}  // namespace

hipError_t launch_reshape(const ReshapeParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * (p.head_dim / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  TraceScope t("reshape_and_cache", stream);
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
