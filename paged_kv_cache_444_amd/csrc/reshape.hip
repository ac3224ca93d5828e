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
//
// A wave takes a patch of 16 consecutive tokens (in input order) by one 32-wide slice of one
// head: lane l moves values 8*(l%4) .. +7 of the slice for token l/4.  When the 16 tokens fill a
// 16-token sub-block in order, as a prefill chunk's do, the wave's K stores cover that slice of
// the sub-block (1 KB) contiguously and each V store instruction writes four whole 32-byte rows
// (16 tokens of one head-dim value).  Other slot patterns (one new token per sequence) are as
// correct, with scattered stores.
//
// FP8 pools keep the same element order with one byte per element: each value is divided by its
// pool's scale (correctly rounded fp32 quotient) and encoded as an OCP E4M3 code, rounding to the
// nearest value with ties to even and saturating at +-448.  K then takes one 8-byte store, V
// eight 1-byte stores.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Thread i of the grid-stride loop: its token, head and first head-dim value, or false when its
// token is past the end.  Waves are numbered (token patch, head, slice) with the slice fastest.
__device__ __forceinline__ bool patch_item(const ReshapeParams& p, int64_t i, int& t, int& h,
                                           int& d0) {
  const int slices = p.head_dim / kSlice;
  const int lane = (int)(i & 63);
  const int64_t w = i >> 6;
  const int sl = (int)(w % slices);
  h = (int)((w / slices) % p.num_kv_heads);
  t = (int)(w / ((int64_t)slices * p.num_kv_heads) * kSub + (lane >> 2));
  d0 = sl * kSlice + 8 * (lane & 3);
  return t < p.num_tokens;
}

// Threads the grid-stride loops cover: 64 per (16-token patch, head, slice).
__host__ __device__ __forceinline__ int64_t patch_threads(const ReshapeParams& p) {
  return ((int64_t)p.num_tokens + kSub - 1) / kSub * p.num_kv_heads * (p.head_dim / kSlice) * 64;
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeParams p) {
  const int D = p.head_dim;
  const int64_t total = patch_threads(p);
  const int64_t pool_slots = p.num_blocks * p.block_size;
  // The stride is a multiple of 64, so i % 64 stays the hardware lane.
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t, h, d0;
    if (!patch_item(p, i, t, h, d0)) continue;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= pool_slots) continue;
    const int64_t blk = slot / p.block_size;
    const int off = (int)(slot % p.block_size);
    const int sb = off / kSub, tt = off % kSub;
    const int64_t src = (int64_t)t * p.token_stride + (int64_t)h * D + d0;
    const uint4 kv = *(const uint4*)(p.key + src);
    const uint4 vv = *(const uint4*)(p.value + src);
    const int64_t tile = ((blk * p.num_kv_heads + h) * p.block_size + (int64_t)sb * kSub) * D;
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

// E4M3 code of y, from the format's fields: sign, 4-bit exponent with bias 7, 3-bit mantissa.
// Magnitudes below 2^-6 are subnormal multiples of 2^-9; larger ones keep the fp32 exponent and
// the top 3 mantissa bits rounded to nearest even (a carry moves into the exponent).  Finite
// magnitudes above 448 saturate to 448 (code 0x7E); NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, y) >> 24) & 0x80u;
  float a = __builtin_fabsf(y);
  if (!(a == a)) return sign | 0x7Fu;
  a = __builtin_fminf(a, 448.f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);  // exact scaling; rint rounds ties to even
  } else {
    const uint32_t u = __builtin_bit_cast(uint32_t, a);
    code = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | code;
}

// Codes of 8 bf16 values (packed in a uint4) divided by `scale`, packed little-endian in a uint2.
__device__ __forceinline__ uint2 quantize8(const uint4& v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t c[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[2 * e] = e4m3_code(__fdiv_rn(__builtin_bit_cast(float, w[e] << 16), scale));
    c[2 * e + 1] = e4m3_code(__fdiv_rn(__builtin_bit_cast(float, w[e] & 0xFFFF0000u), scale));
  }
  return make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                    c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
}

__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ReshapeParams p) {
  const int D = p.head_dim;
  const int64_t total = patch_threads(p);
  const int64_t pool_slots = p.num_blocks * p.block_size;
  uint8_t* kpool = reinterpret_cast<uint8_t*>(p.kpool);
  uint8_t* vpool = reinterpret_cast<uint8_t*>(p.vpool);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t, h, d0;
    if (!patch_item(p, i, t, h, d0)) continue;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= pool_slots) continue;
    const int64_t blk = slot / p.block_size;
    const int off = (int)(slot % p.block_size);
    const int sb = off / kSub, tt = off % kSub;
    const int64_t src = (int64_t)t * p.token_stride + (int64_t)h * D + d0;
    const uint2 kc = quantize8(*(const uint4*)(p.key + src), p.k_scale);
    const uint2 vc = quantize8(*(const uint4*)(p.value + src), p.v_scale);
    const int64_t tile = ((blk * p.num_kv_heads + h) * p.block_size + (int64_t)sb * kSub) * D;
    *(uint2*)(kpool + tile + (d0 / kSlice) * (kSub * kSlice) + tt * kSlice + d0 % kSlice) = kc;
    uint8_t* vdst = vpool + tile + (int64_t)d0 * kSub + tt;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vdst[e * kSub] = (uint8_t)(((e < 4 ? vc.x : vc.y) >> (8 * (e & 3))) & 0xFFu);
  }
}

}  // namespace

hipError_t launch_reshape(const ReshapeParams& p, hipStream_t stream) {
  if (p.head_dim % kSlice != 0) return hipErrorInvalidValue;  // whole 32-wide slices only
  const int64_t total = patch_threads(p);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  TraceScope t("reshape_and_cache", stream);
  if (p.kv_fp8)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
