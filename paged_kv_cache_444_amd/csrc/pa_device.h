// Device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// Tokens per sub-block: the unit in which K/V tiles are laid out inside a physical block.
constexpr int kSub = 16;
// Width of a head-dimension slice in the K layout.
constexpr int kSlice = 32;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowHalfMirror = 0x141;  // lane i of each 8-lane half-row reads lane 7 - i

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl,
                                                               0xF, 0xF, false));
}

// Exchange with the lane 16 positions away inside each 32-lane half (rows 0<->1, 2<->3).
__device__ __forceinline__ float xor16_f32(float x) {
  // ds_swizzle bit-mask mode: and_mask=0x1f, or_mask=0, xor_mask=0x10.
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Sum of two bf16 products added to an fp32 accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Dot product of 8 bf16 pairs packed in two uint4 values, accumulated onto c.
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  c = dot2(a.w, b.w, c);
  return c;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

// Orders LDS traffic between lanes of one wave without a workgroup barrier: LDS operations of a
// wave execute in issue order, so only compiler reordering has to be prevented.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace pa
