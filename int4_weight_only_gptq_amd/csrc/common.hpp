// Shared device-side definitions for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;     // rows of k sharing one scale and zero
constexpr int kWave = 64;       // CDNA wavefront

// bf16 bit pattern of 1.0 in both halves of a dword.
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;
// bf16 bit pattern of 128.0; OR-ing a 4-bit code q into its low mantissa bits
// gives the bf16 value 128 + q exactly (the ulp of [128, 256) is 1).
constexpr uint32_t kBias128x2 = 0x43004300u;

// Four dwords holding the eight codes of one qweight word as bf16 pairs
// (128 + q_t, 128 + q_{t+4}), t = 0..3.  The k order inside the MFMA operand is
// therefore 0,4,1,5,2,6,3,7; the activation operand uses the same order
// (see x_pairs_permuted), so the contraction over k is unchanged.
//
// The mask and the bias are passed through an empty asm so that they sit in
// VGPRs: a VOP3 instruction takes no literal on gfx9, and with both as
// literals the compiler emits an AND and an OR per dword instead of one
// v_and_or_b32.  (No instruction is written in asm: the compiler's hazard
// tracking does not see inside asm, and an asm VALU write can race an MFMA
// still writing the same register.)
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32x4 codes_as_bf16_pairs(uint32_t w) {
  const uint32_t mask = in_vgpr(0x000F000Fu), bias = in_vgpr(kBias128x2);
  u32x4 r;
  r[0] = (w & mask) | bias;
  r[1] = ((w >> 4) & mask) | bias;
  r[2] = ((w >> 8) & mask) | bias;
  r[3] = ((w >> 12) & mask) | bias;
  return r;
}

// Eight consecutive bf16 activations (four dwords, x0..x7) reordered to the
// pairs (x_t, x_{t+4}), t = 0..3, matching codes_as_bf16_pairs.
__device__ __forceinline__ u32x4 x_pairs_permuted(u32x4 d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// fp32 16x16x4 MFMA: lane l gives A[l % 16][l / 16] and B[l / 16][l % 16].
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum of a value over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48), using the gfx950 row-swap permutes; every lane gets the total.
__device__ __forceinline__ float sum_over_rows(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  float s = __builtin_bit_cast(float, (uint32_t)p32[0]) + __builtin_bit_cast(float, (uint32_t)p32[1]);
  uint32_t us = __builtin_bit_cast(uint32_t, s);
  auto p16 = __builtin_amdgcn_permlane16_swap(us, us, false, false);
  return __builtin_bit_cast(float, (uint32_t)p16[0]) + __builtin_bit_cast(float, (uint32_t)p16[1]);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and ignores the other counters (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Slot of 16-byte chunk c (8 bf16 of k) of row r in a K-contiguous LDS tile of
// 8 chunks per row: the XOR spreads the 16 rows one MFMA operand read touches
// over distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return 8 * r + (c ^ (r & 7)); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every direct global->LDS load in flight).  The empty asm with a
// memory clobber keeps the compiler from moving LDS reads or writes across it:
// the s_barrier builtin itself is not a memory operation to the compiler.
// Visibility of another wave's direct loads is the caller's job: each wave
// waits for its own loads (vmcnt) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS copy through a raw buffer resource on `base`: 16 or 4
// bytes per lane from base + voff into lds + lane * bytes (lds is the wave's
// base slot; the hardware adds the lane offset).  The resource covers 2^32 - 1
// bytes from base, so voff must stay below 4 GiB; the resource is formed in
// SGPRs from a wave-uniform base.  The bodies exist only in the device pass:
// the host pass cannot form buffer resources or address-space-3 pointers.
__device__ __forceinline__ void buffer_to_lds16(const void* base, uint32_t voff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                           (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ void buffer_to_lds4(const void* base, uint32_t voff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                           (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
#endif
}

}  // namespace qg
