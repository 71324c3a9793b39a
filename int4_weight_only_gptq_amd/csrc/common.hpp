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

// With the mask and bias already in VGPRs (see codes_as_bf16_pairs below).
__device__ __forceinline__ u32x4 codes_as_bf16_pairs_mb(uint32_t w, uint32_t mask, uint32_t bias) {
  u32x4 r;
  r[0] = (w & mask) | bias;
  r[1] = ((w >> 4) & mask) | bias;
  r[2] = ((w >> 8) & mask) | bias;
  r[3] = ((w >> 12) & mask) | bias;
  return r;
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

// s_waitcnt vmcnt(n) for an n that is a constant only after unrolling (the
// builtin wants a literal): the switch folds to the one wait.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vmcnt_imm(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vmcnt_imm(14)); break;
    case 15: __builtin_amdgcn_s_waitcnt(vmcnt_imm(15)); break;
    case 16: __builtin_amdgcn_s_waitcnt(vmcnt_imm(16)); break;
    case 17: __builtin_amdgcn_s_waitcnt(vmcnt_imm(17)); break;
    case 18: __builtin_amdgcn_s_waitcnt(vmcnt_imm(18)); break;
    case 19: __builtin_amdgcn_s_waitcnt(vmcnt_imm(19)); break;
    case 20: __builtin_amdgcn_s_waitcnt(vmcnt_imm(20)); break;
    case 21: __builtin_amdgcn_s_waitcnt(vmcnt_imm(21)); break;
    case 22: __builtin_amdgcn_s_waitcnt(vmcnt_imm(22)); break;
    case 23: __builtin_amdgcn_s_waitcnt(vmcnt_imm(23)); break;
    case 24: __builtin_amdgcn_s_waitcnt(vmcnt_imm(24)); break;
    case 25: __builtin_amdgcn_s_waitcnt(vmcnt_imm(25)); break;
    case 26: __builtin_amdgcn_s_waitcnt(vmcnt_imm(26)); break;
    case 27: __builtin_amdgcn_s_waitcnt(vmcnt_imm(27)); break;
    case 28: __builtin_amdgcn_s_waitcnt(vmcnt_imm(28)); break;
    case 29: __builtin_amdgcn_s_waitcnt(vmcnt_imm(29)); break;
    case 30: __builtin_amdgcn_s_waitcnt(vmcnt_imm(30)); break;
    case 31: __builtin_amdgcn_s_waitcnt(vmcnt_imm(31)); break;
    case 32: __builtin_amdgcn_s_waitcnt(vmcnt_imm(32)); break;
    case 33: __builtin_amdgcn_s_waitcnt(vmcnt_imm(33)); break;
    case 34: __builtin_amdgcn_s_waitcnt(vmcnt_imm(34)); break;
    case 35: __builtin_amdgcn_s_waitcnt(vmcnt_imm(35)); break;
    case 36: __builtin_amdgcn_s_waitcnt(vmcnt_imm(36)); break;
    case 37: __builtin_amdgcn_s_waitcnt(vmcnt_imm(37)); break;
    case 38: __builtin_amdgcn_s_waitcnt(vmcnt_imm(38)); break;
    case 39: __builtin_amdgcn_s_waitcnt(vmcnt_imm(39)); break;
    case 40: __builtin_amdgcn_s_waitcnt(vmcnt_imm(40)); break;
    case 41: __builtin_amdgcn_s_waitcnt(vmcnt_imm(41)); break;
    case 42: __builtin_amdgcn_s_waitcnt(vmcnt_imm(42)); break;
    case 43: __builtin_amdgcn_s_waitcnt(vmcnt_imm(43)); break;
    case 44: __builtin_amdgcn_s_waitcnt(vmcnt_imm(44)); break;
    case 45: __builtin_amdgcn_s_waitcnt(vmcnt_imm(45)); break;
    case 46: __builtin_amdgcn_s_waitcnt(vmcnt_imm(46)); break;
    case 47: __builtin_amdgcn_s_waitcnt(vmcnt_imm(47)); break;
    case 48: __builtin_amdgcn_s_waitcnt(vmcnt_imm(48)); break;
    case 49: __builtin_amdgcn_s_waitcnt(vmcnt_imm(49)); break;
    case 50: __builtin_amdgcn_s_waitcnt(vmcnt_imm(50)); break;
    case 51: __builtin_amdgcn_s_waitcnt(vmcnt_imm(51)); break;
    case 52: __builtin_amdgcn_s_waitcnt(vmcnt_imm(52)); break;
    case 53: __builtin_amdgcn_s_waitcnt(vmcnt_imm(53)); break;
    case 54: __builtin_amdgcn_s_waitcnt(vmcnt_imm(54)); break;
    case 55: __builtin_amdgcn_s_waitcnt(vmcnt_imm(55)); break;
    case 56: __builtin_amdgcn_s_waitcnt(vmcnt_imm(56)); break;
    case 57: __builtin_amdgcn_s_waitcnt(vmcnt_imm(57)); break;
    case 58: __builtin_amdgcn_s_waitcnt(vmcnt_imm(58)); break;
    case 59: __builtin_amdgcn_s_waitcnt(vmcnt_imm(59)); break;
    case 60: __builtin_amdgcn_s_waitcnt(vmcnt_imm(60)); break;
    case 61: __builtin_amdgcn_s_waitcnt(vmcnt_imm(61)); break;
    case 62: __builtin_amdgcn_s_waitcnt(vmcnt_imm(62)); break;
    case 63: __builtin_amdgcn_s_waitcnt(vmcnt_imm(63)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(63)); break;
  }
}

// Slot of 16-byte chunk c (8 bf16 of k) of row r in a K-contiguous LDS tile of
// 8 chunks per row: the XOR spreads the 16 rows one MFMA operand read touches
// over distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return 8 * r + (c ^ (r & 7)); }

// One ticket of a k split's counter (agent scope); returns the count before.
// acq_rel != 0: an acquire-release increment (the memory model orders the
// slice's partial stores before it and the last slice's reads after it);
// else relaxed, the partials' order then resting on the store-completion wait
// before the increment.
__device__ __forceinline__ uint32_t ticket_add(uint32_t* t, int acq_rel) {
  return acq_rel ? __hip_atomic_fetch_add(t, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT)
                 : __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Loads through a raw buffer resource on a wave-uniform base (SGPRs) with a
// 32-bit per-lane byte offset (below 4 GiB): the lane offset register can
// serve many loads whose bases differ only in the uniform part.
__device__ __forceinline__ u32x4 buffer_load16(const void* base, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b128(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                               voff, 0, 0);
#else
  return u32x4{0u, 0u, 0u, 0u};
#endif
}

__device__ __forceinline__ u32x2 buffer_load8(const void* base, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b64(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                              voff, 0, 0);
#else
  return u32x2{0u, 0u};
#endif
}

__device__ __forceinline__ uint32_t buffer_load4(const void* base, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b32(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                              voff, 0, 0);
#else
  return 0u;
#endif
}

__device__ __forceinline__ uint32_t buffer_load2(const void* base, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b16(__builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, -1, 0x00020000),
                                              voff, 0, 0);
#else
  return 0u;
#endif
}

}  // namespace qg
