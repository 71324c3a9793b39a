// Measurement probes: the sustained bf16 MFMA rate and the shader clock under
// that load, and the HBM copy and read bandwidth.  The BC-250 tuned-GEMM post ("Checking the hardware first") checks
// the machine before tuning: it measures the real clock by comparing a cycle
// counter with a constant-rate counter, and the peak against a register-only
// loop.  These probes give the same two denominators on gfx950; the library's
// products do not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "qgemm.h"

namespace qg {

// Each wave runs `iters` rounds of 8 independent 16x16x32 bf16
// MFMAs (eight accumulator chains) on register operands (no memory traffic in the loop).  Lane 0 of each
// workgroup records the shader cycle counter (s_memtime) and the constant-rate
// counter (s_memrealtime) before and after the loop: clocks[4 b + 0..3] =
// {cycles at start, real time at start, cycles at end, real time at end}.
// The accumulators feed a store guarded by a condition the loop never meets
// (their sum is positive), which keeps the loop from being removed.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  // operands: bf16 pairs of 1/64 and 1/32 (exact; sums stay far from overflow)
  const uint32_t pa = 0x3C803C80u, pb = 0x3D003D00u;
  const u32x4 a = {pa, pa ^ (uint32_t)(lane & 1), pa, pa};
  const u32x4 b = {pb, pb, pb ^ (uint32_t)(lane & 2), pb};
  // eight chains in separate variables (an indexed array of accumulators made
  // the register allocator shuffle them between iterations); distinct
  // starting values keep the chains from being merged
  f32x4 c0 = {1.f, 1.f, 1.f, 1.f}, c1 = {2.f, 2.f, 2.f, 2.f}, c2 = {3.f, 3.f, 3.f, 3.f},
        c3 = {4.f, 4.f, 4.f, 4.f}, c4 = {5.f, 5.f, 5.f, 5.f}, c5 = {6.f, 6.f, 6.f, 6.f},
        c6 = {7.f, 7.f, 7.f, 7.f}, c7 = {8.f, 8.f, 8.f, 8.f};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma16_bf16(a, b, c0);
    c1 = mfma16_bf16(a, b, c1);
    c2 = mfma16_bf16(a, b, c2);
    c3 = mfma16_bf16(a, b, c3);
    c4 = mfma16_bf16(a, b, c4);
    c5 = mfma16_bf16(a, b, c5);
    c6 = mfma16_bf16(a, b, c6);
    c7 = mfma16_bf16(a, b, c7);
  }
  const f32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = t[0] + t[1] + t[2] + t[3];
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    uint64_t* c = clocks + 4 * (int64_t)blockIdx.x;
    c[0] = t0;
    c[1] = r0;
    c[2] = t1;
    c[3] = r1;
  }
  // every term is positive, so a negative sum never happens; the store keeps s live
  if (s < 0.f) clocks[4 * (int64_t)blockIdx.x + 1] = (uint64_t)(-s);
}

hipError_t launch_mfma_probe(int64_t blocks, int iters, uint64_t* clocks, hipStream_t stream) {
  mfma_probe_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(iters, clocks);
  return hipGetLastError();
}

// Bandwidth denominators (the same post measures a large copy and a
// multi-stream add before tuning): a copy and a read-only stream of 16-byte
// lane accesses.  Thread t of a grid of T threads handles the 16-byte chunks
// t, t + T, t + 2T, ...; four of them per loop trip, all loads issued before
// the first use.  The read folds its chunks with XOR and stores only when the
// result equals `key` (never, in practice), which keeps every load live.
__global__ __launch_bounds__(256) void copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t chunks) {
  const int64_t T = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * T < chunks; i += 4 * T) {
    const u32x4 a = src[i], b = src[i + T], c = src[i + 2 * T], d = src[i + 3 * T];
    dst[i] = a;
    dst[i + T] = b;
    dst[i + 2 * T] = c;
    dst[i + 3 * T] = d;
  }
  for (; i < chunks; i += T) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read16_kernel(const u32x4* __restrict__ src, int64_t chunks, uint32_t key,
                                                     uint32_t* __restrict__ sink) {
  const int64_t T = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * T < chunks; i += 4 * T) {
    const u32x4 a = src[i], b = src[i + T], c = src[i + 2 * T], d = src[i + 3 * T];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < chunks; i += T) acc ^= src[i];
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == key) sink[0] = v;
}

// Workgroups of a probe launch: one loop trip (4 chunks per thread) over the
// bytes, at most 16 workgroups per CU (the rest by the grid stride).
static int64_t stream_blocks(int64_t chunks, int64_t blocks) {
  if (blocks > 0) return blocks;
  int64_t b = (chunks + 1023) / 1024;
  return b < 1 ? 1 : (b > 4096 ? 4096 : b);
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int64_t blocks, hipStream_t stream) {
  const int64_t chunks = bytes / 16;
  if (chunks == 0) return hipSuccess;
  copy16_kernel<<<dim3((unsigned)stream_blocks(chunks, blocks)), dim3(256), 0, stream>>>(
      (const u32x4*)src, (u32x4*)dst, chunks);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, int64_t bytes, int64_t blocks, uint32_t key, uint32_t* sink,
                             hipStream_t stream) {
  const int64_t chunks = bytes / 16;
  if (chunks == 0) return hipSuccess;
  read16_kernel<<<dim3((unsigned)stream_blocks(chunks, blocks)), dim3(256), 0, stream>>>((const u32x4*)src,
                                                                                          chunks, key, sink);
  return hipGetLastError();
}

}  // namespace qg
