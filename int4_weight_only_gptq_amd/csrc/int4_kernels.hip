// int4 GPTQ kernels for gfx950: dequant, the m = 1 GEMV, the fused small-M
// kernel and the pipelined MFMA kernel for larger m.
//
// Storage (GPTQ-Int4, group size 128): qweight uint32 [k/8][n] with row 8r+t
// of column j in bits 4t..4t+3 of word (r, j); qzeros uint32 [k/128][n/8] with
// column 8c+t in bits 4t..4t+3 of word (g, c); scales fp16 [k/128][n].
// Weight: w = (q - z) * s.
//
// All three product kernels contract the activations with the exact bf16
// values 128 + q (codes_as_bf16_pairs) and correct the offset per group with
// the group sum of the activations:
//   sum_i x_i (q_i - z) = sum_i x_i (128 + q_i) - (128 + z) sum_i x_i,
// then scale by s in fp32 once per 128-row group.  Nothing is rounded below
// fp32 before the scale is applied.
#include <stdio.h>

#include "common.hpp"
#include "launch.hpp"

namespace qg {

// ---------------------------------------------------------------------------
// dequant: w[i][j] = (float)(q - z) * s, fp32 [k][n]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ qzeros,
                                                      float* __restrict__ w, int64_t n, int64_t k) {
  const int64_t quads = n >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = idx / quads;
  if (r >= (k >> 3)) return;
  const int64_t col = (idx - r * quads) << 2;
  const u32x4 words = *reinterpret_cast<const u32x4*>(qweight + r * n + col);
  const int64_t g = r >> 4;
  const uint32_t zw = qzeros ? qzeros[g * (n >> 3) + (col >> 3)] >> ((col & 7) * 4) : 0u;   // none: z = 0
  const u32x2 sw = *reinterpret_cast<const u32x2*>(scales + g * n + col);
  float s[4] = {half_bits_to_float(sw[0] & 0xFFFFu), half_bits_to_float(sw[0] >> 16),
                half_bits_to_float(sw[1] & 0xFFFFu), half_bits_to_float(sw[1] >> 16)};
  int z[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) z[c] = (int)((zw >> (4 * c)) & 15u);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = (float)((int)((words[c] >> (4 * t)) & 15u) - z[c]) * s[c];
    *reinterpret_cast<f32x4*>(w + (8 * r + t) * n + col) = o;
  }
}

hipError_t launch_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros,
                          float* w, int64_t n, int64_t k, hipStream_t stream) {
  const int64_t threads = (k / 8) * (n / 4);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(qweight, scales, qzeros, w, n, k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// helpers shared by the product kernels
// ---------------------------------------------------------------------------
template <int CPL>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[CPL]) {
  if constexpr (CPL == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p), u = *reinterpret_cast<const u32x4*>(p + 4);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    w[4] = u[0]; w[5] = u[1]; w[6] = u[2]; w[7] = u[3];
  } else if constexpr (CPL == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (CPL == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = *p;
  }
}

// Raw group metadata of CPL consecutive columns: their fp16 scales and the
// word holding their zero nibbles.  Loaded in the load phase and decoded only
// where it is used, so the loads do not force an early wait on everything in
// flight.
template <int CPL>
struct Meta {
  uint32_t s[CPL >= 4 ? CPL / 2 : 1];
  uint32_t z;
};

template <int CPL>
__device__ __forceinline__ Meta<CPL> load_meta(const uint16_t* __restrict__ sp, const uint32_t* __restrict__ zp) {
  Meta<CPL> r;
  if constexpr (CPL == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(sp);
    r.s[0] = v[0];
    r.s[1] = v[1];
    r.s[2] = v[2];
    r.s[3] = v[3];
  } else if constexpr (CPL == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
    r.s[0] = v[0];
    r.s[1] = v[1];
  } else if constexpr (CPL == 2) {
    r.s[0] = *reinterpret_cast<const uint32_t*>(sp);
  } else {
    r.s[0] = *sp;
  }
  r.z = *zp;
  return r;
}

// zshift = 4 * (col % 8): the nibble of the first of the CPL columns; zmask = 0
// without a zero point (z = 0).
template <int CPL>
__device__ __forceinline__ void decode_meta(const Meta<CPL>& mt, int zshift, uint32_t zmask, float (&s)[CPL],
                                            float (&bz)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    s[c] = half_bits_to_float((mt.s[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);
    bz[c] = (float)(128u + (((mt.z & zmask) >> (zshift + 4 * c)) & 15u));
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// ---------------------------------------------------------------------------
// Skinny kernel for m <= 16 tokens (M known at compile time).
//
// A workgroup of W waves owns one strip of 16 * CPL output columns and a range
// of k groups (its k-slice; the whole of k unless the k split is on).  Lane
// (cl = lane % 16, ks = lane / 16) reads the CPL consecutive words of columns
// CPL * cl .. CPL * cl + CPL - 1 of word-row 4s + ks (k-step s of a group), so a
// wave-load covers 4 word-rows x 64 * CPL contiguous bytes.  Wave w takes
// groups w, w + W, w + 2W, ... of the slice and software-pipelines them: the
// loads of its next group are in flight while it computes the current one.
//
// DOT = true (m = 1, the GEMV): per lane v_dot2_f32_bf16 on (128 + q) pairs
// against the 8 activations of its word-row (one load the 16 lanes of a row
// share), per-group offset correction and scale per lane, then the four
// 16-lane rows summed with the row-swap permutes.
// DOT = false: the 16x16x32 bf16 MFMA, operand A = activations loaded per lane
// (token = lane % 16, zero for tokens >= M), operand B = the codes of one word
// (8 consecutive k of one column = one lane's B slice); tile c of a lane is
// column CPL * cl + c of the strip.  A second MFMA against a ones operand
// gives the per-token group sums for the offset correction.
//
// The W wave partials [M][16 * CPL] are summed in LDS.  With ksplit > 1 the
// workgroup partial goes to the workspace and the last workgroup of the strip
// to arrive (counter) adds the ksplit partials in k order and writes Y.
// Blocks are numbered so that consecutive strips, and all k-slices of a
// strip, land on the same XCD (block b runs on XCD b % 8).
// ---------------------------------------------------------------------------
constexpr int64_t kTicketBytes = kSplitCounterBytes;   // counters of up to 16384 strips
constexpr int SK_MAX_SPLIT = 16;              // k-slices per strip at most

// MFMA row tiles of 16 tokens: one up to 16 tokens, two up to 32, ... four up to 64
template <int M, bool DOT>
constexpr int kRowTiles = DOT ? 1 : (M + 15) / 16;

template <int M, bool DOT, int CPL>
struct GroupRegs {
  uint32_t w[4][CPL];                  // codes of the 4 k-steps
  u32x4 xa[kRowTiles<M, DOT>][4];      // activations of the 4 k-steps per row tile (MFMA: the A slices)
  Meta<CPL> meta;
};

// One group's loads.  Every address is in range, so no load carries a
// condition: a load inside an exec-masked branch makes the number of loads in
// flight depend on the path, and the compiler then waits for all of them
// before the current group's arithmetic instead of only for that group's.  The
// caller clamps the pointers: lanes whose columns are past n read column 0 and
// MFMA lanes whose token is past M read token 0 (xr[t] is the lane's row of row
// tile t; GEMV: the one token for every lane); those values reach only outputs
// that are never stored, since MFMA rows and columns are independent.  Without
// a zero point zp is any readable word (zstride 0) and the caller masks z.
template <int M, bool DOT, int CPL>
__device__ __forceinline__ void load_group(GroupRegs<M, DOT, CPL>& r, const uint32_t* __restrict__ qp,
                                           const uint16_t* const (&xr)[kRowTiles<M, DOT>],
                                           const uint16_t* __restrict__ sp, const uint32_t* __restrict__ zp,
                                           int64_t n, int64_t zstride, int64_t g, int ks) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    load_words<CPL>(qp + (g * 16 + 4 * s + ks) * n, r.w[s]);
    // MFMA: the lane's token's 8 k of this word-row; GEMV: the one token's 8 k
    // (the same address for the 16 lanes of a row: one broadcast load)
#pragma unroll
    for (int t = 0; t < kRowTiles<M, DOT>; ++t)
      r.xa[t][s] = *reinterpret_cast<const u32x4*>(xr[t] + 8 * (g * 16 + 4 * s + ks));
  }
  r.meta = load_meta<CPL>(sp + g * n, zp + g * zstride);
}

// ---------------------------------------------------------------------------
// LoRA add in the epilogue: Y += scale * U . B^T, U = X . A^T (fp32 [m][16]).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// Row reduction of the epilogue: q is this lane's sum of squares of its
// rounded outputs of one row (0 without one); the G lanes of an aligned group
// (all on the same row) add theirs with cross-lane swaps, and the group's
// first lane adds the total to row_ss[row] with one atomic.  Every lane of a
// group must come here together.
template <int G>
__device__ __forceinline__ void add_row_sumsq(float* row_ss, float q, int64_t row, bool first, bool valid) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) q += __shfl_xor(q, o, G);
  if (first && valid) atomicAdd(row_ss + row, q);
}

// The LoRA term of one output (row, col): scale * sum_r U[row][r] B[col][r].
// All loads are issued before the first use (one round trip): the U row as
// four 16-byte loads, the B row as two when its 16 entries are aligned (else
// element loads); U's columns past the rank are zero, B is used only below it.
__device__ __forceinline__ float lora_term(const LoraEpi& L, int64_t row, int64_t col) {
  const f32x4* u = reinterpret_cast<const f32x4*>(L.u + row * 16);
  const uint16_t* b = L.b + col * L.ldb;
  f32x4 uu[4];
  float bb[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) uu[i] = u[i];
  // loads from clamped in-range addresses, the rank applied by a select after
  // them: no branch between the loads
  if (L.ldb >= 16 && (L.ldb & 7) == 0 && ((uintptr_t)L.b & 15u) == 0) {
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(b), w1 = *reinterpret_cast<const u32x4*>(b + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bb[2 * i] = bf16_bits_to_float(w0[i] & 0xFFFFu);
      bb[2 * i + 1] = bf16_bits_to_float(w0[i] >> 16);
      bb[8 + 2 * i] = bf16_bits_to_float(w1[i] & 0xFFFFu);
      bb[8 + 2 * i + 1] = bf16_bits_to_float(w1[i] >> 16);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) bb[r] = r < L.rank ? bb[r] : 0.f;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = bf16_bits_to_float(b[r < L.rank ? r : 0]);
      bb[r] = r < L.rank ? v : 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s = __builtin_fmaf(uu[r >> 2][r & 3], bb[r], s);
  return L.scale * s;
}

// The LoRA term of one output with the U row already at hand (16 fp32 values,
// columns past the rank zero): the B row loaded as in lora_term.
__device__ __forceinline__ float lora_term_u(const LoraEpi& L, const float* urow, int64_t col) {
  const uint16_t* b = L.b + col * L.ldb;
  float bb[16];
  if (L.ldb >= 16 && (L.ldb & 7) == 0 && ((uintptr_t)L.b & 15u) == 0) {
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(b), w1 = *reinterpret_cast<const u32x4*>(b + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bb[2 * i] = bf16_bits_to_float(w0[i] & 0xFFFFu);
      bb[2 * i + 1] = bf16_bits_to_float(w0[i] >> 16);
      bb[8 + 2 * i] = bf16_bits_to_float(w1[i] & 0xFFFFu);
      bb[8 + 2 * i + 1] = bf16_bits_to_float(w1[i] >> 16);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) bb[r] = r < L.rank ? bb[r] : 0.f;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = bf16_bits_to_float(b[r < L.rank ? r : 0]);
      bb[r] = r < L.rank ? v : 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s = __builtin_fmaf(urow[r], bb[r], s);
  return L.scale * s;
}

// U = X . A^T in two small launches: partial 16 x 16 tiles of U over k slices
// (workgroup (b, s): rows 16 b .. 16 b + 15, k slice s; its 16 waves take
// interleaved 32-k steps on the 16x16x32 bf16 MFMA with the activations as A
// and lora_A's rows as B, fp32), then the slices summed in slice order.
// Slices of `kps` k (a multiple of 512); partials [b][s][16][16] fp32.
__global__ __launch_bounds__(1024) void lora_u_partial_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                              const uint16_t* __restrict__ a, int64_t lda,
                                                              int rank, int64_t m, int k, int kps,
                                                              float* __restrict__ part) {
  __shared__ float red[16][16][16];   // [wave][row][r]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int kbeg = blockIdx.y * kps, kend = min(k, kbeg + kps);
  const bool xok = row0 + cl < m, aok = cl < rank;
  const uint16_t* xp = x + (xok ? row0 + cl : 0) * ldx + 8 * ks;
  const uint16_t* ap = a + (aok ? cl : 0) * lda + 8 * ks;
  const u32x4 z = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg + 32 * wave; k0 < kend; k0 += 4 * 512) {   // four steps' loads in flight, then the MFMAs
    u32x4 xv[4], av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = k0 + 512 * j;
      xv[j] = xok && kk < kend ? *reinterpret_cast<const u32x4*>(xp + kk) : z;
      av[j] = aok && kk < kend ? *reinterpret_cast<const u32x4*>(ap + kk) : z;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16_bf16(xv[j], av[j], acc);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][4 * ks + v][cl] = acc[v];
  __syncthreads();
  if (tid < 256) {
    const int rr = tid >> 4, c = tid & 15;
    float sum = 0.f;
    for (int w = 0; w < 16; ++w) sum += red[w][rr][c];
    part[((int64_t)blockIdx.x * gridDim.y + blockIdx.y) * 256 + tid] = sum;
  }
}

__global__ __launch_bounds__(256) void lora_u_reduce_kernel(const float* __restrict__ part, int slices, int64_t m,
                                                            float* __restrict__ u) {
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const float* p = part + (int64_t)blockIdx.x * slices * 256 + tid;
  float sum = 0.f;
  for (int s0 = 0; s0 < slices; s0 += 8) {      // eight loads in flight, added in slice order
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = p[(int64_t)(s0 + j < slices ? s0 + j : slices - 1) * 256];
      v[j] = s0 + j < slices ? w : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += v[j];
  }
  if (row < m) u[row * 16 + (tid & 15)] = sum;
}

// k slices of the U product: about 512 workgroups over the row blocks, each
// slice a multiple of 512 k.
void lora_u_split(int64_t m, int64_t k, int* slices, int* kps) {
  const int64_t blocks = (m + 15) / 16, steps = (k + 511) / 512;
  int64_t s = (512 + blocks - 1) / blocks;
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  const int64_t per = (steps + s - 1) / s;
  *kps = (int)(per * 512);
  *slices = (int)((k + *kps - 1) / *kps);
  if (*slices < 1) *slices = 1;
}

int64_t lora_bytes(int64_t m, int64_t k) {
  int slices, kps;
  lora_u_split(m, k, &slices, &kps);
  const int64_t blocks = (m + 15) / 16;
  return ((m * 64 + 255) & ~(int64_t)255) + blocks * slices * 1024;
}

hipError_t launch_lora_u(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda, int rank, int64_t m,
                         int64_t k, float* u, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  int slices, kps;
  lora_u_split(m, k, &slices, &kps);
  const int64_t blocks = (m + 15) / 16;
  float* part = u + ((m * 16 + 63) & ~(int64_t)63);      // after U, 256-byte aligned
  lora_u_partial_kernel<<<dim3((unsigned)blocks, (unsigned)slices), dim3(1024), 0, stream>>>(
      x, ldx, a, lda, rank, m, (int)k, kps, part);
  lora_u_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(part, slices, m, u);
  return hipGetLastError();
}

template <int M, bool DOT, int CPL>
__global__ __launch_bounds__(M > 16 || CPL > 4 ? 512 : 1024) void skinny_int4_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    uint16_t* __restrict__ y, int64_t ldy, int n, int k, int nstrips, int ksplit, int gwg,
    int items_per_xcd, float* __restrict__ partials, uint32_t* __restrict__ tickets, int acq_rel,
    LoraEpi lora) {
  static_assert(!DOT || M == 1, "the VALU variant computes one token");
  constexpr int SW = 16 * CPL;                 // strip width in columns
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  float* plane = reinterpret_cast<float*>(smem);                          // [nw][M][SW]
  __shared__ int last_flag;

  const int item = (blockIdx.x & 7) * items_per_xcd + (blockIdx.x >> 3);
  const int strip = item / ksplit, kslice = item - strip * ksplit;
  if (strip >= nstrips) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int G = k >> 7;
  const int gbeg = kslice * gwg, gend = min(G, gbeg + gwg);
  const int64_t col = (int64_t)strip * SW + CPL * cl;
  const bool live = col < n;
  // clamped pointers (see load_group): columns past n read column 0; MFMA: the
  // lane supplies token 16 t + cl of row tile t (token 0 past M); GEMV: every
  // lane the one token
  constexpr int MT = kRowTiles<M, DOT>;
  const int64_t colc = live ? col : 0;
  const uint32_t* qp = qweight + colc;
  const uint16_t* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xr[t] = x + (!DOT && 16 * t + cl < M ? (int64_t)(16 * t + cl) * ldx : 0);
  const uint16_t* sp = scales + colc;
  const uint32_t* zp = qzeros ? qzeros + (colc >> 3) : reinterpret_cast<const uint32_t*>(scales);
  const int64_t zstride = qzeros ? (int64_t)(n >> 3) : 0;
  const uint32_t zmask = qzeros ? ~0u : 0u;
  const int zshift = (int)(col & 7) * 4;
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

  // first group's loads go out before anything waits (a wave without a group
  // loads the slice's first one and skips the arithmetic); the wave index is
  // made scalar so that the group loop's branches are uniform
  GroupRegs<M, DOT, CPL> ra, rb;
  int g = gbeg + __builtin_amdgcn_readfirstlane(wave);
  const bool busy = g < gend;
  load_group<M, DOT, CPL>(ra, qp, xr, sp, zp, n, zstride, busy ? g : gbeg, ks);

  // the LoRA terms of this thread's outputs in the final reduction (output
  // o = tid + j * blockDim), computed now so that their loads overlap the
  // k loop; added once per output (slice 0 of a split strip)
  float lora_pre[4] = {0.f, 0.f, 0.f, 0.f};
  if (lora.u && kslice == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int o = tid + j * blockDim.x;
      const int token = o / SW, cc = o - token * SW;
      const int64_t cg = (int64_t)strip * SW + cc;
      if (o < M * SW && cg < n) lora_pre[j] = lora_term(lora, token, cg);
    }
  }

  f32x4 total[MT][CPL];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < CPL; ++c) total[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the group's arithmetic, accumulated into total
  auto compute = [&](const GroupRegs<M, DOT, CPL>& cur) {
    float sc[CPL], bz[CPL];
    if constexpr (DOT) {
      float d[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) d[c] = 0.f;
      float xs = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = x_pairs_permuted(cur.xa[0][s]);
#pragma unroll
        for (int t = 0; t < 4; ++t) xs = dot2_bf16(a[t], kOnesBf16x2, xs);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const u32x4 bq = codes_as_bf16_pairs(cur.w[s][c]);
#pragma unroll
          for (int t = 0; t < 4; ++t) d[c] = dot2_bf16(bq[t], a[t], d[c]);
        }
      }
      decode_meta<CPL>(cur.meta, zshift, zmask, sc, bz);
#pragma unroll
      for (int c = 0; c < CPL; ++c) total[0][c][0] += sc[c] * (d[c] - bz[c] * xs);
    } else {
      constexpr int VMAX = M < 4 ? M : 4;
      f32x4 acc[MT][CPL], xsum[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        xsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (MT == 1) {
          const u32x4 a = x_pairs_permuted(cur.xa[0][s]);
          xsum[0] = mfma16_bf16(a, ones, xsum[0]);
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[0][c] = mfma16_bf16(a, codes_as_bf16_pairs(cur.w[s][c]), acc[0][c]);
        } else {
          u32x4 b[CPL];   // one decode of the step's words serves both row tiles
#pragma unroll
          for (int c = 0; c < CPL; ++c) b[c] = codes_as_bf16_pairs(cur.w[s][c]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const u32x4 a = x_pairs_permuted(cur.xa[t][s]);
            xsum[t] = mfma16_bf16(a, ones, xsum[t]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[t][c] = mfma16_bf16(a, b[c], acc[t][c]);
          }
        }
      }
      decode_meta<CPL>(cur.meta, zshift, zmask, sc, bz);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int v = 0; v < VMAX; ++v) total[t][c][v] += sc[c] * (acc[t][c][v] - bz[c] * xsum[t][v]);
    }
  };
  // Two register sets in turn, no copy between them (a copy of registers whose
  // loads are in flight would wait for them): the next group's loads are issued
  // before the current group's arithmetic, which waits for its own loads only.
  // The 64-column MFMA strips of 1024-thread workgroups (128 registers) would
  // spill with both sets live across the arithmetic; they keep one set and a
  // copy, and wait for both groups' loads.  Measured against conditional loads
  // and one set (cold weights): 4096 x 4096 m = 1 / 8 / 15 6.18 / 6.99 / 8.33
  // -> 5.49 / 6.63 / 7.99 µs, m = 33 14.9 -> 12.7 µs, 4096 x 14336 m = 1
  // 10.2 -> 8.7 µs, 5120 x 25600 m = 24 38.0 -> 32.2 µs; the 64-column m = 16
  // strips, one set with unconditional loads: 5120 x 25600 26.1 -> 23.7 µs
  // (11-15% slower than that with both sets).
  constexpr bool kTwoSets = DOT || M > 16 || CPL < 4;
  if (busy) {
    // (the scheduling barriers keep the next group's loads ahead of the current
    // group's first use: scheduled after it, they would go out only once the
    // current group had arrived)
    // Waves with one or two groups run straight-line code: at a loop head the
    // compiler merges the entry and back-edge states and waited there for most
    // of the current group's loads before issuing the next group's.
    if constexpr (kTwoSets) {
      if (g + nw >= gend) {
        compute(ra);
      } else {
        load_group<M, DOT, CPL>(rb, qp, xr, sp, zp, n, zstride, g + nw, ks);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra);
        g += nw;
        if (g + nw >= gend) {
          compute(rb);
        } else {
          for (;;) {
            load_group<M, DOT, CPL>(ra, qp, xr, sp, zp, n, zstride, g + nw, ks);
            __builtin_amdgcn_sched_barrier(0);
            compute(rb);
            g += nw;
            if (g + nw >= gend) { compute(ra); break; }
            load_group<M, DOT, CPL>(rb, qp, xr, sp, zp, n, zstride, g + nw, ks);
            __builtin_amdgcn_sched_barrier(0);
            compute(ra);
            g += nw;
            if (g + nw >= gend) { compute(rb); break; }
          }
        }
      }
    } else {
      for (;;) {
        const bool more = g + nw < gend;
        if (more) load_group<M, DOT, CPL>(rb, qp, xr, sp, zp, n, zstride, g + nw, ks);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra);
        if (!more) break;
        ra = rb;
        g += nw;
      }
    }
  }

  // wave partials [M][SW] -> LDS plane -> sum over the waves
  if constexpr (DOT) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) total[0][c][0] = sum_over_rows(total[0][c][0]);
    if (ks == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) plane[wave * SW + CPL * cl + c] = total[0][c][0];
    }
  } else {
    constexpr int VMAX = M < 4 ? M : 4;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        const int token = 16 * t + 4 * ks + v;
        if (token < M) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) plane[(wave * M + token) * SW + CPL * cl + c] = total[t][c][v];
        }
      }
  }
  __syncthreads();

  float* mine = ksplit > 1 ? partials + ((int64_t)strip * ksplit + kslice) * (M * SW) : nullptr;
  int jo = 0;                              // index of the output within this thread's
  for (int o = tid; o < M * SW; o += blockDim.x, ++jo) {
    const int token = o / SW, cc = o - token * SW;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += plane[(w * M + token) * SW + cc];
    const int64_t cg = (int64_t)strip * SW + cc;
    if (lora.u && kslice == 0 && cg < n) {
      // precomputed for the first four outputs (selects, no indexed registers)
      float pre = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) pre = jo == i ? lora_pre[i] : pre;
      v += jo < 4 ? pre : lora_term(lora, token, cg);
    }
    if (ksplit == 1) {
      const uint32_t yb = f32_to_bf16_bits(v);
      if (cg < n) y[(int64_t)token * ldy + cg] = (uint16_t)yb;
      if (lora.row_ss) {
        const float yf = cg < n ? bf16_bits_to_float(yb) : 0.f;
        add_row_sumsq<(SW < 64 ? SW : 64)>(lora.row_ss, yf * yf, token, cc % 64 == 0, true);
      }
    } else {
      // agent-coherent store: visible to any workgroup once it has completed
      __hip_atomic_store(&mine[o], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (ksplit == 1) return;

  // split k: the last workgroup of the strip adds the partials in k order.
  // Every thread waits for its partial stores to complete before the barrier,
  // then one counter increment per workgroup; partials are only written and
  // read with agent-coherent accesses, so no cache-wide maintenance is needed
  // (acq_rel: the increment orders them by the memory model, at the price of
  // an L2 write-back and invalidate).
  asm volatile("" ::: "memory");             // (no instruction: keeps the stores above the wait)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (tid == 0)
    last_flag = ticket_add(&tickets[strip], acq_rel) == (uint32_t)(ksplit - 1);
  __syncthreads();
  if (!last_flag) return;
  const float* base = partials + (int64_t)strip * ksplit * (M * SW);
  for (int o = tid; o < M * SW; o += blockDim.x) {
    const int token = o / SW, cc = o - token * SW;
    const int64_t cg = (int64_t)strip * SW + cc;
    float part[SK_MAX_SPLIT];
#pragma unroll
    for (int p = 0; p < SK_MAX_SPLIT; ++p)       // all loads in flight, then add in k order
      part[p] = p < ksplit ? __hip_atomic_load(&base[p * (M * SW) + o], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < SK_MAX_SPLIT; ++p) v += part[p];
    const uint32_t yb = f32_to_bf16_bits(v);
    if (cg < n) y[(int64_t)token * ldy + cg] = (uint16_t)yb;
    if (lora.row_ss) {
      const float yf = cg < n ? bf16_bits_to_float(yb) : 0.f;
      add_row_sumsq<(SW < 64 ? SW : 64)>(lora.row_ss, yf * yf, token, cc % 64 == 0, true);
    }
  }
  if (tid == 0) __hip_atomic_store(&tickets[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Small-M kernel with the codes staged in LDS (m <= 16, whole k per
// workgroup).  Same work split as skinny_int4_kernel (a strip of 16 * CPL
// columns per workgroup, wave w takes groups w, w + W, ...), but every group a
// wave owns has its loads issued before any arithmetic: the codes go straight
// to LDS with 16-byte lane loads (buffer_load ... lds: no registers held while
// in flight; one instruction moves 1 KiB of a group's 16 word rows), the
// activations and raw metadata to registers through buffer resources on
// wave-uniform group bases (one lane-offset register serves every group).
// Groups are then computed in issue order, each after an explicit wait for its
// own loads (a wave's vector memory operations complete in order), so the
// arithmetic of group j runs while groups j + 1 .. are still arriving; the
// scheduling barriers keep the compiler from hoisting a later group's decode
// above its wait.  A wave owns NGW = NG or NG - 1 groups (NG at compile time:
// the activation registers and the wait counts depend on it).
//
// Measured (cold weights, HIP-graph replay) against skinny_int4_kernel:
// 4096 x 4096 m = 1 / 8 / 15 5.53 / 6.66 / 8.01 -> 5.03 / 6.12 / 7.21 µs,
// 2048 x 8192 4.98 / 5.38 / 6.27 -> 4.34 / 4.84 / 5.47 µs.  Timing copies
// with parts switched off (4096 x 4096): without arithmetic the time hardly
// changes (4.85 / 6.16 / 6.96 µs), without loads it is 2.9-3.1 µs, so the
// arithmetic is hidden and the loads bound the kernel; the activation loads
// (every strip reads all of X) add 0.3 / 1.2 / 2.3 µs over the codes alone.
// ---------------------------------------------------------------------------
// Activations staged in LDS too (XL): per group the wave copies its M tokens x
// 128 k with direct loads, 1 KiB = 4 tokens x 256 contiguous bytes per
// instruction (MFMA; the GEMV copies its one token's 256 bytes with 4-byte
// lanes), instead of four 16-byte register loads per lane whose 16 tokens each
// touch half a cache line: 4096 x 4096 m = 8 / 15 6.16 / 7.21 -> 5.53 / 6.25
// µs in a timing copy.  The 16-byte chunk c of token t's row sits in slot
// c ^ t, so the 16 lanes of an MFMA operand read (16 tokens, one chunk) hit
// distinct banks.
template <int M, bool DOT, bool XL>
constexpr int kXLoads = XL ? (DOT ? 1 : (M + 3) / 4) : 4;   // activation loads per group and lane

template <int M, bool DOT, int CPL, int NGW, bool XL, bool LORA>
__device__ __forceinline__ void lds_strip_groups(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qweight,
                                                 const uint16_t* __restrict__ scales, const uint32_t* zbase,
                                                 int64_t zstride, uint32_t* codes, uint32_t* xlds, int n, int wave,
                                                 int nw, int lane, const uint32_t (&xo)[4], uint32_t soff, uint32_t zoff,
                                                 const uint32_t (&coff)[CPL], int zshift, uint32_t zmask,
                                                 f32x4 (&total)[CPL], const uint16_t* __restrict__ la_base,
                                                 uint32_t aoff, bool arank, f32x4& uacc) {
  constexpr int SW = 16 * CPL;                 // strip width in columns
  constexpr int GDW = 16 * SW;                 // dwords of codes per group
  constexpr int XI = kXLoads<M, DOT, XL>;
  constexpr int XDW = DOT ? 64 : 256 * XI;     // dwords of activations per group (XL)
  constexpr int LPG = CPL + XI + 2 + (LORA ? 4 : 0);   // vector memory operations per group
  static_assert(NGW * LPG <= 63, "vmcnt range");
  const int cl = lane & 15, ks = lane >> 4;
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  u32x4 xa[XL ? 1 : NGW][4];
  u32x4 la[LORA ? NGW : 1][4];   // LoRA: lane (rank cl, chunk ks) of lora_A per k step
  Meta<CPL> meta[NGW];
#pragma unroll
  for (int j = 0; j < NGW; ++j) {
    const int g = wave + nw * j;
    const uint32_t* gbase = qweight + (int64_t)g * 16 * n;
    uint32_t* lds = codes + (size_t)g * GDW;
#pragma unroll
    for (int i = 0; i < CPL; ++i) buffer_to_lds16(gbase, coff[i], lds + 256 * i);
    const uint16_t* xg = x + (int64_t)g * 128;
    if constexpr (XL) {
      uint32_t* xl = xlds + (size_t)g * XDW;
      if constexpr (DOT) {
        buffer_to_lds4(xg, xo[0], xl);
      } else {
#pragma unroll
        for (int i = 0; i < XI; ++i) buffer_to_lds16(xg, xo[i], xl + 256 * i);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) xa[j][s] = buffer_load16(xg, xo[0] + 64 * s);
    }
    const uint16_t* sg = scales + (int64_t)g * n;
    if constexpr (CPL == 4) {
      const u32x2 v = buffer_load8(sg, soff);
      meta[j].s[0] = v[0];
      meta[j].s[CPL == 4 ? 1 : 0] = v[1];
    } else if constexpr (CPL == 2) {
      meta[j].s[0] = buffer_load4(sg, soff);
    } else {
      meta[j].s[0] = buffer_load2(sg, soff);
    }
    meta[j].z = buffer_load4(zbase + (int64_t)g * zstride, zoff);
    if constexpr (LORA) {
      const uint16_t* ag = la_base + (int64_t)g * 128;
#pragma unroll
      for (int s = 0; s < 4; ++s) la[j][s] = buffer_load16(ag, aoff + 64 * s);
    }
    __builtin_amdgcn_sched_barrier(0);   // groups' loads stay in issue order
  }
  const uint32_t mask = in_vgpr(0x000F000Fu), bias = in_vgpr(kBias128x2);   // VGPR operands of v_and_or_b32
  // the lane's 8 activations of k step s of group j (MFMA: token cl, GEMV: the
  // one token), from registers or from the LDS copy (row cl, chunk 4 s + ks in
  // slot (4 s + ks) ^ cl; rows past the copied ones read row 0)
  const int xrow = cl < 4 * XI ? cl : 0;
  auto xfrag = [&](int j, int s) -> u32x4 {
    if constexpr (!XL) {
      return xa[j][s];
    } else {
      const uint32_t* xl = xlds + (size_t)(wave + nw * j) * XDW;
      if constexpr (DOT) return *reinterpret_cast<const u32x4*>(xl + 4 * (4 * s + ks));
      else return *reinterpret_cast<const u32x4*>(xl + 64 * xrow + 4 * ((4 * s + ks) ^ xrow));
    }
  };
#pragma unroll
  for (int j = 0; j < NGW; ++j) {
    // this group's loads have landed once at most the later groups' are outstanding
    wait_vmcnt((NGW - 1 - j) * LPG);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t* lds = codes + (size_t)(wave + nw * j) * GDW;
    uint32_t w[4][CPL];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t* p = lds + (4 * s + ks) * SW + CPL * cl;
      if constexpr (CPL == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[s][0] = v[0]; w[s][1] = v[1]; w[s][2] = v[2]; w[s][3] = v[3];
      } else if constexpr (CPL == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        w[s][0] = v[0]; w[s][1] = v[1];
      } else {
        w[s][0] = *p;
      }
    }
    float sc[CPL], bz[CPL];
    decode_meta<CPL>(meta[j], zshift, zmask, sc, bz);
    if constexpr (DOT) {
      float d[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) d[c] = 0.f;
      float xs = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 xr = xfrag(j, s);
        if constexpr (LORA) {
          // U[rank cl] += x . lora_A[cl] over this lane's chunk (both in natural order)
          const u32x4 av = arank ? la[j][s] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int t = 0; t < 4; ++t) uacc[0] = dot2_bf16(xr[t], av[t], uacc[0]);
        }
        const u32x4 a = x_pairs_permuted(xr);
#pragma unroll
        for (int t = 0; t < 4; ++t) xs = dot2_bf16(a[t], kOnesBf16x2, xs);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const u32x4 bq = codes_as_bf16_pairs_mb(w[s][c], mask, bias);
#pragma unroll
          for (int t = 0; t < 4; ++t) d[c] = dot2_bf16(bq[t], a[t], d[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) total[c][0] += sc[c] * (d[c] - bz[c] * xs);
    } else {
      constexpr int VMAX = M < 4 ? M : 4;
      f32x4 acc[CPL], xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 xr = xfrag(j, s);
        if constexpr (LORA) {
          // U[token][rank] += x . lora_A^T: tokens as A, ranks as B (natural k order)
          uacc = mfma16_bf16(xr, arank ? la[j][s] : u32x4{0u, 0u, 0u, 0u}, uacc);
        }
        const u32x4 a = x_pairs_permuted(xr);
        xsum = mfma16_bf16(a, ones, xsum);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = mfma16_bf16(a, codes_as_bf16_pairs_mb(w[s][c], mask, bias), acc[c]);
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int v = 0; v < VMAX; ++v) total[c][v] += sc[c] * (acc[c][v] - bz[c] * xsum[v]);
    }
    __builtin_amdgcn_sched_barrier(0);   // nothing of the next group moves above its wait
  }
}

template <int M, bool DOT, int CPL, int NG, bool XL, bool LORA>
__global__ __launch_bounds__(1024) void skinny_lds_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    uint16_t* __restrict__ y, int64_t ldy, int n, int k, int nstrips, int items_per_xcd, int plane_off,
    LoraEpi lora) {
  static_assert(!DOT || M == 1, "the VALU variant computes one token");
  static_assert(M <= 16, "one MFMA row tile");
  constexpr int SW = 16 * CPL;                 // strip width in columns
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  // codes [G][16][SW], with XL the activations [G][rows][128] behind them, and
  // the wave partial plane [nw][M][SW] behind those or, when LDS is short
  // (plane_off 0), over them once every wave is done
  uint32_t* codes = reinterpret_cast<uint32_t*>(smem);
  float* plane = reinterpret_cast<float*>(smem + plane_off);

  const int strip = (blockIdx.x & 7) * items_per_xcd + (blockIdx.x >> 3);
  if (strip >= nstrips) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cl = lane & 15, ks = lane >> 4;
  const int G = k >> 7;
  const int64_t col0 = (int64_t)strip * SW;
  const int64_t col = col0 + CPL * cl;
  const int64_t colc = col < n ? col : 0;
  // lane parts of the addresses as 32-bit byte offsets from wave-uniform bases
  // (columns past n read column 0; MFMA lanes past M read token 0; GEMV: the
  // one token for every lane)
  // activation offsets: registers -- the lane's token row and k chunk ks;
  // LDS copy -- instruction i, lane l: token t = 4 i + l / 16 (token 0 past M),
  // source chunk (l % 16) ^ t; the GEMV copy: dword l of the row
  uint32_t xo[4] = {0u, 0u, 0u, 0u};
  if constexpr (!XL) {
    xo[0] = (uint32_t)(((!DOT && cl < M ? (int64_t)cl * ldx : 0) + 8 * ks) * 2);
  } else if constexpr (DOT) {
    xo[0] = (uint32_t)(4 * lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + ks;
      xo[i] = (uint32_t)(((t < M ? (int64_t)t * ldx : 0) + 8 * (cl ^ t)) * 2);
    }
  }
  uint32_t* xlds = codes + (size_t)G * 16 * SW;
  const uint32_t soff = (uint32_t)(colc * 2);
  const uint32_t zoff = qzeros ? (uint32_t)((colc >> 3) * 4) : 0u;
  const uint32_t* zbase = qzeros ? qzeros : reinterpret_cast<const uint32_t*>(scales);
  const int64_t zstride = qzeros ? (int64_t)(n >> 3) : 0;
  const uint32_t zmask = qzeros ? ~0u : 0u;
  const int zshift = (int)(col & 7) * 4;
  // direct-load lane offsets of the codes: instruction i, lane l -> 16-byte
  // chunk c = 64 i + l of the group, word row c / (SW / 4), columns
  // 4 (c % (SW / 4)) .. + 3 (chunks past n read column 0 of their row);
  // byte offsets from the group's first word row stay below 16 n * 4 <= 2^32
  uint32_t coff[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = 64 * i + lane, row = c / (SW / 4), cc = 4 * (c % (SW / 4));
    coff[i] = (uint32_t)(((int64_t)row * n + (col0 + cc < n ? col0 + cc : 0)) * 4);
  }

  f32x4 total[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) total[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // NG groups for the first G - nw (NG - 1) waves, NG - 1 for the rest (uniform branch)
  // LoRA with U accumulated here: lane (rank cl, chunk ks) reads lora_A row cl
  // (row 0 past the rank; its contribution is zeroed)
  const bool arank = LORA && cl < lora.rank;
  const uint32_t aoff = LORA ? (uint32_t)(((arank ? (int64_t)cl * lora.lda : 0) + 8 * ks) * 2) : 0u;
  f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
  if (wave + nw * (NG - 1) < G) {
    lds_strip_groups<M, DOT, CPL, NG, XL, LORA>(x, qweight, scales, zbase, zstride, codes, xlds, n, wave, nw, lane,
                                                xo, soff, zoff, coff, zshift, zmask, total, lora.a, aoff, arank, uacc);
  } else if constexpr (NG > 1) {
    lds_strip_groups<M, DOT, CPL, NG - 1, XL, LORA>(x, qweight, scales, zbase, zstride, codes, xlds, n, wave, nw,
                                                    lane, xo, soff, zoff, coff, zshift, zmask, total, lora.a, aoff,
                                                    arank, uacc);
  }

  // wave partials [M][SW] -> LDS plane -> sum over the waves (LoRA: the wave
  // partials of U [M][16] behind the plane, summed into U [M][16] after them)
  if (plane_off == 0) __syncthreads();
  float* uplane = plane + nw * M * SW;
  float* utot = uplane + nw * M * 16;
  if constexpr (LORA) {
    if constexpr (DOT) {
      const float u = sum_over_rows(uacc[0]);
      if (ks == 0) uplane[wave * 16 + cl] = u;
    } else {
      constexpr int VMAX = M < 4 ? M : 4;
#pragma unroll
      for (int v = 0; v < VMAX; ++v)
        if (4 * ks + v < M) uplane[(wave * M + 4 * ks + v) * 16 + cl] = uacc[v];
    }
  }
  if constexpr (DOT) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) total[c][0] = sum_over_rows(total[c][0]);
    if (ks == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) plane[wave * SW + CPL * cl + c] = total[c][0];
    }
  } else {
    constexpr int VMAX = M < 4 ? M : 4;
#pragma unroll
    for (int v = 0; v < VMAX; ++v) {
      const int token = 4 * ks + v;
      if (token < M) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) plane[(wave * M + token) * SW + CPL * cl + c] = total[c][v];
      }
    }
  }
  __syncthreads();
  if constexpr (LORA) {
    for (int o = tid; o < M * 16; o += blockDim.x) {   // U summed over the waves in wave order
      float u = 0.f;
      for (int w = 0; w < nw; ++w) u += uplane[w * M * 16 + o];
      utot[o] = u;
    }
    __syncthreads();
  }
  for (int o = tid; o < M * SW; o += blockDim.x) {
    const int token = o / SW, cc = o - token * SW;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += plane[(w * M + token) * SW + cc];
    const int64_t cg = col0 + cc;
    float yf = 0.f;
    if (cg < n) {
      if constexpr (LORA) v += lora_term_u(lora, utot + token * 16, cg);
      else if (lora.u) v += lora_term(lora, token, cg);
      const uint32_t yb = f32_to_bf16_bits(v);
      y[(int64_t)token * ldy + cg] = (uint16_t)yb;
      yf = bf16_bits_to_float(yb);
    }
    if (lora.row_ss) add_row_sumsq<SW>(lora.row_ss, yf * yf, token, cc == 0, true);
  }
}

// ---------------------------------------------------------------------------
// Pipelined MFMA kernel for m > 16.
//
// Workgroup tile BM x BN = (NWM * 16 * FM) tokens x (NWN * 64) columns; wave
// (wm, wn) owns 16 * FM tokens x 64 columns as FM x 4 MFMA tiles of 16 x 16.
// Within a wave's 64 columns, N-fragment c holds columns 4 * l + c (l = lane
// % 16), so one 16-byte LDS read gives a lane the words of its four columns and
// the output of four adjacent columns lands in one lane.
//
// The k loop walks stages of 64 rows (half a quantization group).  Each stage
// is copied global -> LDS with direct buffer loads (no register
// round trip), STAGES deep:
//   activations  BM x 64 bf16, K-contiguous, XOR-swizzled 16-byte chunks
//   codes        8 word rows x BN columns (the qweight words of those 64 rows)
//   metadata     the group's BN fp16 scales and BN / 8 zero words
// The oldest stage is consumed once the wave's vmcnt shows its loads landed
// and a plain s_barrier shows every wave is past the previous stage.
//
// Per 32-row k step a wave turns each column's word into the bf16 pairs
// 128 + q (codes_as_bf16_pairs), reorders its activation fragments to the
// same pair order, and accumulates; a ones-MFMA on the raw activation
// fragments gives the per-token group sums in the accumulator layout.  After
// both stages of a group: total += s * (acc - (128 + z) * sum_x), fp32.
// ---------------------------------------------------------------------------
#ifndef QG_PIPE_INTERLEAVE
#define QG_PIPE_INTERLEAVE 1   // interleave the second k step's decode with the first step's MFMAs
#endif

template <int NWM, int NWN, int FM, bool PREP, bool LORA = false>
struct PipeShape {
  static constexpr int T = 64 * NWM * NWN;               // threads
  static constexpr int NW = NWM * NWN;                   // waves
  static constexpr int BM = NWM * 16 * FM, BN = NWN * 64;
  static constexpr int X_SLOTS = BM * 8;                 // 16-byte activation chunks per stage
  static constexpr int XL = X_SLOTS / T;                 // per thread
  static constexpr bool W16 = (2 * BN) % T == 0;         // words as 16-byte chunks, else dwords
  static constexpr int WL = W16 ? 2 * BN / T : 8 * BN / T;
  // metadata: 64-dword slots, one per wave and load: the BN scales (slot 0), the
  // BN / 8 zero words (slot 1) and, with the prepared activations, the group
  // sums of the BM tokens (slots 2 .. 2 + BM / 64 - 1); other slots are filler
  static constexpr int MSLOTS = 2 + (PREP ? BM / 64 : 0);
  static constexpr int ML = (MSLOTS + NW - 1) / NW;      // metadata loads per thread
  // LoRA: the stage's 16 x 64 block of lora_A (512 dwords, 4-byte loads)
  static constexpr int AL = LORA ? 512 / T : 0;
  static constexpr int LOADS = XL + WL + ML + AL;        // direct loads per thread per stage
  static constexpr int X_DW = 4 * X_SLOTS, W_DW = 8 * BN, M_DW = 64 * NW * ML, A_DW = LORA ? 512 : 0;
  static constexpr int STAGE_DW = X_DW + W_DW + M_DW + A_DW;   // dwords of LDS per stage
  static constexpr int OP = BN + 8;                      // output tile row pitch (bf16)
  static_assert(X_SLOTS % T == 0, "activation chunks per thread");
  static_assert((8 * BN) % T == 0, "word loads per thread");
  static_assert(BN == 128 && BM % 64 == 0, "metadata slots");
  static_assert(!LORA || (512 % T == 0 && NWN == 2), "lora_A block loads; two column waves share U");
};

template <int NWM, int NWN, int FM, int STAGES, bool PREP, bool LORA>
__global__ __launch_bounds__(64 * NWM * NWN) __attribute__((amdgpu_waves_per_eu(2))) void int4_pipe_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    const float* __restrict__ xsum, uint16_t* __restrict__ y, int64_t ldy, int m, int n, int k,
    int tiles_n, int items, int items_per_xcd, int vec_store, int ksplit, int gps,
    float* __restrict__ partials, uint32_t* __restrict__ tickets, int acq_rel, LoraEpi lora) {
  using S = PipeShape<NWM, NWN, FM, PREP, LORA>;
  constexpr int T = S::T, BM = S::BM, BN = S::BN, XL = S::XL, WL = S::WL, LOADS = S::LOADS;
  static_assert(LOADS * (STAGES - 2) <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint32_t psm_i4[];

  // item = tile * ksplit + k-slice; the slices of a tile are consecutive items,
  // so they run on one XCD
  const int item = (blockIdx.x & 7) * items_per_xcd + (blockIdx.x >> 3);
  if (item >= items) return;
  const int t = item / ksplit, kslice = item - t * ksplit;
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  const int gbeg = kslice * gps, gend = min(k >> 7, gbeg + gps);   // this slice's groups
  const int kt0 = 2 * gbeg;                                          // its first stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
  const int cl = lane & 15, ks = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave % NWM) * 16 * FM, wn0 = (wave / NWM) * 64;

  // Direct loads go through buffer resources (base in SGPRs, rebased per
  // stage) with one fixed 32-bit byte offset per lane and load, so a stage's
  // issue costs no vector ALU work.  Rows past m and columns past n load a
  // clamped valid address; their results are discarded.
  uint32_t xoff[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int slot = tid + T * i;
    const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
    const int rl = m0 + r < m ? r : m - 1 - m0;
    xoff[i] = (uint32_t)(((int64_t)rl * ldx + 8 * c) * 2);
  }
  uint32_t woff[WL];
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int slot = tid + T * i;
    int wr, cw;
    if constexpr (S::W16) {
      wr = slot / (BN / 4);
      cw = n0 + 4 * (slot % (BN / 4)) < n ? 4 * (slot % (BN / 4)) : n - 4 - n0;
    } else {
      wr = slot / BN;
      cw = n0 + slot % BN < n ? slot % BN : n - 1 - n0;
    }
    woff[i] = (uint32_t)(((int64_t)wr * n + cw) * 4);
  }
  // metadata slot j = NW * i + wave of load i: 0 scales, 1 zero words,
  // 2.. the group sums of tokens m0 + 64 (j - 2) + lane; others: zero words
  const int zlane = (n0 >> 3) + lane < (n >> 3) ? lane : (n >> 3) - 1 - (n0 >> 3);
  uint32_t moff[S::ML];
#pragma unroll
  for (int i = 0; i < S::ML; ++i) {
    const int j = S::NW * i + wave;
    if (j == 0) {
      moff[i] = (uint32_t)((n0 + 2 * lane < n ? 2 * lane : n - 2 - n0) * 2);
    } else if (j >= 2 && j < S::MSLOTS) {
      const int r = 64 * (j - 2) + lane;
      moff[i] = (uint32_t)((m0 + r < m ? r : m - 1 - m0) * 4);
    } else {
      moff[i] = (uint32_t)(zlane * 4);
    }
  }
  // LoRA: dword d = T i + 64 wave + lane of the stage's lora_A block holds
  // rank r = d / 32, 16-byte slot c = (d % 32) / 4, dword d % 4, where slot c of
  // row r carries the row's chunk c ^ (r & 7) (8 k each): the 16 ranks of an
  // operand read then spread over the banks.  Ranks past the rank read row 0.
  uint32_t aoff[S::AL > 0 ? S::AL : 1];
#pragma unroll
  for (int i = 0; i < S::AL; ++i) {
    const int d = T * i + 64 * wave + lane, r = d >> 5, c = (d & 31) >> 2;
    aoff[i] = (uint32_t)(((r < lora.rank ? (int64_t)r * lora.lda : 0) + 8 * (c ^ (r & 7)) + 2 * (d & 3)) * 2);
  }
  const uint16_t* xbase = x + (int64_t)m0 * ldx;
  const uint32_t* wbase0 = qweight + n0;

  auto issue = [&](int st) {   // local stage st = global stage kt0 + st
    uint32_t* base = psm_i4 + (size_t)(st % STAGES) * S::STAGE_DW;
    const uint16_t* xs_base = xbase + 64 * (int64_t)(kt0 + st);
#pragma unroll
    for (int i = 0; i < XL; ++i) buffer_to_lds16(xs_base, xoff[i], base + 4 * (T * i + 64 * wave));
    uint32_t* wl = base + S::X_DW;
    const uint32_t* ws_base = wbase0 + 8 * (int64_t)(kt0 + st) * n;
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      if constexpr (S::W16) buffer_to_lds16(ws_base, woff[i], wl + 4 * (T * i + 64 * wave));
      else buffer_to_lds4(ws_base, woff[i], wl + T * i + 64 * wave);
    }
    const int64_t g = (kt0 + st) >> 1;
#pragma unroll
    for (int i = 0; i < S::ML; ++i) {
      const int j = S::NW * i + wave;
      // Every wave issues the same number of loads per stage (the waits count
      // them).  Without zero points the zero-word slots load a word of the
      // stage's scale row instead (in bounds: lane offsets stay below n / 2
      // bytes), which is never read.
      if (j == 0) buffer_to_lds4(scales + g * n + n0, moff[i], wl + S::W_DW + 64 * j);
      else if (j >= 2 && j < S::MSLOTS) buffer_to_lds4(xsum + g * m + m0, moff[i], wl + S::W_DW + 64 * j);
      else if (qzeros) buffer_to_lds4(qzeros + g * (n >> 3) + (n0 >> 3), moff[i], wl + S::W_DW + 64 * j);
      else buffer_to_lds4(scales + g * n + n0, moff[i], wl + S::W_DW + 64 * j);
    }
    if constexpr (LORA) {
      uint32_t* al = wl + S::W_DW + S::M_DW;
      const uint16_t* abase = lora.a + 64 * (int64_t)(kt0 + st);
#pragma unroll
      for (int i = 0; i < S::AL; ++i) buffer_to_lds4(abase, aoff[i], al + T * i + 64 * wave);
    }
  };

  f32x4 total[FM][4], acc[FM][4], xs[PREP ? 1 : FM];
  f32x4 uacc[LORA ? FM : 1];   // LoRA: this wave's share of U for its rows (rank = lane % 16)
#pragma unroll
  for (int f = 0; f < (LORA ? FM : 1); ++f) uacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wn = wave / NWM;     // column wave: takes U for k step wn of each stage
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c) total[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

  const int ktiles = 2 * (gend - gbeg);   // stages of this slice
  // raw fragments of one k step: FM activation chunks and one 16-byte word read
  u32x4 fa[FM], fw;
  auto read_step = [&](int kt, int s) {
    const uint32_t* st = psm_i4 + (size_t)(kt % STAGES) * S::STAGE_DW;
    const u32x4* la = reinterpret_cast<const u32x4*>(st);
#pragma unroll
    for (int f = 0; f < FM; ++f) fa[f] = la[swz(wm0 + 16 * f + cl, 4 * s + ks)];
    fw = *reinterpret_cast<const u32x4*>(st + S::X_DW + (4 * s + ks) * BN + wn0 + 4 * cl);
  };

  // LoRA add (once per output: slice 0 of a split tile): total starts at
  // scale * U[rows] . B[cols]^T, four 16x16x4 fp32 MFMAs per 16 x 16 block
  // with the block's rows of U as A and its fragment's columns 4 l + c of B
  // as B; MFMA j takes rank index r = 4 k4 + j (k4 = lane / 16) from both, so
  // a lane's operands are four consecutive entries of a U row (one 16-byte
  // load) and of a B row (one 8-byte load when B's rows hold 16 aligned
  // entries; else element loads).  The result lands in the layout of total.
  // The operands are loaded before the prologue's stage loads and multiplied
  // once the first stage has landed.  U's columns past the rank are zero; B
  // is used only below the rank (clamped addresses, selects after the loads).
  const bool lora_on = lora.u && kslice == 0;
  f32x4 ua[FM];
  float bb[4][4];
  if (lora_on) {
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int64_t row = m0 + wm0 + 16 * f + cl;
      const f32x4 v = *reinterpret_cast<const f32x4*>(lora.u + (row < m ? row : m - 1) * 16 + 4 * ks);
      ua[f] = row < m ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool bvec = lora.ldb >= 16 && (lora.ldb & 3) == 0 && ((uintptr_t)lora.b & 7u) == 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t col = n0 + wn0 + 4 * cl + c;
      const uint16_t* brow = lora.b + (col < n ? col : n - 1) * lora.ldb;
      uint32_t h[4];
      if (bvec) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(brow + 4 * ks);
        h[0] = w[0] & 0xFFFFu; h[1] = w[0] >> 16; h[2] = w[1] & 0xFFFFu; h[3] = w[1] >> 16;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = brow[4 * ks + j < lora.rank ? 4 * ks + j : 0];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j][c] = (col < n && 4 * ks + j < lora.rank) ? bf16_bits_to_float(h[j]) : 0.f;
    }
  }

  // all STAGES buffers start filling; stage 0 must land before the first read
#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < ktiles) issue(st);
  if (ktiles >= STAGES) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 1)));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  lds_barrier();
  read_step(0, 0);
  if (lora_on) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int c = 0; c < 4; ++c) total[f][c] = mfma16_f32(ua[f][j], bb[j][c], total[f][c]);
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) total[f][c][v] *= lora.scale;
  }

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < (ktiles >> 1); ++g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kt = 2 * g + h;
      u32x4 bn[4];   // the second k step's decoded words, decoded under the first step's MFMAs
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // reorder / decode this step's fragments (their LDS reads were issued
        // one step earlier, under the previous step's MFMAs); prepared
        // activations are already in pair order
        u32x4 ap[FM], b[4];
#pragma unroll
        for (int f = 0; f < FM; ++f) ap[f] = PREP ? fa[f] : x_pairs_permuted(fa[f]);
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = s == 0 ? codes_as_bf16_pairs(fw[c]) : bn[c];
        if (s == 0) read_step(kt, 1);
        const bool first = h == 0 && s == 0;   // first k step of the group
        // the ones-MFMA sums the reordered activations; a sum's order does not matter
#pragma unroll
        for (int f = 0; f < FM; ++f) {
          if constexpr (!PREP) xs[f] = mfma16_bf16(ap[f], ones, first ? zero : xs[f]);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[f][c] = mfma16_bf16(ap[f], b[c], first ? zero : acc[f][c]);
        }
        if constexpr (LORA) {
          // U[rows][rank] += x . lora_A^T for this k step, by one of the two column
          // waves (the other takes the stage's other step): lora_A row cl, chunk
          // 4 s + ks, in the activations' pair order
          if (wn == s) {
            const uint32_t* al = psm_i4 + (size_t)(kt % STAGES) * S::STAGE_DW + S::X_DW + S::W_DW + S::M_DW;
            const int q = 4 * s + ks;
            const u32x4 raw = *reinterpret_cast<const u32x4*>(al + 32 * cl + 4 * (q ^ (cl & 7)));
            const u32x4 av = cl < lora.rank ? x_pairs_permuted(raw) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int f = 0; f < FM; ++f) uacc[f] = mfma16_bf16(ap[f], av, uacc[f]);
          }
        }
        if (s == 0) {
          // the second step's words (fw now holds them once the reads above
          // land) are decoded while the first step's MFMAs run: the matrix
          // core and the vector ALU then work side by side.  Scheduling
          // order of this step: its own decode, the next step's LDS reads,
          // four MFMAs (covering the read latency), then one MFMA per three
          // decode instructions.
#pragma unroll
          for (int c = 0; c < 4; ++c) bn[c] = codes_as_bf16_pairs(fw[c]);
          if constexpr (PREP && QG_PIPE_INTERLEAVE) {
            __builtin_amdgcn_sched_group_barrier(0x002, 28, 0);   // VALU: this step's decode
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);    // DS reads of the next step
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);    // MFMA
#pragma unroll
            for (int i = 0; i < 12; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU: next step's decode
            }
          }
        }
      }
      // the group's scales, zeros (and prepared group sums), read while stage
      // kt is still ours
      float sc[4], bz[4];
      f32x4 gs[FM];   // group sums of this lane's accumulator rows 4 ks + v
      if (h == 1) {
        const uint32_t* lm = psm_i4 + (size_t)(kt % STAGES) * S::STAGE_DW + S::X_DW + S::W_DW;
#pragma unroll
        for (int f = 0; f < FM; ++f)
          gs[f] = PREP ? *reinterpret_cast<const f32x4*>(lm + 128 + wm0 + 16 * f + 4 * ks) : xs[PREP ? 0 : f];
        const int col = wn0 + 4 * cl;
        const u32x2 sv = *reinterpret_cast<const u32x2*>(lm + (col >> 1));
        const uint32_t zw = qzeros ? lm[BN / 2 + (col >> 3)] >> (4 * (col & 7)) : 0u;
        sc[0] = half_bits_to_float(sv[0] & 0xFFFFu);
        sc[1] = half_bits_to_float(sv[0] >> 16);
        sc[2] = half_bits_to_float(sv[1] & 0xFFFFu);
        sc[3] = half_bits_to_float(sv[1] >> 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) bz[c] = (float)(128u + ((zw >> (4 * c)) & 15u));
      }
      // Stage kt is fully read (fragments and metadata sit in registers).  With
      // the MFMAs above in flight: wait for this wave's loads of stage kt + 1,
      // meet the other waves (after which every wave is done with stage kt and
      // all of stage kt + 1 has landed), refill stage kt's buffer with stage
      // kt + STAGES and read the first fragments of stage kt + 1.
      if (kt + 1 < ktiles) {
        if (kt + STAGES - 1 < ktiles) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 2)));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        lds_barrier();
        if (kt + STAGES < ktiles) issue(kt + STAGES);
        read_step(kt + 1, 0);
      }
      if (h == 1) {
        // end of group g: scale and remove the 128 + z offset
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              total[f][c][v] = __builtin_fmaf(sc[c], __builtin_fmaf(-bz[c], gs[f][v], acc[f][c][v]),
                                              total[f][c][v]);
      }
    }
  }
  if constexpr (LORA) {
    // total += scale * U . B^T for this slice's U (the sum over slices is linear,
    // so every slice adds its own).  The two column waves' shares of U meet in
    // LDS (the stages are done); then four 16x16x4 fp32 MFMAs per 16 x 16 block
    // with a block's U rows as A and its columns of B as B, as for a precomputed U.
    __syncthreads();
    float* ul = reinterpret_cast<float*>(psm_i4);   // [NWN][BM][16]
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) ul[(wn * BM + wm0 + 16 * f + 4 * ks + v) * 16 + cl] = uacc[f][v];
    __syncthreads();
    f32x4 ua[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int row = wm0 + 16 * f + cl;
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(ul + row * 16 + 4 * ks);
      const f32x4 u1 = *reinterpret_cast<const f32x4*>(ul + (BM + row) * 16 + 4 * ks);
      ua[f] = u0 + u1;
    }
    float bb[4][4];
    const bool bvec = lora.ldb >= 16 && (lora.ldb & 3) == 0 && ((uintptr_t)lora.b & 7u) == 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t col = n0 + wn0 + 4 * cl + c;
      const uint16_t* brow = lora.b + (col < n ? col : n - 1) * lora.ldb;
      uint32_t hh[4];
      if (bvec) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(brow + 4 * ks);
        hh[0] = w[0] & 0xFFFFu; hh[1] = w[0] >> 16; hh[2] = w[1] & 0xFFFFu; hh[3] = w[1] >> 16;
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) hh[jj] = brow[4 * ks + jj < lora.rank ? 4 * ks + jj : 0];
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        bb[jj][c] = (col < n && 4 * ks + jj < lora.rank) ? bf16_bits_to_float(hh[jj]) : 0.f;
    }
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x4 lt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) lt = mfma16_f32(ua[f][jj], bb[jj][c], lt);
#pragma unroll
        for (int v = 0; v < 4; ++v) total[f][c][v] = __builtin_fmaf(lora.scale, lt[v], total[f][c][v]);
      }
  }
  if (ksplit > 1) {
    // Split k: every slice stores its fp32 partial tile with agent-coherent
    // stores and takes a ticket; the last slice of the tile to arrive adds the
    // partials in slice order (deterministic) and writes Y.  No fences: the
    // partials are only written and read with agent-coherent accesses, and
    // every thread waits for its stores before the ticket is taken (or, with
    // acq_rel, the ticket orders them).
    // fragment order: element pair (f, v, c / 2) of thread tid at
    // ((f * 4 + v) * 2 + c / 2) * T + tid (8-byte words), so that each store
    // instruction of a wave covers 512 contiguous bytes; the last slice reads
    // with the same thread mapping
    uint64_t* mine = reinterpret_cast<uint64_t*>(partials) + ((int64_t)t * ksplit + kslice) * (BM * BN / 2);
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          // (the element is copied to a scalar first: a bit cast applied to a
          // vector element directly read element 0 whatever the index)
          const float lo = total[f][2 * h2][v], hi = total[f][2 * h2 + 1][v];
          const uint64_t pair = (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                                ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
          __hip_atomic_store(&mine[((f * 4 + v) * 2 + h2) * T + tid], pair, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (tid == 0)
      psm_i4[0] = ticket_add(&tickets[t], acq_rel) == (uint32_t)(ksplit - 1);
    __syncthreads();
    if (!psm_i4[0]) return;
    const uint64_t* base = reinterpret_cast<const uint64_t*>(partials) + (int64_t)t * ksplit * (BM * BN / 2);
    // slice by slice: the 8 FM pairs of a slice are loaded together (one round
    // trip per slice, not per element), then added; each element still sums
    // the slices in slice order
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c) total[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < ksplit; ++p) {
      const uint64_t* sl = base + (int64_t)p * (BM * BN / 2);
      uint64_t pr[FM][4][2];
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            pr[f][v][h2] = __hip_atomic_load(&sl[((f * 4 + v) * 2 + h2) * T + tid], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            total[f][2 * h2][v] += __builtin_bit_cast(float, (uint32_t)pr[f][v][h2]);
            total[f][2 * h2 + 1][v] += __builtin_bit_cast(float, (uint32_t)(pr[f][v][h2] >> 32));
          }
    }
    if (tid == 0) __hip_atomic_store(&tickets[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // output tile through LDS, then 16-byte (or 8-byte) row stores
  uint16_t* osm = reinterpret_cast<uint16_t*>(psm_i4);
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = wm0 + 16 * f + 4 * ks + v;
      u32x2 o;
      o[0] = pack_bf16x2(total[f][0][v], total[f][1][v]);
      o[1] = pack_bf16x2(total[f][2][v], total[f][3][v]);
      *reinterpret_cast<u32x2*>(&osm[row * S::OP + wn0 + 4 * cl]) = o;
    }
  __syncthreads();
  constexpr int CPR = BN / 8;
  for (int c = tid; c < BM * CPR; c += T) {
    const int r = c / CPR, cc = c - r * CPR;
    const int gr = m0 + r, gc = n0 + 8 * cc;
    const bool in = gr < m && gc < n;
    const uint16_t* src = &osm[r * S::OP + 8 * cc];
    if (in) {
      uint16_t* dst = y + (int64_t)gr * ldy + gc;
      if (vec_store) {
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      } else {
        reinterpret_cast<u32x2*>(dst)[0] = reinterpret_cast<const u32x2*>(src)[0];
        reinterpret_cast<u32x2*>(dst)[1] = reinterpret_cast<const u32x2*>(src)[1];
      }
    }
    if (lora.row_ss) {   // the CPR lanes of a row: one aligned group
      float q = 0.f;
      if (in) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_bits_to_float(w[i] & 0xFFFFu), hi = bf16_bits_to_float(w[i] >> 16);
          q = __builtin_fmaf(lo, lo, q);
          q = __builtin_fmaf(hi, hi, q);
        }
      }
      add_row_sumsq<CPR>(lora.row_ss, q, gr, cc == 0, gr < m);
    }
  }
}

// ---------------------------------------------------------------------------
// launch shapes of the skinny kernel
// ---------------------------------------------------------------------------
#ifndef QG_SKINNY_MIN_STRIPS
#define QG_SKINNY_MIN_STRIPS 256   // strips wanted before widening them
#endif
#ifndef QG_SKINNY_WAVES
#define QG_SKINNY_WAVES 16         // waves per workgroup at most
#endif
#ifndef QG_SKINNY_MAX_GPW
#define QG_SKINNY_MAX_GPW 6        // groups per wave above which k is split
#endif
#ifndef QG_SKINNY_WIDE_M
#define QG_SKINNY_WIDE_M 1         // tokens from which wide strips pay for a k split
#endif
#ifndef QG_SKINNY_GPW_MIN
#define QG_SKINNY_GPW_MIN 1        // groups per wave the wave count aims at (at least)
#endif
// More strips than CUs: 8-wave workgroups, so that two fit on a CU and the
// strips take one pass instead of two (257-383 strips with 16 waves took two):
// 2048 x 5632 m = 1 / 8 / 15 6.38 / 7.49 / 8.83 -> 5.45 / 6.61 / 7.90 µs,
// 4096 x 11008 m = 8 12.6 -> 11.6 µs, 2048 x 9216 m = 8 8.50 -> 7.11 µs.
#ifndef QG_SKINNY_MANY_STRIPS
#define QG_SKINNY_MANY_STRIPS 257  // strips from which workgroups have 8 waves (two per CU)
#endif
#ifndef QG_SKINNY_LONG_G
#define QG_SKINNY_LONG_G 48        // groups from which MFMA strips (m >= 8) use 8-wave workgroups
#endif
// 128-column strips (m <= 16, MFMA) where k is split anyway and each slice
// keeps at least QG_SKINNY_CPL8_MIN_GPS groups: half the activation reads per
// column (every workgroup reads X over its k range), one 512-thread workgroup
// per CU.  Same-process A/B, cold weights, against 64-column strips:
// 25600 x 5120 m = 2 / 8 / 16 24.9 / 22.9 / 26.3 -> 18.2 / 20.1 / 23.1 µs,
// 32768 x 8192 m = 8 41.9 -> 31.2 µs, 25600 x 7168 m = 16 34.9 -> 29.2 µs,
// 28672 x 4096 m = 16 (28 groups per slice) 23.1 -> 21.2 µs; but 14336 x
// 4096 m = 16 (14 groups per slice) 13.4 -> 15.7 µs.
#ifndef QG_SKINNY_CPL8
#define QG_SKINNY_CPL8 1
#endif
#ifndef QG_SKINNY_CPL8_MIN_GPS
#define QG_SKINNY_CPL8_MIN_GPS 20
#endif
#ifndef QG_SKINNY_CPL8_MIN_STRIPS
#define QG_SKINNY_CPL8_MIN_STRIPS 192   // 128-column strips without a split: at least this many
#endif

int64_t split_workspace_bytes(int64_t nstrips, int64_t ksplit, int64_t m, int cpl) {
  return kTicketBytes + nstrips * ksplit * m * 16 * cpl * 4;
}

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int64_t workspace_bytes, bool dot) {
  SkinnyPlan p{};
  const int64_t G = k / 128;
  // widest strip the registers allow: 64 columns up to 32 tokens, 32 up to 48,
  // 16 above (each row tile adds accumulators and double-buffered activations)
  const int cplmax = dot || m <= 32 ? 4 : (m <= 48 ? 2 : 1);
  // widest strip that still leaves enough strips for the CUs
  p.cpl = 1;
  if ((n + 63) / 64 >= QG_SKINNY_MIN_STRIPS) p.cpl = 4;
  else if ((n + 31) / 32 >= QG_SKINNY_MIN_STRIPS) p.cpl = 2;
  // When 32-column strips are so many (>= 384) that they take 8-wave
  // workgroups at 1.5-2 per CU, 64-column strips at one 16-wave workgroup per
  // CU (192-256 of them) balance the CUs, load 16 bytes per lane and halve the
  // activation reads (every strip reads all of X): 4096 x 14336 m = 1 / 8 / 16
  // 12.8 / 13.8 / 17.2 -> 10.3 / 10.9 / 12.5 µs.
  if (p.cpl == 2 && (n + 31) / 32 >= 384) {
    const int64_t s4 = (n + 63) / 64;
    if (s4 >= 192 && s4 <= 256) p.cpl = 4;
  }
  if (p.cpl > cplmax) p.cpl = cplmax;
  const int sw = 16 * p.cpl;
  p.nstrips = (int)((n + sw - 1) / sw);
  // more strips than CUs: 8-wave workgroups so that two fit on a CU; few: 16 waves.
  // One group per wave: every wave's loads go out at once (a wave waits for
  // all of its loads in flight at each group, so a chain of groups costs a
  // memory latency per link).  Long k with m >= 8: 8 waves (longer chains,
  // and a k split chosen for them) measured faster than 16: 25600 x 5120
  // m = 16 33.3 -> 28.7 µs, 8192 x 8192 m = 8 / 16 14.2 / 17.0 -> 13.5 / 15.2 µs;
  // at 4096 x 4096 and for the GEMV they were slower.
  const bool long_k = !dot && m >= 8 && G >= QG_SKINNY_LONG_G;
  // above 16 tokens (two row tiles) the kernel is bounded to 512 threads
  const int64_t wcap = (p.nstrips >= QG_SKINNY_MANY_STRIPS || long_k || m > 16) ? (QG_SKINNY_WAVES < 8 ? QG_SKINNY_WAVES : 8)
                                                               : QG_SKINNY_WAVES;
  p.waves = (int)(G < QG_SKINNY_GPW_MIN ? 1 : (G / QG_SKINNY_GPW_MIN < wcap ? G / QG_SKINNY_GPW_MIN : wcap));
  // k split only when each wave would otherwise walk a long chain of groups
  int64_t ks = 1;
  const int64_t per_wave = (G + p.waves - 1) / p.waves;
  if (per_wave > QG_SKINNY_MAX_GPW && (int64_t)p.nstrips * 4 <= kTicketBytes) {
    ks = (per_wave + 3) / 4;
    if (ks > SK_MAX_SPLIT) ks = SK_MAX_SPLIT;
  }
  // Without a split, 64-column strips that need two workgroups per CU (more
  // than 256) become 128-column strips in one pass of one 8-wave workgroup per
  // CU when those still cover most CUs (same-process A/B, cold weights:
  // 4096 x 28672 m = 4 / 8 / 16 16.3 / 17.0 / 19.2 -> 15.8 / 16.3 / 18.1 µs,
  // 5120 x 25600 m = 8 / 16 20.2 / 23.5 -> 18.7 / 21.6 µs, 4096 x 32768 m = 16
  // 19.2 -> 18.2 µs).
  if (QG_SKINNY_CPL8 && !dot && m <= 16 && ks == 1 && p.cpl == 4 && p.nstrips > 256) {
    const int64_t s8 = (n + 127) / 128;
    if (s8 >= QG_SKINNY_CPL8_MIN_STRIPS && s8 <= 256 && G <= 8 * QG_SKINNY_MAX_GPW) {
      p.cpl = 8;
      p.nstrips = (int)s8;
      p.waves = (int)(G < 8 ? (G > 0 ? G : 1) : 8);
    }
  }
  // When k is long enough to be split anyway, take the widest strip whose
  // count, times a split of at most SK_MAX_SPLIT, still fills the CUs: every
  // workgroup reads X over its k range (X traffic = strips x m x k x 2 bytes,
  // 4m / (16 CPL) times the codes' traffic) and wider strips load more code
  // bytes per instruction.  Measured at k = 25600, n = 5120: m = 1 40 -> 29 µs,
  // m = 2 39 -> 27 µs, m = 16 57 -> 35 µs.
  const int cplwide = QG_SKINNY_CPL8 && !dot && m <= 16 ? 8 : cplmax;
  if ((dot || m >= QG_SKINNY_WIDE_M) && ks > 1 && p.cpl < cplwide) {
    for (int c = cplwide; c > p.cpl; c /= 2) {
      const int64_t strips = (n + 16 * c - 1) / (16 * c);
      // (128-column strips: 512-thread workgroups, twice the accumulators)
      const int64_t wc = (strips >= QG_SKINNY_MANY_STRIPS || long_k || m > 16 || c > 4)
                             ? (QG_SKINNY_WAVES < 8 ? QG_SKINNY_WAVES : 8)
                             : QG_SKINNY_WAVES;
      const int64_t wv = G < QG_SKINNY_GPW_MIN ? 1 : (G / QG_SKINNY_GPW_MIN < wc ? G / QG_SKINNY_GPW_MIN : wc);
      const int64_t pw = (G + wv - 1) / wv;
      int64_t kc = (pw + 3) / 4;
      const int64_t fill = (QG_SKINNY_MIN_STRIPS + strips - 1) / strips;
      if (kc < fill) kc = fill;
      if (c == 8) {
        // one 512-thread workgroup per CU (the registers allow no second): as
        // many slices as fit one pass, and only when each slice keeps a long
        // chain of groups
        kc = 256 / strips;
        if (kc < 2 || G / kc < QG_SKINNY_CPL8_MIN_GPS) continue;
        if (split_workspace_bytes(strips, kc, m, c) > workspace_bytes) continue;   // (no split: not these)
      }
      if (kc > SK_MAX_SPLIT || kc > G || strips * 4 > kTicketBytes) continue;
      p.cpl = c;
      p.nstrips = (int)strips;
      p.waves = (int)wv;
      ks = kc;
      break;
    }
  }
#ifdef QG_SKINNY_FORCE_CPL   // launch-shape sweeps: strip width, k split and waves fixed from m on
  if (m >= QG_SKINNY_FORCE_MINM) {
    p.cpl = QG_SKINNY_FORCE_CPL;
    p.nstrips = (int)((n + 16 * p.cpl - 1) / (16 * p.cpl));
    ks = QG_SKINNY_FORCE_KS < G ? QG_SKINNY_FORCE_KS : (G > 0 ? G : 1);
    p.waves = QG_SKINNY_FORCE_WAVES;
  }
#endif
  const int sw2 = 16 * p.cpl;
  int64_t gwg = (G + ks - 1) / ks;
  ks = G > 0 ? (G + gwg - 1) / gwg : 1;
  int64_t need = ks > 1 ? split_workspace_bytes(p.nstrips, ks, m, p.cpl) : 0;
  if (need > workspace_bytes) {       // no room for the partials: one slice per strip
    ks = 1;
    gwg = G;
    need = 0;
  }
  p.ksplit = (int)ks;
  p.gwg = (int)gwg;
  p.ws_bytes = need;
  // no more waves than groups in a slice: a wave without a group would still
  // load one and widen the partial plane
  if (gwg >= 1 && p.waves > gwg) p.waves = (int)gwg;
  const int64_t items = (int64_t)p.nstrips * p.ksplit;
  p.items_per_xcd = (int)((items + 7) / 8);
  p.blocks = (int64_t)p.items_per_xcd * 8;
  p.lds = (size_t)p.waves * m * sw2 * 4;   // the wave partial plane
  (void)dot;
  return p;
}

template <int M, bool DOT, int CPL>
static void skinny_launch(const Int4Args& a, const SkinnyPlan& p, void* ws, hipStream_t stream) {
  uint32_t* tickets = (uint32_t*)ws;
  float* partials = ws ? (float*)((char*)ws + kTicketBytes) : nullptr;
  skinny_int4_kernel<M, DOT, CPL><<<dim3((unsigned)p.blocks), dim3(64 * p.waves), p.lds, stream>>>(
      a.x, a.ldx, a.qweight, a.scales, a.qzeros, a.y, a.ldy, (int)a.n, (int)a.k, p.nstrips,
      p.ksplit, p.gwg, p.items_per_xcd, partials, tickets, a.split_acq_rel, a.lora);
}

template <int M, bool DOT>
static void skinny_launch_c(const Int4Args& a, const SkinnyPlan& p, void* ws, hipStream_t stream) {
  if constexpr (M <= 32) {
    if constexpr (M <= 16 && !DOT && QG_SKINNY_CPL8) {
      if (p.cpl == 8) {
        skinny_launch<M, DOT, 8>(a, p, ws, stream);
        return;
      }
    }
    if (p.cpl == 4) skinny_launch<M, DOT, 4>(a, p, ws, stream);
    else if (p.cpl == 2) skinny_launch<M, DOT, 2>(a, p, ws, stream);
    else skinny_launch<M, DOT, 1>(a, p, ws, stream);
  } else if constexpr (M <= 48) {   // the planner caps the strip width by the token count
    if (p.cpl >= 2) skinny_launch<M, DOT, 2>(a, p, ws, stream);
    else skinny_launch<M, DOT, 1>(a, p, ws, stream);
  } else {
    skinny_launch<M, DOT, 1>(a, p, ws, stream);
  }
}

// Launch shape of skinny_lds_kernel for a small-M plan, or ng = 0 where it does
// not apply: a k split, m > 16, more than 64 groups, or more strips than one
// pass over the CUs takes (its LDS holds all of a strip's codes).  NG groups
// per wave: 1 up to 16 groups, 2 up to 32, 4 up to 64; waves = ceil(G / NG).
struct LdsPlan {
  int ng, waves, plane_off;
  bool xl;   // activations staged in LDS as well
  size_t lds;
};

// More strips than CUs: at least two groups per wave (half the waves), so two
// workgroups share a CU at 16 waves: 2048 x 5632 (352 strips) m = 1 / 8 / 15
// 5.76 / 6.91 / 8.17 -> 5.05 / 6.11 / 7.16 µs (the register-staged kernel:
// 5.48 / 6.62 / 7.91).  Padding the LDS to one workgroup per CU for 256
// strips changed nothing (within 1%).
#ifndef QG_LDS_MANY_NG
#define QG_LDS_MANY_NG 2
#endif

static LdsPlan plan_lds(int64_t m, const SkinnyPlan& p, int64_t k, bool dot, bool lora = false) {
  LdsPlan r{0, 0, 0, false, 0};
  const int64_t G = k / 128;
  if (m > 16 || p.ksplit != 1 || G < 1 || p.cpl > 4) return r;
  int ng = G <= 16 ? 1 : (G <= 32 ? 2 : (G <= 64 ? 4 : 0));
  if (p.nstrips > 256 && ng > 0 && ng < QG_LDS_MANY_NG && G > 8) ng = G <= 32 ? 2 : 4;
  const int la = lora ? 4 : 0;                                 // lora_A loads per group
  if (ng == 0 || ng * (p.cpl + 6 + la) > 63) return r;
  const int waves = (int)((G + ng - 1) / ng);
  // epilogue: the wave partial plane, and with LoRA the wave partials of U and U
  const size_t plane = (size_t)waves * m * 16 * p.cpl * 4 + (lora ? (size_t)(waves + 1) * m * 16 * 4 : 0);
  const int xi = dot ? 1 : (int)((m + 3) / 4);                 // activation loads per group
  // the activations join the codes in LDS when both fit (strips of 16 and 32
  // columns) and the workgroups still take one pass; else they go to registers
  for (int xl = 1; xl >= 0; --xl) {
    if (xl && (p.cpl > 2 || ng * (p.cpl + xi + 2 + la) > 63)) continue;
    const size_t codes = (size_t)G * 16 * 16 * p.cpl * 4 + (xl ? (size_t)G * (dot ? 256 : 1024 * xi) : 0);
    size_t lds = codes + plane;
    int plane_off = (int)codes;
    if (lds > 160 * 1024) {
      lds = codes > plane ? codes : plane;
      plane_off = 0;
    }
    if (lds > 160 * 1024) continue;
    const int64_t by_lds = (int64_t)(160 * 1024 / lds), by_waves = 32 / waves;
    const int64_t per_cu = by_lds < by_waves ? by_lds : by_waves;
    if (per_cu < 1 || p.nstrips > 256 * per_cu) continue;
    r.ng = ng;
    r.waves = waves;
    r.plane_off = plane_off;
    r.xl = xl != 0;
    r.lds = lds;
    return r;
  }
  return r;
}

// The strip plan without a k split (the strip width by n alone), for the
// LDS-staged kernel where the register-staged plan would split k.
static SkinnyPlan plan_whole_k(int64_t m, int64_t n, int64_t k, bool dot) {
  SkinnyPlan p = plan_skinny(m, n, k, 0, dot);
  const int cplmax = dot || m <= 32 ? 4 : (m <= 48 ? 2 : 1);
  int cpl = 1;
  if ((n + 63) / 64 >= QG_SKINNY_MIN_STRIPS) cpl = 4;
  else if ((n + 31) / 32 >= QG_SKINNY_MIN_STRIPS) cpl = 2;
  if (cpl == 2 && (n + 31) / 32 >= 384) {
    const int64_t s4 = (n + 63) / 64;
    if (s4 >= 192 && s4 <= 256) cpl = 4;
  }
  if (cpl > cplmax) cpl = cplmax;
  p.cpl = cpl;
  p.nstrips = (int)((n + 16 * cpl - 1) / (16 * cpl));
  p.ksplit = 1;
  p.gwg = (int)(k / 128);
  p.ws_bytes = 0;
  p.items_per_xcd = (p.nstrips + 7) / 8;
  p.blocks = (int64_t)p.items_per_xcd * 8;
  return p;
}

#ifndef QG_LDS_PREFER_WHOLE_K
#define QG_LDS_PREFER_WHOLE_K 1
#endif

// The plan the small-M paths launch: the register-staged plan, or the
// LDS-staged kernel over the whole k where the register-staged plan splits k
// (or has no LDS-staged form) and the whole-k strips fill the CUs.  Measured
// (cold weights): 32-column strips and the GEMV gain, 16-column strips with
// m >= 2 lose (the split's extra workgroups hide more latency there):
// 8192 x 8192 m = 8 / 16 13.0 / 14.5 -> 11.6 / 13.8 µs, 7168 x 8192 m = 15
// 13.1 -> 12.6 µs, 8192 x 5632 m = 1 13.7 -> 12.9 µs, but 8192 x 5632
// m = 16 15.6 -> 21.2 µs.
static SkinnyPlan plan_small_m(int64_t m, int64_t n, int64_t k, int64_t ws_bytes, bool dot) {
  const SkinnyPlan p = plan_skinny(m, n, k, ws_bytes, dot);
  if (QG_LDS_PREFER_WHOLE_K && m <= 16 && (p.ksplit > 1 || plan_lds(m, p, k, dot).ng == 0)) {
    const SkinnyPlan q = plan_whole_k(m, n, k, dot);
    if (q.nstrips >= QG_SKINNY_MIN_STRIPS && (dot || q.cpl >= 2) && plan_lds(m, q, k, dot).ng > 0) return q;
  }
  return p;
}

template <int M, bool DOT, int CPL, int NG, bool XL, bool LORA>
static void lds_launch_k(const Int4Args& a, const SkinnyPlan& p, const LdsPlan& l, hipStream_t stream) {
  skinny_lds_kernel<M, DOT, CPL, NG, XL, LORA><<<dim3((unsigned)p.blocks), dim3(64 * l.waves), l.lds, stream>>>(
      a.x, a.ldx, a.qweight, a.scales, a.qzeros, a.y, a.ldy, (int)a.n, (int)a.k, p.nstrips, p.items_per_xcd,
      l.plane_off, a.lora);
}

template <int M, bool DOT, int CPL, int NG>
static void lds_launch(const Int4Args& a, const SkinnyPlan& p, const LdsPlan& l, hipStream_t stream) {
  const bool lora = a.lora.a != nullptr;
  if constexpr (CPL <= 2) {
    if (l.xl) {
      if (lora) lds_launch_k<M, DOT, CPL, NG, true, true>(a, p, l, stream);
      else lds_launch_k<M, DOT, CPL, NG, true, false>(a, p, l, stream);
      return;
    }
  }
  if (lora) lds_launch_k<M, DOT, CPL, NG, false, true>(a, p, l, stream);
  else lds_launch_k<M, DOT, CPL, NG, false, false>(a, p, l, stream);
}

template <int M, bool DOT, int CPL>
static void lds_launch_n(const Int4Args& a, const SkinnyPlan& p, const LdsPlan& l, hipStream_t stream) {
  if (l.ng == 4) lds_launch<M, DOT, CPL, 4>(a, p, l, stream);
  else if (l.ng == 2) lds_launch<M, DOT, CPL, 2>(a, p, l, stream);
  else lds_launch<M, DOT, CPL, 1>(a, p, l, stream);
}

// Launches the LDS-staged kernel when it applies (returns false otherwise).
template <int M, bool DOT>
static bool lds_launch_c(const Int4Args& a, const SkinnyPlan& p, hipStream_t stream) {
  if constexpr (M > 16) {
    return false;
  } else {
    const LdsPlan l = plan_lds(M, p, a.k, DOT, a.lora.a != nullptr);
    if (l.ng == 0) return false;
    if (p.cpl == 4) lds_launch_n<M, DOT, 4>(a, p, l, stream);
    else if (p.cpl == 2) lds_launch_n<M, DOT, 2>(a, p, l, stream);
    else lds_launch_n<M, DOT, 1>(a, p, l, stream);
    return true;
  }
}

// Where U goes (measured, cold weights, rank 16; ratio to the plain product):
// the LDS-staged small-M kernel accumulates it from the activations it already
// holds -- 4096 x 4096 m = 1 / 8 / 15 1.52 / 1.49 / 1.51 (two extra launches
// first: 1.97 / 1.82 / 1.72), 2048 x 8192 1.30 / 1.35 / 1.32 (2.05 / 1.99 /
// 1.89).  The MFMA tiles recompute U in every column tile (an extra 16-column
// MFMA per k step and row fragment, +12.5%), which beats two launches only
// for short products: 4096 x 4096 m = 130 1.13 (1.20), but 25600 x 5120
// m = 512 1.16 (1.08) and 5120 x 25600 m = 2048 1.20 (1.05); so the tiles
// take U in the launch up to 2^34 flops.  The register-staged small-M kernel
// (k splits, 17..64 tokens) has no registers to spare for it.
#ifndef QG_LORA_TILE_MAX_FLOPS
#define QG_LORA_TILE_MAX_FLOPS 17179869184.0
#endif
bool lora_in_launch(const Int4Args& a, int path, int64_t ws_bytes) {
  if (path == 3) return 2.0 * (double)a.m * (double)a.n * (double)a.k <= QG_LORA_TILE_MAX_FLOPS;
  if (a.m > 16) return false;
  const bool dot = path == 1;
  const SkinnyPlan p = plan_small_m(dot ? 1 : a.m, a.n, a.k, ws_bytes, dot);
  return plan_lds(dot ? 1 : a.m, p, a.k, dot, true).ng > 0;
}

hipError_t launch_gemv_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const SkinnyPlan p = plan_small_m(1, a.n, a.k, ws ? ws_bytes : 0, true);
  if (!lds_launch_c<1, true>(a, p, stream)) skinny_launch_c<1, true>(a, p, ws, stream);
  return hipGetLastError();
}

hipError_t launch_fused_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const SkinnyPlan p = plan_small_m(a.m, a.n, a.k, ws ? ws_bytes : 0, false);
  switch (a.m) {
    case 1: if (!lds_launch_c<1, false>(a, p, stream)) skinny_launch_c<1, false>(a, p, ws, stream); break;
    case 2: if (!lds_launch_c<2, false>(a, p, stream)) skinny_launch_c<2, false>(a, p, ws, stream); break;
    case 3: if (!lds_launch_c<3, false>(a, p, stream)) skinny_launch_c<3, false>(a, p, ws, stream); break;
    case 4: if (!lds_launch_c<4, false>(a, p, stream)) skinny_launch_c<4, false>(a, p, ws, stream); break;
    case 5: if (!lds_launch_c<5, false>(a, p, stream)) skinny_launch_c<5, false>(a, p, ws, stream); break;
    case 6: if (!lds_launch_c<6, false>(a, p, stream)) skinny_launch_c<6, false>(a, p, ws, stream); break;
    case 7: if (!lds_launch_c<7, false>(a, p, stream)) skinny_launch_c<7, false>(a, p, ws, stream); break;
    case 8: if (!lds_launch_c<8, false>(a, p, stream)) skinny_launch_c<8, false>(a, p, ws, stream); break;
    case 9: if (!lds_launch_c<9, false>(a, p, stream)) skinny_launch_c<9, false>(a, p, ws, stream); break;
    case 10: if (!lds_launch_c<10, false>(a, p, stream)) skinny_launch_c<10, false>(a, p, ws, stream); break;
    case 11: if (!lds_launch_c<11, false>(a, p, stream)) skinny_launch_c<11, false>(a, p, ws, stream); break;
    case 12: if (!lds_launch_c<12, false>(a, p, stream)) skinny_launch_c<12, false>(a, p, ws, stream); break;
    case 13: if (!lds_launch_c<13, false>(a, p, stream)) skinny_launch_c<13, false>(a, p, ws, stream); break;
    case 14: if (!lds_launch_c<14, false>(a, p, stream)) skinny_launch_c<14, false>(a, p, ws, stream); break;
    case 15: if (!lds_launch_c<15, false>(a, p, stream)) skinny_launch_c<15, false>(a, p, ws, stream); break;
    case 16: if (!lds_launch_c<16, false>(a, p, stream)) skinny_launch_c<16, false>(a, p, ws, stream); break;
    // two MFMA row tiles (the automatic path sends 16 < m <= 32 here when n is small)
    case 17: skinny_launch_c<17, false>(a, p, ws, stream); break;
    case 18: skinny_launch_c<18, false>(a, p, ws, stream); break;
    case 19: skinny_launch_c<19, false>(a, p, ws, stream); break;
    case 20: skinny_launch_c<20, false>(a, p, ws, stream); break;
    case 21: skinny_launch_c<21, false>(a, p, ws, stream); break;
    case 22: skinny_launch_c<22, false>(a, p, ws, stream); break;
    case 23: skinny_launch_c<23, false>(a, p, ws, stream); break;
    case 24: skinny_launch_c<24, false>(a, p, ws, stream); break;
    case 25: skinny_launch_c<25, false>(a, p, ws, stream); break;
    case 26: skinny_launch_c<26, false>(a, p, ws, stream); break;
    case 27: skinny_launch_c<27, false>(a, p, ws, stream); break;
    case 28: skinny_launch_c<28, false>(a, p, ws, stream); break;
    case 29: skinny_launch_c<29, false>(a, p, ws, stream); break;
    case 30: skinny_launch_c<30, false>(a, p, ws, stream); break;
    case 31: skinny_launch_c<31, false>(a, p, ws, stream); break;
    case 32: skinny_launch_c<32, false>(a, p, ws, stream); break;
    // three and four row tiles (the automatic path sends 32 < m <= 64 here when
    // the planned workgroups take a single pass over the CUs)
    case 33: skinny_launch_c<33, false>(a, p, ws, stream); break;
    case 34: skinny_launch_c<34, false>(a, p, ws, stream); break;
    case 35: skinny_launch_c<35, false>(a, p, ws, stream); break;
    case 36: skinny_launch_c<36, false>(a, p, ws, stream); break;
    case 37: skinny_launch_c<37, false>(a, p, ws, stream); break;
    case 38: skinny_launch_c<38, false>(a, p, ws, stream); break;
    case 39: skinny_launch_c<39, false>(a, p, ws, stream); break;
    case 40: skinny_launch_c<40, false>(a, p, ws, stream); break;
    case 41: skinny_launch_c<41, false>(a, p, ws, stream); break;
    case 42: skinny_launch_c<42, false>(a, p, ws, stream); break;
    case 43: skinny_launch_c<43, false>(a, p, ws, stream); break;
    case 44: skinny_launch_c<44, false>(a, p, ws, stream); break;
    case 45: skinny_launch_c<45, false>(a, p, ws, stream); break;
    case 46: skinny_launch_c<46, false>(a, p, ws, stream); break;
    case 47: skinny_launch_c<47, false>(a, p, ws, stream); break;
    case 48: skinny_launch_c<48, false>(a, p, ws, stream); break;
    case 49: skinny_launch_c<49, false>(a, p, ws, stream); break;
    case 50: skinny_launch_c<50, false>(a, p, ws, stream); break;
    case 51: skinny_launch_c<51, false>(a, p, ws, stream); break;
    case 52: skinny_launch_c<52, false>(a, p, ws, stream); break;
    case 53: skinny_launch_c<53, false>(a, p, ws, stream); break;
    case 54: skinny_launch_c<54, false>(a, p, ws, stream); break;
    case 55: skinny_launch_c<55, false>(a, p, ws, stream); break;
    case 56: skinny_launch_c<56, false>(a, p, ws, stream); break;
    case 57: skinny_launch_c<57, false>(a, p, ws, stream); break;
    case 58: skinny_launch_c<58, false>(a, p, ws, stream); break;
    case 59: skinny_launch_c<59, false>(a, p, ws, stream); break;
    case 60: skinny_launch_c<60, false>(a, p, ws, stream); break;
    case 61: skinny_launch_c<61, false>(a, p, ws, stream); break;
    case 62: skinny_launch_c<62, false>(a, p, ws, stream); break;
    case 63: skinny_launch_c<63, false>(a, p, ws, stream); break;
    case 64: skinny_launch_c<64, false>(a, p, ws, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Activation preparation for the pipelined kernel (with a workspace): each
// 8-element chunk of X copied in the pair order of codes_as_bf16_pairs, and the
// fp32 sum of every 128-row group per token, xsum[g][token].  The MFMA loop
// then needs neither the reorder nor a ones-MFMA.  Thread = (token, chunk);
// the 16 threads of a group are 16 consecutive lanes (k % 128 == 0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void int4_prep_kernel(const uint16_t* __restrict__ x, int64_t ldx, int m,
                                                        int k, uint16_t* __restrict__ xp,
                                                        float* __restrict__ xsum) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = k >> 3;
  if (t >= (int64_t)m * cpr) return;   // whole 16-lane groups leave together
  const int row = (int)(t / cpr), c = (int)(t - (int64_t)row * cpr);
  const u32x4 v = *reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx + 8 * c);
  *reinterpret_cast<u32x4*>(xp + (int64_t)row * k + 8 * c) = x_pairs_permuted(v);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) sum = dot2_bf16(v[i], kOnesBf16x2, sum);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 16);
  if ((c & 15) == 0) xsum[(int64_t)(c >> 4) * m + row] = sum;
}

// Workspace of the pipelined path: the counters (64 KiB; per-tile tickets of
// the k split, zero between calls), the prepared activations [m][k] bf16,
// xsum [k/128][m] fp32, then the split's fp32 partial tiles.

// Launch shapes of the pipelined kernel, smallest tile first.
struct PipeCfg {
  int bm, bn, stages, threads;
  size_t lds;
};

template <int NWM, int NWN, int FM, int STAGES, bool PREP, bool LORA = false>
static PipeCfg pipe_cfg() {
  using S = PipeShape<NWM, NWN, FM, PREP, LORA>;
  size_t lds = (size_t)STAGES * S::STAGE_DW * 4;
  const size_t out = (size_t)S::BM * S::OP * 2;
  return PipeCfg{S::BM, S::BN, STAGES, S::T, lds > out ? lds : out};
}

// Plan of the pipelined path: tile, k split, preparation.  A launch takes
// ceil(items / (256 CUs x workgroups per CU)) rounds; measured round times
// relative to 256 x 128 (one workgroup per CU) with the whole of k: 128 x 128
// (one per CU) 0.62-0.66, 64 x 128 (three per CU) 0.8-0.9.  A k slice of
// 1/ks of the groups costs 1/ks of that plus the partial exchange; slices keep
// at least QG_PIPE_MIN_GPS groups.  The split needs the preparation workspace
// (it rides behind it) and at most 16384 tiles (the counters).
// cfg 0: 64 x 128, 1: 128 x 128, 2: 256 x 128.
#ifndef QG_PIPE_T128
#define QG_PIPE_T128 0.65
#endif
#ifndef QG_PIPE_T64
#define QG_PIPE_T64 0.85
#endif
#ifndef QG_PIPE_MIN_GPS
#define QG_PIPE_MIN_GPS 4
#endif
// Costs in rounds of a full-k 256 x 128 tile (≈ 0.0192 us per k row on this
// chip): a slice pays QG_PIPE_FILL stages of pipeline fill and drain, and a
// split writes and re-reads items x BM x 128 fp32 partials at ~4 TB/s.
#ifndef QG_PIPE_FILL
#define QG_PIPE_FILL 3.0
#endif
#ifndef QG_PIPE_US_PER_K
#define QG_PIPE_US_PER_K 0.0192
#endif
#ifndef QG_PIPE_PARTIAL_BPUS
#define QG_PIPE_PARTIAL_BPUS 4.0e6   // bytes per microsecond of partial traffic
#endif
#ifndef QG_PIPE_MAX_SPLIT
#define QG_PIPE_MAX_SPLIT 8
#endif

struct MfmaPlan {
  int cfg, ksplit, gps;
  bool prep;
  int64_t tiles, ws_bytes;
};

static const int kCfgBM[3] = {64, 128, 256};

static MfmaPlan plan_mfma(int64_t m, int64_t n, int64_t k, int64_t ws_bytes) {
  const int64_t G = k / 128, tn = (n + 127) / 128;
  // prepared activations, group sums, then (256-byte aligned) the split's partials
  const int64_t prep_bytes = (kTicketBytes + m * k * 2 + G * m * 4 + 255) & ~(int64_t)255;
  MfmaPlan best{2, 1, (int)G, ws_bytes >= prep_bytes, ((m + 255) / 256) * tn, 0};
  best.ws_bytes = best.prep ? prep_bytes : 0;
  double best_cost = 1e300;
  const double tcost[3] = {QG_PIPE_T64, QG_PIPE_T128, 1.0};
  const int per_cu[3] = {3, 1, 1};
  for (int cfg = 0; cfg < 3; ++cfg) {
    const int64_t tiles = ((m + kCfgBM[cfg] - 1) / kCfgBM[cfg]) * tn;
    for (int ks = 1; ks <= QG_PIPE_MAX_SPLIT; ++ks) {
      const int64_t gps = (G + ks - 1) / ks;
      if (ks > 1 && (gps < QG_PIPE_MIN_GPS || (G + gps - 1) / gps != ks)) continue;
      int64_t need = best.prep ? prep_bytes : 0;
      if (ks > 1) {
        if (!best.prep || tiles > kTicketBytes / 4) break;
        need = prep_bytes + tiles * ks * kCfgBM[cfg] * 128 * 4;
        if (need > ws_bytes) break;
      }
      const int64_t items = tiles * ks;
      const double rounds = (double)((items + 256 * per_cu[cfg] - 1) / (256 * per_cu[cfg]));
      const double round_us = QG_PIPE_US_PER_K * (double)k;                  // full-k 256 x 128 round
      double cost = rounds * tcost[cfg] * (2.0 * gps + QG_PIPE_FILL) / (2.0 * G);
      if (ks > 1) cost += (double)items * kCfgBM[cfg] * 128 * 4 * 2 / QG_PIPE_PARTIAL_BPUS / round_us;
#ifdef QG_PIPE_FORCE
      if (cfg != QG_PIPE_FORCE) continue;
#endif
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best.cfg = cfg;
        best.ksplit = ks;
        best.gps = (int)gps;
        best.tiles = tiles;
        best.ws_bytes = need;
      }
    }
  }
  return best;
}

#ifndef QG_PIPE_S128
#define QG_PIPE_S128 4     // LDS stages of the 128 x 128 tile
#endif
#ifndef QG_PIPE_S64
#define QG_PIPE_S64 4      // LDS stages of the 64 x 128 tile
#endif

template <bool PREP>
static PipeCfg pipe_cfg_of(int which) {
  switch (which) {
    case 2: return pipe_cfg<4, 2, 4, 4, PREP>();
    case 1: return pipe_cfg<2, 2, 4, QG_PIPE_S128, PREP>();
    default: return pipe_cfg<1, 2, 4, QG_PIPE_S64, PREP>();
  }
}

// LDS of a workgroup must fit the 160 KiB of a CU (the kernel has no static
// LDS: the k split's ticket flag lives in the dynamic area once the stages
// are done).  With LoRA the stages also carry a block of lora_A; where four
// such stages would not fit, three are used.
constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kPipeStaticLds = 0;

template <int NWM, int NWN, int FM, int STAGES, bool PREP>
static void pipe_launch(const Int4Args& a, const MfmaPlan& p, const uint16_t* x, int64_t ldx,
                        const float* xsum, float* partials, uint32_t* tickets, hipStream_t stream) {
  using SL = PipeShape<NWM, NWN, FM, PREP, true>;
  constexpr int LSTAGES = (size_t)STAGES * SL::STAGE_DW * 4 + kPipeStaticLds <= kLdsBytes ? STAGES : STAGES - 1;
  static_assert((size_t)STAGES * PipeShape<NWM, NWN, FM, PREP>::STAGE_DW * 4 + kPipeStaticLds <= kLdsBytes,
                "LDS budget");
  static_assert((size_t)LSTAGES * SL::STAGE_DW * 4 + kPipeStaticLds <= kLdsBytes && LSTAGES >= 3, "LDS budget");
  const bool lora = a.lora.a != nullptr;
  const PipeCfg c = lora ? pipe_cfg<NWM, NWN, FM, LSTAGES, PREP, true>() : pipe_cfg<NWM, NWN, FM, STAGES, PREP>();
  const int tiles_n = (int)((a.n + c.bn - 1) / c.bn);
  const int items = (int)(p.tiles * p.ksplit), per_xcd = (items + 7) / 8;
  const int vec = ((uintptr_t)a.y & 15u) == 0 && a.ldy % 8 == 0;
  if (lora)
    int4_pipe_kernel<NWM, NWN, FM, LSTAGES, PREP, true><<<dim3((unsigned)(per_xcd * 8)), dim3(c.threads), c.lds,
                                                           stream>>>(
        x, ldx, a.qweight, a.scales, a.qzeros, xsum, a.y, a.ldy, (int)a.m, (int)a.n, (int)a.k, tiles_n, items,
        per_xcd, vec, p.ksplit, p.gps, partials, tickets, a.split_acq_rel, a.lora);
  else
    int4_pipe_kernel<NWM, NWN, FM, STAGES, PREP, false><<<dim3((unsigned)(per_xcd * 8)), dim3(c.threads), c.lds,
                                                           stream>>>(
        x, ldx, a.qweight, a.scales, a.qzeros, xsum, a.y, a.ldy, (int)a.m, (int)a.n, (int)a.k, tiles_n, items,
        per_xcd, vec, p.ksplit, p.gps, partials, tickets, a.split_acq_rel, a.lora);
}

template <bool PREP>
static void pipe_dispatch(const Int4Args& a, const MfmaPlan& p, const uint16_t* x, int64_t ldx,
                          const float* xsum, float* partials, uint32_t* tickets, hipStream_t stream) {
  switch (p.cfg) {
    case 2: pipe_launch<4, 2, 4, 4, PREP>(a, p, x, ldx, xsum, partials, tickets, stream); break;
    case 1: pipe_launch<2, 2, 4, QG_PIPE_S128, PREP>(a, p, x, ldx, xsum, partials, tickets, stream); break;
    default: pipe_launch<1, 2, 4, QG_PIPE_S64, PREP>(a, p, x, ldx, xsum, partials, tickets, stream); break;
  }
}

hipError_t launch_mfma_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const MfmaPlan p = plan_mfma(a.m, a.n, a.k, ws ? ws_bytes : 0);
  if (p.prep) {
    uint32_t* tickets = (uint32_t*)ws;
    uint16_t* xp = (uint16_t*)((char*)ws + kTicketBytes);
    float* xsum = (float*)(xp + a.m * a.k);
    float* partials = (float*)((char*)ws + ((kTicketBytes + a.m * a.k * 2 + (a.k / 128) * a.m * 4 + 255) & ~(int64_t)255));
    const int64_t threads = a.m * (a.k / 8);
    int4_prep_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(
        a.x, a.ldx, (int)a.m, (int)a.k, xp, xsum);
    pipe_dispatch<true>(a, p, xp, a.k, xsum, partials, tickets, stream);
  } else {
    pipe_dispatch<false>(a, p, a.x, a.ldx, nullptr, nullptr, nullptr, stream);
  }
  return hipGetLastError();
}

int64_t workspace_int4(int64_t m, int64_t n, int64_t k, int path) {
  if (m == 0 || n == 0 || k == 0) return 0;
  if (path == 3) return plan_mfma(m, n, k, INT64_MAX).ws_bytes;
  return plan_small_m(m, n, k, INT64_MAX, path == 1).ws_bytes;
}

void describe_int4(int64_t m, int64_t n, int64_t k, int path, int64_t ws_bytes, char* buf,
                   size_t len) {
  if (path == 1 || path == 2) {
    const int64_t mp = path == 1 ? 1 : m;
    const SkinnyPlan p = plan_small_m(mp, n, k, ws_bytes, path == 1);
    const bool dot = path == 1;
    const LdsPlan l = plan_lds(mp, p, k, dot);
    if (l.ng > 0) {
      snprintf(buf, len, "skinny_lds_kernel<%lld,%s,%d,%d,%s> grid=%lld block=%d lds=%lld ksplit=1 groups=%d",
               (long long)mp, dot ? "dot" : "mfma", p.cpl, l.ng, l.xl ? "xlds" : "xreg", (long long)p.blocks,
               64 * l.waves, (long long)l.lds, p.gwg);
    } else {
      snprintf(buf, len, "skinny_int4_kernel<%lld,%s,%d> grid=%lld block=%d lds=%lld ksplit=%d groups=%d",
               (long long)mp, dot ? "dot" : "mfma", p.cpl, (long long)p.blocks, 64 * p.waves, (long long)p.lds,
               p.ksplit, p.gwg);
    }
  } else {
    const MfmaPlan p = plan_mfma(m, n, k, ws_bytes);
    const PipeCfg c = p.prep ? pipe_cfg_of<true>(p.cfg) : pipe_cfg_of<false>(p.cfg);
    const long long items = p.tiles * p.ksplit;
    snprintf(buf, len, "int4_pipe_kernel<%d,%d,%d,%s> grid=%lld block=%d lds=%lld ksplit=%d groups=%d", c.bm,
             c.bn, c.stages, p.prep ? "prep" : "ones", ((items + 7) / 8) * 8, c.threads, (long long)c.lds,
             p.ksplit, p.gps);
  }
}

// ---------------------------------------------------------------------------
// zero fill of a strided 16-bit matrix
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero16_kernel(uint16_t* p, int64_t rows, int64_t cols,
                                                     int64_t ld) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows * cols) {
    const int64_t r = i / cols;
    p[r * ld + (i - r * cols)] = 0;
  }
}

hipError_t launch_zero16(uint16_t* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  zero16_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(p, rows, cols, ld);
  return hipGetLastError();
}

}  // namespace qg
