// int4 GPTQ kernels for gfx950: dequant, the m = 1 GEMV, the fused small-M
// kernel and the LDS-tiled MFMA kernel.
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
  const uint32_t zw = qzeros[g * (n >> 3) + (col >> 3)] >> ((col & 7) * 4);
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
  if constexpr (CPL == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (CPL == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = *p;
  }
}

// Scales of CPL consecutive columns (fp32) and their zero points plus 128.
template <int CPL>
__device__ __forceinline__ void load_group_meta(const uint16_t* __restrict__ scales,
                                                const uint32_t* __restrict__ qzeros, int64_t n,
                                                int64_t g, int64_t col, float (&s)[CPL],
                                                float (&bz)[CPL]) {
  const uint16_t* sp = scales + g * n + col;
  if constexpr (CPL == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
    s[0] = half_bits_to_float(v[0] & 0xFFFFu); s[1] = half_bits_to_float(v[0] >> 16);
    s[2] = half_bits_to_float(v[1] & 0xFFFFu); s[3] = half_bits_to_float(v[1] >> 16);
  } else if constexpr (CPL == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(sp);
    s[0] = half_bits_to_float(v & 0xFFFFu); s[1] = half_bits_to_float(v >> 16);
  } else {
    s[0] = half_bits_to_float(*sp);
  }
  const uint32_t zw = qzeros[g * (n >> 3) + (col >> 3)] >> ((col & 7) * 4);
#pragma unroll
  for (int c = 0; c < CPL; ++c) bz[c] = (float)(128u + ((zw >> (4 * c)) & 15u));
}

// Raw group metadata of CPL consecutive columns: their fp16 scales and the
// word holding their zero nibbles.  Loaded in the load phase and decoded only
// where it is used, so the loads do not force an early wait on everything in
// flight.
template <int CPL>
struct Meta {
  uint32_t s[CPL == 4 ? 2 : 1];
  uint32_t z;
};

template <int CPL>
__device__ __forceinline__ Meta<CPL> load_meta(const uint16_t* __restrict__ scales,
                                               const uint32_t* __restrict__ qzeros, int64_t n,
                                               int64_t g, int64_t col) {
  Meta<CPL> r;
  const uint16_t* sp = scales + g * n + col;
  if constexpr (CPL == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
    r.s[0] = v[0];
    r.s[1] = v[1];
  } else if constexpr (CPL == 2) {
    r.s[0] = *reinterpret_cast<const uint32_t*>(sp);
  } else {
    r.s[0] = *sp;
  }
  r.z = qzeros[g * (n >> 3) + (col >> 3)];
  return r;
}

// zshift = 4 * (col % 8): the nibble of the first of the CPL columns.
template <int CPL>
__device__ __forceinline__ void decode_meta(const Meta<CPL>& mt, int zshift, float (&s)[CPL],
                                            float (&bz)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    s[c] = half_bits_to_float((mt.s[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);
    bz[c] = (float)(128u + ((mt.z >> (zshift + 4 * c)) & 15u));
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
// against the activation slice staged once in LDS, per-group offset
// correction and scale per lane, then the four 16-lane rows summed with the
// row-swap permutes.
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
constexpr int64_t kTicketBytes = 64 << 10;   // counters of up to 16384 strips
constexpr int SK_MAX_SPLIT = 16;              // k-slices per strip at most
constexpr size_t kSkinnyMaxLds = 150 << 10;    // of the 160 KiB of a gfx950 CU

template <int M, bool DOT, int CPL>
struct GroupRegs {
  uint32_t w[4][CPL];                  // codes of the 4 k-steps
  u32x4 xa[DOT ? 1 : 4];               // MFMA: the A slices of the 4 k-steps
  Meta<CPL> meta;
};

// gok: the group is in range; live: this lane's columns are in range; xrow:
// this lane supplies activation row (token) cl.  The activation row does not
// depend on the lane's columns.
template <int M, bool DOT, int CPL>
__device__ __forceinline__ void load_group(GroupRegs<M, DOT, CPL>& r, bool gok, bool live, bool xrow,
                                           const uint32_t* __restrict__ qp,
                                           const uint16_t* __restrict__ xp,
                                           const uint16_t* __restrict__ scales,
                                           const uint32_t* __restrict__ qzeros, int64_t n,
                                           int64_t g, int64_t col, int ks) {
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const bool ok = gok && live;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (ok) {
      load_words<CPL>(qp + (g * 16 + 4 * s + ks) * n, r.w[s]);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) r.w[s][c] = 0u;
    }
    if constexpr (!DOT)
      r.xa[s] = (gok && xrow) ? *reinterpret_cast<const u32x4*>(xp + 8 * (g * 16 + 4 * s + ks)) : zero4;
  }
  if (ok) {
    r.meta = load_meta<CPL>(scales, qzeros, n, g, col);
  } else {
    r.meta.z = 0u;
#pragma unroll
    for (int i = 0; i < (CPL == 4 ? 2 : 1); ++i) r.meta.s[i] = 0u;
  }
}

template <int M, bool DOT, int CPL>
__global__ __launch_bounds__(1024) void skinny_int4_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    uint16_t* __restrict__ y, int64_t ldy, int n, int k, int nstrips, int ksplit, int gwg,
    int items_per_xcd, float* __restrict__ partials, uint32_t* __restrict__ tickets) {
  static_assert(!DOT || M == 1, "the VALU variant computes one token");
  constexpr int SW = 16 * CPL;                 // strip width in columns
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nw = blockDim.x >> 6;
  float* plane = reinterpret_cast<float*>(smem);                          // [nw][M][SW]
  u32x4* xl = reinterpret_cast<u32x4*>(smem + (size_t)nw * M * SW * 4);   // DOT: [k-slice chunks]
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
  const bool xrow = cl < M;
  const uint32_t* qp = qweight + (live ? col : 0);
  const uint16_t* xp = x + (xrow ? (int64_t)cl * ldx : 0);
  const int zshift = (int)(col & 7) * 4;
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

  // first group's loads go out before anything waits
  GroupRegs<M, DOT, CPL> cur, nxt;
  int g = gbeg + wave;
  load_group<M, DOT, CPL>(cur, g < gend, live, xrow, qp, xp, scales, qzeros, n, g, col, ks);

  if constexpr (DOT) {
    // the activation row of this k-slice, in pair order, once per workgroup
    const int chunks = (gend - gbeg) * 16;
    for (int c = tid; c < chunks; c += blockDim.x)
      xl[c] = x_pairs_permuted(*reinterpret_cast<const u32x4*>(x + (int64_t)gbeg * 128 + 8 * c));
    __syncthreads();
  }

  f32x4 total[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) total[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (; g < gend; g += nw) {
    const int gn = g + nw;
    load_group<M, DOT, CPL>(nxt, gn < gend, live, xrow, qp, xp, scales, qzeros, n, gn, col, ks);
    float sc[CPL], bz[CPL];
    if constexpr (DOT) {
      float d[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) d[c] = 0.f;
      float xs = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = xl[(g - gbeg) * 16 + 4 * s + ks];
#pragma unroll
        for (int t = 0; t < 4; ++t) xs = dot2_bf16(a[t], kOnesBf16x2, xs);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const u32x4 bq = codes_as_bf16_pairs(cur.w[s][c]);
#pragma unroll
          for (int t = 0; t < 4; ++t) d[c] = dot2_bf16(bq[t], a[t], d[c]);
        }
      }
      decode_meta<CPL>(cur.meta, zshift, sc, bz);
#pragma unroll
      for (int c = 0; c < CPL; ++c) total[c][0] += sc[c] * (d[c] - bz[c] * xs);
    } else {
      constexpr int VMAX = M < 4 ? M : 4;
      f32x4 acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = x_pairs_permuted(cur.xa[s]);
        xsum = mfma16_bf16(a, ones, xsum);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = mfma16_bf16(a, codes_as_bf16_pairs(cur.w[s][c]), acc[c]);
      }
      decode_meta<CPL>(cur.meta, zshift, sc, bz);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int v = 0; v < VMAX; ++v) total[c][v] += sc[c] * (acc[c][v] - bz[c] * xsum[v]);
    }
    cur = nxt;
  }

  // wave partials [M][SW] -> LDS plane -> sum over the waves
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

  float* mine = ksplit > 1 ? partials + ((int64_t)strip * ksplit + kslice) * (M * SW) : nullptr;
  for (int o = tid; o < M * SW; o += blockDim.x) {
    const int token = o / SW, cc = o - token * SW;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += plane[(w * M + token) * SW + cc];
    const int64_t cg = (int64_t)strip * SW + cc;
    if (ksplit == 1) {
      if (cg < n) y[(int64_t)token * ldy + cg] = (uint16_t)f32_to_bf16_bits(v);
    } else {
      // agent-coherent store: visible to any workgroup once it has completed
      __hip_atomic_store(&mine[o], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (ksplit == 1) return;

  // split k: the last workgroup of the strip adds the partials in k order.
  // Every thread waits for its partial stores to complete before the barrier,
  // then one counter increment per workgroup; partials are only written and
  // read with agent-coherent accesses, so no cache-wide maintenance is needed.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(&tickets[strip], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(ksplit - 1);
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
    if (cg < n) y[(int64_t)token * ldy + cg] = (uint16_t)f32_to_bf16_bits(v);
  }
  if (tid == 0) __hip_atomic_store(&tickets[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// LDS-tiled MFMA kernel for m > 16.  Workgroup tile 128 tokens x 128 columns,
// four waves in 2 x 2 (64 x 64 each, 4 x 4 MFMA tiles of 16 x 16).  One k group
// (128 rows) per iteration: the activation tile (128 x 128 bf16, stored in
// the permuted pair order) and the packed words (16 x 128) are staged in LDS;
// the next group's global loads are in flight while the current one computes.
// Each wave turns its words into bf16 B operands itself; the per-token group
// sums come from v_dot2 on the A operands it already holds.
// ---------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128;
constexpr int XS_STRIDE = 128 + 8;   // bf16 per LDS row of the activation tile
constexpr int WS_STRIDE = 128 + 4;   // words per LDS row of the code tile

__global__ __launch_bounds__(256) void mfma_int4_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    uint16_t* __restrict__ y, int64_t ldy, int m, int n, int k, int tiles_m) {
  __shared__ __attribute__((aligned(16))) uint16_t xs_lds[TBM * XS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint32_t ws_lds[16 * WS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int wm0 = (wave & 1) * 64, wn0 = (wave >> 1) * 64;
  const int G = k >> 7;

  // staging assignment: activation chunks (row, 8-wide k chunk), word chunks
  u32x4 xreg[8];
  u32x4 wreg[2];
  auto load_tiles = [&](int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, kc = c & 15;
      const int tok = m0 + row;
      xreg[i] = tok < m ? *reinterpret_cast<const u32x4*>(x + (int64_t)tok * ldx + (int64_t)g * 128 + 8 * kc)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int wr = c >> 5, cc = c & 31;
      const int colw = n0 + 4 * cc;
      wreg[i] = colw < n ? *reinterpret_cast<const u32x4*>(qweight + ((int64_t)g * 16 + wr) * n + colw)
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, kc = c & 15;
      *reinterpret_cast<u32x4*>(&xs_lds[row * XS_STRIDE + 8 * kc]) = x_pairs_permuted(xreg[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int wr = c >> 5, cc = c & 31;
      *reinterpret_cast<u32x4*>(&ws_lds[wr * WS_STRIDE + 4 * cc]) = wreg[i];
    }
  };

  const int64_t mycol = (int64_t)n0 + wn0 + 4 * cl;   // columns mycol + c, c = 0..3
  const bool colok = mycol < n;

  f32x4 total[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c) total[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (G > 0) load_tiles(0);
  for (int g = 0; g < G; ++g) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (g + 1 < G) load_tiles(g + 1);
    float sc[4], bz[4];
    if (colok) {
      load_group_meta<4>(scales, qzeros, n, g, mycol, sc, bz);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) { sc[c] = 0.f; bz[c] = 0.f; }
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float xsp[4] = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        a[f] = *reinterpret_cast<const u32x4*>(&xs_lds[(wm0 + 16 * f + cl) * XS_STRIDE + 32 * s + 8 * ks]);
      const u32x4 wv = *reinterpret_cast<const u32x4*>(&ws_lds[(4 * s + ks) * WS_STRIDE + wn0 + 4 * cl]);
      u32x4 b[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = codes_as_bf16_pairs(wv[c]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
#pragma unroll
        for (int t = 0; t < 4; ++t) xsp[f] = dot2_bf16(a[f][t], kOnesBf16x2, xsp[f]);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[f][c] = mfma16_bf16(a[f], b[c], acc[f][c]);
      }
    }
    // group sums per token: A rows are lane % 16, accumulator rows are 4*ks + v
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float rs = sum_over_rows(xsp[f]);
      float xsv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) xsv[v] = __shfl(rs, 4 * ks + v);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) total[f][c][v] += sc[c] * (acc[f][c][v] - bz[c] * xsv[v]);
    }
  }

  if (colok) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = m0 + wm0 + 16 * f + 4 * ks + v;
        if (tok < m) {
          u32x2 o;
          o[0] = pack_bf16x2(total[f][0][v], total[f][1][v]);
          o[1] = pack_bf16x2(total[f][2][v], total[f][3][v]);
          *reinterpret_cast<u32x2*>(y + (int64_t)tok * ldy + mycol) = o;
        }
      }
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

int64_t split_workspace_bytes(int64_t nstrips, int64_t ksplit, int64_t m, int cpl) {
  return kTicketBytes + nstrips * ksplit * m * 16 * cpl * 4;
}

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int64_t workspace_bytes, bool dot) {
  SkinnyPlan p{};
  const int64_t G = k / 128;
  // widest strip that still leaves enough strips for the CUs
  p.cpl = 1;
  if ((n + 63) / 64 >= QG_SKINNY_MIN_STRIPS) p.cpl = 4;
  else if ((n + 31) / 32 >= QG_SKINNY_MIN_STRIPS) p.cpl = 2;
  const int sw = 16 * p.cpl;
  p.nstrips = (int)((n + sw - 1) / sw);
  // many strips: 8-wave workgroups so that two fit on a CU; few: 16 waves
  const int64_t wcap = p.nstrips >= 384 ? (QG_SKINNY_WAVES < 8 ? QG_SKINNY_WAVES : 8) : QG_SKINNY_WAVES;
  p.waves = (int)(G < 2 ? 1 : (G / 2 < wcap ? G / 2 : wcap));
  // k split only when each wave would otherwise walk a long chain of groups
  int64_t ks = 1;
  const int64_t per_wave = (G + p.waves - 1) / p.waves;
  if (per_wave > QG_SKINNY_MAX_GPW && (int64_t)p.nstrips * 4 <= kTicketBytes) {
    ks = (per_wave + 3) / 4;
    if (ks > SK_MAX_SPLIT) ks = SK_MAX_SPLIT;
  }
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
  const int64_t items = (int64_t)p.nstrips * p.ksplit;
  p.items_per_xcd = (int)((items + 7) / 8);
  p.blocks = (int64_t)p.items_per_xcd * 8;
  p.lds = (size_t)p.waves * m * sw * 4 + (dot ? (size_t)gwg * 16 * 16 : 0);
  return p;
}

template <int M, bool DOT, int CPL>
static void skinny_launch(const Int4Args& a, const SkinnyPlan& p, void* ws, hipStream_t stream) {
  uint32_t* tickets = (uint32_t*)ws;
  float* partials = ws ? (float*)((char*)ws + kTicketBytes) : nullptr;
  skinny_int4_kernel<M, DOT, CPL><<<dim3((unsigned)p.blocks), dim3(64 * p.waves), p.lds, stream>>>(
      a.x, a.ldx, a.qweight, a.scales, a.qzeros, a.y, a.ldy, (int)a.n, (int)a.k, p.nstrips,
      p.ksplit, p.gwg, p.items_per_xcd, partials, tickets);
}

template <int M, bool DOT>
static void skinny_launch_c(const Int4Args& a, const SkinnyPlan& p, void* ws, hipStream_t stream) {
  if (p.cpl == 4) skinny_launch<M, DOT, 4>(a, p, ws, stream);
  else if (p.cpl == 2) skinny_launch<M, DOT, 2>(a, p, ws, stream);
  else skinny_launch<M, DOT, 1>(a, p, ws, stream);
}

hipError_t launch_gemv_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const SkinnyPlan p = plan_skinny(1, a.n, a.k, ws ? ws_bytes : 0, true);
  if (p.lds <= kSkinnyMaxLds) {
    skinny_launch_c<1, true>(a, p, ws, stream);
  } else {
    // the k-slice's activations do not fit in LDS: the MFMA variant needs none
    skinny_launch_c<1, false>(a, plan_skinny(1, a.n, a.k, ws ? ws_bytes : 0, false), ws, stream);
  }
  return hipGetLastError();
}

hipError_t launch_fused_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const SkinnyPlan p = plan_skinny(a.m, a.n, a.k, ws ? ws_bytes : 0, false);
  switch (a.m) {
    case 1: skinny_launch_c<1, false>(a, p, ws, stream); break;
    case 2: skinny_launch_c<2, false>(a, p, ws, stream); break;
    case 3: skinny_launch_c<3, false>(a, p, ws, stream); break;
    case 4: skinny_launch_c<4, false>(a, p, ws, stream); break;
    case 5: skinny_launch_c<5, false>(a, p, ws, stream); break;
    case 6: skinny_launch_c<6, false>(a, p, ws, stream); break;
    case 7: skinny_launch_c<7, false>(a, p, ws, stream); break;
    case 8: skinny_launch_c<8, false>(a, p, ws, stream); break;
    case 9: skinny_launch_c<9, false>(a, p, ws, stream); break;
    case 10: skinny_launch_c<10, false>(a, p, ws, stream); break;
    case 11: skinny_launch_c<11, false>(a, p, ws, stream); break;
    case 12: skinny_launch_c<12, false>(a, p, ws, stream); break;
    case 13: skinny_launch_c<13, false>(a, p, ws, stream); break;
    case 14: skinny_launch_c<14, false>(a, p, ws, stream); break;
    case 15: skinny_launch_c<15, false>(a, p, ws, stream); break;
    case 16: skinny_launch_c<16, false>(a, p, ws, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_int4(const Int4Args& a, hipStream_t stream) {
  const int tiles_m = (int)((a.m + TBM - 1) / TBM);
  const int tiles_n = (int)((a.n + TBN - 1) / TBN);
  const unsigned blocks = (unsigned)tiles_m * (unsigned)tiles_n;
  mfma_int4_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(a.x, a.ldx, a.qweight, a.scales,
                                                            a.qzeros, a.y, a.ldy, (int)a.m,
                                                            (int)a.n, (int)a.k, tiles_m);
  return hipGetLastError();
}

int64_t workspace_int4(int64_t m, int64_t n, int64_t k, int path) {
  if (path == 3 || m == 0 || n == 0 || k == 0) return 0;
  return plan_skinny(m, n, k, INT64_MAX, path == 1).ws_bytes;
}

void describe_int4(int64_t m, int64_t n, int64_t k, int path, int64_t ws_bytes, char* buf,
                   size_t len) {
  if (path == 1 || path == 2) {
    SkinnyPlan p = plan_skinny(path == 1 ? 1 : m, n, k, ws_bytes, path == 1);
    const bool dot = path == 1 && p.lds <= kSkinnyMaxLds;
    if (path == 1 && !dot) p = plan_skinny(1, n, k, ws_bytes, false);
    snprintf(buf, len, "skinny_int4_kernel<%lld,%s,%d> grid=%lld block=%d lds=%lld ksplit=%d groups=%d",
             path == 1 ? 1LL : (long long)m, dot ? "dot" : "mfma", p.cpl, (long long)p.blocks,
             64 * p.waves, (long long)p.lds, p.ksplit, p.gwg);
  } else {
    const long long tiles = ((m + TBM - 1) / TBM) * ((n + TBN - 1) / TBN);
    snprintf(buf, len, "mfma_int4_kernel grid=%lld block=256 lds=%d", tiles,
             (int)(TBM * XS_STRIDE * 2 + 16 * WS_STRIDE * 4));
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
