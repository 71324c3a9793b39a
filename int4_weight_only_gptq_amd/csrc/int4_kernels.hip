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

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// ---------------------------------------------------------------------------
// m = 1 GEMV (VALU).  A workgroup owns 16*CPL output columns; its waves split
// the k groups.  Lane (cl = lane % 16, ks = lane / 16) reads CPL consecutive
// words of word-row 4s + ks (s = 0..3 within a group), so the 16 lanes of a row
// read 64*CPL contiguous bytes.  Products use v_dot2_f32_bf16 on the pairs of
// (128 + q) and the activations; the per-group offset correction and scale are
// applied per lane.  The four 16-lane rows are then summed with the gfx950
// row-swap permutes and the waves through LDS.
// ---------------------------------------------------------------------------
template <int CPL>
__global__ __launch_bounds__(1024) void gemv_int4_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qzeros,
                                                         uint16_t* __restrict__ y, int n, int k) {
  constexpr int NB = 16 * CPL;
  __shared__ float plane[16][NB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t col = (int64_t)blockIdx.x * NB + CPL * cl;
  const bool live = col < n;
  const int G = k >> 7;
  const int g0 = (wave * G) / nwaves, g1 = ((wave + 1) * G) / nwaves;
  const uint32_t* qp = qweight + (live ? col : 0);

  float total[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) total[c] = 0.f;

  for (int g = g0; g < g1; ++g) {
    u32x4 xv[4];
    uint32_t wv[4][CPL];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t r = (int64_t)g * 16 + 4 * s + ks;
      xv[s] = *reinterpret_cast<const u32x4*>(x + 8 * r);
      if (live) {
        load_words<CPL>(qp + r * n, wv[s]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) wv[s][c] = 0u;
      }
    }
    float sc[CPL], bz[CPL];
    if (live) {
      load_group_meta<CPL>(scales, qzeros, n, g, col, sc, bz);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) { sc[c] = 0.f; bz[c] = 0.f; }
    }
    float d[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) d[c] = 0.f;
    float xs = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 a = x_pairs_permuted(xv[s]);
#pragma unroll
      for (int t = 0; t < 4; ++t) xs = dot2_bf16(a[t], kOnesBf16x2, xs);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const u32x4 b = codes_as_bf16_pairs(wv[s][c]);
#pragma unroll
        for (int t = 0; t < 4; ++t) d[c] = dot2_bf16(b[t], a[t], d[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) total[c] += sc[c] * (d[c] - bz[c] * xs);
  }

#pragma unroll
  for (int c = 0; c < CPL; ++c) total[c] = sum_over_rows(total[c]);
  if (ks == 0 && live) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) plane[wave][CPL * cl + c] = total[c];
  }
  __syncthreads();
  if ((int)threadIdx.x < NB) {
    const int64_t cc = (int64_t)blockIdx.x * NB + threadIdx.x;
    if (cc < n) {
      float acc = 0.f;
      for (int w = 0; w < nwaves; ++w) acc += plane[w][threadIdx.x];
      y[cc] = (uint16_t)f32_to_bf16_bits(acc);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused small-M kernel, M = 1..16 tokens known at compile time.  Same column
// ownership and word stream as the GEMV; the contraction runs on the
// 16x16x32 bf16 MFMA: operand A = activations (row = token, rows >= M are
// zero), operand B = the codes of one word per lane (8 consecutive k of one
// column is exactly one lane's B slice).  Tile c of a lane holds column
// 16*CPL*block + CPL*(lane%16) + c.  A second MFMA against a ones operand
// gives the per-token group sums for the offset correction.  Accumulators are
// compile-time sized VGPR arrays; the cross-wave partial plane holds M tokens.
// ---------------------------------------------------------------------------
template <int M, int CPL>
__global__ __launch_bounds__(1024) void fused_int4_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    uint16_t* __restrict__ y, int64_t ldy, int n, int k) {
  constexpr int NB = 16 * CPL;
  constexpr int VMAX = M < 4 ? M : 4;   // accumulator rows that can hold a token
  extern __shared__ float plane[];      // [nwaves][M][NB]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t col = (int64_t)blockIdx.x * NB + CPL * cl;
  const bool live = col < n;
  const bool xrow = cl < M;
  const int G = k >> 7;
  const int g0 = (wave * G) / nwaves, g1 = ((wave + 1) * G) / nwaves;
  const uint32_t* qp = qweight + (live ? col : 0);
  const uint16_t* xp = x + (xrow ? (int64_t)cl * ldx : 0);
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  f32x4 total[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) total[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = g0; g < g1; ++g) {
    u32x4 xv[4];
    uint32_t wv[4][CPL];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t r = (int64_t)g * 16 + 4 * s + ks;
      xv[s] = xrow ? *reinterpret_cast<const u32x4*>(xp + 8 * r) : zero4;
      if (live) {
        load_words<CPL>(qp + r * n, wv[s]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) wv[s][c] = 0u;
      }
    }
    float sc[CPL], bz[CPL];
    if (live) {
      load_group_meta<CPL>(scales, qzeros, n, g, col, sc, bz);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) { sc[c] = 0.f; bz[c] = 0.f; }
    }
    f32x4 acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 a = x_pairs_permuted(xv[s]);
      xsum = mfma16_bf16(a, ones, xsum);
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = mfma16_bf16(a, codes_as_bf16_pairs(wv[s][c]), acc[c]);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
      for (int v = 0; v < VMAX; ++v) total[c][v] += sc[c] * (acc[c][v] - bz[c] * xsum[v]);
    }
  }

  // accumulator (c, v) of this lane is token 4*ks + v, column CPL*cl + c of the block
#pragma unroll
  for (int v = 0; v < VMAX; ++v) {
    const int token = 4 * ks + v;
    if (token < M && live) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) plane[(wave * M + token) * NB + CPL * cl + c] = total[c][v];
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < M * NB; o += blockDim.x) {
    const int token = o / NB, cc = o - token * NB;
    const int64_t cg = (int64_t)blockIdx.x * NB + cc;
    if (cg < n) {
      float acc = 0.f;
      for (int w = 0; w < nwaves; ++w) acc += plane[(w * M + token) * NB + cc];
      y[(int64_t)token * ldy + cg] = (uint16_t)f32_to_bf16_bits(acc);
    }
  }
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
// launch shapes
// ---------------------------------------------------------------------------
static int pick_cpl(int64_t n) {
  // widest per-lane load that still gives enough workgroups for 256 CUs
  if ((n + 63) / 64 >= 384) return 4;
  if ((n + 31) / 32 >= 384) return 2;
  return 1;
}

static int pick_waves(int64_t k) {
  const int64_t groups = k / 128;
  return (int)(groups < 16 ? (groups < 1 ? 1 : groups) : 16);
}

hipError_t launch_gemv_int4(const Int4Args& a, hipStream_t stream) {
  const int cpl = pick_cpl(a.n);
  const int nw = pick_waves(a.k);
  const unsigned blocks = (unsigned)((a.n + 16 * cpl - 1) / (16 * cpl));
  const dim3 grid(blocks), block(64 * nw);
  const int n = (int)a.n, k = (int)a.k;
  if (cpl == 4)
    gemv_int4_kernel<4><<<grid, block, 0, stream>>>(a.x, a.qweight, a.scales, a.qzeros, a.y, n, k);
  else if (cpl == 2)
    gemv_int4_kernel<2><<<grid, block, 0, stream>>>(a.x, a.qweight, a.scales, a.qzeros, a.y, n, k);
  else
    gemv_int4_kernel<1><<<grid, block, 0, stream>>>(a.x, a.qweight, a.scales, a.qzeros, a.y, n, k);
  return hipGetLastError();
}

template <int M, int CPL>
static void fused_launch(const Int4Args& a, int nw, hipStream_t stream) {
  const unsigned blocks = (unsigned)((a.n + 16 * CPL - 1) / (16 * CPL));
  const size_t lds = (size_t)nw * M * 16 * CPL * sizeof(float);
  fused_int4_kernel<M, CPL><<<dim3(blocks), dim3(64 * nw), lds, stream>>>(
      a.x, a.ldx, a.qweight, a.scales, a.qzeros, a.y, a.ldy, (int)a.n, (int)a.k);
}

template <int M>
static void fused_launch_m(const Int4Args& a, hipStream_t stream) {
  const int cpl = pick_cpl(a.n);
  const int nw = pick_waves(a.k);
  if (cpl == 4) fused_launch<M, 4>(a, nw, stream);
  else if (cpl == 2) fused_launch<M, 2>(a, nw, stream);
  else fused_launch<M, 1>(a, nw, stream);
}

hipError_t launch_fused_int4(const Int4Args& a, hipStream_t stream) {
  switch (a.m) {
    case 1: fused_launch_m<1>(a, stream); break;
    case 2: fused_launch_m<2>(a, stream); break;
    case 3: fused_launch_m<3>(a, stream); break;
    case 4: fused_launch_m<4>(a, stream); break;
    case 5: fused_launch_m<5>(a, stream); break;
    case 6: fused_launch_m<6>(a, stream); break;
    case 7: fused_launch_m<7>(a, stream); break;
    case 8: fused_launch_m<8>(a, stream); break;
    case 9: fused_launch_m<9>(a, stream); break;
    case 10: fused_launch_m<10>(a, stream); break;
    case 11: fused_launch_m<11>(a, stream); break;
    case 12: fused_launch_m<12>(a, stream); break;
    case 13: fused_launch_m<13>(a, stream); break;
    case 14: fused_launch_m<14>(a, stream); break;
    case 15: fused_launch_m<15>(a, stream); break;
    case 16: fused_launch_m<16>(a, stream); break;
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

void describe_int4(int64_t m, int64_t n, int64_t k, int path, char* buf, size_t len) {
  if (path == 1 || path == 2) {
    const int cpl = pick_cpl(n), nw = pick_waves(k);
    const long long blocks = (n + 16 * cpl - 1) / (16 * cpl);
    if (path == 1)
      snprintf(buf, len, "gemv_int4_kernel<%d> grid=%lld block=%d lds=%d", cpl, blocks, 64 * nw,
               16 * 16 * cpl * 4);
    else
      snprintf(buf, len, "fused_int4_kernel<%lld,%d> grid=%lld block=%d lds=%lld", (long long)m, cpl,
               blocks, 64 * nw, (long long)nw * m * 16 * cpl * 4);
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
