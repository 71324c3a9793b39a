// Dense bf16/fp16 GEMMs with fp32 accumulation for gfx950: the forward (NT),
// input-gradient (NN) and weight-gradient (TN) products of a linear layer.
//
//   NT: C[M][N] = A[M][K] . B[N][K]^T
//   NN: C[M][N] = A[M][K] . B[K][N]
//   TN: C[M][N] = A[K][M]^T . B[K][N]
//
// The MFMA kernel keeps both operands K-contiguous in LDS ([row][k]), which is
// what a 16x16x32 MFMA lane slice needs (8 consecutive k of one row/column).
// Operands that are M- or N-contiguous in memory (A of TN, B of NN and TN) are
// transposed on the way in: a thread loads an 8 x 8 block (8 k-rows of 8
// elements), transposes it in registers with byte permutes and writes 8
// K-contiguous rows.
#include "common.hpp"
#include "launch.hpp"

namespace qg {

constexpr int DBM = 128, DBN = 128, DBK = 64;
constexpr int DSTRIDE = DBK + 8;   // 16-bit elements per LDS row

// 8 x 8 transpose of 16-bit elements: in[r] holds row r (8 elements), out[j]
// receives column j = (in[0][j], in[1][j], ..., in[7][j]).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) out[j][p] = __builtin_amdgcn_perm(in[2 * p + 1][j >> 1], in[2 * p][j >> 1], sel);
  }
}

// Stage a K-contiguous operand tile (rows x DBK) from global memory.
// rows = 128: 1024 chunks of 8 elements, 4 per thread.
__device__ __forceinline__ void load_kcontig(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                             int64_t rows, int64_t k0, int64_t K, u32x4 (&reg)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, kc = c & 7;
    const int64_t gr = row0 + r, gk = k0 + 8 * kc;
    reg[i] = (gr < rows && gk < K) ? *reinterpret_cast<const u32x4*>(p + gr * ld + gk)
                                   : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_kcontig(uint16_t* lds, const u32x4 (&reg)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4*>(&lds[r * DSTRIDE + 8 * kc]) = reg[i];
  }
}

// Stage an MN-contiguous operand tile: memory [K][rows], 8 k-blocks x 16
// row-blocks of 8 x 8 = 128 blocks; threads 0..127 of `half` take one each.
__device__ __forceinline__ void load_mncontig(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                              int64_t rows, int64_t k0, int64_t K, int slot,
                                              u32x4 (&reg)[8]) {
  const int kb = slot >> 4, rb = slot & 15;
  const int64_t gr = row0 + 8 * rb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t gk = k0 + 8 * kb + e;
    reg[e] = (gr < rows && gk < K) ? *reinterpret_cast<const u32x4*>(p + gk * ld + gr)
                                   : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_mncontig(uint16_t* lds, int slot, const u32x4 (&reg)[8]) {
  const int kb = slot >> 4, rb = slot & 15;
  u32x4 t[8];
  transpose8x8(reg, t);
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&lds[(8 * rb + j) * DSTRIDE + 8 * kb]) = t[j];
}

template <int LAYOUT, int DTYPE>
__global__ __launch_bounds__(256) void dense_mfma_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                         const uint16_t* __restrict__ B, int64_t ldb,
                                                         uint16_t* __restrict__ C, int64_t ldc,
                                                         int M, int N, int K, int tiles_m) {
  constexpr bool A_T = (LAYOUT == 2);            // A stored [K][M]
  constexpr bool B_T = (LAYOUT != 0);            // B stored [K][N]
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[DBM * DSTRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t b_lds[DBN * DSTRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = (int64_t)tm * DBM, n0 = (int64_t)tn * DBN;
  const int wm0 = (wave & 1) * 64, wn0 = (wave >> 1) * 64;

  // register staging for the next k tile
  u32x4 ra[A_T ? 8 : 4];
  u32x4 rb[B_T ? 8 : 4];
  // threads 0..127 stage A blocks and 128..255 B blocks when both are transposed;
  // when only one is transposed, every thread stages the K-contiguous one and
  // threads 0..127 the transposed one.
  auto load = [&](int64_t k0) {
    if constexpr (A_T) {
      if (tid < 128) load_mncontig(A, lda, m0, M, k0, K, tid, ra);
    } else {
      load_kcontig(A, lda, m0, M, k0, K, ra);
    }
    if constexpr (B_T) {
      const int slot = A_T ? tid - 128 : tid;
      if (slot >= 0 && slot < 128) load_mncontig(B, ldb, n0, N, k0, K, slot, rb);
    } else {
      load_kcontig(B, ldb, n0, N, k0, K, rb);
    }
  };
  auto store = [&]() {
    if constexpr (A_T) {
      if (tid < 128) store_mncontig(a_lds, tid, ra);
    } else {
      store_kcontig(a_lds, ra);
    }
    if constexpr (B_T) {
      const int slot = A_T ? tid - 128 : tid;
      if (slot >= 0 && slot < 128) store_mncontig(b_lds, slot, rb);
    } else {
      store_kcontig(b_lds, rb);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (K + DBK - 1) / DBK;
  if (ktiles > 0) load(0);
  for (int kt = 0; kt < ktiles; ++kt) {
    __syncthreads();
    store();
    __syncthreads();
    if (kt + 1 < ktiles) load((int64_t)(kt + 1) * DBK);
#pragma unroll
    for (int s = 0; s < DBK / 32; ++s) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        a[f] = *reinterpret_cast<const u32x4*>(&a_lds[(wm0 + 16 * f + cl) * DSTRIDE + 32 * s + 8 * ks]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        b[c] = *reinterpret_cast<const u32x4*>(&b_lds[(wn0 + 4 * cl + c) * DSTRIDE + 32 * s + 8 * ks]);
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[f][c] = DTYPE == 0 ? mfma16_bf16(a[f], b[c], acc[f][c]) : mfma16_f16(a[f], b[c], acc[f][c]);
    }
  }

  // lane (cl, ks) holds rows 4*ks + v of tile f and columns wn0 + 4*cl + c
  const int64_t col = n0 + wn0 + 4 * cl;
  if (col < N) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = m0 + wm0 + 16 * f + 4 * ks + v;
        if (row < M) {
          u32x2 o;
          if constexpr (DTYPE == 0) {
            o[0] = pack_bf16x2(acc[f][0][v], acc[f][1][v]);
            o[1] = pack_bf16x2(acc[f][2][v], acc[f][3][v]);
          } else {
            o[0] = pack_f16x2(acc[f][0][v], acc[f][1][v]);
            o[1] = pack_f16x2(acc[f][2][v], acc[f][3][v]);
          }
          *reinterpret_cast<u32x2*>(C + row * ldc + col) = o;
        }
      }
    }
  }
}

// Any shape, any alignment: one thread per output element, fp32 accumulation.
template <int DTYPE>
__device__ __forceinline__ float load_elem(const uint16_t* p) {
  if constexpr (DTYPE == 0) return (float)__builtin_bit_cast(__bf16, *p);
  else return (float)__builtin_bit_cast(_Float16, *p);
}

template <int LAYOUT, int DTYPE>
__global__ __launch_bounds__(256) void dense_generic_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                            const uint16_t* __restrict__ B, int64_t ldb,
                                                            uint16_t* __restrict__ C, int64_t ldc,
                                                            int64_t M, int64_t N, int64_t K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * N) return;
  const int64_t r = i / N, c = i - r * N;
  float acc = 0.f;
  for (int64_t p = 0; p < K; ++p) {
    const float a = load_elem<DTYPE>(LAYOUT == 2 ? A + p * lda + r : A + r * lda + p);
    const float b = load_elem<DTYPE>(LAYOUT == 0 ? B + c * ldb + p : B + p * ldb + c);
    acc = __builtin_fmaf(a, b, acc);
  }
  if constexpr (DTYPE == 0) C[r * ldc + c] = (uint16_t)f32_to_bf16_bits(acc);
  else C[r * ldc + c] = __builtin_bit_cast(uint16_t, (_Float16)acc);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the MFMA kernel's vector loads/stores fit this problem.
static bool mfma_fits(const DenseArgs& a) {
  if (!aligned16(a.A) || !aligned16(a.B) || ((uintptr_t)a.C & 7u)) return false;
  if (a.lda % 8 || a.ldb % 8 || a.ldc % 4 || a.N % 4) return false;
  const int64_t a_contig = a.layout == 2 ? a.M : a.K;
  const int64_t b_contig = a.layout == 0 ? a.K : a.N;
  if (a_contig % 8 || b_contig % 8) return false;
  return a.M < (1LL << 31) && a.N < (1LL << 31) && a.K < (1LL << 31);
}

template <int LAYOUT, int DTYPE>
static void dense_dispatch(const DenseArgs& a, hipStream_t stream) {
  const uint16_t* A = a.A;
  const uint16_t* B = a.B;
  if (mfma_fits(a)) {
    const int tiles_m = (int)((a.M + DBM - 1) / DBM), tiles_n = (int)((a.N + DBN - 1) / DBN);
    dense_mfma_kernel<LAYOUT, DTYPE><<<dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream>>>(
        A, a.lda, B, a.ldb, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m);
  } else {
    const int64_t total = a.M * a.N;
    dense_generic_kernel<LAYOUT, DTYPE><<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
        A, a.lda, B, a.ldb, a.C, a.ldc, a.M, a.N, a.K);
  }
}

hipError_t launch_dense(const DenseArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.K == 0) return launch_zero16(a.C, a.M, a.N, a.ldc, stream);
  switch (a.layout * 2 + a.dtype) {
    case 0: dense_dispatch<0, 0>(a, stream); break;
    case 1: dense_dispatch<0, 1>(a, stream); break;
    case 2: dense_dispatch<1, 0>(a, stream); break;
    case 3: dense_dispatch<1, 1>(a, stream); break;
    case 4: dense_dispatch<2, 0>(a, stream); break;
    case 5: dense_dispatch<2, 1>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
