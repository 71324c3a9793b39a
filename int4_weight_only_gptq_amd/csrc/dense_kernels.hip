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
#include <type_traits>
#include "launch.hpp"

namespace qg {

constexpr int DBK = 64;
constexpr int SPLIT_MAX = 4;   // k slices of a dense tile at most (the exchange loads three others at once)
constexpr int DSTRIDE = DBK + 8;   // 16-bit elements per LDS row (144 bytes)

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

// Stage an MN-contiguous operand tile: memory [K][rows], 8 k-blocks x rows/8
// row-blocks of 8 x 8 elements; block `slot` is (k-block slot % 8, row-block
// slot / 8), one per thread.
__device__ __forceinline__ void load_mncontig(const uint16_t* __restrict__ p, int64_t ld, int64_t row0,
                                              int64_t rows, int64_t k0, int64_t K, int slot,
                                              u32x4 (&reg)[8]) {
  const int kb = slot & 7, rb = slot >> 3;
  const int64_t gr = row0 + 8 * rb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t gk = k0 + 8 * kb + e;
    reg[e] = (gr < rows && gk < K) ? *reinterpret_cast<const u32x4*>(p + gk * ld + gr)
                                   : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_mncontig(uint16_t* lds, int slot, const u32x4 (&reg)[8]) {
  const int kb = slot & 7, rb = slot >> 3;
  u32x4 t[8];
  transpose8x8(reg, t);
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&lds[(8 * rb + j) * DSTRIDE + 8 * kb]) = t[j];
}

// Tile kernel: BM x BN output tile per workgroup of 4 waves (2 x 2, each
// BM/2 x BN/2 = FM x FN MFMA tiles of 16 x 16), k tiles of 64 double-buffered in
// LDS with one barrier per k tile: the next tile's global loads are in flight
// while the current one is multiplied, and are written to the other buffer
// after.  B fragment c of a wave holds columns wn0 + 16c + lane % 16, the
// standard mapping (lanes 0..15 read 16 consecutive LDS rows, conflict-free
// with the 144-byte row pitch).  The epilogue converts the accumulators into an
// output tile in LDS and writes it with 16-byte row-contiguous stores.
// Workgroup b works on tile (b % 8) * tiles_per_xcd + b / 8, so each XCD gets
// a contiguous, row-major range of tiles (shared A panels in its L2).
template <int BM, int BN>
struct DenseSmem {
  static constexpr int kA = BM * DSTRIDE, kB = BN * DSTRIDE;          // halves per buffer
  static constexpr int kMain = 2 * (kA + kB);                          // two buffers
  static constexpr int kOut = BM * (BN + 8);                           // epilogue tile
  static constexpr int kHalves = kMain > kOut ? kMain : kOut;
};

template <int LAYOUT, int DTYPE, int BM, int BN>
__global__ __launch_bounds__(256) void dense_tile_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                         const uint16_t* __restrict__ B, int64_t ldb,
                                                         uint16_t* __restrict__ C, int64_t ldc, int M,
                                                         int N, int K, int tiles_n, int tiles,
                                                         int tiles_per_xcd, int vec_store, BatchStrides bs) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  constexpr bool A_T = (LAYOUT == 2);            // A stored [K][M]
  constexpr bool B_T = (LAYOUT != 0);            // B stored [K][N]
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  constexpr int ACH = BM / 32, BCH = BN / 32;    // 16-byte chunks per thread, K-contiguous staging
  using SM = DenseSmem<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint16_t dsm[];

  const int t = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm0 = (wave & 1) * WM, wn0 = (wave >> 1) * WN;

  u32x4 ra[A_T ? 8 : ACH];
  u32x4 rb[B_T ? 8 : BCH];
  auto load = [&](int64_t k0) {
    if constexpr (A_T) {
      if (tid < BM) load_mncontig(A, lda, m0, M, k0, K, tid, ra);
    } else {
#pragma unroll
      for (int i = 0; i < ACH; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        const int64_t gr = m0 + r, gk = k0 + 8 * kc;
        ra[i] = (gr < M && gk < K) ? *reinterpret_cast<const u32x4*>(A + gr * lda + gk) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (B_T) {
      if (tid < BN) load_mncontig(B, ldb, n0, N, k0, K, tid, rb);
    } else {
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        const int64_t gr = n0 + r, gk = k0 + 8 * kc;
        rb[i] = (gr < N && gk < K) ? *reinterpret_cast<const u32x4*>(B + gr * ldb + gk) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int buf) {
    uint16_t* la = dsm + buf * SM::kA;
    uint16_t* lb = dsm + 2 * SM::kA + buf * SM::kB;
    if constexpr (A_T) {
      if (tid < BM) store_mncontig(la, tid, ra);
    } else {
#pragma unroll
      for (int i = 0; i < ACH; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        *reinterpret_cast<u32x4*>(&la[r * DSTRIDE + 8 * kc]) = ra[i];
      }
    }
    if constexpr (B_T) {
      if (tid < BN) store_mncontig(lb, tid, rb);
    } else {
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        *reinterpret_cast<u32x4*>(&lb[r * DSTRIDE + 8 * kc]) = rb[i];
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (K + DBK - 1) / DBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load((int64_t)(kt + 1) * DBK);
    const uint16_t* la = dsm + buf * SM::kA;
    const uint16_t* lb = dsm + 2 * SM::kA + buf * SM::kB;
#pragma unroll
    for (int s = 0; s < DBK / 32; ++s) {
      u32x4 a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f)
        a[f] = *reinterpret_cast<const u32x4*>(&la[(wm0 + 16 * f + cl) * DSTRIDE + 32 * s + 8 * ks]);
#pragma unroll
      for (int c = 0; c < FN; ++c)
        b[c] = *reinterpret_cast<const u32x4*>(&lb[(wn0 + 16 * c + cl) * DSTRIDE + 32 * s + 8 * ks]);
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int c = 0; c < FN; ++c)
          acc[f][c] = DTYPE == 0 ? mfma16_bf16(a[f], b[c], acc[f][c]) : mfma16_f16(a[f], b[c], acc[f][c]);
    }
    if (kt + 1 < ktiles) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: accumulators -> output tile in LDS -> 16-byte stores
  constexpr int OP = BN + 8;                     // halves per LDS output row
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm0 + 16 * f + 4 * ks + v, col = wn0 + 16 * c + cl;
        uint16_t h;
        if constexpr (DTYPE == 0) h = (uint16_t)f32_to_bf16_bits(acc[f][c][v]);
        else h = __builtin_bit_cast(uint16_t, (_Float16)acc[f][c][v]);
        dsm[row * OP + col] = h;
      }
  __syncthreads();
  constexpr int CPR = BN / 8;                    // 16-byte chunks per tile row
  for (int c = tid; c < BM * CPR; c += 256) {
    const int r = c / CPR, cc = c - r * CPR;
    const int64_t gr = m0 + r, gc = n0 + 8 * cc;
    if (gr >= M || gc >= N) continue;
    const uint16_t* src = &dsm[r * OP + 8 * cc];
    if (vec_store && gc + 8 <= N) {
      *reinterpret_cast<u32x4*>(C + gr * ldc + gc) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int e = 0; e < 8 && gc + e < N; ++e) C[gr * ldc + gc + e] = src[e];
    }
  }
}

// Pipeline kernel for all three layouts (K % 64 == 0, operands 16-byte
// vectorizable).  Tile BM x BN per workgroup of 4 waves (2 x 2, each
// (BM/2) x (BN/2)), k tiles of 64 in a STAGES-deep ring of LDS buffers filled
// by direct global-to-LDS loads (no staging registers): while tile kt is
// multiplied, tiles kt+1 .. kt+STAGES-1 are in flight.  One barrier per k tile,
// operand fragments read one 32-k step ahead of the MFMAs that use them.
//
// Operand tiles are stored in LDS in their memory orientation, in 16-byte
// chunks, with an XOR swizzle instead of padding (a direct load fills 64
// consecutive chunks per instruction):
//  * K-contiguous operand (A of NT/NN, B of NT): rows = m or n, 8 chunks of 8 k;
//    chunk c of row r sits at 8r + (c ^ (r & 7)).  A fragment is one 16-byte
//    read of row (lane % 16), chunk 4s + lane / 16.
//  * MN-contiguous operand (A of TN, B of NN and TN): rows = k, R/8 chunks of
//    8 m or n; chunk c of row k sits at k*R/8 + (c ^ f(k)), f(k) = 2((k & 3) |
//    ((k >> 1) & 4)).  A fragment is two transposing reads
//    (ds_read_b64_tr_b16): in each 16-lane group, lane 4r + q supplies columns
//    4q..4q+3 of k-row r and lane j receives column j of the 4 rows, i.e. 4
//    consecutive k of one column; the swizzle puts the 16 rows one read
//    touches two to a bank slot (the minimum for 512 bytes).
// Rows or columns past M or N load a clamped valid address; their results
// are discarded.
__device__ __forceinline__ int fmn(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }
// the same XOR limited to a row of R / 8 chunks (R = 64: 8 chunks)
template <int R>
__device__ __forceinline__ int fmn_r(int k) { return fmn(k) & (R / 8 - 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

// 8 consecutive k of column `col` (0 .. R-1) from an MN-contiguous stage
// region with R columns (R/8 chunks per k-row); kb = first k (multiple of 8).
template <int R>
__device__ __forceinline__ u32x4 read_mn_frag(const u32x4* region, int kb, int col0, int lane) {
  const int j = lane & 15, r = j >> 2, q = j & 3;
  const int c = (col0 >> 3) + (q >> 1);
  const int k1 = kb + r, k2 = kb + 4 + r;
  const uint16_t* h1 = reinterpret_cast<const uint16_t*>(region + k1 * (R / 8) + (c ^ fmn_r<R>(k1))) + 4 * (q & 1);
  const uint16_t* h2 = reinterpret_cast<const uint16_t*>(region + k2 * (R / 8) + (c ^ fmn_r<R>(k2))) + 4 * (q & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h1));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h2));
  u32x4 out;
  out[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  out[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  out[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  out[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return out;
}

template <int LAYOUT, int DTYPE, int BM, int BN, int STAGES, int NWV = 4, int WGM = 2, bool KSPLIT = false>
__global__ __launch_bounds__(64 * NWV) void dense_pipe_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_n, int tiles,
    int tiles_per_xcd, int vec_store, BatchStrides bs, int ksplit, int kps, float* __restrict__ partials,
    uint32_t* __restrict__ tickets, int acq_rel, int band_w) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  constexpr bool A_MN = (LAYOUT == 2);           // A stored [K][M]
  constexpr bool B_MN = (LAYOUT != 0);           // B stored [K][N]
  // NWV waves as a WGM x (NWV / WGM) grid over the tile: 4 waves (one per
  // SIMD) or 8 (two per SIMD)
  constexpr int T = 64 * NWV;
  constexpr int WM = BM / WGM, WN = BN / (NWV / WGM), FM = WM / 16, FN = WN / 16;
  constexpr int A_SLOTS = BM * 8, B_SLOTS = BN * 8;           // 16-byte chunks per stage
  constexpr int STAGE = A_SLOTS + B_SLOTS;
  constexpr int A_LOADS = A_SLOTS / T, B_LOADS = B_SLOTS / T;   // per thread per stage
  static_assert(A_SLOTS % T == 0 && B_SLOTS % T == 0 && (NWV == 4 || NWV == 8), "loads per thread");
  constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(LOADS * (STAGES - 1) <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) u32x4 psm[];

  // item = tile * ksplit + k slice (the slices of a tile are consecutive
  // items, so they run on one XCD); slice s takes k tiles [s kps, (s + 1) kps)
  const int item = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (!KSPLIT) ksplit = 1;   // (the exchange below is compiled only into split kernels)
  if (item >= tiles * ksplit) return;
  const int t = item / ksplit, kslice = item - t * ksplit;
  // tile order: bands of band_w tile columns, row-major inside a band, so that
  // an XCD's run of consecutive tiles is a block of rows x band_w columns
  // sharing operand panels in its L2 (band_w = tiles_n: plain row-major)
  const int tiles_m = tiles / tiles_n, band = t / (tiles_m * band_w);
  const int bw = min(band_w, tiles_n - band * band_w), in_band = t - band * tiles_m * band_w;
  const int tm = in_band / bw, tn = band * band_w + (in_band - tm * bw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wm0 = (wave % WGM) * WM, wn0 = (wave / WGM) * WN;
  const int kt0 = kslice * kps;
  A += A_MN ? (int64_t)kt0 * DBK * lda : (int64_t)kt0 * DBK;
  B += B_MN ? (int64_t)kt0 * DBK * ldb : (int64_t)kt0 * DBK;

  // source of each of this thread's chunks (chunk tid + 256 i of the operand's
  // stage region), at k tile 0; later tiles add k0 (K-contiguous) or k0 * ld
  const uint16_t* asrc[A_LOADS];
  const uint16_t* bsrc[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int slot = tid + T * i;
    if constexpr (A_MN) {
      const int k = slot / (BM / 8), c = (slot % (BM / 8)) ^ fmn_r<BM>(k);
      const int64_t gm = m0 + 8 * c < M ? m0 + 8 * c : (int64_t)M - 8;
      asrc[i] = A + (int64_t)k * lda + gm;
    } else {
      const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
      const int64_t gr = m0 + r < M ? m0 + r : (int64_t)M - 1;
      asrc[i] = A + gr * lda + 8 * c;
    }
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int slot = tid + T * i;
    if constexpr (B_MN) {
      const int k = slot / (BN / 8), c = (slot % (BN / 8)) ^ fmn_r<BN>(k);
      const int64_t gn = n0 + 8 * c < N ? n0 + 8 * c : (int64_t)N - 8;
      bsrc[i] = B + (int64_t)k * ldb + gn;
    } else {
      const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
      const int64_t gr = n0 + r < N ? n0 + r : (int64_t)N - 1;
      bsrc[i] = B + gr * ldb + 8 * c;
    }
  }
  const int64_t astep = A_MN ? (int64_t)DBK * lda : DBK;      // source advance per k tile
  const int64_t bstep = B_MN ? (int64_t)DBK * ldb : DBK;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = K / DBK - kt0 < kps ? K / DBK - kt0 : kps;   // this slice's k tiles
  // direct load j (0 .. LOADS-1) of stage st: each wave-instruction fills 64
  // consecutive chunks of the stage's buffer
  auto issue1 = [&](int st, int j) {
    u32x4* base = psm + (size_t)(st % STAGES) * STAGE;
    if (j < A_LOADS)
      __builtin_amdgcn_global_load_lds((void*)(asrc[j] + st * astep), (void*)(base + T * j + 64 * wave), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((void*)(bsrc[j - A_LOADS] + st * bstep),
                                       (void*)(base + A_SLOTS + T * (j - A_LOADS) + 64 * wave), 16, 0, 0);
  };
  // operand fragment j (0 .. FM-1: rows of A, FM .. FM+FN-1: columns of B) of
  // k step s (32 k) of stage kt
  //
  // An M/N-contiguous fragment (column col0 + l % 16 of 8 k-rows) takes two
  // transposed 8-byte reads at k-rows kb + r and kb + 4 + r (r = (l % 16) / 4,
  // kb = 32 s + 8 (l / 16)).  Both rows get the same chunk XOR of the stage
  // layout, 2 (r | 4 (l / 16 % 2)), for either k step, and it only touches
  // the even part of the chunk index, so a fragment's address is a per-lane
  // base for its column group plus constant offsets for s and the row half.
  const int r4 = (lane & 15) >> 2, q4 = lane & 3;
  auto mn_base = [&](int R, int col0) {    // halfword offset in the operand region
    const int x = (2 * (r4 | 4 * (ks & 1))) & (R / 8 - 1);
    return ((8 * ks + r4) * (R / 8) + (((col0 >> 3) ^ x) | (q4 >> 1))) * 8 + 4 * (q4 & 1);
  };
  auto read_mn = [&](const u32x4* region, int R, int base, int s) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(region) + base + 32 * s * R;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h + 4 * R));
    u32x4 out;
    out[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    out[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    out[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    out[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return out;
  };
  auto read1 = [&](int kt, int s, int j, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
    const u32x4* la = psm + (size_t)(kt % STAGES) * STAGE;
    const u32x4* lb = la + A_SLOTS;
    const int ch = 4 * s + ks;
    if (j < FM) {
      if constexpr (A_MN) a[j] = read_mn(la, BM, mn_base(BM, wm0 + 16 * j), s);
      else a[j] = la[swz(wm0 + 16 * j + cl, ch)];
    } else {
      const int c = j - FM;
      if constexpr (B_MN) b[c] = read_mn(lb, BN, mn_base(BN, wn0 + 16 * c), s);
      else b[c] = lb[swz(wn0 + 16 * c + cl, ch)];
    }
  };
  // the FN MFMAs of accumulator row f
  auto mma_row = [&](int f, const u32x4 (&a)[FM], const u32x4 (&b)[FN]) {
#pragma unroll
    for (int c = 0; c < FN; ++c)
      acc[f][c] = DTYPE == 0 ? mfma16_bf16(a[f], b[c], acc[f][c]) : mfma16_f16(a[f], b[c], acc[f][c]);
  };
  constexpr int NFRAG = FM + FN, RROWS = FM / 2;   // fragment reads spread over the first FM/2 rows

  // Every buffer starts filled.  Per k tile kt (its first k step already in
  // registers r0), with scheduling barriers fixing the order:
  //  1. MFMA rows of the first k step, the second k step read into r1
  //     between rows 0 .. FM/2-1;
  //  2. one barrier: stage kt + 1 has landed for every wave, and nobody reads
  //     stage kt any more (all reads of it are complete); stage kt's buffer
  //     is refilled with stage kt + STAGES;
  //  3. MFMA rows of the second k step, the first k step of kt + 1 read into
  //     r0 between rows 0 .. FM/2-1.
  // So the matrix unit waits for neither an operand read nor a load issue,
  // only at the one barrier per k tile.  Where the barrier and the refill go
  // is measured per operand form: with K-contiguous operands the barrier
  // follows the first k step and the refill loads are spread over the rows of
  // the second; with a transposed operand (whose loads take longer to land)
  // the barrier comes right after the reads of r1, half-way through the
  // first k step, and the refill is issued at once, a whole k tile before
  // it is needed.
  constexpr bool EARLY = A_MN || B_MN;
#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < ktiles)
#pragma unroll
      for (int j = 0; j < LOADS; ++j) issue1(st, j);
  if (ktiles >= STAGES) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 1)));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  u32x4 r0a[FM], r0b[FN], r1a[FM], r1b[FN];
#pragma unroll
  for (int j = 0; j < NFRAG; ++j) read1(0, 0, j, r0a, r0b);
  // one k tile; refill = kt + STAGES < ktiles, next = kt + 1 < ktiles, either
  // compile-time (std::true_type / false_type) or run-time uniform flags
  auto tile = [&](int kt, auto refill, auto next) {
    constexpr int BAR_ROW = EARLY ? RROWS : FM;        // first-step rows before the barrier
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & ~(0xF << 8));     // r0 complete
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < BAR_ROW; ++f) {
      mma_row(f, r0a, r0b);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NFRAG; ++j)
        if (j * RROWS / NFRAG == f) read1(kt, 1, j, r1a, r1b);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage kt + 1 landed (with a refill ahead, stages kt + 2 .. kt + STAGES - 1
    // may stay in flight; without, fewer were issued and all are waited for),
    // and this wave's reads of stage kt are complete
    if (refill) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 2)) & ~(0xF << 8));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~(0xF << 8));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (EARLY) {
      if (refill) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) issue1(kt + STAGES, j);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = BAR_ROW; f < FM; ++f) mma_row(f, r0a, r0b);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      mma_row(f, r1a, r1b);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!EARLY) {
        if (refill) {
#pragma unroll
          for (int j = 0; j < LOADS; ++j)
            if (j * FM / LOADS == f) issue1(kt + STAGES, j);
        }
      }
      if (next) {
#pragma unroll
        for (int j = 0; j < NFRAG; ++j)
          if (j * RROWS / NFRAG == f) read1(kt + 1, 0, j, r0a, r0b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (!EARLY) {
    // K-contiguous operands: the last tiles in loops of their own, branch-free
    using T_ = std::true_type;
    using F_ = std::false_type;
    int kt = 0;
    for (; kt + STAGES < ktiles; ++kt) tile(kt, T_{}, T_{});
    for (; kt + 1 < ktiles; ++kt) tile(kt, F_{}, T_{});
    tile(kt, F_{}, F_{});
  } else {
    // with transposed reads, separate loops made the register allocator
    // shuffle accumulators between loops; one loop with uniform flags
    for (int kt = 0; kt < ktiles; ++kt) tile(kt, kt + STAGES < ktiles, kt + 1 < ktiles);
  }
  __syncthreads();

  if constexpr (KSPLIT) {
    // Split k: every slice stores its fp32 accumulators (fragment order:
    // element pair h of (f, c) of thread tid at ((f FN + c) 2 + h) T + tid,
    // 8-byte agent-coherent stores, 512 contiguous bytes per wave and store),
    // waits for them and takes a ticket; the last slice of the tile to arrive
    // adds the slices in slice order (its own from registers) and goes on to
    // the epilogue.  The exchange's ordering is that of the int4 split (acq_rel:
    // an acquire-release ticket).
    __shared__ int last_slice;
    uint64_t* part64 = reinterpret_cast<uint64_t*>(partials);
    uint64_t* mine = part64 + ((int64_t)t * ksplit + kslice) * (FM * FN * 2 * T);
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int c = 0; c < FN; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float lo = acc[f][c][2 * h], hi = acc[f][c][2 * h + 1];
          const uint64_t pair = (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                                ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
          __hip_atomic_store(&mine[((f * FN + c) * 2 + h) * T + tid], pair, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
    asm volatile("" ::: "memory");   // (no instruction: keeps the stores above the wait)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (tid == 0) last_slice = ticket_add(&tickets[t], acq_rel) == (uint32_t)(ksplit - 1);
    __syncthreads();
    if (!last_slice) return;
    // the O = ksplit - 1 other slices' pairs, FG row fragments per batch of
    // loads (at most 32 pairs in flight per thread), added in slice order
    constexpr int SLICE = FM * FN * 2 * T, PAIRS = FN * 2;
    const uint64_t* base = part64 + (int64_t)t * ksplit * SLICE;
    auto reduce = [&](auto o_) {
      constexpr int O = decltype(o_)::value;
      constexpr int FG0 = 32 / (O * PAIRS), FG = FG0 < 1 ? 1 : (FG0 > FM ? FM : FG0);
#pragma unroll
      for (int f0 = 0; f0 < FM; f0 += FG) {
        uint64_t w[FG][O][PAIRS];
#pragma unroll
        for (int g = 0; g < FG; ++g)
#pragma unroll
          for (int j = 0; j < O; ++j) {
            const int q = j < kslice ? j : j + 1;
            const uint64_t* src = base + (int64_t)q * SLICE + (f0 + g) * FN * 2 * T + tid;
#pragma unroll
            for (int e = 0; e < PAIRS; ++e)
              w[g][j][e] = f0 + g < FM ? __hip_atomic_load(src + e * T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
          }
#pragma unroll
        for (int g = 0; g < FG; ++g) {
          const int f = f0 + g;
          if (f >= FM) break;
#pragma unroll
          for (int c = 0; c < FN; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int e = c * 2 + h;
              float lo = 0.f, hi = 0.f;
#pragma unroll
              for (int p = 0; p <= O; ++p) {
                const int jp = p < kslice ? p : p - 1;   // (selects: no indexed registers)
                uint64_t v = w[g][0][e];
#pragma unroll
                for (int j = 1; j < O; ++j) v = jp == j ? w[g][j][e] : v;
                lo += p == kslice ? acc[f][c][2 * h] : __builtin_bit_cast(float, (uint32_t)v);
                hi += p == kslice ? acc[f][c][2 * h + 1] : __builtin_bit_cast(float, (uint32_t)(v >> 32));
              }
              acc[f][c][2 * h] = lo;
              acc[f][c][2 * h + 1] = hi;
            }
        }
      }
    };
    if (ksplit == 2) reduce(std::integral_constant<int, 1>{});
    else if (ksplit == 3) reduce(std::integral_constant<int, 2>{});
    else reduce(std::integral_constant<int, 3>{});
    if (tid == 0) __hip_atomic_store(&tickets[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // epilogue: accumulators -> output tile in LDS -> 16-byte stores
  uint16_t* osm = reinterpret_cast<uint16_t*>(psm);
  constexpr int OP = BN + 8;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm0 + 16 * f + 4 * ks + v, col = wn0 + 16 * c + cl;
        uint16_t h;
        if constexpr (DTYPE == 0) h = (uint16_t)f32_to_bf16_bits(acc[f][c][v]);
        else h = __builtin_bit_cast(uint16_t, (_Float16)acc[f][c][v]);
        osm[row * OP + col] = h;
      }
  __syncthreads();
  constexpr int CPR = BN / 8;
  for (int c = tid; c < BM * CPR; c += T) {
    const int r = c / CPR, cc = c - r * CPR;
    const int64_t gr = m0 + r, gc = n0 + 8 * cc;
    if (gr >= M || gc >= N) continue;
    const uint16_t* src = &osm[r * OP + 8 * cc];
    if (vec_store && gc + 8 <= N) {
      *reinterpret_cast<u32x4*>(C + gr * ldc + gc) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int e = 0; e < 8 && gc + e < N; ++e) C[gr * ldc + gc + e] = src[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Products with one output dimension of at most 16 (the rank-16 LoRA factors:
// C[t][16] = X . A_l^T, dU = dY . B_l, dB_l = dY^T . U, dA_l = dU^T . X).
// They stream one large operand once and are bound by HBM, so the kernel is
// built for bytes in flight, not for MFMA throughput: one workgroup owns a
// 16 x 16 output tile, its W waves take interleaved 32-row k steps (U of
// them per round, all loads issued before any MFMA), and the W partial
// tiles are summed through LDS at the end.
//
// A K-contiguous operand (A of NT and NN, B of NT) is loaded straight into
// the MFMA fragment (lane: row l % 16, 8 consecutive k).  An M/N-contiguous
// one (B of NN and TN, A of TN) is loaded as 32 k-rows x 16 columns (64
// lanes x 16 bytes) into a wave-private LDS buffer and read back transposed
// with ds_read_b64_tr_b16 (two reads of 4 k-rows each); no barrier is needed
// since only the wave itself touches its buffer.
// ---------------------------------------------------------------------------
constexpr int SK_W = 16;

// 8 consecutive k (kb .. kb+7) of column j (0..15) from a wave buffer of
// 32 k-rows x 16 columns (k-row k at chunks 2k, 2k+1).
__device__ __forceinline__ u32x4 read16_frag(const u32x4* buf, int kb, int lane) {
  const int j = lane & 15, r = j >> 2, q = j & 3;
  const uint16_t* h1 = reinterpret_cast<const uint16_t*>(buf + 2 * (kb + r) + (q >> 1)) + 4 * (q & 1);
  const uint16_t* h2 = reinterpret_cast<const uint16_t*>(buf + 2 * (kb + 4 + r) + (q >> 1)) + 4 * (q & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h1));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(h2));
  u32x4 out;
  out[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  out[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  out[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  out[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return out;
}

// Raw 16 bytes of operand P for k step k0: a fragment (K-contiguous: row
// r0 + l % 16, k0 + 8 (l / 16)) or a staging chunk (MN-contiguous: k-row
// k0 + l / 2, columns r0 + 8 (l % 2)).  Past K: zeros (they enter the sum);
// past the row / column count: a clamped valid address (result discarded).
template <bool MN>
__device__ __forceinline__ u32x4 load_sk(const uint16_t* __restrict__ p, int64_t ld, int rows, int K,
                                         int r0, int k0, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  if constexpr (MN) {
    const int kr = k0 + (lane >> 1);
    int c = r0 + 8 * (lane & 1);
    if (c >= rows) c = r0;                 // a whole chunk past the end (rows % 8 == 0)
    return kr < K ? *reinterpret_cast<const u32x4*>(p + (int64_t)kr * ld + c) : z;
  } else {
    const int r = r0 + (lane & 15) < rows ? r0 + (lane & 15) : rows - 1;
    const int kc = k0 + 8 * (lane >> 4);
    return kc < K ? *reinterpret_cast<const u32x4*>(p + (int64_t)r * ld + kc) : z;
  }
}

// U k steps per round per wave: 4 when at most one operand is staged, 2 when
// both are (TN), so that the LDS of two workgroups fits on a CU.
template <int LAYOUT, int DTYPE>
__global__ __launch_bounds__(64 * SK_W) void dense_splitk16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_n, int tiles,
    int tiles_per_xcd, BatchStrides bs) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  constexpr bool A_MN = (LAYOUT == 2), B_MN = (LAYOUT != 0);
  constexpr int U = (A_MN && B_MN) ? 2 : 4;
  constexpr int NSTAGED = (A_MN ? 1 : 0) + (B_MN ? 1 : 0);
  constexpr int STAGE_CHUNKS = SK_W * U * 64 * NSTAGED;   // 16-byte chunks
  constexpr int RED_CHUNKS = SK_W * 64;                    // f32x4 partial tiles
  __shared__ u32x4 smem[STAGE_CHUNKS > RED_CHUNKS ? STAGE_CHUNKS : RED_CHUNKS];
  // consecutive tiles (adjacent 16-wide strips) run on one XCD and share its L2
  const int t = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = (t / tiles_n) * 16, j0 = (t % tiles_n) * 16;
  const int ksteps = (K + 31) >> 5;
  u32x4* sa = smem + (size_t)wave * U * 64 * NSTAGED;   // this wave's staging buffers
  u32x4* sb = sa + (A_MN ? U * 64 : 0);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < ksteps; s0 += SK_W * U) {
    u32x4 ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = 32 * (s0 + SK_W * u);   // past K loads zeros
      ra[u] = load_sk<A_MN>(A, lda, M, K, i0, k0, lane);
      rb[u] = load_sk<B_MN>(B, ldb, N, K, j0, k0, lane);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (A_MN) sa[64 * u + lane] = ra[u];
      if constexpr (B_MN) sb[64 * u + lane] = rb[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = 8 * (lane >> 4);
      const u32x4 a = A_MN ? read16_frag(sa + 64 * u, kb, lane) : ra[u];
      const u32x4 b = B_MN ? read16_frag(sb + 64 * u, kb, lane) : rb[u];
      acc = DTYPE == 0 ? mfma16_bf16(a, b, acc) : mfma16_f16(a, b, acc);
    }
  }
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  __syncthreads();   // staging buffers are reused for the partial tiles
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 tot = red[lane];
#pragma unroll
    for (int w = 1; w < SK_W; ++w) tot += red[w * 64 + lane];
    const int col = j0 + (lane & 15);
    if (col < N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i0 + 4 * (lane >> 4) + v;
        if (row < M) {
          uint16_t h;
          if constexpr (DTYPE == 0) h = (uint16_t)f32_to_bf16_bits(tot[v]);
          else h = __builtin_bit_cast(uint16_t, (_Float16)tot[v]);
          C[(int64_t)row * ldc + col] = h;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Products with K <= 32 (Y += U . B_l^T and dX += dU . A_l of a rank-16
// adapter): a rank-K outer product whose cost is writing C.  Each wave owns a
// 64 x 64 tile of C and does one k step of 16 MFMAs; N-fragment c of a 64-column
// block holds columns 4 * l + c (l = lane % 16), so a lane ends with 4
// adjacent columns of 16 rows and 16 lanes store one 128-byte row segment.
// A (K-contiguous) and NT's B load straight into fragments; NN's B ([K][N])
// is staged per wave (K rows x 64 columns) and read back transposed.
// ---------------------------------------------------------------------------
template <int LAYOUT, int DTYPE>
__global__ __launch_bounds__(256) void dense_smallk_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_n, int tiles,
    int tiles_per_xcd, int vec_store, BatchStrides bs) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  constexpr bool B_MN = (LAYOUT == 1);
  __shared__ u32x4 bstage[B_MN ? 4 * 256 : 1];   // per wave: 32 k-rows x 64 columns
  const int t = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int lane = threadIdx.x & 63, cl = lane & 15, ks = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = (t / tiles_n) * 64, n0 = (t % tiles_n) * 256 + 64 * wave;
  const u32x4 z = {0u, 0u, 0u, 0u};

  u32x4 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int r = m0 + 16 * f + cl < M ? m0 + 16 * f + cl : M - 1;
    a[f] = 8 * ks < K ? *reinterpret_cast<const u32x4*>(A + (int64_t)r * lda + 8 * ks) : z;
  }
  if constexpr (!B_MN) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = n0 + 4 * cl + c < N ? n0 + 4 * cl + c : N - 1;
      b[c] = 8 * ks < K ? *reinterpret_cast<const u32x4*>(B + (int64_t)col * ldb + 8 * ks) : z;
    }
  } else {
    // Stage rows k of B[k][n0 .. n0+63] with the columns reordered so that
    // position 16 (col % 4) + col / 4 holds column col: fragment c's columns
    // 4 l + c then sit at positions 16 c .. 16 c + 15.  A 16-byte chunk of
    // columns 8 ch .. 8 ch + 7 becomes the pairs (x_e, x_{e+4}), e = 0..3, at
    // positions 16 e + 2 ch (+1).  Past K zeros, past N a clamped chunk.
    uint32_t* buf = reinterpret_cast<uint32_t*>(bstage + 256 * wave);   // 32 rows x 32 dwords
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kr = 8 * p + (lane >> 3), ch = lane & 7;
      int c0 = n0 + 8 * ch;
      if (c0 >= N) c0 = N - 8;
      const u32x4 v = kr < K ? *reinterpret_cast<const u32x4*>(B + (int64_t)kr * ldb + c0) : z;
      const u32x4 pv = x_pairs_permuted(v);
#pragma unroll
      for (int e = 0; e < 4; ++e) buf[32 * kr + 8 * e + ch] = pv[e];
    }
    // fragment c: 8 consecutive k of position 16 c + (lane % 16), two
    // transposing reads of 4 k-rows each (lane 4 r + q addresses row r,
    // positions 4 q .. 4 q + 3 of the 16)
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(buf);
    const int r = cl >> 2, q = cl & 3;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hb + (8 * ks + r) * 64 + 16 * c + 4 * q));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hb + (8 * ks + 4 + r) * 64 + 16 * c + 4 * q));
      b[c][0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
      b[c][1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
      b[c][2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
      b[c][3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[f][c] = DTYPE == 0 ? mfma16_bf16(a[f], b[c], f32x4{0.f, 0.f, 0.f, 0.f})
                             : mfma16_f16(a[f], b[c], f32x4{0.f, 0.f, 0.f, 0.f});

  const int col = n0 + 4 * cl;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + 16 * f + 4 * ks + v;
      if (row >= M || col >= N) continue;
      uint16_t h[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (DTYPE == 0) h[c] = (uint16_t)f32_to_bf16_bits(acc[f][c][v]);
        else h[c] = __builtin_bit_cast(uint16_t, (_Float16)acc[f][c][v]);
      }
      uint16_t* dst = C + (int64_t)row * ldc + col;
      if (vec_store && col + 4 <= N) {
        u32x2 o;
        o[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        o[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
        for (int c = 0; c < 4 && col + c < N; ++c) dst[c] = h[c];
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
                                                            int64_t M, int64_t N, int64_t K, BatchStrides bs) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
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

// ---------------------------------------------------------------------------
// FP32 products (A, B and C fp32, fp32 accumulation) on the 16x16x4 fp32 MFMA.
// Tile 128 x 128 per workgroup of 4 waves (2 x 2, 64 x 64 each), k tiles of 32
// staged through registers into two LDS buffers, one barrier per k tile.
//
// One MFMA takes one value per lane per operand (lane l: row or column l % 16,
// k index l / 16 of its 4).  The k order inside a 16-k group is permuted so
// that a K-contiguous fragment is one 16-byte read: lane group g holds
// k = 16q + 4g .. 16q + 4g + 3 and MFMA j (0..3) of the group uses element j,
// i.e. MFMA j covers k = 16q + 4g + j over the four lane groups g.  Both
// operands use the same order, so each of the 16 k of the group enters the
// sum exactly once.  An M/N-contiguous fragment gathers the same four k with
// four 4-byte reads.  LDS rows are padded by 16 bytes (K-contiguous: 36
// floats per row; M/N-contiguous: 132 floats per k-row) so that the 16 rows a
// fragment read touches fall in distinct banks.
// ---------------------------------------------------------------------------
constexpr int FBK = 32;                  // k per stage
constexpr int FKP = FBK + 4;             // floats per LDS row, K-contiguous operand
constexpr int FMP = 128 + 4;             // floats per LDS k-row, M/N-contiguous operand
constexpr int F32_REGION = 128 * FKP > FBK * FMP ? 128 * FKP : FBK * FMP;   // floats per operand buffer

// BM = 128 or 64 rows per tile (waves of 64 x 64 or 32 x 64): the 64-row tile
// for products whose 128-row tiles would leave CUs idle in their last round.
template <int LAYOUT, int BM = 128, int NWF = 4>
__global__ __launch_bounds__(64 * NWF) void dense_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ B, int64_t ldb,
                                                        float* __restrict__ C, int64_t ldc, int M, int N,
                                                        int K, int tiles_n, int tiles, int tiles_per_xcd,
                                                        BatchStrides bs) {
  A += blockIdx.y * bs.a;   // batch blockIdx.y
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  constexpr bool A_MN = (LAYOUT == 2), B_MN = (LAYOUT != 0);
  static_assert(BM == 128 || BM == 64, "tile rows");
  static_assert(NWF == 4 || NWF == 8, "waves");
  // NWF waves as 2 x (NWF / 2): 4 waves of (BM / 2) x 64, or 8 of (BM / 2) x 32
  constexpr int TF = 64 * NWF, WNF = 128 / (NWF / 2);
  constexpr int FM = BM / 32, FN = WNF / 16;
  constexpr int AL = BM * 8 / TF;            // float4 loads of A per thread and k tile
  constexpr int BLD = 128 * 8 / TF;          // of B
  __shared__ __attribute__((aligned(16))) float fsm[2][2][F32_REGION];   // [buffer][A, B]

  const int t = (blockIdx.x & 7) * tiles_per_xcd + (blockIdx.x >> 3);
  if (t >= tiles) return;
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 15, ks = lane >> 4;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * 128;
  const int wm0 = (wave & 1) * (BM / 2), wn0 = (wave >> 1) * WNF;

  // AL (A) and BLD (B) float4 per thread and k tile; past the edges: zeros.
  // An operand of R rows (R = BM or 128): K-contiguous, 8 float4 per row;
  // M/N-contiguous, R / 4 float4 per k-row.
  f32x4 ra[AL], rb[BLD];
  auto load_op = [&](const float* __restrict__ P, int64_t ld, int64_t r0, int64_t rows, bool mn, int64_t k0,
                     auto& reg) {
    constexpr int L = sizeof(reg) / sizeof(reg[0]), R = L * TF / 8;   // rows of this operand's tile
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int c = tid + TF * i;
      if (mn) {
        const int64_t gk = k0 + c / (R / 4), gr = r0 + 4 * (c % (R / 4));
        reg[i] = (gk < K && gr < rows) ? *reinterpret_cast<const f32x4*>(P + gk * ld + gr)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int64_t gr = r0 + c / 8, gk = k0 + 4 * (c % 8);
        reg[i] = (gr < rows && gk < K) ? *reinterpret_cast<const f32x4*>(P + gr * ld + gk)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_op = [&](float* region, bool mn, const auto& reg) {
    constexpr int L = sizeof(reg) / sizeof(reg[0]), R = L * TF / 8;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int c = tid + TF * i;
      if (mn) *reinterpret_cast<f32x4*>(region + (c / (R / 4)) * FMP + 4 * (c % (R / 4))) = reg[i];
      else *reinterpret_cast<f32x4*>(region + (c / 8) * FKP + 4 * (c % 8)) = reg[i];
    }
  };
  auto load = [&](int64_t k0) {
    load_op(A, lda, m0, M, A_MN, k0, ra);
    load_op(B, ldb, n0, N, B_MN, k0, rb);
  };
  auto store = [&](int buf) {
    store_op(fsm[buf][0], A_MN, ra);
    store_op(fsm[buf][1], B_MN, rb);
  };
  // the four k (16q + 4 ks + j, j = 0..3) of row or column `r` of a region
  auto frag = [&](const float* region, bool mn, int r, int q) {
    if (mn) {
      const float* p = region + (16 * q + 4 * ks) * FMP + r;
      return f32x4{p[0], p[FMP], p[2 * FMP], p[3 * FMP]};
    }
    return *reinterpret_cast<const f32x4*>(region + r * FKP + 16 * q + 4 * ks);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[f][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (K + FBK - 1) / FBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load((int64_t)(kt + 1) * FBK);
#pragma unroll
    for (int q = 0; q < FBK / 16; ++q) {
      f32x4 a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) a[f] = frag(fsm[buf][0], A_MN, wm0 + 16 * f + cl, q);
#pragma unroll
      for (int c = 0; c < FN; ++c) b[c] = frag(fsm[buf][1], B_MN, wn0 + 16 * c + cl, q);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int c = 0; c < FN; ++c) acc[f][c] = mfma16_f32(a[f][j], b[c][j], acc[f][c]);
    }
    if (kt + 1 < ktiles) store(buf ^ 1);
    __syncthreads();
  }

  // lane (cl, ks) holds rows 4 ks + v, column cl of each 16 x 16 block: 16 lanes
  // store 64 contiguous bytes of a row
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t gr = m0 + wm0 + 16 * f + 4 * ks + v, gc = n0 + wn0 + 16 * c + cl;
        if (gr < M && gc < N) C[gr * ldc + gc] = acc[f][c][v];
      }
}

// Any fp32 shape and alignment: one thread per output element.
template <int LAYOUT>
__global__ __launch_bounds__(256) void dense_generic_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                                const float* __restrict__ B, int64_t ldb,
                                                                float* __restrict__ C, int64_t ldc, int64_t M,
                                                                int64_t N, int64_t K, BatchStrides bs) {
  A += blockIdx.y * bs.a;
  B += blockIdx.y * bs.b;
  C += blockIdx.y * bs.c;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * N) return;
  const int64_t r = i / N, c = i - r * N;
  float acc = 0.f;
  for (int64_t p = 0; p < K; ++p) {
    const float a = LAYOUT == 2 ? A[p * lda + r] : A[r * lda + p];
    const float b = LAYOUT == 0 ? B[c * ldb + p] : B[p * ldb + c];
    acc = __builtin_fmaf(a, b, acc);
  }
  C[r * ldc + c] = acc;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static BatchStrides strides(const DenseArgs& a) { return BatchStrides{a.sa, a.sb, a.sc}; }

// Whether the tile kernel's 16-byte operand loads fit this problem.
static bool mfma_fits(const DenseArgs& a) {
  if (!aligned16(a.A) || !aligned16(a.B)) return false;
  if (a.lda % 8 || a.ldb % 8 || a.sa % 8 || a.sb % 8) return false;
  const int64_t a_contig = a.layout == 2 ? a.M : a.K;
  const int64_t b_contig = a.layout == 0 ? a.K : a.N;
  if (a_contig % 8 || b_contig % 8) return false;
  return a.M < (1LL << 31) && a.N < (1LL << 31) && a.K < (1LL << 31);
}

#ifndef QG_DENSE_BIG_MIN_TILES
#define QG_DENSE_BIG_MIN_TILES 160     // 256 x 128 tiles wanted before using them
#endif

template <int LAYOUT, int DTYPE, int BM, int BN>
static void tile_launch(const DenseArgs& a, hipStream_t stream) {
  const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = (int)((a.N + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n, per_xcd = (tiles + 7) / 8;
  const int vec = aligned16(a.C) && a.ldc % 8 == 0 && a.sc % 8 == 0;
  const size_t lds = (size_t)DenseSmem<BM, BN>::kHalves * 2;
  dense_tile_kernel<LAYOUT, DTYPE, BM, BN><<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(256), lds, stream>>>(
      a.A, a.lda, a.B, a.ldb, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, vec, strides(a));
}

#ifndef QG_DENSE_PIPE_STAGES
#define QG_DENSE_PIPE_STAGES 3
#endif
// Waves of the 256 x 256 and 256 x 128 tiles: 8, two per SIMD, so that one
// wave's MFMAs run while the other waits on LDS or the barrier (4: one per
// SIMD).  Measured against 4 waves (bf16 training trio, same-process A/B):
// 256 x 256 as 128 x 64 per wave, NN 2048 x 5632 x 2048 73.6 -> 61.9 µs, TN
// 2-9% faster, NT within 5%; then 256 x 128 as 64 x 64 (NT) or 128 x 32 (NN,
// TN) per wave, NN 1024 x 5632 x 2048 48.8 -> 41.3 µs, 4096 x 2048 x 5632
// 121.6 -> 109.0 µs, NT 4096 x 5632 x 2048 97.9 -> 91.9 µs, 2.5% over the trio.
#ifndef QG_DENSE_W128
#define QG_DENSE_W128 8     // waves of the 256 x 128 tile
#endif
#ifndef QG_DENSE_G128
#define QG_DENSE_G128 0     // of which along M (0: 2 for NN, 4 for NT and TN)
#endif
// The 128 x 128 tile: 4 stages, 8 waves of 64 x 32 (NN 2048 x 2048 x 5632
// 82.7 -> 77.3 µs, NT 2048 x 2048 x 5632 58.5 -> 56.5 µs against 4 waves of
// 64 x 64; 2 stages, so that two workgroups share a CU, were slower).
#ifndef QG_DENSE_T0_STAGES
#define QG_DENSE_T0_STAGES 4
#endif
#ifndef QG_DENSE_T0_WAVES
#define QG_DENSE_T0_WAVES 8
#endif
#ifndef QG_DENSE_T0_WGM
#define QG_DENSE_T0_WGM 2
#endif
#ifndef QG_DENSE_W256
#define QG_DENSE_W256 8     // waves of the 256 x 256 tile (128 x 64 each)
#endif

// Tile columns per band of the pipelined kernels' tile order: an XCD's 32 CUs
// run about 32 consecutive items at a time, and a block of r rows x w columns
// of tiles reads r BM + w BN operand rows (of k) into that XCD's L2, least
// near w = sqrt(32 BM / BN) tiles (power of two, at least 32 / tiles_m).
#ifndef QG_DENSE_BAND
#define QG_DENSE_BAND 1      // 0: row-major tile order
#endif
static int band_width(int tiles_m, int tiles_n, int per_xcd, int ksplit, int BM, int BN) {
  if (!QG_DENSE_BAND) return tiles_n;
  const int conc = (per_xcd < 32 ? per_xcd : 32) / ksplit;
  const int conc_tiles = conc > 1 ? conc : 1;
  int w = 1;
  while ((double)(2 * w) * (2 * w) <= 2.0 * conc_tiles * BM / BN) w *= 2;   // nearest power of two in log
  const int wmin = (conc_tiles + tiles_m - 1) / tiles_m;
  if (w < wmin) w = wmin;
  return w < tiles_n ? w : tiles_n;
}

template <int LAYOUT, int DTYPE, int BM, int BN, int STAGES, int NWV = 4, int WGM = 2, bool KSPLIT = false>
static void pipe_launch(const DenseArgs& a, hipStream_t stream, int ksplit = 1) {
  if (!KSPLIT) ksplit = 1;
  const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = (int)((a.N + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n, per_xcd = (tiles * ksplit + 7) / 8;
  const int ktiles = (int)(a.K / DBK), kps = (ktiles + ksplit - 1) / ksplit;
  uint32_t* tickets = ksplit > 1 ? (uint32_t*)a.ws : nullptr;
  float* partials = ksplit > 1 ? (float*)((char*)a.ws + kSplitCounterBytes) : nullptr;
  const int vec = aligned16(a.C) && a.ldc % 8 == 0 && a.sc % 8 == 0;
  const size_t main_bytes = (size_t)STAGES * (BM + BN) * 8 * 16;
  const size_t out_bytes = (size_t)BM * (BN + 8) * 2;
  const size_t lds = main_bytes > out_bytes ? main_bytes : out_bytes;
  dense_pipe_kernel<LAYOUT, DTYPE, BM, BN, STAGES, NWV, WGM, KSPLIT>
      <<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(64 * NWV), lds, stream>>>(
      a.A, a.lda, a.B, a.ldb, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, vec, strides(a),
      ksplit, kps, partials, tickets, a.split_acq_rel, band_width(tiles_m, tiles_n, per_xcd, ksplit, BM, BN));
}

// k split of the pipelined 128 x 128 or 256 x 128 tile, for products whose
// tiles fill at most half of the 256 CUs over a long k: s = min(4, 256 /
// tiles) slices of at least 16 k tiles (1024 k) each; the slices' fp32
// partials (s x BM x 128 x 4 bytes per tile) ride behind the split counters.
// Of the two tiles the one whose tiles x slices fills more CUs is taken; on a
// tie, 256 x 128 for NN (its more efficient tile) and 128 x 128 for NT and TN.
// NT never splits the 256 x 128 tile: its unsplit 128 x 128 and 64 x 128
// tiles fill the chip well, and the larger exchange (128 KiB per slice, about
// 8-9 µs at 256 busy CUs) lost (2048 x 2048 x 5632 1.12x, 1024 x 2048 x 5632
// 1.03x).  Same-process A/B, bf16, split time / best unsplit time: NT
// 256 x 2048 x 8192 0.53, 1024 x 1024 x 8192 0.58, 512 x 2048 x 5632 0.69,
// 1024 x 2048 x 5632 0.82, 512 x 4096 x 4096 0.87; NN 512 x 2048 x 5632 0.47
// (128 x 128 tiles), 1024 x 2048 x 5632 0.66, 2048 x 2048 x 5632 0.84 (256 x
// 128); TN 256 x 2048 x 8192 0.40, 1024 x 2048 x 5632 0.71, 2048 x 2048 x
// 5632 0.94.
#ifndef QG_DENSE_SPLIT_TILES
#define QG_DENSE_SPLIT_TILES 128
#endif
#ifndef QG_DENSE_SPLIT_MIN_KT
#define QG_DENSE_SPLIT_MIN_KT 16
#endif
struct DenseSplit {
  int bm = 0;        // rows of the split tile (columns: 128); 0: no split
  int s = 1;         // k slices
  int64_t tiles = 0;
  int64_t bytes() const { return kSplitCounterBytes + tiles * s * bm * 128 * 4; }
};
static DenseSplit plan_dense_split(const DenseArgs& a) {
  DenseSplit best;
  if (a.batch != 1 || a.dtype == 2 || a.K % DBK != 0 || a.M < 128 || a.N < 128) return best;
  for (int bm : {256, 128}) {
    if (bm == 256 && a.layout == 0) continue;
    const int64_t tiles = ((a.M + bm - 1) / bm) * ((a.N + 127) / 128);
    if (tiles > QG_DENSE_SPLIT_TILES || tiles > kSplitCounterBytes / 4) continue;
    int s = (int)(256 / tiles);
    if (s > SPLIT_MAX) s = SPLIT_MAX;
    while (s > 1 && (a.K / DBK) / s < QG_DENSE_SPLIT_MIN_KT) --s;
    if (s < 2) continue;
    const int64_t items = tiles * s, best_items = best.tiles * best.s;
    const bool tie_to_this = bm == 128 && a.layout != 1;
    if (items > best_items || (items == best_items && tie_to_this)) {
      best.bm = bm;
      best.s = s;
      best.tiles = tiles;
    }
  }
  return best;
}

int64_t dense_workspace_bytes(const DenseArgs& a) {
  if (!mfma_fits(a)) return 0;
  const DenseSplit p = plan_dense_split(a);
  return p.bm ? p.bytes() : 0;
}

#ifndef QG_SPLITK16_MIN_K
#define QG_SPLITK16_MIN_K 256     // k below which the 16 x 16 split-k tile is not worth it
#endif

// Tile of the pipelined kernel: each of these runs one workgroup per CU, so a
// launch takes ceil(tiles / 256) rounds of one tile time.  Measured tile times
// relative to 256 x 128: 256 x 256 (128 x 128 per wave, accumulators in AGPRs)
// costs 1.4-1.6x for twice the work, 128 x 128 about 0.6x for half of it,
// 64 x 128 about 0.4x for a quarter of it.
// -1: 64 x 128, 0: 128 x 128, 1: 256 x 128, 2: 256 x 256.
#ifndef QG_DENSE_T256X256
#define QG_DENSE_T256X256 1.5
#endif
#ifndef QG_DENSE_T128X128
#define QG_DENSE_T128X128 0.6
#endif
#ifndef QG_DENSE_T64X128
#define QG_DENSE_T64X128 0.4
#endif
// rounds-model cost of tile t (2: 256 x 256, 1: 256 x 128, 0: 128 x 128,
// -1: 64 x 128) over an M x N output (batch products)
static double pipe_cost(int t, int64_t M, int64_t N, int64_t batch) {
  auto rounds = [batch](int64_t tiles) { return (double)((tiles * batch + 255) / 256); };
  switch (t) {
    case 2: return rounds(((M + 255) / 256) * ((N + 255) / 256)) * QG_DENSE_T256X256;
    case 1: return rounds(((M + 255) / 256) * ((N + 127) / 128));
    case 0: return rounds(((M + 127) / 128) * ((N + 127) / 128)) * QG_DENSE_T128X128;
    default: return rounds(((M + 63) / 64) * ((N + 127) / 128)) * QG_DENSE_T64X128;
  }
}

static int pick_pipe_tile(int64_t M, int64_t N, int64_t batch) {
#ifdef QG_DENSE_FORCE_TILE
  return QG_DENSE_FORCE_TILE;       // tile sweeps
#endif
  const double c2 = pipe_cost(2, M, N, batch), c1 = pipe_cost(1, M, N, batch);
  const double c0 = pipe_cost(0, M, N, batch), cm = pipe_cost(-1, M, N, batch);
  if (c2 <= c1 && c2 < c0 && c2 < cm) return 2;     // ties: 256 x 256 measured 3-4% ahead
  if (c1 <= c0 && c1 <= cm) return 1;
  return c0 <= cm ? 0 : -1;
}

// Two row bands when a tile size leaves its last round mostly empty: the first
// band is whole rounds of 256-row tiles (256 x 256 or 256 x 128), the rest gets
// its own tile choice, each band one launch on the stream.  Returns the first
// band's rows (a multiple of 256) or 0 when one launch is cheaper; a second
// launch is charged QG_DENSE_BAND_GAP of a 256 x 128 round.
#ifndef QG_DENSE_BAND_GAP
#define QG_DENSE_BAND_GAP 0.1
#endif
static int64_t pick_row_bands(int64_t M, int64_t N, int64_t batch, int* t1, int* t2) {
#ifdef QG_DENSE_FORCE_TILE
  return 0;
#endif
  if (batch != 1) return 0;
  const int one = pick_pipe_tile(M, N, 1);
  double best = pipe_cost(one, M, N, 1);
  int64_t m1_best = 0;
  for (int t = 1; t <= 2; ++t) {
    const int64_t tn = t == 2 ? (N + 255) / 256 : (N + 127) / 128;
    for (int64_t r = 1; r <= 8; ++r) {
      const int64_t m1 = (256 * r / tn) * 256;
      if (m1 <= 0 || m1 >= M) break;
      const int other = pick_pipe_tile(M - m1, N, 1);
      const double c = pipe_cost(t, m1, N, 1) + pipe_cost(other, M - m1, N, 1) + QG_DENSE_BAND_GAP;
      if (c < best - 1e-9) {
        best = c;
        m1_best = m1;
        *t1 = t;
        *t2 = other;
      }
    }
  }
  return m1_best;
}

template <int LAYOUT, int DTYPE>
static void dense_dispatch(const DenseArgs& a, hipStream_t stream) {
  if (mfma_fits(a) && (a.M <= 16 || a.N <= 16) && a.K >= QG_SPLITK16_MIN_K) {
    const int tiles_n = (int)((a.N + 15) / 16);
    const int tiles = (int)(((a.M + 15) / 16) * tiles_n), per_xcd = (tiles + 7) / 8;
    dense_splitk16_kernel<LAYOUT, DTYPE><<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(64 * SK_W), 0, stream>>>(
        a.A, a.lda, a.B, a.ldb, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, strides(a));
  } else if (LAYOUT != 2 && mfma_fits(a) && a.K <= 32 && a.M >= 64 && a.N >= 256) {
    const int tiles_n = (int)((a.N + 255) / 256);
    const int tiles = (int)(((a.M + 63) / 64) * tiles_n), per_xcd = (tiles + 7) / 8;
    const int vec = ((uintptr_t)a.C & 7u) == 0 && a.ldc % 4 == 0 && a.sc % 4 == 0;
    dense_smallk_kernel<LAYOUT, DTYPE><<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(256), 0, stream>>>(
        a.A, a.lda, a.B, a.ldb, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, vec, strides(a));
  } else if (mfma_fits(a) && a.K % DBK == 0 && a.M >= 128 && a.N >= 128) {
    const DenseSplit sp = a.ws ? plan_dense_split(a) : DenseSplit{};
    if (sp.bm && sp.bytes() <= a.ws_bytes) {
      const int split = sp.s;
      if (sp.bm == 128)
        pipe_launch<LAYOUT, DTYPE, 128, 128, QG_DENSE_T0_STAGES, QG_DENSE_T0_WAVES, QG_DENSE_T0_WGM, true>(a, stream,
                                                                                                       split);
      else
        pipe_launch<LAYOUT, DTYPE, 256, 128, QG_DENSE_PIPE_STAGES, QG_DENSE_W128,
                    QG_DENSE_G128 ? QG_DENSE_G128 : (LAYOUT == 1 ? 2 : 4), true>(a, stream, split);
      return;
    }
    auto launch_tile = [&](int t, const DenseArgs& b) {
      switch (t) {
        case 2: pipe_launch<LAYOUT, DTYPE, 256, 256, 2, QG_DENSE_W256>(b, stream); break;
        case 1:
          pipe_launch<LAYOUT, DTYPE, 256, 128, QG_DENSE_PIPE_STAGES, QG_DENSE_W128,
                      QG_DENSE_G128 ? QG_DENSE_G128 : (LAYOUT == 1 ? 2 : 4)>(b, stream);
          break;
        case 0: pipe_launch<LAYOUT, DTYPE, 128, 128, QG_DENSE_T0_STAGES, QG_DENSE_T0_WAVES, QG_DENSE_T0_WGM>(b, stream); break;
        default: pipe_launch<LAYOUT, DTYPE, 64, 128, 4>(b, stream); break;
      }
    };
    int t1 = 0, t2 = 0;
    const int64_t m1 = pick_row_bands(a.M, a.N, a.batch, &t1, &t2);
    if (m1 > 0) {
      // rows [0, m1) and [m1, M): A's rows (its columns for TN) and C's rows
      DenseArgs lo = a, hi = a;
      lo.M = m1;
      hi.M = a.M - m1;
      hi.A = a.A + (LAYOUT == 2 ? m1 : m1 * a.lda);
      hi.C = a.C + m1 * a.ldc;
      launch_tile(t1, lo);
      launch_tile(t2, hi);
    } else {
      launch_tile(pick_pipe_tile(a.M, a.N, a.batch), a);
    }
  } else if (mfma_fits(a)) {
    const int64_t big = ((a.M + 255) / 256) * ((a.N + 127) / 128);
    if (big >= QG_DENSE_BIG_MIN_TILES) tile_launch<LAYOUT, DTYPE, 256, 128>(a, stream);
    else tile_launch<LAYOUT, DTYPE, 128, 128>(a, stream);
  } else {
    const int64_t total = a.M * a.N;
    dense_generic_kernel<LAYOUT, DTYPE><<<dim3((unsigned)((total + 255) / 256), (unsigned)a.batch), dim3(256), 0, stream>>>(
        a.A, a.lda, a.B, a.ldb, a.C, a.ldc, a.M, a.N, a.K, strides(a));
  }
}

// Waves of the 128 x 128 fp32 tile: 8 (two per SIMD, 64 x 32 each) for NN and
// TN, 4 (64 x 64) for NT.  Eight against four, same-process A/B: NN 2048 x
// 2048 x 5632 440 -> 405 µs, TN 1-3% faster at every size; NT mixed (2048 x
// 5632 x 2048 538 -> 464 µs, but 4096 tokens 6-8% slower).
#ifndef QG_F32_WAVES
#define QG_F32_WAVES 0    // 0: by layout as above
#endif
#ifndef QG_F32_T64
#define QG_F32_T64 0.55   // time of a round of 64 x 128 fp32 tiles relative to 128 x 128
#endif

template <int LAYOUT>
static void dense_dispatch_f32(const DenseArgs& a, hipStream_t stream) {
  const float* A = reinterpret_cast<const float*>(a.A);
  const float* B = reinterpret_cast<const float*>(a.B);
  float* C = reinterpret_cast<float*>(a.C);
  const int64_t a_contig = LAYOUT == 2 ? a.M : a.K, b_contig = LAYOUT == 0 ? a.K : a.N;
  const bool vec = aligned16(A) && aligned16(B) && a.lda % 4 == 0 && a.ldb % 4 == 0 && a.sa % 4 == 0 &&
                   a.sb % 4 == 0 && a_contig % 4 == 0 && b_contig % 4 == 0 && a.M < (1LL << 31) &&
                   a.N < (1LL << 31) && a.K < (1LL << 31);
  if (vec) {
    // 64-row tiles where they take fewer rounds of the CUs, weighted by their
    // relative time per round
    const int tiles_n = (int)((a.N + 127) / 128);
    const int64_t t128 = ((a.M + 127) / 128) * tiles_n, t64 = ((a.M + 63) / 64) * tiles_n;
    auto rounds = [&](int64_t t) { return (double)((t * a.batch + 255) / 256); };
    if (rounds(t64) * QG_F32_T64 < rounds(t128)) {
      const int tiles = (int)t64, per_xcd = (tiles + 7) / 8;
      dense_f32_kernel<LAYOUT, 64><<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(256), 0, stream>>>(
          A, a.lda, B, a.ldb, C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, strides(a));
    } else {
      const int tiles = (int)t128, per_xcd = (tiles + 7) / 8;
      constexpr int W = QG_F32_WAVES ? QG_F32_WAVES : (LAYOUT == 0 ? 4 : 8);
      dense_f32_kernel<LAYOUT, 128, W><<<dim3((unsigned)(per_xcd * 8), (unsigned)a.batch), dim3(64 * W), 0,
                                         stream>>>(
          A, a.lda, B, a.ldb, C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_n, tiles, per_xcd, strides(a));
    }
  } else {
    const int64_t total = a.M * a.N;
    dense_generic_f32_kernel<LAYOUT><<<dim3((unsigned)((total + 255) / 256), (unsigned)a.batch), dim3(256), 0,
                                       stream>>>(A, a.lda, B, a.ldb, C, a.ldc, a.M, a.N, a.K, strides(a));
  }
}

hipError_t launch_dense(const DenseArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.K == 0) {
    // fp32: each element is two zero halves at twice the leading dimension
    const int w = a.dtype == 2 ? 2 : 1;
    for (int64_t b = 0; b < a.batch; ++b) {
      const hipError_t e = launch_zero16(a.C + w * b * a.sc, a.M, w * a.N, w * a.ldc, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (a.dtype == 2) {
    switch (a.layout) {
      case 0: dense_dispatch_f32<0>(a, stream); break;
      case 1: dense_dispatch_f32<1>(a, stream); break;
      case 2: dense_dispatch_f32<2>(a, stream); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
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
