// Internal launchers (host side) of the gfx950 kernels.  Arguments are already
// validated by the C ABI layer; every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// LoRA add in the epilogue of an int4 product: Y += scale * U . B^T with
// U = X . A^T (fp32, columns >= rank zero).  Either U was computed beforehand
// (u: [m][16]) or the product's kernel accumulates it from lora_A itself (a).
struct LoraEpi {
  const float* u;         // precomputed U, or nullptr
  const uint16_t* b;      // lora_B bf16 [n][ldb], the first `rank` entries of each row used
  int64_t ldb;
  int rank;
  float scale;
  const uint16_t* a;      // lora_A bf16 [rank][lda] for U inside the product's launch, or nullptr
  int64_t lda;
  float* row_ss;          // row reduction: += sum over j of y[r][j]^2 (rounded outputs), or nullptr
};

struct Int4Args {
  const uint16_t* x;
  int64_t ldx;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  uint16_t* y;
  int64_t ldy;
  int64_t m, n, k;
  LoraEpi lora;           // zero-initialised: no adapter
  int split_acq_rel = 0;  // 1: the k split's ticket is an acquire-release RMW
};

// U[m][16] = X . A^T in fp32 for lora_A bf16 [rank][lda] (rank <= 16; the
// other columns of U are written as zeros).  u points at lora_bytes(m, k)
// bytes: U, then (256-byte aligned) the partial tiles of its k slices.
hipError_t launch_lora_u(const uint16_t* x, int64_t ldx, const uint16_t* a, int64_t lda, int rank, int64_t m,
                         int64_t k, float* u, hipStream_t stream);
int64_t lora_bytes(int64_t m, int64_t k);

hipError_t launch_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros,
                          float* w, int64_t n, int64_t k, hipStream_t stream);
// Launch shape of the skinny (m <= 16) kernel: strips of 16 * cpl columns,
// `waves` waves per workgroup, k split into `ksplit` slices of `gwg` groups.
struct SkinnyPlan {
  int cpl, nstrips, waves, ksplit, gwg, items_per_xcd;
  int64_t blocks;
  size_t lds;
  int64_t ws_bytes;
};
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int64_t workspace_bytes, bool dot);
int64_t split_workspace_bytes(int64_t nstrips, int64_t ksplit, int64_t m, int cpl);

// Bytes at the front of an int4 workspace that hold the split counters (zero
// between calls).
constexpr int64_t kSplitCounterBytes = 64 << 10;

// ws may be NULL (then no k split); ws_bytes is its size.
hipError_t launch_gemv_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream);
hipError_t launch_fused_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream);
// With ws_bytes >= workspace_int4(m, n, k, 3): a preparation pass into ws first.
hipError_t launch_mfma_int4(const Int4Args& a, void* ws, int64_t ws_bytes, hipStream_t stream);

// True when the kernel that path (1 GEMV, 2 fused, 3 MFMA) launches for these
// arguments and workspace accumulates the LoRA intermediate U itself (lora.a).
bool lora_in_launch(const Int4Args& a, int path, int64_t ws_bytes);

// Workspace bytes a path (1 GEMV, 2 fused, 3 MFMA) can use; 0 if none.
int64_t workspace_int4(int64_t m, int64_t n, int64_t k, int path);
// Text description of the kernel and launch shape of a path.
void describe_int4(int64_t m, int64_t n, int64_t k, int path, int64_t ws_bytes, char* buf, size_t len);

// Writes zeros to a rows x cols matrix of 16-bit elements with leading dimension ld.
hipError_t launch_zero16(uint16_t* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

struct DenseArgs {
  int layout;  // 0 NT, 1 NN, 2 TN
  int dtype;   // 0 bf16, 1 fp16
  int64_t M, N, K;
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  uint16_t* C;
  int64_t ldc;
  int64_t batch;           // >= 1 products, operand b at A + b sa, B + b sb, C + b sc
  int64_t sa, sb, sc;      // batch strides in elements (0 when batch == 1)
  void* ws = nullptr;      // optional workspace: k split counters, then fp32 partials
  int64_t ws_bytes = 0;
  int split_acq_rel = 0;   // 1: the k split's ticket is an acquire-release RMW
};
// Workspace bytes that let a dense product split k (0 when it would not).
int64_t dense_workspace_bytes(const DenseArgs& a);

// batch strides as one kernel argument
struct BatchStrides {
  int64_t a, b, c;
};

hipError_t launch_dense(const DenseArgs& a, hipStream_t stream);

// register-resident bf16 MFMA loop with clock stamps (measurement probe)
hipError_t launch_mfma_probe(int64_t blocks, int iters, uint64_t* clocks, hipStream_t stream);
// 16-byte copy and read-only streams over `bytes` (measurement probes); blocks 0 = automatic
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int64_t blocks, hipStream_t stream);
hipError_t launch_read_probe(const void* src, int64_t bytes, int64_t blocks, uint32_t key, uint32_t* sink,
                             hipStream_t stream);

}  // namespace qg
