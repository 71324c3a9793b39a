// C ABI of the library: argument validation, path choice and launch.
// Declarations and the contract of each entry point are in include/qgemm.h.
#include "qgemm.h"

#include <hip/hip_runtime.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"

// Scratch of qgemm_int4_noalloc: one copy per GPU the library runs on, held
// until the process ends.  Host code never passes this name to a kernel: on
// the host it is a stand-in, not a device address; the device address comes
// from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[QG_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;
std::atomic<int32_t> g_split_order{QG_SPLIT_ORDER_HW};

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return QG_OK;
  g_last_hip_error = (int32_t)e;
  return QG_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Validation shared by the int4 entry points; returns QG_OK or the error.
int32_t check_int4(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                   const uint32_t* qzeros, const void* y, int64_t ldy, int64_t m, int64_t n,
                   int64_t k, int32_t group_size) {
  if (m < 0 || n < 0 || k < 0) return QG_ERR_SHAPE;
  if (group_size != 128) return QG_ERR_UNSUPPORTED;
  if (k % 128 != 0 || n % 8 != 0) return QG_ERR_SHAPE;
  // the kernels address a stage of activations and codes with 32-bit byte
  // offsets: 256 rows of x (ldx <= 2^22) and 8 word rows of qweight (n <= 2^26)
  if (n > (int64_t)1 << 26 || k > (int64_t)1 << 22) return QG_ERR_SHAPE;
  if (m == 0 || n == 0) return QG_OK;
  if (y == nullptr) return QG_ERR_NULL;
  if (ldy < n) return QG_ERR_SHAPE;
  if (!aligned(y, 8) || ldy % 4 != 0) return QG_ERR_ALIGN;
  if (k == 0) return QG_OK;
  if (x == nullptr || qweight == nullptr || scales == nullptr) return QG_ERR_NULL;   // qzeros may be null
  if (ldx < k || ldx > (int64_t)1 << 22) return QG_ERR_SHAPE;
  if (!aligned(x, 16) || ldx % 8 != 0) return QG_ERR_ALIGN;
  if (!aligned(qweight, 16) || !aligned(scales, 8) || !aligned(qzeros, 4)) return QG_ERR_ALIGN;
  return QG_OK;
}

// Automatic choice: m = 1 the GEMV; m <= 16 the small-M kernel (one MFMA row
// tile); 16 < m <= 32 the small-M kernel with two row tiles when n is below
// kRowTileMaxN, m <= 24 or its workgroups take at most two passes; 32 < m <= 64 the small-M kernel with three or four
// row tiles when its planned workgroups take a single pass over the 256 CUs,
// or two passes at k > 8192 and m <= 48; else the MFMA tiles.  Measured (cold weights): the tiles pad every wave to 64
// rows and at small n leave CUs idle (4096 x 4096 m = 17 21.0 -> 9.7 µs,
// 2048 x 8192 m = 17 17.6 -> 7.7 µs, 4096 x 14336 m = 20 28.8 -> 14.7 µs); at
// n >= 20480 the row tiles still win to m = 24 (5120 x 25600 m = 17
// 38.9 -> 31.0 µs); above that, in at most two passes (5120 x 25600 m = 28 / 32
// 39.5 / 39.5 -> 34.4 / 37.3 µs, 4096 x 28672 m = 32 35.3 -> 29.4 µs), not in
// more (8192 x 28672 m = 32, 896 workgroups: 55.1 vs 68.0 µs).  Above 32 tokens the
// small-M time grows with m and with every further pass over the CUs: in one
// pass 4096 x 4096 m = 33 / 48 / 56 21.2 / 21.4 / 21.5 -> 14.9 / 17.8 / 21.0 µs,
// 2048 x 8192 m = 48 17.9 -> 11.8 µs, 8192 x 4096 m = 48 31.9 -> 23.1 µs,
// 1024 x 4096 m = 64 16.0 -> 7.9 µs.  In two passes the row tiles win at long
// k (14336 x 4096 m = 33 / 40 / 48 40.1 / 40.3 / 40.3 -> 30.8 / 33.8 / 36.8 µs,
// 11008 x 4096 m = 33 / 40 35.5 / 35.5 -> 30.1 / 32.7 µs, m = 48 even) and not
// at k <= 8192 (8192 x 8192 m = 33 / 40 32.0 / 32.2 vs 32.9 / 35.5 µs,
// 4096 x 11008 m = 48 29.7 vs 31.9 µs).
#ifndef QG_ROWTILE_MAX_N
#define QG_ROWTILE_MAX_N 20480
#endif
constexpr int64_t kRowTileMaxN = QG_ROWTILE_MAX_N;
#ifndef QG_ROWTILE_MAX_BLOCKS
#define QG_ROWTILE_MAX_BLOCKS 256   // one workgroup per CU
#endif
constexpr int64_t kOnePassBlocks = QG_ROWTILE_MAX_BLOCKS;
constexpr int64_t kTwoPassMinK = 8192;    // two passes only above this k (and m <= 48)

int32_t resolve_path(int64_t m, int64_t n, int64_t k, int32_t path) {
  if (path != QG_PATH_AUTO) return path;
  if (m == 1) return QG_PATH_GEMV;
  if (m <= 16) return QG_PATH_FUSED;
  if (m <= 64) {
    const int64_t blocks = qg::plan_skinny(m, n, k, INT64_MAX, false).blocks;
    if (m <= 32 && (n < kRowTileMaxN || m <= 24 || blocks <= 2 * kOnePassBlocks)) return QG_PATH_FUSED;
    if (blocks <= kOnePassBlocks || (m <= 48 && k > kTwoPassMinK && blocks <= 2 * kOnePassBlocks))
      return QG_PATH_FUSED;
  }
  return QG_PATH_MFMA;
}

int32_t check_path(int64_t m, int32_t path) {
  if (path < QG_PATH_AUTO || path > QG_PATH_MFMA) return QG_ERR_UNSUPPORTED;
  if (path == QG_PATH_GEMV && m > 1) return QG_ERR_UNSUPPORTED;
  if (path == QG_PATH_FUSED && m > 16) return QG_ERR_UNSUPPORTED;
  return QG_OK;
}

// Bytes of the LoRA intermediate U (fp32 [m][16]) and its k-slice partials at
// the end of the workspace.
int64_t lora_u_bytes(int64_t m, int64_t k) { return qg::lora_bytes(m, k); }

int32_t run_int4(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                 const uint32_t* qzeros, void* y, int64_t ldy, int64_t m, int64_t n, int64_t k,
                 int32_t group_size, int32_t path, void* ws, int64_t ws_bytes, void* stream,
                 const qg::LoraEpi* lora = nullptr, const void* lora_a = nullptr, int64_t lda_a = 0,
                 float* row_ss = nullptr) {
  int32_t st = check_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size);
  if (st != QG_OK) return st;
  st = check_path(m, path);
  if (st != QG_OK) return st;
  if (ws_bytes < 0) return QG_ERR_SHAPE;
  if (ws != nullptr && !aligned(ws, 16)) return QG_ERR_ALIGN;
  if (m == 0 || n == 0) return QG_OK;
  hipStream_t s = (hipStream_t)stream;
  if (k == 0) return hip_status(qg::launch_zero16((uint16_t*)y, m, n, ldy, s));
  qg::Int4Args a{(const uint16_t*)x, ldx, qweight, scales, qzeros, (uint16_t*)y, ldy, m, n, k};
  a.split_acq_rel = g_split_order.load(std::memory_order_relaxed) == QG_SPLIT_ORDER_ACQ_REL;
  a.lora.row_ss = row_ss;
  if (ws == nullptr) ws_bytes = 0;
  const int32_t rp = resolve_path(m, n, k, path);
  if (lora != nullptr) {
    // the path keeps the 256-byte aligned front part of the workspace; the
    // product's kernel accumulates U = X . A^T itself where it can (one
    // launch), else U goes to the end of the workspace first (two small
    // launches) and the product adds the LoRA term in its epilogue
    const int64_t rest = (ws_bytes - lora_u_bytes(m, k)) & ~(int64_t)255;
    a.lora = *lora;
    a.lora.a = (const uint16_t*)lora_a;
    a.lora.lda = lda_a;
    a.lora.row_ss = row_ss;
    if (!qg::lora_in_launch(a, rp, rest)) {
      float* u = (float*)((char*)ws + rest);
      st = hip_status(qg::launch_lora_u((const uint16_t*)x, ldx, (const uint16_t*)lora_a, lda_a, lora->rank, m,
                                        k, u, s));
      if (st != QG_OK) return st;
      a.lora.u = u;
      a.lora.a = nullptr;
    }
    ws_bytes = rest;
    if (ws_bytes == 0) ws = nullptr;
  }
  switch (rp) {
    case QG_PATH_GEMV: return hip_status(qg::launch_gemv_int4(a, ws, ws_bytes, s));
    case QG_PATH_FUSED: return hip_status(qg::launch_fused_int4(a, ws, ws_bytes, s));
    default: return hip_status(qg::launch_mfma_int4(a, ws, ws_bytes, s));
  }
}

// Device address of `scratch` on the current device, looked up once per device
// with that device current; the split counters (its first 64 KiB) are cleared
// then with a fill kernel on `stream`, ordered before the first product.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t qgemm_int4_lora_rss(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                            int64_t ldb_b, int32_t rank, float lora_scale, float* row_sumsq, void* y,
                            int64_t ldy, int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                            void* workspace, int64_t workspace_bytes, void* stream);

int32_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return QG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || !aligned(p, 256)) return QG_ERR_HIP;
    const int64_t halves = qg::kSplitCounterBytes / 2;
    e = qg::launch_zero16((uint16_t*)p, 1, halves, halves, stream);
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}

}  // namespace

extern "C" {

int32_t qg_abi_version(void) { return QG_ABI_VERSION; }

const char* qg_status_str(int32_t status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_NULL: return "a required pointer is NULL";
    case QG_ERR_SHAPE: return "invalid shape or leading dimension";
    case QG_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case QG_ERR_DTYPE: return "unknown dtype";
    case QG_ERR_LAYOUT: return "unknown layout";
    case QG_ERR_UNSUPPORTED: return "unsupported group size or path for this m";
    case QG_ERR_HIP: return "HIP launch error";
    case QG_ERR_SCRATCH: return "the problem needs more scratch than the static buffer holds";
    default: return "unknown status";
  }
}

int32_t qg_last_hip_error(void) { return g_last_hip_error; }

int32_t qg_set_split_order(int32_t order) {
  if (order != QG_SPLIT_ORDER_HW && order != QG_SPLIT_ORDER_ACQ_REL) return QG_ERR_UNSUPPORTED;
  g_split_order.store(order, std::memory_order_relaxed);
  return QG_OK;
}

int32_t qg_split_order(void) { return g_split_order.load(std::memory_order_relaxed); }

int32_t qgemm_int4(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                   const uint32_t* qzeros, void* y, int64_t ldy, int64_t m, int64_t n, int64_t k,
                   int32_t group_size, void* workspace, int64_t workspace_bytes, void* stream) {
  return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, QG_PATH_AUTO,
                  workspace, workspace_bytes, stream);
}

int32_t qgemm_int4_noalloc(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, void* y, int64_t ldy, int64_t m, int64_t n, int64_t k,
                           int32_t group_size, void* stream) {
  int32_t st = check_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size);
  if (st != QG_OK) return st;
  if (m == 0 || n == 0 || k == 0) return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size,
                                                  QG_PATH_AUTO, nullptr, 0, stream);
  const int64_t need = qg::workspace_int4(m, n, k, resolve_path(m, n, k, QG_PATH_AUTO));
  if (need > (int64_t)QG_NOALLOC_SCRATCH_BYTES) return QG_ERR_SCRATCH;
  void* ws = nullptr;
  st = noalloc_scratch((hipStream_t)stream, &ws);
  if (st != QG_OK) return st;
  return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, QG_PATH_AUTO, ws, need,
                  stream);
}

int32_t qgemm_int4_path(const void* x, int64_t ldx, const uint32_t* qweight,
                        const uint16_t* scales, const uint32_t* qzeros, void* y, int64_t ldy,
                        int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                        void* workspace, int64_t workspace_bytes, void* stream) {
  return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, path, workspace,
                  workspace_bytes, stream);
}

int32_t qgemm_int4_epilogue(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                            int64_t ldb_b, int32_t rank, float lora_scale, float* row_sumsq, void* y,
                            int64_t ldy, int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                            void* workspace, int64_t workspace_bytes, void* stream) {
  if (row_sumsq != nullptr && !aligned(row_sumsq, 4)) return QG_ERR_ALIGN;
  if (lora_a == nullptr) {
    const int32_t st = check_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size);
    if (st != QG_OK) return st;
    if (m == 0 || n == 0 || k == 0)   // k == 0: zeros, whose squares add nothing
      return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, path, workspace,
                      workspace_bytes, stream);
    return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, path, workspace,
                    workspace_bytes, stream, nullptr, nullptr, 0, row_sumsq);
  }
  return qgemm_int4_lora_rss(x, ldx, qweight, scales, qzeros, lora_a, lda_a, lora_b, ldb_b, rank, lora_scale,
                             row_sumsq, y, ldy, m, n, k, group_size, path, workspace, workspace_bytes, stream);
}

int32_t qgemm_int4_lora(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                        int64_t ldb_b, int32_t rank, float lora_scale, void* y, int64_t ldy, int64_t m,
                        int64_t n, int64_t k, int32_t group_size, int32_t path, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return qgemm_int4_lora_rss(x, ldx, qweight, scales, qzeros, lora_a, lda_a, lora_b, ldb_b, rank, lora_scale,
                             nullptr, y, ldy, m, n, k, group_size, path, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int32_t qgemm_int4_lora_rss(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                            int64_t ldb_b, int32_t rank, float lora_scale, float* row_sumsq, void* y,
                            int64_t ldy, int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                            void* workspace, int64_t workspace_bytes, void* stream) {
  if (rank < 1 || rank > 16) return QG_ERR_SHAPE;
  if (m > 0 && n > 0 && k > 0) {
    if (lora_a == nullptr || lora_b == nullptr) return QG_ERR_NULL;
    if (lda_a < k || lda_a > (int64_t)1 << 22 || ldb_b < rank) return QG_ERR_SHAPE;
    if (!aligned(lora_a, 16) || lda_a % 8 != 0 || !aligned(lora_b, 2)) return QG_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < lora_u_bytes(m, k)) return QG_ERR_SHAPE;
  }
  if (m > 0 && n > 0 && k == 0)      // U = 0: the plain product (zeros)
    return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, path, workspace,
                    workspace_bytes, stream);
  const qg::LoraEpi l{nullptr, (const uint16_t*)lora_b, ldb_b, rank, lora_scale, nullptr, 0, nullptr};
  return run_int4(x, ldx, qweight, scales, qzeros, y, ldy, m, n, k, group_size, path, workspace,
                  workspace_bytes, stream, &l, lora_a, lda_a, row_sumsq);
}

}  // namespace

extern "C" {

int64_t qgemm_int4_lora_workspace_size(int64_t m, int64_t n, int64_t k, int32_t path) {
  const int64_t base = qgemm_int4_workspace_size(m, n, k, path);
  if (base < 0) return base;
  return ((base + 255) & ~(int64_t)255) + lora_u_bytes(m, k);
}

int64_t qgemm_int4_workspace_size(int64_t m, int64_t n, int64_t k, int32_t path) {
  if (m < 0 || n < 0 || k < 0 || k % 128 != 0 || n % 8 != 0) return -QG_ERR_SHAPE;
  if (n > (int64_t)1 << 30 || k > (int64_t)1 << 30) return -QG_ERR_SHAPE;
  if (check_path(m, path) != QG_OK) return -QG_ERR_UNSUPPORTED;
  return qg::workspace_int4(m, n, k, resolve_path(m, n, k, path));
}

int32_t qgemm_int4_describe(int64_t m, int64_t n, int64_t k, int32_t path, int64_t workspace_bytes,
                            char* buf, int64_t len) {
  if (buf == nullptr || len <= 0) return QG_ERR_NULL;
  buf[0] = 0;
  if (m < 0 || n < 0 || k < 0 || k % 128 != 0 || n % 8 != 0) return QG_ERR_SHAPE;
  if (check_path(m, path) != QG_OK) return QG_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) {
    snprintf(buf, (size_t)len, "none");
    return QG_OK;
  }
  if (k == 0) {
    snprintf(buf, (size_t)len, "zero16_kernel");
    return QG_OK;
  }
  qg::describe_int4(m, n, k, resolve_path(m, n, k, path), workspace_bytes < 0 ? 0 : workspace_bytes, buf,
                    (size_t)len);
  return QG_OK;
}

int32_t qgemm_int4_dequant(const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, float* w, int64_t n, int64_t k,
                           int32_t group_size, void* stream) {
  if (n < 0 || k < 0) return QG_ERR_SHAPE;
  if (group_size != 128) return QG_ERR_UNSUPPORTED;
  if (k % 128 != 0 || n % 8 != 0) return QG_ERR_SHAPE;
  if (n == 0 || k == 0) return QG_OK;
  if (qweight == nullptr || scales == nullptr || w == nullptr) return QG_ERR_NULL;   // qzeros may be null
  if (!aligned(qweight, 16) || !aligned(scales, 8) || !aligned(qzeros, 4) || !aligned(w, 16))
    return QG_ERR_ALIGN;
  return hip_status(qg::launch_dequant(qweight, scales, qzeros, w, n, k, (hipStream_t)stream));
}

static int32_t run_dense(int32_t layout, int32_t dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, int64_t sa, const void* B, int64_t ldb, int64_t sb,
                         void* C, int64_t ldc, int64_t sc, void* stream, void* ws = nullptr,
                         int64_t ws_bytes = 0) {
  if (ws_bytes < 0) return QG_ERR_SHAPE;
  if (ws != nullptr && !aligned(ws, 16)) return QG_ERR_ALIGN;
  if (layout < QG_NT || layout > QG_TN) return QG_ERR_LAYOUT;
  if (dtype != QG_BF16 && dtype != QG_FP16 && dtype != QG_FP32) return QG_ERR_DTYPE;
  const uintptr_t esize = dtype == QG_FP32 ? 4 : 2;
  if (M < 0 || N < 0 || K < 0 || batch < 0 || batch > 65535) return QG_ERR_SHAPE;
  if (sa < 0 || sb < 0 || sc < 0) return QG_ERR_SHAPE;
  if (M == 0 || N == 0 || batch == 0) return QG_OK;
  if (C == nullptr) return QG_ERR_NULL;
  if (ldc < N) return QG_ERR_SHAPE;
  if (batch > 1 && sc < (M - 1) * ldc + N) return QG_ERR_SHAPE;     // outputs must not overlap
  if (!aligned(C, esize)) return QG_ERR_ALIGN;
  if (K > 0) {
    if (A == nullptr || B == nullptr) return QG_ERR_NULL;
    const int64_t a_row = layout == QG_TN ? M : K;
    const int64_t b_row = layout == QG_NT ? K : N;
    if (lda < a_row || ldb < b_row) return QG_ERR_SHAPE;
    if (!aligned(A, esize) || !aligned(B, esize)) return QG_ERR_ALIGN;
  }
  if (batch == 1) sa = sb = sc = 0;
  qg::DenseArgs a{layout, dtype, M, N, K, (const uint16_t*)A, lda, (const uint16_t*)B, ldb,
                  (uint16_t*)C, ldc, batch, sa, sb, sc};
  a.ws = ws;
  a.ws_bytes = ws ? ws_bytes : 0;
  a.split_acq_rel = g_split_order.load(std::memory_order_relaxed) == QG_SPLIT_ORDER_ACQ_REL;
  return hip_status(qg::launch_dense(a, (hipStream_t)stream));
}

int32_t gemm_dense(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
  return run_dense(layout, dtype, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, stream);
}

int32_t gemm_dense_ws(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                      int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  return run_dense(layout, dtype, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, stream, workspace,
                   workspace_bytes);
}

int64_t gemm_dense_workspace_size(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K) {
  if (layout < QG_NT || layout > QG_TN) return -(int64_t)QG_ERR_LAYOUT;
  if (dtype != QG_BF16 && dtype != QG_FP16 && dtype != QG_FP32) return -(int64_t)QG_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return -(int64_t)QG_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0 || dtype == QG_FP32) return 0;
  // the split needs the pipelined tiles, whose 16-byte loads need aligned
  // operands: the size assumes 16-byte aligned A and B with leading
  // dimensions equal to the contiguous extents
  qg::DenseArgs a{layout, dtype, M, N, K, (const uint16_t*)nullptr, 0, (const uint16_t*)nullptr, 0,
                  (uint16_t*)nullptr, N, 1, 0, 0, 0};
  a.lda = layout == QG_TN ? M : K;
  a.ldb = layout == QG_NT ? K : N;
  return qg::dense_workspace_bytes(a);
}

int32_t gemm_dense_batched(int32_t layout, int32_t dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                           int64_t stride_b, void* C, int64_t ldc, int64_t stride_c, void* stream) {
  return run_dense(layout, dtype, batch, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                   stream);
}

int32_t qg_probe_copy(const void* src, void* dst, int64_t bytes, int64_t blocks, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || blocks < 0 || blocks > 65536) return QG_ERR_SHAPE;
  if (bytes == 0) return QG_OK;
  if (!src || !dst) return QG_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_copy_probe(src, dst, bytes, blocks, (hipStream_t)stream));
}

int32_t qg_probe_read(const void* src, int64_t bytes, int64_t blocks, uint32_t key, uint32_t* sink,
                      void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || blocks < 0 || blocks > 65536) return QG_ERR_SHAPE;
  if (bytes == 0) return QG_OK;
  if (!src || !sink) return QG_ERR_NULL;
  if (!aligned(src, 16) || !aligned(sink, 4)) return QG_ERR_ALIGN;
  return hip_status(qg::launch_read_probe(src, bytes, blocks, key, sink, (hipStream_t)stream));
}

int32_t qg_probe_mfma_bf16(int64_t blocks, int32_t iters, uint64_t* clocks, void* stream) {
  if (!clocks) return QG_ERR_NULL;
  if (blocks < 1 || blocks > 65536 || iters < 1) return QG_ERR_SHAPE;
  if (((uintptr_t)clocks & 7u) != 0) return QG_ERR_ALIGN;
  return hip_status(qg::launch_mfma_probe(blocks, iters, clocks, (hipStream_t)stream));
}

}  // extern "C"
