/*
 * qgemm.h -- C ABI of the MI355X (gfx950) int4 GPTQ and dense GEMM library.
 *
 * The products are the linear-layer matmuls of the pages:
 *   - the GPTQ int4 weight-only linear layer (GPTQModel pull request #3645,
 *     "What changed": one fused kernel for m <= 15 tokens, the matrix-core
 *     kernel from m = 16; mi50grad README, "Project Structure" and "Model":
 *     an int4 GEMV with a DPP reduction, GPTQ-Int4 with group size 128);
 *   - the dense bf16/fp16 training products with fp32 accumulation (BC-250
 *     tuned-GEMM post, "Where the time went": forward, input-gradient and
 *     weight-gradient products, each a different memory layout).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no memory, keeps no state between calls and may be called from
 *     several host threads at once.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Matrices are row-major; a leading dimension (ld*) is the distance in
 *     elements between consecutive rows and must be >= the row length.
 *   - Every argument is validated on the host before anything is launched.  An
 *     invalid call returns a non-zero qg_status and enqueues nothing.  After a
 *     launch, a HIP launch error is reported as QG_ERR_HIP; the HIP error code is
 *     then available from qg_last_hip_error() on the calling thread.
 *   - Sizes of zero are valid: m == 0 or n == 0 enqueue nothing (pointers may be
 *     NULL); k == 0 writes zeros to the output.
 *   - No C++ exception crosses this boundary.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 1

/* Return codes (qg_status values, returned as int32_t). */
#define QG_OK 0
#define QG_ERR_NULL 1        /* a required pointer is NULL                         */
#define QG_ERR_SHAPE 2       /* bad size or ld (see each call), k % 128, n % 8    */
#define QG_ERR_ALIGN 3       /* a pointer or leading dimension is misaligned       */
#define QG_ERR_DTYPE 4       /* unknown dtype code                                 */
#define QG_ERR_LAYOUT 5      /* unknown layout code                                */
#define QG_ERR_UNSUPPORTED 6 /* group size != 128, or a forced path that cannot take m */
#define QG_ERR_HIP 7         /* the HIP runtime rejected a launch                  */
#define QG_ERR_SCRATCH 8     /* qgemm_int4_noalloc: the problem needs more scratch
                                than QG_NOALLOC_SCRATCH_BYTES                        */

/* dtype codes of gemm_dense */
#define QG_BF16 0
#define QG_FP16 1
#define QG_FP32 2

/* layout codes of gemm_dense (row-major definitions, see gemm_dense) */
#define QG_NT 0
#define QG_NN 1
#define QG_TN 2

/* path codes of qgemm_int4_path */
#define QG_PATH_AUTO 0  /* m == 1: GEMV; 2 <= m <= 16: fused small-M; 16 < m <= 32: fused small-M
                           with two row tiles when n < 20480, m <= 24 or its workgroups fit two
                           passes over the 256 CUs; 32 < m <= 64: fused
                           small-M with three or four row tiles when its workgroups fit one
                           pass over the 256 CUs (two passes at k > 8192 and m <= 48);
                           otherwise MFMA tiles */
#define QG_PATH_GEMV 1  /* m must be 1                                                   */
#define QG_PATH_FUSED 2 /* 1 <= m <= 16                                                   */
#define QG_PATH_MFMA 3  /* any m >= 1                                                    */

/* Version of this ABI (QG_ABI_VERSION of the built library). */
int32_t qg_abi_version(void);

/* Static, NUL-terminated description of a qg_status value. */
const char* qg_status_str(int32_t status);

/* HIP error code (hipError_t as int) of the last QG_ERR_HIP on this thread. */
int32_t qg_last_hip_error(void);

/*
 * Ordering of the k split's partial-sum exchange on the int4 paths.  When k is
 * split, every k slice of an output tile stores its fp32 partials, takes a
 * ticket from a counter in the workspace, and the slice that takes the last
 * ticket adds the partials in slice order (a deterministic result) and writes
 * Y; the sums are the same in both orders below, bit for bit.
 *
 *   QG_SPLIT_ORDER_HW (the default): partials are stored and read with
 *     agent-scope atomic accesses, every thread waits for the completion of
 *     its stores before its workgroup's ticket is taken, and the ticket
 *     increment is relaxed.  The order rests on the GPU's store-completion
 *     counter (an agent-scope store completes at the point where every CU
 *     sees it), not on the HIP memory model.
 *   QG_SPLIT_ORDER_ACQ_REL: the ticket increment is an agent-scope
 *     acquire-release read-modify-write, so the memory model itself orders
 *     the partials before their sum.  On gfx950 it costs an L2 write-back and
 *     invalidate per workgroup of a split launch: measured (cold weights)
 *     25600 x 5120 m = 16 26.2 -> 47.6 µs, 14336 x 4096 m = 8 11.8 -> 13.9 µs,
 *     25600 x 5120 m = 2048 (MFMA tiles) 695 -> 710 µs.
 *
 * Process-wide; applies to launches made after the call (calls that overlap
 * it on another thread may take either order).  qg_set_split_order returns
 * QG_OK, or QG_ERR_UNSUPPORTED (nothing changed) for another value;
 * qg_split_order returns the current order.
 */
#define QG_SPLIT_ORDER_HW 0
#define QG_SPLIT_ORDER_ACQ_REL 1
int32_t qg_set_split_order(int32_t order);
int32_t qg_split_order(void);

/*
 * qgemm_int4 -- Y = X . W^T with GPTQ int4 weights (GPTQModel #3645, "What
 * changed" and "Accuracy"; mi50grad README, "Model": group size 128).
 *
 *   Y[r][j] = bf16_rne( sum_i X[r][i] * W[i][j] ),  accumulated in fp32,
 *   W[i][j] = (q[i][j] - z[i/128][j]) * s[i/128][j]  (exact in fp32).
 *
 *   x        bf16 [m][ldx], k <= ldx <= 2^22, ldx % 8 == 0, 16-byte aligned.
 *   qweight  uint32 [k/8][n], 16-byte aligned.  Word (r, j) holds the 4-bit
 *            codes of rows 8r..8r+7 of output column j; row 8r+t is in bits
 *            4t..4t+3 (least significant nibble first).
 *   scales   fp16 bit patterns [k/128][n], 8-byte aligned.
 *   qzeros   uint32 [k/128][n/8], 4-byte aligned.  Word (g, c) holds the 4-bit
 *            zero points of columns 8c..8c+7; column 8c+t in bits 4t..4t+3.
 *            The stored nibble is z itself (no +1 offset).  NULL: weights
 *            without a zero point, W[i][j] = q[i][j] * s[i/128][j] (the AWQ
 *            GEMV variant of the mi50grad README, "Project Structure", which
 *            skips the zero-point subtraction); every path accepts it.
 *   y        bf16 [m][ldy] output, ldy >= n, ldy % 4 == 0, 8-byte aligned.
 *   m >= 0 tokens, 0 <= n <= 2^26 output columns (n % 8 == 0), 0 <= k <= 2^22
 *   input rows (k % 128 == 0), group_size must be 128.
 *   workspace, workspace_bytes
 *            optional device scratch (16-byte aligned).  The small-M paths
 *            use it to split k over several workgroups; the MFMA path (m > 16)
 *            to hold the activations in the decode's pair order and their
 *            per-group sums (a preparation pass before the tiles run).
 *            qgemm_int4_workspace_size gives the size that enables either.
 *            Its first 64 KiB hold the split's counters: they must be zero
 *            before the first use with this library, and each call leaves them
 *            zero again (the rest holds per-call data).  NULL or a smaller size
 *            is valid: the call then runs without the split / preparation
 *            (same accuracy contract; the summation order may differ).  Calls
 *            that share a workspace must not run concurrently.
 *
 * The path is chosen from m (see QG_PATH_AUTO).  x and y must not overlap the
 * weights or the workspace.  Errors: QG_ERR_NULL, QG_ERR_SHAPE, QG_ERR_ALIGN,
 * QG_ERR_UNSUPPORTED, QG_ERR_HIP.
 */
int32_t qgemm_int4(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                   const uint32_t* qzeros, void* y, int64_t ldy, int64_t m, int64_t n, int64_t k,
                   int32_t group_size, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qgemm_int4_lora -- qgemm_int4 with a LoRA adapter added in the product's
 * epilogue (the BC-250 post trains rank-16 LoRA adapters on every linear layer,
 * "Where the time went"; the mi50grad README, "Key Optimizations", fuses a
 * linear layer's epilogue into its kernel launch):
 *
 *   Y[r][j] = bf16_rne( sum_i X[r][i] W[i][j]  +  lora_scale * sum_t U[r][t] B[j][t] ),
 *   U[r][t] = sum_i X[r][i] A[t][i]   (fp32, not rounded to bf16).
 *
 *   lora_a   bf16 [rank][lda_a] (A, the adapter's down projection),
 *            k <= lda_a <= 2^22, lda_a % 8 == 0, 16-byte aligned.
 *   lora_b   bf16 [n][ldb_b] (B, the up projection), ldb_b >= rank, 2-byte aligned.
 *   rank     1..16.
 *   path     as qgemm_int4_path (QG_PATH_AUTO chooses from m).
 *   workspace, workspace_bytes
 *            required: its end holds U and the partial tiles of U's k
 *            slices (round_up(64 m, 256) + 1 KiB per 16 rows and slice; the
 *            minimum is qgemm_int4_lora_workspace_size with path data
 *            excluded); the front part, rounded down to 256 bytes, serves the
 *            path as in qgemm_int4 (same counter contract).
 *            qgemm_int4_lora_workspace_size gives the size that also enables
 *            the path's split / preparation.
 *
 * One launch where it pays: the LDS-staged small-M kernel (m <= 16, k up to
 * 64 groups, strips in one pass) and the MFMA tiles of products up to 2^34
 * flops accumulate U from the activations they already hold, in fp32, and add
 * the LoRA term to the product's fp32 accumulators in the same kernel (each k
 * slice adds its own share of U when k is split).  Otherwise (the
 * register-staged small-M kernel: long-k splits and 17..64 tokens; larger
 * MFMA products) U is computed first by two small kernels on the same stream
 * into the end of the workspace (k slices in parallel, then their sum in slice
 * order), and the product adds the term in its epilogue (once per output).
 * Other arguments, limits and errors as qgemm_int4 (plus QG_ERR_SHAPE for a
 * bad rank or a workspace without room for U).
 */
int32_t qgemm_int4_lora(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                        int64_t ldb_b, int32_t rank, float lora_scale, void* y, int64_t ldy, int64_t m,
                        int64_t n, int64_t k, int32_t group_size, int32_t path, void* workspace,
                        int64_t workspace_bytes, void* stream);

/*
 * qgemm_int4_epilogue -- qgemm_int4 with the fused epilogues of a linear layer
 * in the product's launch (mi50grad README, "Key Optimizations": the FFN
 * down-projection's GEMV, all-reduce and RMSNorm in one kernel, the RMSNorm's
 * sum of squares taken over the whole output row; BC-250 post, "Where the
 * time went": LoRA adapters on every linear layer):
 *
 *   - the LoRA add of qgemm_int4_lora when lora_a != NULL (same arguments,
 *     limits and workspace rule); lora_a == NULL: no adapter (lora_b, rank and
 *     lora_scale are ignored; the workspace is optional as in qgemm_int4);
 *   - the row reduction of an RMSNorm when row_sumsq != NULL: fp32 [m] device
 *     vector (4-byte aligned), to which the call adds, for every row r,
 *       row_sumsq[r] += sum_j float(Y[r][j])^2,
 *     the squares of the rounded bf16 outputs accumulated in fp32.  Zero it
 *     first for a fresh sum.  The partial sums of the column strips / tiles
 *     are added with fp32 atomics, so their order (and the last bits) can
 *     differ from call to call; Y itself is deterministic.
 *
 * Other arguments, limits and errors as qgemm_int4 / qgemm_int4_lora.
 */
int32_t qgemm_int4_epilogue(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const void* lora_a, int64_t lda_a, const void* lora_b,
                            int64_t ldb_b, int32_t rank, float lora_scale, float* row_sumsq, void* y,
                            int64_t ldy, int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes for qgemm_int4_lora (U plus what the path can use); < 0: -error. */
int64_t qgemm_int4_lora_workspace_size(int64_t m, int64_t n, int64_t k, int32_t path);

/*
 * qgemm_int4_noalloc -- qgemm_int4 for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and path choice as qgemm_int4
 * called with a workspace of qgemm_int4_workspace_size(m, n, k, QG_PATH_AUTO)
 * bytes, but the workspace is a static device buffer of the library
 * (QG_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends): the call
 * allocates and frees nothing.
 *
 * The first call on a device looks the buffer up and clears its split
 * counters with a small fill kernel on `stream`; every call leaves them zero
 * again.  All calls on one GPU share the buffer: calls that overlap on one
 * GPU (other streams or host threads) race and must be serialised by the
 * caller.  A problem whose workspace would exceed the buffer (for the MFMA
 * path, roughly m * k * 2 bytes of prepared activations: e.g. m = 2048,
 * k = 25600) returns QG_ERR_SCRATCH and launches nothing.  Other errors as
 * qgemm_int4.
 */
#define QG_NOALLOC_SCRATCH_BYTES 33554432 /* 32 MiB */
int32_t qgemm_int4_noalloc(const void* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, void* y, int64_t ldy, int64_t m, int64_t n, int64_t k,
                           int32_t group_size, void* stream);

/*
 * qgemm_int4_path -- qgemm_int4 with the kernel path forced (QG_PATH_* code),
 * for same-process A/B measurement and per-path testing.  A path that cannot
 * take m returns QG_ERR_UNSUPPORTED.  Same arguments and results otherwise.
 */
int32_t qgemm_int4_path(const void* x, int64_t ldx, const uint32_t* qweight,
                        const uint16_t* scales, const uint32_t* qzeros, void* y, int64_t ldy,
                        int64_t m, int64_t n, int64_t k, int32_t group_size, int32_t path,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qgemm_int4_workspace_size -- bytes of workspace with which qgemm_int4_path
 * (m, n, k, path) runs its preferred k split; 0 when it uses none.  Negative
 * sizes or n % 8, k % 128 != 0 return -QG_ERR_SHAPE; an invalid path returns
 * -QG_ERR_UNSUPPORTED.  Launches nothing.
 */
int64_t qgemm_int4_workspace_size(int64_t m, int64_t n, int64_t k, int32_t path);

/*
 * qgemm_int4_describe -- names the kernel and launch shape that qgemm_int4_path
 * would use for (m, n, k, path) with a workspace of workspace_bytes, e.g.
 * "skinny_int4_kernel<8,mfma,1> grid=512 block=256 lds=40960 ksplit=8 groups=4",
 * into buf (NUL-terminated, truncated to len bytes).  Launches nothing.
 * Errors: QG_ERR_NULL (buf), QG_ERR_SHAPE, QG_ERR_UNSUPPORTED.
 */
int32_t qgemm_int4_describe(int64_t m, int64_t n, int64_t k, int32_t path, int64_t workspace_bytes,
                            char* buf, int64_t len);

/*
 * qgemm_int4_dequant -- the dequantised weights themselves, for a bit-exact
 * check of the decode every int4 path shares (same storage as qgemm_int4).
 * GPTQModel #3645, "What changed" and "Accuracy": the codec decodes to exact
 * values that the matmul then accumulates in FP32; for GPTQ int4 with fp16
 * scales (mi50grad README, "Model": GPTQ-Int4, group size 128) the exact
 * decoded value is the fp32 product below (4-bit difference times an 11-bit
 * significand: at most 15 significant bits, so no rounding):
 *
 *   w[i][j] = (float)(q[i][j] - z[i/128][j]) * s[i/128][j],  fp32 [k][n], n-contiguous.
 *
 * qzeros NULL: z = 0, as in qgemm_int4.  w must be 16-byte aligned.  Errors as
 * qgemm_int4.
 */
int32_t qgemm_int4_dequant(const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, float* w, int64_t n, int64_t k,
                           int32_t group_size, void* stream);

/*
 * gemm_dense -- C = op(A) . op(B) in bf16 or fp16 with fp32 accumulation
 * (BC-250 tuned-GEMM post, "Where the time went" and "Tuning the kernels": the
 * three products of a linear layer, each a different memory layout, with FP32
 * accumulation).  Row-major definitions:
 *
 *   QG_NT  forward:          C[M][N] = A[M][K] . B[N][K]^T   (lda >= K, ldb >= K)
 *   QG_NN  input gradient:   C[M][N] = A[M][K] . B[K][N]     (lda >= K, ldb >= N)
 *   QG_TN  weight gradient:  C[M][N] = A[K][M]^T . B[K][N]   (lda >= M, ldb >= N)
 *
 * A, B and C share the dtype (QG_BF16 or QG_FP16); C is rounded to nearest even
 * from the fp32 accumulator, ldc >= N.  Pointers must be 2-byte aligned; any
 * sizes are accepted (1x1x1 included).  QG_FP32: A, B and C fp32 with fp32
 * products and accumulation (the post tunes and validates FP32 in all three
 * layouts as well), pointers 4-byte aligned; leading dimensions in elements.  Errors: QG_ERR_NULL, QG_ERR_SHAPE,
 * QG_ERR_ALIGN, QG_ERR_DTYPE, QG_ERR_LAYOUT, QG_ERR_HIP.
 */
int32_t gemm_dense(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/*
 * gemm_dense_ws -- gemm_dense with a workspace, which lets products with few
 * output tiles and a long K split K over several workgroups (bf16 / fp16, batch
 * 1, on the pipelined 128 x 128 or 256 x 128 tiles: at most 128 tiles, up to 4
 * k slices of at least 1024 k each, the tile whose tiles x slices covers more
 * of the 256 CUs; NT splits only the 128 x 128 tile).
 * Each slice stores its fp32 partial tile; the last slice of a tile to arrive
 * adds them in slice order (deterministic for a given size) and rounds once,
 * so the accuracy contract is that of gemm_dense (the summation order
 * differs).  The exchange is ordered as qg_set_split_order selects.
 *
 *   workspace, workspace_bytes
 *            optional device scratch (16-byte aligned); NULL or fewer bytes
 *            than gemm_dense_workspace_size asks for: no split.  As for
 *            qgemm_int4, its first 64 KiB hold the split's counters, which
 *            must be zero before the first use with this library and are
 *            zero again after each call (the same workspace may serve both
 *            entry points); calls that share a workspace must not overlap.
 *
 * Other arguments and errors as gemm_dense (plus QG_ERR_SHAPE for a negative
 * workspace_bytes and QG_ERR_ALIGN for a misaligned workspace).
 */
int32_t gemm_dense_ws(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                      int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* workspace,
                      int64_t workspace_bytes, void* stream);

/*
 * gemm_dense_workspace_size -- bytes of workspace with which gemm_dense_ws
 * splits K for this (layout, dtype, M, N, K), assuming 16-byte aligned
 * operands with leading dimensions equal to their contiguous extents; 0 when
 * it would not split (QG_FP32, short K, enough tiles).  A negative value is
 * -qg_status for invalid arguments.
 */
int64_t gemm_dense_workspace_size(int32_t layout, int32_t dtype, int64_t M, int64_t N, int64_t K);

/*
 * gemm_dense_batched -- `batch` independent gemm_dense products in one launch:
 * the attention layers' batched products, which the BC-250 tuned-GEMM post
 * tunes and validates ("Tuning the kernels", "Checking the results are right"):
 *
 *   C_b = op(A_b) . op(B_b),  A_b = A + b * stride_a, B_b = B + b * stride_b,
 *   C_b = C + b * stride_c  (strides in elements), b = 0 .. batch-1,
 *
 * each product as gemm_dense defines it (same layouts, dtypes, rounding and
 * leading dimensions).  0 <= batch <= 65535; strides >= 0 (an input stride of
 * 0 reuses one operand for every product); when batch > 1 the outputs must not
 * overlap: stride_c >= (M - 1) * ldc + N.  batch == 1 ignores the strides.
 * Errors as gemm_dense.
 */
int32_t gemm_dense_batched(int32_t layout, int32_t dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                           int64_t stride_b, void* C, int64_t ldc, int64_t stride_c, void* stream);

/*
 * Measurement probe (not a product): the sustained bf16 MFMA rate and the
 * shader clock under that load, the two denominators the BC-250 tuned-GEMM
 * post ("Checking the hardware first") establishes before tuning -- a
 * register-only matrix loop, and a cycle counter compared with a
 * constant-rate counter.
 *
 * Launches `blocks` workgroups of 4 waves; every wave runs `iters` rounds of 8
 * independent 16x16x32 bf16 MFMAs on register operands, i.e.
 *   flops = blocks * 4 * iters * 8 * 16384.
 * clocks: device buffer of blocks * 4 uint64_t (8-byte aligned), written as
 * {shader cycles at start, constant counter at start, shader cycles at end,
 * constant counter at end} per workgroup (s_memtime / s_memrealtime; the
 * constant counter runs at 100 MHz on this GPU family, so the clock in MHz is
 * 100 * cycles / constant ticks).
 * 1 <= blocks <= 65536, iters >= 1; errors: QG_ERR_NULL, QG_ERR_SHAPE,
 * QG_ERR_ALIGN, QG_ERR_HIP.
 */
int32_t qg_probe_mfma_bf16(int64_t blocks, int32_t iters, uint64_t* clocks, void* stream);

/*
 * Measurement probes (not products): the bandwidth denominators.  The BC-250
 * tuned-GEMM post ("Checking the hardware first") measures a large copy and a
 * multi-stream add before tuning; the int4 paths at m <= 16 are judged against
 * a measured copy of this kind, and against a read-only stream because they
 * mostly read.
 *
 * qg_probe_copy: dst[0 .. bytes) = src[0 .. bytes) with 16-byte lane loads and
 *   stores (device buffers, 16-byte aligned, must not overlap).
 * qg_probe_read: reads src[0 .. bytes) with 16-byte lane loads and folds it by
 *   XOR; the device word *sink (4-byte aligned) is written only when a
 *   thread's fold equals `key`, so the caller chooses a key and treats *sink
 *   as scratch.
 * bytes % 16 == 0, 0 <= bytes; blocks: workgroups of 256 threads, 1..65536,
 * or 0 for one loop trip of four 16-byte chunks per thread (at most 4096
 * workgroups; larger sizes loop over the grid).  Errors: QG_ERR_NULL,
 * QG_ERR_SHAPE, QG_ERR_ALIGN, QG_ERR_HIP.
 */
int32_t qg_probe_copy(const void* src, void* dst, int64_t bytes, int64_t blocks, void* stream);
int32_t qg_probe_read(const void* src, int64_t bytes, int64_t blocks, uint32_t key, uint32_t* sink,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
