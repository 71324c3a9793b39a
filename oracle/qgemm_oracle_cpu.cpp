// Plain C++ CPU oracle for the int4 GPTQ linear layer and the dense products.
// TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
// benchmark's CPU-baseline leg load it; the GPU library never does, and the two
// share no code, header or table.
//
// What it computes (fp64 results, written out from the definitions):
//  * int4 GPTQ weights (GPTQModel pull request #3645, "What changed" and
//    "Accuracy"; the mi50grad README, "Model": GPTQ-Int4, group size 128).
//    Output column j, input row i, group g = floor(i / group):
//      q = floor(qweight[i/8][j] / 16^(i mod 8)) mod 16
//      z = floor(qzeros[g][j/8] / 16^(j mod 8)) mod 16    (z = 0 without qzeros:
//          the AWQ-style variant of the mi50grad README, "Project Structure")
//      s = the IEEE binary16 value of scales[g][j]
//      W32[i][j] = fp32((q - z) * s)   -- exact; checked against the fp64 product
//      Y[r][j]   = sum over i ascending of x[r][i] * W32[i][j], in fp64,
//    x the bfloat16 value of X[r][i].
//  * dense products C = op(A) op(B) of bf16 or fp16 operands (the BC-250 tuned
//    GEMM post, "Where the time went": forward, input-gradient and
//    weight-gradient products; "Checking the results are right": float64 CPU
//    reference), row-major:
//      NT: C[M][N] = A[M][K] . B[N][K]^T
//      NN: C[M][N] = A[M][K] . B[K][N]
//      TN: C[M][N] = A[K][M]^T . B[K][N]
//    summed over k ascending in fp64.
//
// Every decoding is written from the IEEE field definitions (sign, biased
// exponent, fraction, the subnormal branch), not by a hardware conversion.
// Work is split over output columns (int4) or rows (dense) on std::threads;
// each output is one thread's ascending sum, so the result does not depend on
// the thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <thread>
#include <vector>

namespace {

double decode_ieee(uint32_t bits, int exp_bits, int man_bits) {
  const uint32_t sign = (bits >> (exp_bits + man_bits)) & 1u;
  const uint32_t e = (bits >> man_bits) & ((1u << exp_bits) - 1u);
  const uint32_t f = bits & ((1u << man_bits) - 1u);
  const int bias = (1 << (exp_bits - 1)) - 1;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(f), 1 - bias - man_bits);  // subnormal: 0.f * 2^(1-bias)
  } else if (e == (1u << exp_bits) - 1u) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = std::ldexp(static_cast<double>(f + (1u << man_bits)), static_cast<int>(e) - bias - man_bits);
  }
  return sign ? -v : v;
}

double fp16_of(uint16_t b) { return decode_ieee(b, 5, 10); }
double bf16_of(uint16_t b) { return decode_ieee(b, 8, 7); }

// the 4-bit field t of a word, by division (not by shifting)
int64_t nibble(uint32_t word, int t) {
  uint64_t p = 1;
  for (int i = 0; i < t; ++i) p *= 16;
  return static_cast<int64_t>((static_cast<uint64_t>(word) / p) % 16);
}

struct Int4 {
  const uint32_t* qweight;  // [k/8][n]
  const uint16_t* scales;   // [k/group][n]
  const uint32_t* qzeros;   // [k/group][n/8] or null
  int64_t k, n, group;
};

// W32 of column j over all k rows; returns false when (q - z) * s is not exact in fp32
bool dequant_column(const Int4& w, int64_t j, float* col) {
  for (int64_t i = 0; i < w.k; ++i) {
    const int64_t g = i / w.group;
    const int64_t q = nibble(w.qweight[(i / 8) * w.n + j], static_cast<int>(i % 8));
    const int64_t z = w.qzeros ? nibble(w.qzeros[g * (w.n / 8) + j / 8], static_cast<int>(j % 8)) : 0;
    const double s = fp16_of(w.scales[g * w.n + j]);
    const double exact = static_cast<double>(q - z) * s;
    col[i] = static_cast<float>(exact);
    if (static_cast<double>(col[i]) != exact) return false;
  }
  return true;
}

int thread_count(int requested) {
  if (requested > 0) return requested;
  const unsigned h = std::thread::hardware_concurrency();
  return h ? static_cast<int>(h) : 1;
}

// run body(t) for t in [0, threads) and join
template <class F>
void parallel(int threads, F body) {
  std::vector<std::thread> pool;
  for (int t = 1; t < threads; ++t) pool.emplace_back(body, t);
  body(0);
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int oc_hardware_threads(void) { return thread_count(0); }

// bit patterns -> fp64 values; kind 0 = fp16, 1 = bf16
void oc_decode16(const uint16_t* bits, int64_t count, int32_t kind, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = kind ? bf16_of(bits[i]) : fp16_of(bits[i]);
}

// W32[k][n]; returns 0, 1 if some (q - z) * s was not exact in fp32, 2 on a bad shape
int32_t oc_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int64_t k,
                   int64_t n, int64_t group, float* w) {
  if (k < 0 || n < 0 || group <= 0 || k % group || k % 8 || n % 8) return 2;
  const Int4 p{qweight, scales, qzeros, k, n, group};
  std::vector<float> col(static_cast<size_t>(k));
  for (int64_t j = 0; j < n; ++j) {
    if (!dequant_column(p, j, col.data())) return 1;
    for (int64_t i = 0; i < k; ++i) w[i * n + j] = col[static_cast<size_t>(i)];
  }
  return 0;
}

// Y[nrows][ncols] for the listed rows of X (bf16 [.][ldx]) and columns of W;
// rows/cols null means all m rows / all n columns.  Returns as oc_dequant.
int32_t oc_qgemm_int4_at(const uint16_t* x, int64_t ldx, const uint32_t* qweight, const uint16_t* scales,
                         const uint32_t* qzeros, int64_t m, int64_t k, int64_t n, int64_t group,
                         const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols, double* y,
                         int32_t threads) {
  if (k < 0 || n < 0 || m < 0 || group <= 0 || k % group || k % 8 || n % 8 || ldx < k) return 2;
  if (!rows) nrows = m;
  if (!cols) ncols = n;
  const Int4 p{qweight, scales, qzeros, k, n, group};
  // activations decoded once, fp64 [nrows][k]
  std::vector<double> xv(static_cast<size_t>(nrows * k));
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t src = rows ? rows[r] : r;
    for (int64_t i = 0; i < k; ++i) xv[static_cast<size_t>(r * k + i)] = bf16_of(x[src * ldx + i]);
  }
  const int T = static_cast<int>(std::min<int64_t>(thread_count(threads), ncols > 0 ? ncols : 1));
  std::vector<int> bad(static_cast<size_t>(T), 0);
  parallel(T, [&](int t) {
    std::vector<float> col(static_cast<size_t>(k));
    for (int64_t c = t; c < ncols; c += T) {
      const int64_t j = cols ? cols[c] : c;
      if (!dequant_column(p, j, col.data())) { bad[static_cast<size_t>(t)] = 1; return; }
      for (int64_t r = 0; r < nrows; ++r) {
        const double* xr = xv.data() + r * k;
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) acc += xr[i] * static_cast<double>(col[static_cast<size_t>(i)]);
        y[r * ncols + c] = acc;
      }
    }
  });
  for (int b : bad) if (b) return 1;
  return 0;
}

// C[M][N] (fp64) = op(A) op(B); layout 0 = NT, 1 = NN, 2 = TN; kind 0 = fp16, 1 = bf16.
// Operands are dense row-major: NT A[M][K] B[N][K]; NN A[M][K] B[K][N]; TN A[K][M] B[K][N].
int32_t oc_dense(int32_t layout, int32_t kind, int64_t M, int64_t N, int64_t K, const uint16_t* a,
                 const uint16_t* b, double* c, int32_t threads) {
  if (M < 0 || N < 0 || K < 0 || layout < 0 || layout > 2) return 2;
  auto val = [kind](uint16_t v) { return kind ? bf16_of(v) : fp16_of(v); };
  auto A = [&](int64_t r, int64_t kk) { return val(layout == 2 ? a[kk * M + r] : a[r * K + kk]); };
  auto B = [&](int64_t kk, int64_t j) { return val(layout == 0 ? b[j * K + kk] : b[kk * N + j]); };
  const int T = static_cast<int>(std::min<int64_t>(thread_count(threads), M > 0 ? M : 1));
  parallel(T, [&](int t) {
    for (int64_t r = t; r < M; r += T)
      for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) acc += A(r, kk) * B(kk, j);
        c[r * N + j] = acc;
      }
  });
  return 0;
}

}  // extern "C"
