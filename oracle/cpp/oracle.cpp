// Plain C++17 CPU oracle, float64 throughout, OpenMP over output rows.
// TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
// benchmark's CPU-baseline leg load it; the product path never does. It
// shares no code, header or constant with the HIP library (it includes only
// the C++ standard library) and none with the numpy oracle beside it, which
// it is checked against.
//
// What it computes (the same definitions as the numpy oracle, written again):
//  * "Pytorch Op for blackwell distributed gemm", Usage and Note on Tensor
//    Layouts: D = alpha * (A @ B^T) + beta * C, A (M, K), B (N, K) row-major
//    (or B given (K, N), i.e. B^T itself), C and D (M, N); beta == 0 means C
//    is not read. Element types bf16 (the top half of a binary32) and OCP
//    E4M3FN ("float_e4m3", Limitations).
//  * "Distributed GEMM", Background (Figures 3-4) and Approach: the
//    all-gather form (AllGather1D_TilingCD_RotatingA: stage t multiplies
//    slice (rank + t) mod P into rows of that slice), the reduce-scatter
//    form (ReduceScatter1D_TilingA_RotatingC: stage t computes row block
//    (rank + 1 + t) mod P, the own block last, which adds the incoming
//    partials) and their column duals (RotatingB, TilingB).
//  * p04 problem statement, "Computation and communication example" and
//    "Interface, layout, and parameters": the per-token-slot FFN
//    z = x w1[l] + b1[l], h = LN_x(u) * silu(LN_gate(g)), y = h wout[l] +
//    bout[l] (LayerNorm with the population variance, eps added), and the
//    All-to-All dispatch / combine as layout maps.
//  * "Add dist GEMM attention and FFN backend", Structure: the SwiGLU hidden
//    silu(x w1) * (x w3) of the gathered rows, w1 | w3 side by side.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

enum { kBf16 = 0, kE4m3 = 1 };
enum { kNK = 0, kKN = 1 };

double bf16_value(uint16_t bits) {
  const uint32_t w = uint32_t(bits) << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return double(f);
}

// OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities.
double e4m3_value(uint8_t bits) {
  if ((bits & 0x7F) == 0x7F) return std::numeric_limits<double>::quiet_NaN();
  const double sign = (bits & 0x80) ? -1.0 : 1.0;
  const int e = (bits >> 3) & 0xF;
  const int m = bits & 0x7;
  const double mag = e == 0 ? (m / 8.0) * std::ldexp(1.0, -6) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return sign * mag;
}

double value(const void* base, int dtype, int64_t i) {
  return dtype == kE4m3 ? e4m3_value(static_cast<const uint8_t*>(base)[i])
                        : bf16_value(static_cast<const uint16_t*>(base)[i]);
}

// rows x cols of a row-major operand, decoded
std::vector<double> decoded(const void* base, int dtype, int64_t rows, int64_t cols) {
  std::vector<double> out(size_t(rows * cols));
  for (int64_t i = 0; i < rows * cols; ++i) out[size_t(i)] = value(base, dtype, i);
  return out;
}

// B as an (N, K) matrix from either layout
std::vector<double> b_as_nk(const void* b, int dtype, int layout, int64_t N, int64_t K) {
  std::vector<double> out(size_t(N * K));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      out[size_t(n * K + k)] = layout == kNK ? value(b, dtype, n * K + k) : value(b, dtype, k * N + n);
  return out;
}

double dot(const double* x, const double* y, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k) s += x[k] * y[k];
  return s;
}

double silu(double t) { return t / (1.0 + std::exp(-t)); }

// LayerNorm of v[0..n) into out: (v - mean) / sqrt(var + eps) * gamma + beta
void layer_norm(const double* v, int64_t n, const double* gamma, const double* beta, double eps, double* out) {
  double mean = 0.0;
  for (int64_t i = 0; i < n; ++i) mean += v[i];
  mean /= double(n);
  double var = 0.0;
  for (int64_t i = 0; i < n; ++i) var += (v[i] - mean) * (v[i] - mean);
  var /= double(n);
  const double inv = 1.0 / std::sqrt(var + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = (v[i] - mean) * inv * gamma[i] + beta[i];
}

}  // namespace

extern "C" {

// out[0..n) = the values of n stored elements of type dtype (0 bf16, 1 e4m3).
void orc_decode(const void* bits, int dtype, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = value(bits, dtype, i);
}

// All-gather form: D (P*m, n_out) from P slices of (m, K); with swiglu the
// product has N = 2 n_out columns [u | v] and D = silu(u) * v + beta * C.
void orc_gemm_ag(const void* const* a_slices, int P, int rank, int64_t m, int64_t N, int64_t K, int dtype,
                 int b_layout, const void* b, const uint16_t* c, double alpha, double beta, int swiglu,
                 double* d) {
  const std::vector<double> B = b_as_nk(b, dtype, b_layout, N, K);
  const int64_t n_out = swiglu ? N / 2 : N;
  for (int t = 0; t < P; ++t) {
    const int s = (rank + t) % P;           // stage t: slice (rank + t) mod P
    const std::vector<double> A = decoded(a_slices[s], dtype, m, K);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
      const int64_t row = int64_t(s) * m + i;
      for (int64_t j = 0; j < n_out; ++j) {
        double out;
        if (swiglu) {
          const double u = alpha * dot(&A[size_t(i * K)], &B[size_t(j * K)], K);
          const double v = alpha * dot(&A[size_t(i * K)], &B[size_t((n_out + j) * K)], K);
          out = silu(u) * v;
        } else {
          out = alpha * dot(&A[size_t(i * K)], &B[size_t(j * K)], K);
        }
        if (beta != 0.0) out += beta * bf16_value(c[row * n_out + j]);
        d[row * n_out + j] = out;
      }
    }
  }
}

// Reduce-scatter form: out (M, N) = alpha * A B^T block by block, own block
// last, plus incoming[j] (m, N) for j != rank (NULL entries add nothing).
void orc_gemm_rs(const uint16_t* a, int64_t M, int64_t N, int64_t K, int P, int rank, int b_layout,
                 const uint16_t* b, const uint16_t* const* incoming, double alpha, double* out) {
  const std::vector<double> B = b_as_nk(b, kBf16, b_layout, N, K);
  const std::vector<double> A = decoded(a, kBf16, M, K);
  const int64_t m = M / P;
  for (int t = 0; t < P; ++t) {
    const int blk = (rank + 1 + t) % P;     // stage t: block (rank + 1 + t) mod P
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
      const int64_t row = int64_t(blk) * m + i;
      for (int64_t j = 0; j < N; ++j) {
        double v = alpha * dot(&A[size_t(row * K)], &B[size_t(j * K)], K);
        if (blk == rank && incoming)
          for (int q = 0; q < P; ++q)
            if (q != rank && incoming[q]) v += bf16_value(incoming[q][i * N + j]);
        out[row * N + j] = v;
      }
    }
  }
}

// All-gather with rotating B: A (M, K) local, B in P slices of n rows ((n, K),
// or (K, n) column blocks in the (K, N) layout); stage t writes columns of
// slice (rank + t) mod P.
void orc_gemm_ag_rotb(const void* a, const void* const* b_slices, int P, int rank, int64_t M, int64_t n,
                      int64_t K, int dtype, int b_layout, const uint16_t* c, double alpha, double beta,
                      double* d) {
  const std::vector<double> A = decoded(a, dtype, M, K);
  const int64_t N = int64_t(P) * n;
  for (int t = 0; t < P; ++t) {
    const int s = (rank + t) % P;
    const std::vector<double> Bs = b_as_nk(b_slices[s], dtype, b_layout, n, K);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
      for (int64_t j = 0; j < n; ++j) {
        const int64_t col = int64_t(s) * n + j;
        double v = alpha * dot(&A[size_t(i * K)], &Bs[size_t(j * K)], K);
        if (beta != 0.0) v += beta * bf16_value(c[i * N + col]);
        d[i * N + col] = v;
      }
  }
}

// Reduce-scatter with tiled B: column blocks of n = N/P, own block last,
// which adds incoming[j] (M, n) for j != rank.
void orc_gemm_rs_tileb(const uint16_t* a, int64_t M, int64_t N, int64_t K, int P, int rank, int b_layout,
                       const uint16_t* b, const uint16_t* const* incoming, double alpha, double* out) {
  const std::vector<double> B = b_as_nk(b, kBf16, b_layout, N, K);
  const std::vector<double> A = decoded(a, kBf16, M, K);
  const int64_t n = N / P;
  for (int t = 0; t < P; ++t) {
    const int blk = (rank + 1 + t) % P;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
      for (int64_t j = 0; j < n; ++j) {
        const int64_t col = int64_t(blk) * n + j;
        double v = alpha * dot(&A[size_t(i * K)], &B[size_t(col * K)], K);
        if (blk == rank && incoming)
          for (int q = 0; q < P; ++q)
            if (q != rank && incoming[q]) v += bf16_value(incoming[q][i * n + j]);
        out[i * N + col] = v;
      }
  }
}

// Per-slot FFN forward: y [PB, L, D] from x [PB, L, D], w1 [L, D, 2H],
// b1 [L, 2H], wout [L, H, D], bout [L, D] and the four [H] norm vectors.
void orc_ffn_slot_forward(const uint16_t* x, int64_t PB, int64_t L, int64_t D, int64_t H, const uint16_t* w1,
                          const uint16_t* b1, const uint16_t* wout, const uint16_t* bout, const uint16_t* gx,
                          const uint16_t* bx, const uint16_t* gg, const uint16_t* bg, double eps, double* y) {
  const std::vector<double> GX = decoded(gx, kBf16, 1, H), BX = decoded(bx, kBf16, 1, H);
  const std::vector<double> GG = decoded(gg, kBf16, 1, H), BG = decoded(bg, kBf16, 1, H);
  for (int64_t l = 0; l < L; ++l) {
    // w1[l] as (2H, D) and wout[l] as (D, H): rows of the contraction
    const std::vector<double> W1 = b_as_nk(w1 + l * D * 2 * H, kBf16, kKN, 2 * H, D);
    const std::vector<double> WO = b_as_nk(wout + l * H * D, kBf16, kKN, D, H);
    const std::vector<double> B1 = decoded(b1 + l * 2 * H, kBf16, 1, 2 * H);
    const std::vector<double> BO = decoded(bout + l * D, kBf16, 1, D);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < PB; ++r) {
      std::vector<double> xr(static_cast<size_t>(D)), z(static_cast<size_t>(2 * H)), a(static_cast<size_t>(H)),
          g(static_cast<size_t>(H)), h(static_cast<size_t>(H));
      for (int64_t k = 0; k < D; ++k) xr[size_t(k)] = bf16_value(x[(r * L + l) * D + k]);
      for (int64_t j = 0; j < 2 * H; ++j) z[size_t(j)] = dot(xr.data(), &W1[size_t(j * D)], D) + B1[size_t(j)];
      layer_norm(z.data(), H, GX.data(), BX.data(), eps, a.data());        // LN_x(u), u = z[:H]
      layer_norm(z.data() + H, H, GG.data(), BG.data(), eps, g.data());    // LN_gate(g), g = z[H:]
      for (int64_t j = 0; j < H; ++j) h[size_t(j)] = a[size_t(j)] * silu(g[size_t(j)]);
      for (int64_t j = 0; j < D; ++j) y[(r * L + l) * D + j] = dot(h.data(), &WO[size_t(j * H)], H) + BO[size_t(j)];
    }
  }
}

// SwiGLU hidden of the gathered rows: h (P*S, F) = silu(x w1) * (x w3), x
// the P shards (S, D) in rank order, w13 (D, 2F) = [w1 | w3].
void orc_swiglu_hidden(const uint16_t* const* x_shards, int P, int64_t S, int64_t D, int64_t F,
                       const uint16_t* w13, double* h) {
  const std::vector<double> W = b_as_nk(w13, kBf16, kKN, 2 * F, D);
  for (int s = 0; s < P; ++s) {
    const std::vector<double> X = decoded(x_shards[s], kBf16, S, D);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < S; ++i)
      for (int64_t j = 0; j < F; ++j) {
        const double u = dot(&X[size_t(i * D)], &W[size_t(j * D)], D);
        const double v = dot(&X[size_t(i * D)], &W[size_t((F + j) * D)], D);
        h[(int64_t(s) * S + i) * F + j] = silu(u) * v;
      }
  }
}

// dispatch = A2A(split 1, concat 0): out[s*B + b, l, :] = in_s[b, rank*L + l, :]
void orc_dispatch(const void* const* inputs, int P, int rank, int64_t B, int64_t T, int64_t D, int elem_bytes,
                  void* out) {
  const int64_t L = T / P, row = D * elem_bytes;
  for (int s = 0; s < P; ++s)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t l = 0; l < L; ++l)
        std::memcpy(static_cast<char*>(out) + ((int64_t(s) * B + b) * L + l) * row,
                    static_cast<const char*>(inputs[s]) + (b * T + int64_t(rank) * L + l) * row, size_t(row));
}

// combine = A2A(split 0, concat 1): out[b, s*L + l, :] = Y_s[rank*B + b, l, :]
void orc_combine(const void* const* ys, int P, int rank, int64_t B, int64_t L, int64_t D, int elem_bytes,
                 void* out) {
  const int64_t row = D * elem_bytes;
  for (int s = 0; s < P; ++s)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t l = 0; l < L; ++l)
        std::memcpy(static_cast<char*>(out) + (b * P * L + int64_t(s) * L + l) * row,
                    static_cast<const char*>(ys[s]) + ((int64_t(rank) * B + b) * L + l) * row, size_t(row));
}

}  // extern "C"
