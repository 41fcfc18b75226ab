// Host-side preparation of one SVDQuant layer (fp64, C++17, std::thread).
//
// Stage 2 of "Quantization Method -- SVDQuant" (svdq-int4-flux.1-depth-dev
// model card) moves activation outliers into the weight with a per-input-
// channel factor lambda; stage 3 splits the smoothed weight by SVD into a
// 16-bit rank-r branch L1 L2 and a residual R, which is quantized to 4 bits
// ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", "Background:
// SVDQuant and Nunchaku").  The pages name no SVD algorithm; this file uses a
// randomized block subspace iteration (Halko, Martinsson, Tropp 2011) with a
// one-sided Jacobi SVD (Hestenes) of the projected block.
//
// Layout: the smoothed weight is held as A = W_hat^T, i.e. [N][K] row-major
// like the input weight, A[n][k] = lambda_k * weight[n][k].

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "svdq.h"
#include "svdq_internal.h"

namespace {

// ------------------------------------------------------------------ rounding
// Round a finite double to a binary floating-point format with `frac` stored
// fraction bits, exponent bias `bias` and `ebits` exponent bits; round to
// nearest, ties to even; overflow gives infinity.  Returns the bit pattern.
uint32_t round_double_to_format(double v, int frac, int ebits) {
  const int bias = (1 << (ebits - 1)) - 1;
  const int emax = bias;           // largest unbiased exponent of a finite value
  const int emin = 1 - bias;       // smallest normal exponent
  uint64_t b;
  std::memcpy(&b, &v, 8);
  const uint32_t sign = static_cast<uint32_t>(b >> 63) << (frac + ebits);
  const uint32_t inf = ((1u << ebits) - 1) << frac;
  const int e = static_cast<int>((b >> 52) & 0x7FF);
  uint64_t m = b & ((1ull << 52) - 1);
  if (e == 0x7FF) return sign | inf | (m ? (1u << (frac - 1)) : 0u);
  if (e == 0 && m == 0) return sign;
  int exp;
  if (e == 0) {  // double subnormal: far below any target's range
    return sign;
  }
  exp = e - 1023;
  m |= (1ull << 52);  // 53-bit significand, value = m * 2^(exp-52)
  // number of low bits to drop so the kept integer counts units of the
  // target's ulp at this exponent (subnormal targets use the emin ulp)
  int unit_exp = (exp >= emin ? exp : emin) - frac;  // ulp exponent
  int shift = unit_exp - (exp - 52);
  uint64_t q;
  if (shift >= 64) {
    q = 0;  // far below half of the smallest subnormal
  } else {
    q = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
  }
  // q counts ulps of 2^unit_exp; renormalize into the format's fields
  if (exp < emin) {
    // subnormal target (q < 2^frac) or rounded up into the smallest normal
    return sign | static_cast<uint32_t>(q);  // q == 2^frac encodes emin exactly
  }
  if (q == (1ull << (frac + 1))) {  // rounding carried into the next binade
    q >>= 1;
    ++exp;
  }
  if (exp > emax) return sign | inf;
  return sign | (static_cast<uint32_t>(exp + bias) << frac) |
         static_cast<uint32_t>(q & ((1ull << frac) - 1));
}

inline uint16_t to_fp16(double v) { return static_cast<uint16_t>(round_double_to_format(v, 10, 5)); }
inline uint16_t to_bf16(double v) { return static_cast<uint16_t>(round_double_to_format(v, 7, 8)); }

inline double bf16_value(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline double fp16_value(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

// ------------------------------------------------------------------ threads
int worker_count() {
  unsigned hc = std::thread::hardware_concurrency();
  int n = hc ? static_cast<int>(hc) : 4;
  return std::max(1, std::min(n, 64));
}

template <class F>
void parallel_for(int64_t n, int64_t grain, F&& f) {
  const int nt = static_cast<int>(std::min<int64_t>(worker_count(), (n + grain - 1) / grain));
  if (nt <= 1) {
    f(0, n);
    return;
  }
  std::atomic<int64_t> next{0};
  auto body = [&]() {
    for (;;) {
      const int64_t b = next.fetch_add(grain);
      if (b >= n) break;
      f(b, std::min(n, b + grain));
    }
  };
  std::vector<std::thread> ts;
  ts.reserve(nt - 1);
  for (int i = 0; i < nt - 1; ++i) ts.emplace_back(body);
  body();
  for (auto& t : ts) t.join();
}

// ------------------------------------------------------------------ RNG
// Counter-based splitmix64 (Steele, Lea, Flood 2014) + Box-Muller.
inline uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

inline double gaussian(uint64_t seed, uint64_t idx) {
  const uint64_t a = splitmix64(seed ^ splitmix64(2 * idx));
  const uint64_t b = splitmix64(seed ^ splitmix64(2 * idx + 1));
  const double u1 = (static_cast<double>(a >> 11) + 1.0) * 0x1.0p-53;  // (0, 1]
  const double u2 = static_cast<double>(b >> 11) * 0x1.0p-53;
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}

// ------------------------------------------------------------------ dense kernels
// Y[n][c] = sum_k A[n][k] * Z[k][c];  A [N][K], Z [K][b], Y [N][b] (row-major)
void mul_A_Z(const std::vector<double>& A, int N, int K, const std::vector<double>& Z, int b,
             std::vector<double>& Y) {
  Y.assign(static_cast<size_t>(N) * b, 0.0);
  constexpr int RB = 8;
  parallel_for((N + RB - 1) / RB, 4, [&](int64_t lo, int64_t hi) {
    for (int64_t blk = lo; blk < hi; ++blk) {
      const int n0 = static_cast<int>(blk * RB), n1 = std::min(N, n0 + RB);
      for (int k = 0; k < K; ++k) {
        const double* z = &Z[static_cast<size_t>(k) * b];
        for (int n = n0; n < n1; ++n) {
          const double a = A[static_cast<size_t>(n) * K + k];
          double* y = &Y[static_cast<size_t>(n) * b];
          for (int c = 0; c < b; ++c) y[c] += a * z[c];
        }
      }
    }
  });
}

// Z[k][c] = sum_n A[n][k] * Q[n][c];  A [N][K], Q [N][b], Z [K][b]
void mul_At_Q(const std::vector<double>& A, int N, int K, const std::vector<double>& Q, int b,
              std::vector<double>& Z) {
  Z.assign(static_cast<size_t>(K) * b, 0.0);
  constexpr int KB = 64;
  parallel_for((K + KB - 1) / KB, 1, [&](int64_t lo, int64_t hi) {
    for (int64_t blk = lo; blk < hi; ++blk) {
      const int k0 = static_cast<int>(blk * KB), k1 = std::min(K, k0 + KB);
      for (int n = 0; n < N; ++n) {
        const double* q = &Q[static_cast<size_t>(n) * b];
        const double* a = &A[static_cast<size_t>(n) * K];
        for (int k = k0; k < k1; ++k) {
          const double av = a[k];
          double* z = &Z[static_cast<size_t>(k) * b];
          for (int c = 0; c < b; ++c) z[c] += av * q[c];
        }
      }
    }
  });
}

// Orthonormalize the b columns of Y [len][b] (row-major) in place by
// classical Gram-Schmidt applied twice.  A column that vanishes is replaced
// by a fresh random vector.  Returns false if that keeps failing.
bool orthonormalize(std::vector<double>& Y, int len, int b, uint64_t seed) {
  std::vector<double> col(static_cast<size_t>(b) * len);  // column-major copy
  for (int i = 0; i < len; ++i)
    for (int c = 0; c < b; ++c) col[static_cast<size_t>(c) * len + i] = Y[static_cast<size_t>(i) * b + c];
  std::vector<double> coef(b);
  for (int c = 0; c < b; ++c) {
    double* v = &col[static_cast<size_t>(c) * len];
    bool ok = false;
    for (int attempt = 0; attempt < 4 && !ok; ++attempt) {
      const double norm0 = std::sqrt(std::inner_product(v, v + len, v, 0.0));
      for (int pass = 0; pass < 2; ++pass) {
        for (int p = 0; p < c; ++p) {
          const double* u = &col[static_cast<size_t>(p) * len];
          coef[p] = std::inner_product(u, u + len, v, 0.0);
        }
        for (int p = 0; p < c; ++p) {
          const double* u = &col[static_cast<size_t>(p) * len];
          const double cp = coef[p];
          for (int i = 0; i < len; ++i) v[i] -= cp * u[i];
        }
      }
      const double nrm = std::sqrt(std::inner_product(v, v + len, v, 0.0));
      if (nrm > 1e-13 * norm0 && nrm > 1e-300) {
        for (int i = 0; i < len; ++i) v[i] /= nrm;
        ok = true;
      } else {
        for (int i = 0; i < len; ++i)
          v[i] = gaussian(seed ^ 0xA5A5A5A5ull, (static_cast<uint64_t>(c) << 40) + (attempt + 1) * 1000003ull + i);
      }
    }
    if (!ok) return false;
  }
  for (int i = 0; i < len; ++i)
    for (int c = 0; c < b; ++c) Y[static_cast<size_t>(i) * b + c] = col[static_cast<size_t>(c) * len + i];
  return true;
}

// One-sided Jacobi (Hestenes) on the b rows of B [b][K]: finds an orthogonal
// J [b][b] with the rows of B' = J^T B mutually orthogonal.  B is replaced by
// B' and J returned row-major (J[c][p]).  Returns false on non-convergence.
bool one_sided_jacobi(std::vector<double>& B, int b, int K, std::vector<double>& J) {
  J.assign(static_cast<size_t>(b) * b, 0.0);
  for (int i = 0; i < b; ++i) J[static_cast<size_t>(i) * b + i] = 1.0;
  std::vector<double> nrm(b);
  for (int sweep = 0; sweep < 80; ++sweep) {
    for (int p = 0; p < b; ++p) {
      const double* x = &B[static_cast<size_t>(p) * K];
      nrm[p] = std::inner_product(x, x + K, x, 0.0);
    }
    int rotations = 0;
    for (int p = 0; p < b - 1; ++p) {
      for (int q = p + 1; q < b; ++q) {
        double* x = &B[static_cast<size_t>(p) * K];
        double* y = &B[static_cast<size_t>(q) * K];
        const double alpha = nrm[p], beta = nrm[q];
        const double gamma = std::inner_product(x, x + K, y, 0.0);
        if (std::fabs(gamma) <= 1e-15 * std::sqrt(alpha * beta) || gamma == 0.0) continue;
        ++rotations;
        const double zeta = (beta - alpha) / (2.0 * gamma);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
        for (int i = 0; i < K; ++i) {
          const double xi = x[i], yi = y[i];
          x[i] = cs * xi - sn * yi;
          y[i] = sn * xi + cs * yi;
        }
        for (int i = 0; i < b; ++i) {
          double& jp = J[static_cast<size_t>(i) * b + p];
          double& jq = J[static_cast<size_t>(i) * b + q];
          const double a0 = jp, a1 = jq;
          jp = cs * a0 - sn * a1;
          jq = sn * a0 + cs * a1;
        }
        nrm[p] = std::inner_product(x, x + K, x, 0.0);
        nrm[q] = std::inner_product(y, y + K, y, 0.0);
      }
    }
    if (rotations == 0) return true;
  }
  return false;
}

bool all_finite_bf16(const uint16_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if ((p[i] & 0x7F80) == 0x7F80) return false;
  return true;
}

}  // namespace

namespace svdq {

int validate_shape(int K, int N, int rank, int group) {
  if (K <= 0 || N <= 0 || rank < 0 || group <= 0) return SVDQ_ERR_INVALID_ARG;
  if (rank > K || rank > N) return SVDQ_ERR_INVALID_ARG;
  if (group != SVDQ_GROUP) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (K % group != 0 || N % 8 != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK)
    return SVDQ_ERR_UNSUPPORTED_SHAPE;
  return SVDQ_OK;
}

int validate_shape_mx(int K, int N, int rank) {
  if (K <= 0 || N <= 0 || rank < 0) return SVDQ_ERR_INVALID_ARG;
  if (rank > K || rank > N) return SVDQ_ERR_INVALID_ARG;
  if (K % 128 != 0 || N % 8 != 0 || rank % 16 != 0 || rank > SVDQ_MAX_RANK) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  return SVDQ_OK;
}

}  // namespace svdq

extern "C" int svdq_prepared_bytes_mxfp4(int K, int N, int rank, size_t* bytes_out) {
  if (!bytes_out) return SVDQ_ERR_INVALID_ARG;
  const int st = svdq::validate_shape_mx(K, N, rank);
  if (st != SVDQ_OK) return st;
  const size_t k = static_cast<size_t>(K), n = static_cast<size_t>(N), r = static_cast<size_t>(rank);
  *bytes_out = n * k / 2 + (k / 32) * n + 2 * r * (k + n) + 4 * k;
  return SVDQ_OK;
}

extern "C" int svdq_prepared_bytes(int K, int N, int rank, int group, size_t* bytes_out) {
  if (!bytes_out) return SVDQ_ERR_INVALID_ARG;
  const int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  const size_t k = static_cast<size_t>(K), n = static_cast<size_t>(N), r = static_cast<size_t>(rank);
  *bytes_out = n * k / 2 + 2 * (k / group) * n + 2 * r * (k + n) + 4 * k;
  return SVDQ_OK;
}

namespace {

// Stages 2 and 3 shared by both encodings: smoothing factors, the low-rank
// split (or the given factors) and the fp64 residual A = W_hat - L1 L2,
// stored [N][K].  Inputs are checked for finiteness first.
int smooth_split_residual(const uint16_t* weight, int K, int N, const float* act_absmax, float alpha,
                          int rank, const uint16_t* lora_down_in, const uint16_t* lora_up_in,
                          int power_iters, uint64_t seed, float* smooth_inv, uint16_t* lora_down,
                          uint16_t* lora_up, double* sigma_out, std::vector<double>& A) {
  const size_t NK = static_cast<size_t>(N) * K;
  if (!all_finite_bf16(weight, NK)) return SVDQ_ERR_NUMERIC;
  for (int k = 0; k < K; ++k)
    if (!std::isfinite(act_absmax[k]) || act_absmax[k] < 0.0f) return SVDQ_ERR_NUMERIC;
  if (lora_down_in && (!all_finite_bf16(lora_down_in, static_cast<size_t>(rank) * K) ||
                       !all_finite_bf16(lora_up_in, static_cast<size_t>(rank) * N)))
    return SVDQ_ERR_NUMERIC;

  // ---- stage 2: smoothing factors
  std::vector<double> wmax(K, 0.0);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      wmax[k] = std::max(wmax[k], std::fabs(bf16_value(weight[static_cast<size_t>(n) * K + k])));
  std::vector<double> lam(K);
  const double eps = 1e-5;
  for (int k = 0; k < K; ++k) {
    const double a = std::max(static_cast<double>(act_absmax[k]), eps);
    const double w = std::max(wmax[k], eps);
    double l0;
    if (alpha == 0.5f) l0 = std::sqrt(a / w);
    else l0 = std::pow(a, static_cast<double>(alpha)) / std::pow(w, 1.0 - static_cast<double>(alpha));
    const float si = static_cast<float>(1.0 / l0);
    if (!(si > 0.0f) || !std::isfinite(si)) return SVDQ_ERR_NUMERIC;
    smooth_inv[k] = si;
    lam[k] = 1.0 / static_cast<double>(si);
  }
  A.assign(NK, 0.0);
  parallel_for(N, 64, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n)
      for (int k = 0; k < K; ++k)
        A[n * K + k] = lam[k] * bf16_value(weight[n * K + k]);
  });

  // ---- stage 3: low-rank split (bf16 factors)
  if (rank > 0) {
    if (lora_down_in) {
      std::memcpy(lora_down, lora_down_in, sizeof(uint16_t) * rank * K);
      std::memcpy(lora_up, lora_up_in, sizeof(uint16_t) * rank * N);
      if (sigma_out)
        for (int i = 0; i < rank; ++i) sigma_out[i] = NAN;
    } else {
      const int mn = std::min(K, N);
      const int b = std::min(mn, rank + std::max(16, rank / 2));
      const int iters = power_iters > 0 ? power_iters : 8;
      std::vector<double> Om(static_cast<size_t>(K) * b), Y, Z;
      for (size_t i = 0; i < Om.size(); ++i) Om[i] = gaussian(seed, i);
      mul_A_Z(A, N, K, Om, b, Y);  // Y = A Omega   [N][b]
      if (!orthonormalize(Y, N, b, seed + 1)) return SVDQ_ERR_NUMERIC;
      for (int it = 0; it < iters; ++it) {
        mul_At_Q(A, N, K, Y, b, Z);  // Z = A^T Q  [K][b]
        if (!orthonormalize(Z, K, b, seed + 2 + 2 * it)) return SVDQ_ERR_NUMERIC;
        mul_A_Z(A, N, K, Z, b, Y);
        if (!orthonormalize(Y, N, b, seed + 3 + 2 * it)) return SVDQ_ERR_NUMERIC;
      }
      mul_At_Q(A, N, K, Y, b, Z);  // Z = A^T Q = B^T  [K][b]
      std::vector<double> Bm(static_cast<size_t>(b) * K);  // B = Q^T A  [b][K]
      for (int k = 0; k < K; ++k)
        for (int c = 0; c < b; ++c) Bm[static_cast<size_t>(c) * K + k] = Z[static_cast<size_t>(k) * b + c];
      std::vector<double> J;
      if (!one_sided_jacobi(Bm, b, K, J)) return SVDQ_ERR_NUMERIC;
      std::vector<double> sig(b);
      for (int c = 0; c < b; ++c) {
        const double* x = &Bm[static_cast<size_t>(c) * K];
        sig[c] = std::sqrt(std::inner_product(x, x + K, x, 0.0));
      }
      std::vector<int> order(b);
      std::iota(order.begin(), order.end(), 0);
      std::stable_sort(order.begin(), order.end(), [&](int i, int j) { return sig[i] > sig[j]; });
      // L1 = U_r Sigma_r: the rotated rows of B;  L2^T = Q J (columns in order)
      for (int i = 0; i < rank; ++i) {
        const double* x = &Bm[static_cast<size_t>(order[i]) * K];
        for (int k = 0; k < K; ++k) lora_down[static_cast<size_t>(i) * K + k] = to_bf16(x[k]);
        if (sigma_out) sigma_out[i] = sig[order[i]];
      }
      parallel_for(N, 256, [&](int64_t lo, int64_t hi) {
        for (int64_t n = lo; n < hi; ++n)
          for (int i = 0; i < rank; ++i) {
            double s = 0.0;
            for (int c = 0; c < b; ++c) s += Y[n * b + c] * J[static_cast<size_t>(c) * b + order[i]];
            lora_up[n * rank + i] = to_bf16(s);
          }
      });
    }
    // ---- residual against the bf16 factors that run: R = W_hat - L1 L2
    std::vector<double> l1(static_cast<size_t>(K) * rank);  // [K][r]
    for (int i = 0; i < rank; ++i)
      for (int k = 0; k < K; ++k) l1[static_cast<size_t>(k) * rank + i] = bf16_value(lora_down[static_cast<size_t>(i) * K + k]);
    parallel_for(N, 16, [&](int64_t lo, int64_t hi) {
      std::vector<double> l2(rank);
      for (int64_t n = lo; n < hi; ++n) {
        for (int i = 0; i < rank; ++i) l2[i] = bf16_value(lora_up[n * rank + i]);
        for (int k = 0; k < K; ++k) {
          const double* a = &l1[static_cast<size_t>(k) * rank];
          double s = 0.0;
          for (int i = 0; i < rank; ++i) s += a[i] * l2[i];
          A[n * K + k] -= s;
        }
      }
    });
  }

  return SVDQ_OK;
}

}  // namespace

extern "C" int svdq_prepare_weights_ex(const uint16_t* weight, int K, int N, const float* act_absmax,
                                       float alpha, int rank, int group, const uint16_t* lora_down_in,
                                       const uint16_t* lora_up_in, int power_iters, uint64_t seed,
                                       float* smooth_inv, uint8_t* w_codes, uint16_t* w_scales,
                                       uint16_t* lora_down, uint16_t* lora_up, double* sigma_out) {
  int st = svdq::validate_shape(K, N, rank, group);
  if (st != SVDQ_OK) return st;
  if (!weight || !act_absmax || !smooth_inv || !w_codes || !w_scales) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if ((lora_down_in == nullptr) != (lora_up_in == nullptr)) return SVDQ_ERR_INVALID_ARG;
  if (!(alpha > 0.0f && alpha < 1.0f)) return SVDQ_ERR_INVALID_ARG;
  std::vector<double> A;
  st = smooth_split_residual(weight, K, N, act_absmax, alpha, rank, lora_down_in, lora_up_in, power_iters, seed,
                             smooth_inv, lora_down, lora_up, sigma_out, A);
  if (st != SVDQ_OK) return st;

  // ---- 4-bit residual: per (group, output channel) symmetric, fp16 scale
  const int G = K / group;
  std::atomic<int> bad{0};
  parallel_for(N, 16, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n) {
      const double* r = &A[n * K];
      uint8_t* dst = w_codes + n * (K / 2);
      for (int g = 0; g < G; ++g) {
        double amax = 0.0;
        for (int k = g * group; k < (g + 1) * group; ++k) amax = std::max(amax, std::fabs(r[k]));
        const uint16_t sh = to_fp16(amax / 7.0);
        const double s = fp16_value(sh);
        if (!std::isfinite(s)) {
          bad.store(1);
          return;
        }
        w_scales[static_cast<size_t>(g) * N + n] = sh;
        for (int k = g * group; k < (g + 1) * group; k += 2) {
          int q0 = 0, q1 = 0;
          if (s != 0.0) {
            q0 = static_cast<int>(std::max(-8.0, std::min(7.0, std::nearbyint(r[k] / s))));
            q1 = static_cast<int>(std::max(-8.0, std::min(7.0, std::nearbyint(r[k + 1] / s))));
          }
          dst[k / 2] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
        }
      }
    }
  });
  if (bad.load()) return SVDQ_ERR_NUMERIC;
  return SVDQ_OK;
}

extern "C" int svdq_prepare_weights(const uint16_t* weight, int K, int N, const float* act_absmax,
                                    float alpha, int rank, int group, float* smooth_inv,
                                    uint8_t* w_codes, uint16_t* w_scales, uint16_t* lora_down,
                                    uint16_t* lora_up) {
  return svdq_prepare_weights_ex(weight, K, N, act_absmax, alpha, rank, group, nullptr, nullptr, 0,
                                 0x5356445175616E74ull, smooth_inv, w_codes, w_scales, lora_down,
                                 lora_up, nullptr);
}

extern "C" int svdq_prepare_weights_mxfp4(const uint16_t* weight, int K, int N, const float* act_absmax,
                                          float alpha, int rank, const uint16_t* lora_down_in,
                                          const uint16_t* lora_up_in, int power_iters, uint64_t seed,
                                          float* smooth_inv, uint8_t* w_codes, uint8_t* w_scales,
                                          uint16_t* lora_down, uint16_t* lora_up, double* sigma_out) {
  int st = svdq::validate_shape_mx(K, N, rank);
  if (st != SVDQ_OK) return st;
  if (!weight || !act_absmax || !smooth_inv || !w_codes || !w_scales) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if ((lora_down_in == nullptr) != (lora_up_in == nullptr)) return SVDQ_ERR_INVALID_ARG;
  if (!(alpha > 0.0f && alpha < 1.0f)) return SVDQ_ERR_INVALID_ARG;
  std::vector<double> A;
  st = smooth_split_residual(weight, K, N, act_absmax, alpha, rank, lora_down_in, lora_up_in, power_iters, seed,
                             smooth_inv, lora_down, lora_up, sigma_out, A);
  if (st != SVDQ_OK) return st;

  // ---- MXFP4 residual: per (output channel, block of 32 along K), scale
  // 2^e with e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an
  // all-zero block), elements rounded to E2M1 with ties to even and
  // saturation at 6; a value rounding to zero is code 0.
  const int B = K / 32;
  parallel_for(N, 16, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n) {
      const double* r = &A[n * K];
      uint8_t* dst = w_codes + n * (K / 2);
      for (int b = 0; b < B; ++b) {
        double amax = 0.0;
        for (int k = b * 32; k < (b + 1) * 32; ++k) amax = std::max(amax, std::fabs(r[k]));
        int e = amax == 0.0 ? -127 : std::ilogb(amax) - 2;
        e = std::max(-127, std::min(127, e));
        w_scales[n * B + b] = static_cast<uint8_t>(e + 127);
        for (int k = b * 32; k < (b + 1) * 32; k += 2) {
          uint32_t c[2];
          for (int t = 0; t < 2; ++t) {
            const double v = std::ldexp(r[k + t], -e);
            const double a = std::fabs(v);
            uint32_t q = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
            if (v < 0.0 && q != 0) q |= 8u;
            c[t] = q;
          }
          dst[k / 2] = static_cast<uint8_t>(c[0] | (c[1] << 4));
        }
      }
    }
  });
  return SVDQ_OK;
}

// ---------------------------------------------------------------------------
// AWQ W4A16 preparation ("Bringing Nunchaku 4-bit Diffusion Inference to
// Diffusers", "Introducing Nunchaku Lite": 4-bit weights with 16-bit
// activations for the modulation projections; "Native loading in Diffusers":
// int4, group 64).  Activation-aware channel scale t_k = max(a_k, 1e-4)^alpha
// normalized by sqrt(max t * min t), a_k = mean |x_cal[:, k]|; alpha from a
// 20-point grid minimizing the calibration output error unless given;
// asymmetric unsigned INT4 per (output channel, group of 64) of W diag(t).
namespace {

struct AwqGroupQuant {
  uint16_t s_bits;
  double s;
  int z;
};

inline AwqGroupQuant awq_group(const double* w, int n) {
  double mx = w[0], mn = w[0];
  for (int i = 1; i < n; ++i) {
    mx = std::max(mx, w[i]);
    mn = std::min(mn, w[i]);
  }
  AwqGroupQuant g;
  g.s_bits = to_fp16(std::max(mx - mn, 1e-5) / 15.0);
  g.s = fp16_value(g.s_bits);
  g.z = static_cast<int>(std::max(0.0, std::min(15.0, std::nearbyint(-mn / g.s))));
  return g;
}

inline int awq_code(double w, const AwqGroupQuant& g) {
  return static_cast<int>(std::max(0.0, std::min(15.0, std::nearbyint(w / g.s) + g.z)));
}

// Channel scale for one alpha: stored inverse (fp32) and the fp64 scale the
// weight side uses, t = 1 / fp64(inv).
void awq_scales(const std::vector<double>& a, double alpha, std::vector<float>& inv, std::vector<double>& t) {
  const size_t K = a.size();
  std::vector<double> u(K);
  double mx = 0.0, mn = INFINITY;
  for (size_t k = 0; k < K; ++k) {
    u[k] = std::pow(std::max(a[k], 1e-4), alpha);
    mx = std::max(mx, u[k]);
    mn = std::min(mn, u[k]);
  }
  const double norm = std::sqrt(mx * mn);
  inv.resize(K);
  t.resize(K);
  for (size_t k = 0; k < K; ++k) {
    inv[k] = static_cast<float>(1.0 / (u[k] / norm));
    t[k] = 1.0 / static_cast<double>(inv[k]);
  }
}

}  // namespace

extern "C" int svdq_awq_prepare(const uint16_t* weight, int K, int N, const uint16_t* x_cal, int Mc, double alpha,
                                int group, float* inv_scale, uint8_t* w_codes, uint16_t* w_scales,
                                uint8_t* w_zeros, double* alpha_out) {
  if (K <= 0 || N <= 0 || Mc <= 0 || group <= 0) return SVDQ_ERR_INVALID_ARG;
  if (group != SVDQ_GROUP || K % group != 0 || N % 32 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
  if (!weight || !x_cal || !inv_scale || !w_codes || !w_scales || !w_zeros) return SVDQ_ERR_INVALID_ARG;
  if (!(alpha < 1.0) || std::isnan(alpha)) return SVDQ_ERR_INVALID_ARG;   // alpha < 0: search
  const size_t NK = static_cast<size_t>(N) * K;
  if (!all_finite_bf16(weight, NK) || !all_finite_bf16(x_cal, static_cast<size_t>(Mc) * K)) return SVDQ_ERR_NUMERIC;
  std::vector<double> W(NK), X(static_cast<size_t>(Mc) * K), a(K, 0.0);
  for (size_t i = 0; i < NK; ++i) W[i] = bf16_value(weight[i]);
  for (size_t i = 0; i < X.size(); ++i) X[i] = bf16_value(x_cal[i]);
  for (int m = 0; m < Mc; ++m)
    for (int k = 0; k < K; ++k) a[k] += std::fabs(X[static_cast<size_t>(m) * K + k]);
  for (int k = 0; k < K; ++k) a[k] /= Mc;
  const int G = K / group;

  double chosen = alpha;
  if (alpha < 0.0) {
    // reference outputs X W^T on the calibration rows
    std::vector<double> ref(static_cast<size_t>(Mc) * N);
    parallel_for(N, 64, [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n)
        for (int m = 0; m < Mc; ++m) {
          const double* x = &X[static_cast<size_t>(m) * K];
          const double* w = &W[n * K];
          double s = 0.0;
          for (int k = 0; k < K; ++k) s += x[k] * w[k];
          ref[static_cast<size_t>(m) * N + n] = s;
        }
    });
    double best = INFINITY;
    for (int gi = 0; gi < 20; ++gi) {
      const double al = gi / 20.0;
      std::vector<float> inv;
      std::vector<double> t;
      awq_scales(a, al, inv, t);
      std::vector<double> part(N, 0.0);
      parallel_for(N, 16, [&](int64_t lo, int64_t hi) {
        std::vector<double> wq(K), ws(group);
        for (int64_t n = lo; n < hi; ++n) {
          for (int g = 0; g < G; ++g) {
            for (int i = 0; i < group; ++i) ws[i] = W[n * K + g * group + i] * t[g * group + i];
            const AwqGroupQuant q = awq_group(ws.data(), group);
            for (int i = 0; i < group; ++i)
              wq[g * group + i] = (awq_code(ws[i], q) - q.z) * q.s * static_cast<double>(inv[g * group + i]);
          }
          double e = 0.0;
          for (int m = 0; m < Mc; ++m) {
            const double* x = &X[static_cast<size_t>(m) * K];
            double s = 0.0;
            for (int k = 0; k < K; ++k) s += x[k] * wq[k];
            const double d = ref[static_cast<size_t>(m) * N + n] - s;
            e += d * d;
          }
          part[n] = e;
        }
      });
      double loss = 0.0;
      for (int n = 0; n < N; ++n) loss += part[n];
      if (loss < best) {
        best = loss;
        chosen = al;
      }
    }
  }
  std::vector<float> inv;
  std::vector<double> t;
  awq_scales(a, chosen, inv, t);
  for (int k = 0; k < K; ++k) {
    if (!std::isfinite(inv[k]) || !(inv[k] > 0.0f)) return SVDQ_ERR_NUMERIC;
    inv_scale[k] = inv[k];
  }
  std::atomic<int> bad{0};
  parallel_for(N, 16, [&](int64_t lo, int64_t hi) {
    std::vector<double> ws(group);
    for (int64_t n = lo; n < hi; ++n)
      for (int g = 0; g < G; ++g) {
        for (int i = 0; i < group; ++i) ws[i] = W[n * K + g * group + i] * t[g * group + i];
        const AwqGroupQuant q = awq_group(ws.data(), group);
        if (!std::isfinite(q.s)) bad.store(1);
        w_scales[n * G + g] = q.s_bits;
        w_zeros[n * G + g] = static_cast<uint8_t>(q.z);
        uint8_t* dst = w_codes + n * (K / 2) + g * (group / 2);
        for (int i = 0; i < group; i += 2)
          dst[i / 2] = static_cast<uint8_t>(awq_code(ws[i], q) | (awq_code(ws[i + 1], q) << 4));
      }
  });
  if (bad.load()) return SVDQ_ERR_NUMERIC;
  if (alpha_out) *alpha_out = chosen;
  return SVDQ_OK;
}
