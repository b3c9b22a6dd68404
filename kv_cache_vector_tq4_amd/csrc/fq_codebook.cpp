// Host-side builder of a layer's quantizer: Lloyd-Max codebook, rotation,
// QJL matrix. "FlashQuant" page, "TurboQuant" steps 2-3 (Haar rotation,
// Gaussian Lloyd-Max with closed-form centroids) and "QJL" (Gaussian
// projection S); "TurboQuant" blog, "Couche 1" (randomized Walsh-Hadamard).
// Everything is computed in double and rounded once to fp32 on output.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "fq.h"
#include "fq_internal.h"

namespace {

// SplitMix64 (Steele, Lea & Flood 2014), addressed by counter: output i of
// the stream started at `seed`.
inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline double uniform_at(uint64_t seed, uint64_t i) {
  return (static_cast<double>(splitmix64_at(seed, i) >> 11) + 0.5) * 0x1.0p-53;
}

// n standard normals by Box-Muller; pair p uses uniforms 2p and 2p+1.
void gaussians(uint64_t seed, size_t n, double* out) {
  const double two_pi = 6.283185307179586476925286766559;
  for (size_t p = 0; 2 * p < n; ++p) {
    double u1 = uniform_at(seed, 2 * p), u2 = uniform_at(seed, 2 * p + 1);
    double r = std::sqrt(-2.0 * std::log(u1));
    out[2 * p] = r * std::cos(two_pi * u2);
    if (2 * p + 1 < n) out[2 * p + 1] = r * std::sin(two_pi * u2);
  }
}

double npdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.39894228040143267794; }

// P(a < Z <= b), evaluated on the side of zero where it does not cancel.
double nmass(double a, double b) {
  const double r2 = 0.70710678118654752440;
  if (a >= 0) return 0.5 * std::erfc(a * r2) - 0.5 * std::erfc(b * r2);
  return 0.5 * std::erfc(-b * r2) - 0.5 * std::erfc(-a * r2);
}

// Phi^{-1}(p) by bisection on the CDF (only the starting point of Lloyd).
double nquantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    double cdf = 0.5 * std::erfc(-mid * 0.70710678118654752440);
    if (cdf < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

void lloyd_max(int bits, std::vector<double>& lev, std::vector<double>& bnd) {
  const int L = 1 << bits;
  lev.resize(L);
  bnd.resize(L - 1);
  for (int i = 0; i < L; ++i) lev[i] = nquantile((i + 0.5) / L);
  std::vector<double> nl(L);
  for (int it = 0; it < 200000; ++it) {
    for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
    double delta = 0;
    for (int i = 0; i < L; ++i) {
      double a = i == 0 ? -INFINITY : bnd[i - 1];
      double b = i == L - 1 ? INFINITY : bnd[i];
      nl[i] = (npdf(a) - npdf(b)) / nmass(a, b);
      delta = std::fmax(delta, std::fabs(nl[i] - lev[i]));
    }
    lev = nl;
    if (delta < 1e-15) break;
  }
  std::vector<double> sym(L);
  for (int i = 0; i < L; ++i) sym[i] = 0.5 * (lev[i] - lev[L - 1 - i]);
  lev = sym;
  for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
}

// ---- spherical marginal ("TurboQuant" blog, "Étape 2" / "Couche 2") ----
// A coordinate of a uniform point on the unit sphere in R^d has density
// proportional to w(x) = (1 - x^2)^(p - 1) on (-1, 1), p = (d - 1) / 2. On a cell
// (a, b] the first moment has the closed form ((1 - a^2)^p - (1 - b^2)^p) / (2p)
// (same unnormalized scale as w); the mass is integrated numerically with
// composite Gauss-Legendre (GL_N nodes on GL_PANELS equal panels).
constexpr int GL_N = 20, GL_PANELS = 16;

// Nodes / weights of the GL_N-point Gauss-Legendre rule on [-1, 1]: roots of P_n by
// Newton's method from the Chebyshev-like guesses cos(pi (i + 3/4) / (n + 1/2)),
// P_n and P_n' from the three-term recurrence; w_i = 2 / ((1 - x_i^2) P_n'(x_i)^2).
void gauss_legendre(double* x, double* w) {
  const int n = GL_N;
  for (int i = 0; i < n; ++i) {
    double z = std::cos(3.14159265358979323846 * (i + 0.75) / (n + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double pk = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = pk;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-17) break;
    }
    x[i] = z;
    w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

double sphere_weight_mass(double a, double b, double p, const double* gx, const double* gw) {
  double sum = 0;
  const double h = (b - a) / GL_PANELS;
  for (int j = 0; j < GL_PANELS; ++j) {
    const double c = a + (j + 0.5) * h, r = 0.5 * h;
    for (int i = 0; i < GL_N; ++i) {
      const double x = c + r * gx[i];
      const double u = 1.0 - x * x;
      if (u > 0) sum += gw[i] * r * std::exp((p - 1.0) * std::log(u));
    }
  }
  return sum;
}

double sphere_m1(double a, double b, double p) {
  auto t = [&](double x) {
    const double u = 1.0 - x * x;
    return u > 0 ? std::exp(p * std::log(u)) : 0.0;
  };
  return (t(a) - t(b)) / (2.0 * p);
}

// Lloyd fixed point for the spherical marginal in R^d: starts from the Gaussian
// codebook scaled by 1/sqrt(d) (the quantizer of this log-concave law is unique,
// so the start only sets the number of steps), iterates until the largest level
// change is below 1e-15, then makes the levels exactly antisymmetric.
void lloyd_max_sphere(int bits, int d, std::vector<double>& lev, std::vector<double>& bnd) {
  const int L = 1 << bits;
  const double p = 0.5 * (d - 1);
  std::vector<double> g, gb;
  lloyd_max(bits, g, gb);
  lev.resize(L);
  bnd.resize(L - 1);
  for (int i = 0; i < L; ++i) lev[i] = std::fmin(0.999, std::fmax(-0.999, g[i] / std::sqrt(static_cast<double>(d))));
  double gx[GL_N], gw[GL_N];
  gauss_legendre(gx, gw);
  std::vector<double> nl(L);
  for (int it = 0; it < 200000; ++it) {
    for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
    double delta = 0;
    for (int i = 0; i < L; ++i) {
      const double a = i == 0 ? -1.0 : bnd[i - 1];
      const double b = i == L - 1 ? 1.0 : bnd[i];
      nl[i] = sphere_m1(a, b, p) / sphere_weight_mass(a, b, p, gx, gw);
      delta = std::fmax(delta, std::fabs(nl[i] - lev[i]));
    }
    lev = nl;
    if (delta < 1e-15) break;
  }
  std::vector<double> sym(L);
  for (int i = 0; i < L; ++i) sym[i] = 0.5 * (lev[i] - lev[L - 1 - i]);
  lev = sym;
  for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
}

// Haar orthogonal matrix: Householder QR of a Gaussian matrix, Q with the
// columns' signs flipped so that diag(R) > 0. a: d x d row-major, overwritten.
void haar_from_gaussian(int d, std::vector<double>& a, std::vector<double>& q) {
  std::vector<double> vs(static_cast<size_t>(d) * d, 0.0);  // Householder vectors, row k
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0;
    for (int i = k; i < d; ++i) norm2 += a[i * d + k] * a[i * d + k];
    double nrm = std::sqrt(norm2);
    double x0 = a[k * d + k];
    double alpha = x0 >= 0 ? -nrm : nrm;
    double* v = &vs[static_cast<size_t>(k) * d];
    for (int i = k; i < d; ++i) v[i] = a[i * d + k];
    v[k] -= alpha;
    double vn2 = 0;
    for (int i = k; i < d; ++i) vn2 += v[i] * v[i];
    rdiag[k] = alpha;
    if (vn2 == 0) continue;
    double inv = 1.0 / std::sqrt(vn2);
    for (int i = k; i < d; ++i) v[i] *= inv;
    for (int j = k; j < d; ++j) {
      double dot = 0;
      for (int i = k; i < d; ++i) dot += v[i] * a[i * d + j];
      for (int i = k; i < d; ++i) a[i * d + j] -= 2.0 * dot * v[i];
    }
  }
  // Q = H_0 H_1 ... H_{d-1}: apply the reflectors to I in reverse order.
  q.assign(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &vs[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0;
      for (int i = k; i < d; ++i) dot += v[i] * q[i * d + j];
      for (int i = k; i < d; ++i) q[i * d + j] -= 2.0 * dot * v[i];
    }
  }
  for (int j = 0; j < d; ++j)
    if (rdiag[j] < 0)
      for (int i = 0; i < d; ++i) q[i * d + j] = -q[i * d + j];
}

}  // namespace

extern "C" fq_status fq_build_codebook(int bits, int head_dim, int rotation, uint64_t rot_seed,
                                       uint64_t qjl_seed, int qjl_dim, float* levels,
                                       float* boundaries, float* rotation_matrix,
                                       float* rotation_t, float* wht_signs, float* qjl_matrix,
                                       float* qjl_matrix_t) {
  if (!levels || !boundaries) return FQ_ERR_INVALID_ARG;
  if (rotation != FQ_ROT_HAAR && rotation != FQ_ROT_WHT) return FQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 4) return FQ_ERR_UNSUPPORTED;
  if (head_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  if (qjl_dim != 0 && qjl_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  const int d = head_dim;
  const double inv_sqrt_d = 1.0 / std::sqrt(static_cast<double>(d));

  std::vector<double> lev, bnd;
  lloyd_max(bits, lev, bnd);
  for (size_t i = 0; i < lev.size(); ++i) levels[i] = static_cast<float>(lev[i] * inv_sqrt_d);
  for (size_t i = 0; i < bnd.size(); ++i) boundaries[i] = static_cast<float>(bnd[i] * inv_sqrt_d);

  std::vector<double> pi(static_cast<size_t>(d) * d);
  if (rotation == FQ_ROT_HAAR) {
    if (rotation_matrix || rotation_t) {
      std::vector<double> g(static_cast<size_t>(d) * d);
      gaussians(rot_seed, g.size(), g.data());
      haar_from_gaussian(d, g, pi);
    }
  } else {
    std::vector<double> s(d);
    for (int j = 0; j < d; ++j) s[j] = (splitmix64_at(rot_seed, j) >> 63) ? -1.0 : 1.0;
    if (wht_signs)
      for (int j = 0; j < d; ++j) wht_signs[j] = static_cast<float>(s[j]);
    // Pi[i][j] = H[i][j] s_j / sqrt(d); Sylvester H[i][j] = (-1)^popcount(i & j).
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double h = (__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -1.0 : 1.0;
        pi[i * d + j] = h * s[j] * inv_sqrt_d;
      }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      if (rotation_matrix) rotation_matrix[i * d + j] = static_cast<float>(pi[i * d + j]);
      if (rotation_t) rotation_t[j * d + i] = static_cast<float>(pi[i * d + j]);
    }

  if (qjl_dim > 0 && (qjl_matrix || qjl_matrix_t)) {
    std::vector<double> s(static_cast<size_t>(qjl_dim) * d);
    gaussians(qjl_seed, s.size(), s.data());
    for (int i = 0; i < qjl_dim; ++i)
      for (int j = 0; j < d; ++j) {
        const float x = static_cast<float>(s[static_cast<size_t>(i) * d + j]);
        if (qjl_matrix) qjl_matrix[i * d + j] = x;
        if (qjl_matrix_t) qjl_matrix_t[j * qjl_dim + i] = x;
      }
  }
  return FQ_OK;
}

namespace {

// Round-to-nearest-even bf16 of a finite fp32 value, as bits.
inline uint32_t bf16_bits_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

inline float bf16_to_float(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline uint32_t f16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

// Accumulator row r of row tile T of the 32x32 matrix-core products holds this
// rotated coordinate (lane half h = (r / 4) % 2 owns coordinates 64h .. 64h+63).
inline int perm_row(int T, int r) { return 64 * ((r >> 2) & 1) + 16 * T + 4 * (r >> 3) + (r & 3); }

}  // namespace

extern "C" fq_status fq_pack_mfma_operands(const float* rotation_matrix, const float* qjl_matrix,
                                           int head_dim, void* out, size_t out_bytes) {
  if (!rotation_matrix || !out || out_bytes < FQ_MFMA_OPERAND_BYTES) return FQ_ERR_INVALID_ARG;
  if (head_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  const int d = head_dim;
  uint32_t* o = static_cast<uint32_t*>(out);  // 4 matrices x 32 fragments x 64 lanes x 4 dwords
  const int per_matrix = 32 * 64 * 4;
  for (int f = 0; f < 32; ++f) {
    const int T = f >> 3, s = f & 7;
    for (int l = 0; l < 64; ++l) {
      const int row = perm_row(T, l & 31);
      const int col = 64 * (l >> 5) + 8 * s;
      for (int q = 0; q < 4; ++q) {
        uint32_t ph = 0, pl = 0, sh = 0, sl = 0;
        for (int half = 0; half < 2; ++half) {
          const int e = 2 * q + half;
          const float x = rotation_matrix[row * d + col + e];
          const uint32_t hb = bf16_bits_rne(x);
          const uint32_t lb = bf16_bits_rne(x - bf16_to_float(hb));
          ph |= hb << (16 * half);
          pl |= lb << (16 * half);
          if (qjl_matrix) {
            const float y = qjl_matrix[row * d + col + e];
            const _Float16 yh = static_cast<_Float16>(y);
            sh |= f16_bits(y) << (16 * half);
            sl |= f16_bits(y - static_cast<float>(yh)) << (16 * half);
          }
        }
        const int idx = (f * 64 + l) * 4 + q;
        o[0 * per_matrix + idx] = ph;
        o[1 * per_matrix + idx] = pl;
        o[2 * per_matrix + idx] = sh;
        o[3 * per_matrix + idx] = sl;
      }
    }
  }
  return FQ_OK;
}

extern "C" fq_status fq_build_levels(int bits, int head_dim, int kind, float* levels, float* boundaries) {
  if (!levels || !boundaries) return FQ_ERR_INVALID_ARG;
  if (kind != FQ_CB_GAUSSIAN && kind != FQ_CB_SPHERE) return FQ_ERR_INVALID_ARG;
  if (bits < 2 || bits > 4) return FQ_ERR_UNSUPPORTED;
  if (head_dim < 3 || head_dim > 256) return FQ_ERR_UNSUPPORTED;
  std::vector<double> lev, bnd;
  double scale = 1.0;
  if (kind == FQ_CB_GAUSSIAN) {
    lloyd_max(bits, lev, bnd);
    scale = 1.0 / std::sqrt(static_cast<double>(head_dim));
  } else {
    lloyd_max_sphere(bits, head_dim, lev, bnd);
  }
  for (size_t i = 0; i < lev.size(); ++i) levels[i] = static_cast<float>(lev[i] * scale);
  for (size_t i = 0; i < bnd.size(); ++i) boundaries[i] = static_cast<float>(bnd[i] * scale);
  return FQ_OK;
}
