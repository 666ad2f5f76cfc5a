// Host construction of the codec tables, float64.  Runs once per codec.
#include "host_codec.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <stdexcept>
#include <thread>

namespace tq {
namespace {

// SplitMix64 output finaliser (Steele, Lea, Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): xor-shift 30, multiply,
// xor-shift 27, multiply, xor-shift 31.
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Run f(j) for j in [lo, hi) on a few host threads (large matrices only).
template <class F>
void parallel_for(int lo, int hi, F f) {
  const int n = hi - lo;
  int nt = (int)std::min<unsigned>(std::max(1u, std::thread::hardware_concurrency()), 16u);
  if (n < 256 || nt == 1) {
    for (int j = lo; j < hi; ++j) f(j);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t) {
    th.emplace_back([=, &f] {
      for (int j = lo + t; j < hi; j += nt) f(j);
    });
  }
  for (auto &x : th) x.join();
}

}  // namespace

double gaussian(uint64_t seed, uint64_t group, int mat, uint64_t elem) {
  // key = mix(seed) ^ ((16 g + mat) << 32); h_t = mix(key ^ (2 e + t))
  const uint64_t key = mix64(seed) ^ ((16ull * group + (uint64_t)mat) << 32);
  const uint64_t h0 = mix64(key ^ (2ull * elem));
  const uint64_t h1 = mix64(key ^ (2ull * elem + 1ull));
  const double u1 = ((double)(h0 >> 11) + 1.0) * 0x1.0p-53;  // (0, 1]
  const double u2 = (double)(h1 >> 11) * 0x1.0p-53;          // [0, 1)
  // Box and Muller (1958): one normal deviate from two uniforms.
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(2.0 * M_PI * u2);
}

void gaussian_matrix(uint64_t seed, uint64_t group, int mat, int rows, int cols, double *out) {
  const uint64_t total = (uint64_t)rows * (uint64_t)cols;
  for (uint64_t e = 0; e < total; ++e) out[e] = gaussian(seed, group, mat, e);
}

void orthogonal_factor(int n, const double *a, double *q) {
  // Column-major working copy: w[j*n + i] = A[i][j].
  std::vector<double> w((size_t)n * n), v((size_t)n * n, 0.0), rdiag(n);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) w[(size_t)j * n + i] = a[(size_t)i * n + j];

  for (int k = 0; k < n; ++k) {
    double *col = &w[(size_t)k * n];
    double norm2 = 0.0;
    for (int i = k; i < n; ++i) norm2 += col[i] * col[i];
    const double norm = std::sqrt(norm2);
    if (k == n - 1) {  // last column: no reflection, R_kk = w_kk
      rdiag[k] = col[k];
      break;
    }
    // Reflect x = col[k:] onto alpha e_1 with alpha = -sign(x_0) ||x||.
    const double alpha = col[k] >= 0.0 ? -norm : norm;
    double *vk = &v[(size_t)k * n];
    double vn2 = 0.0;
    for (int i = k; i < n; ++i) {
      vk[i] = col[i] - (i == k ? alpha : 0.0);
      vn2 += vk[i] * vk[i];
    }
    rdiag[k] = alpha;
    if (vn2 == 0.0) continue;  // column already reduced
    const double inv = 1.0 / std::sqrt(vn2);
    for (int i = k; i < n; ++i) vk[i] *= inv;
    for (int i = k; i < n; ++i) col[i] = (i == k ? alpha : 0.0);
    // Trailing columns: w_j -= 2 v (v . w_j)
    parallel_for(k + 1, n, [&](int j) {
      double *wj = &w[(size_t)j * n];
      double s = 0.0;
      for (int i = k; i < n; ++i) s += vk[i] * wj[i];
      s *= 2.0;
      for (int i = k; i < n; ++i) wj[i] -= s * vk[i];
    });
  }
  // Q = H_0 H_1 ... H_{n-2}, accumulated backwards on the identity
  // (column-major, qc[j*n + i] = Q[i][j]).
  std::vector<double> qc((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) qc[(size_t)i * n + i] = 1.0;
  for (int k = n - 2; k >= 0; --k) {
    const double *vk = &v[(size_t)k * n];
    parallel_for(k, n, [&](int j) {
      double *qj = &qc[(size_t)j * n];
      double s = 0.0;
      for (int i = k; i < n; ++i) s += vk[i] * qj[i];
      s *= 2.0;
      if (s != 0.0)
        for (int i = k; i < n; ++i) qj[i] -= s * vk[i];
    });
  }
  // Make diag(R) positive: flip column k of Q where R_kk < 0.
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      const double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;
      q[(size_t)i * n + j] = sgn * qc[(size_t)j * n + i];
    }
}

namespace {

// Continued fraction of the incomplete beta (DLMF 8.17.22):
// I_x(a,b) = x^a (1-x)^b / (a B(a,b)) / F,  F = 1 + d1/(1 + d2/(1 + ...)).
// Returns 1/F, with F evaluated by the modified Lentz method; converges fast
// for x < (a+1)/(a+b+2).
double beta_cf(double x, double a, double b) {
  const double tiny = 1e-300, eps = 1e-16;
  double f = 1.0, c = 1.0, d = 0.0;
  for (int i = 1; i < 20000; ++i) {
    const int m = i / 2;
    double coef;
    if (i & 1)
      coef = -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
    else
      coef = m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    d = 1.0 + coef * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + coef / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    const double delta = c * d;
    f *= delta;
    if (std::fabs(delta - 1.0) < eps) break;
  }
  return 1.0 / f;
}

struct CoordLaw {
  int d;
  double log_c;  // log of Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2))
  explicit CoordLaw(int d_) : d(d_) {
    log_c = std::lgamma(0.5 * d) - std::lgamma(0.5 * (d - 1)) - 0.5 * std::log(M_PI);
  }
  // F(x) = 1/2 + sgn(x)/2 I_{x^2}(1/2, (d-1)/2)   (substitute s = x^2)
  double cdf(double x) const {
    if (x <= -1.0) return 0.0;
    if (x >= 1.0) return 1.0;
    const double ib = incomplete_beta(x * x, 0.5, 0.5 * (d - 1));
    return x >= 0.0 ? 0.5 + 0.5 * ib : 0.5 - 0.5 * ib;
  }
  // (1 - x^2)^((d-1)/2) scaled by C/(d-1): antiderivative of -x f(x)
  double moment_term(double x) const {
    if (std::fabs(x) >= 1.0) return 0.0;
    return std::exp(log_c - std::log((double)(d - 1)) + 0.5 * (d - 1) * std::log1p(-x * x));
  }
  double first_moment(double a, double b) const { return moment_term(a) - moment_term(b); }
  // f(x) = C (1 - x^2)^((d-3)/2) inside (-1, 1)
  double density(double x) const {
    if (std::fabs(x) >= 1.0) return 0.0;
    return std::exp(log_c + 0.5 * (d - 3) * std::log1p(-x * x));
  }
  // F^{-1}(p) by bisection on the increasing CDF (start values only)
  double quantile(double p) const {
    double lo = -1.0, hi = 1.0;
    for (int i = 0; i < 200 && lo < hi; ++i) {
      const double mid = 0.5 * (lo + hi);
      if (mid <= lo || mid >= hi) break;
      if (cdf(mid) < p)
        lo = mid;
      else
        hi = mid;
    }
    return 0.5 * (lo + hi);
  }
};

}  // namespace

double incomplete_beta(double x, double a, double b) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lbeta = std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b);
  const double front = std::exp(a * std::log(x) + b * std::log1p(-x) - lbeta);
  if (x < (a + 1.0) / (a + b + 2.0)) return front * beta_cf(x, a, b) / a;
  return 1.0 - front * beta_cf(1.0 - x, b, a) / b;
}

Codebook lloyd_max(int d, int bits) {
  if (d < 2 || bits < 1 || bits > 8) throw std::invalid_argument("lloyd_max: bad d or bits");
  const int L = 1 << bits;
  CoordLaw law(d);
  std::vector<double> c(L), t(L - 1), edge(L + 1), mass(L), next(L);
  // start at the law's own quantiles: inside (-1, 1) for every d and L, and
  // the answer itself for d = 3 (uniform law); symmetric by construction
  for (int k = 0; k < L / 2; ++k) {
    c[L / 2 + k] = law.quantile((L / 2 + k + 0.5) / L);
    c[L / 2 - 1 - k] = -c[L / 2 + k];
  }
  // next = T(c): boundaries at the midpoints, centroids at the cell means
  auto lloyd_map = [&]() {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    edge[0] = -1.0;
    edge[L] = 1.0;
    for (int k = 0; k + 1 < L; ++k) edge[k + 1] = t[k];
    for (int k = 0; k < L; ++k) mass[k] = law.cdf(edge[k + 1]) - law.cdf(edge[k]);
    for (int k = 0; k < L; ++k) next[k] = law.first_moment(edge[k], edge[k + 1]) / mass[k];
  };
  const double sd = std::sqrt((double)d);
  int it = 0;
  // phase 1: Lloyd's iteration until its moves are below 1e-3 / sqrt(d)
  for (int pass = 0; pass < 100000; ++pass) {
    lloyd_map();
    ++it;
    double step = 0.0;
    for (int k = 0; k < L; ++k) {
      const double sym = 0.5 * (next[k] - next[L - 1 - k]);  // f_d is even
      step = std::max(step, std::fabs(sym - c[k]));
      c[k] = sym;
    }
    if (step < 1e-3 / sd) break;
  }
  // phase 2: Newton on c = T(c).  c'_k depends on c only through its cell
  // edges t_{k-1}, t_k: dc'_k/dt_k = f(t_k)(t_k - c'_k)/P_k and
  // dc'_k/dt_{k-1} = f(t_{k-1})(c'_k - t_{k-1})/P_k, with t_k = (c_k + c_{k+1})/2,
  // so (J_T - I) delta = c - T(c) is tridiagonal (Thomas algorithm).
  std::vector<double> lo(L), up(L), sub(L), dia(L), sup(L), rhs(L), delta(L);
  double prev = HUGE_VAL;
  for (int pass = 0; pass < 100; ++pass) {
    lloyd_map();
    for (int k = 0; k < L; ++k) {
      up[k] = k + 1 < L ? law.density(t[k]) * (t[k] - next[k]) / mass[k] : 0.0;
      lo[k] = k > 0 ? law.density(t[k - 1]) * (next[k] - t[k - 1]) / mass[k] : 0.0;
      sub[k] = 0.5 * lo[k];
      dia[k] = 0.5 * (lo[k] + up[k]) - 1.0;
      sup[k] = 0.5 * up[k];
      rhs[k] = c[k] - next[k];
    }
    for (int k = 1; k < L; ++k) {  // forward elimination
      const double w = sub[k] / dia[k - 1];
      dia[k] -= w * sup[k - 1];
      rhs[k] -= w * rhs[k - 1];
    }
    delta[L - 1] = rhs[L - 1] / dia[L - 1];
    for (int k = L - 2; k >= 0; --k) delta[k] = (rhs[k] - sup[k] * delta[k + 1]) / dia[k];
    double size = 0.0;
    for (int k = 0; k < L; ++k) size = std::max(size, std::fabs(delta[k]));
    if (!(size < prev)) break;  // at the rounding floor of T
    for (int k = 0; k < L; ++k) next[k] = c[k] + delta[k];
    for (int k = 0; k < L; ++k) c[k] = 0.5 * (next[k] - next[L - 1 - k]);
    prev = size;
    ++it;
    if (size < 1e-13 / sd) break;
  }
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  edge[0] = -1.0;
  edge[L] = 1.0;
  for (int k = 0; k + 1 < L; ++k) edge[k + 1] = t[k];
  double e = 0.0;
  for (int k = 0; k < L; ++k) e += c[k] * c[k] * (law.cdf(edge[k + 1]) - law.cdf(edge[k]));
  Codebook cb;
  cb.centroids = c;
  cb.boundaries = t;
  cb.distortion = 1.0 - d * e;
  cb.iterations = it;
  return cb;
}

bool build_cell_table(const std::vector<float> &bounds, int min_radius, CellTable &out) {
  const double margin = 1.0 / 16.0;
  double gap = 2.0;
  for (size_t k = 0; k + 1 < bounds.size(); ++k) {
    const double g = (double)bounds[k + 1] - (double)bounds[k];
    if (!(g > 0.0)) return false;
    gap = std::min(gap, g);
  }
  // a widened cell spans (1 + 2 margin) / scale < gap
  const float scale = (float)((1.0 + 2.0 * margin) / gap * 1.01);
  const int radius = std::max((int)std::ceil((double)scale) + 2, min_radius);
  std::vector<uint32_t> words(2 * (2 * radius + 1));
  for (int r = -radius; r <= radius; ++r) {
    const double lo = (r - 0.5 - margin) / (double)scale, hi = (r + 0.5 + margin) / (double)scale;
    float t = 1e30f;
    uint32_t below = 0;
    int inside = 0;
    for (size_t k = 0; k < bounds.size(); ++k) {
      const double b = bounds[k];
      if (b < lo) {
        ++below;
      } else if (b <= hi) {
        t = bounds[k];
        ++inside;
      }
    }
    if (inside > 1) return false;
    std::memcpy(&words[2 * (r + radius)], &t, 4);
    words[2 * (r + radius) + 1] = below;
  }
  out.scale = scale;
  out.radius = radius;
  out.words.swap(words);
  return true;
}

}  // namespace tq
