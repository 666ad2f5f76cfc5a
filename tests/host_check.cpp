// Host-code check built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitizers.py: runs the codec's host construction
// (Gaussian streams, Householder QR, Lloyd–Max, cell tables) over the shapes
// the library accepts and checks the invariants each must meet.  Prints "ok"
// and exits 0, or names the first failure and exits 1.
#include <cmath>
#include <cstdio>
#include <vector>

#include "../kv_cache_compression_tq_amd/csrc/host_codec.h"

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      std::fprintf(stderr, "FAIL: " __VA_ARGS__); \
      std::fprintf(stderr, "\n");                \
      ++fails;                                   \
    }                                            \
  } while (0)

int main() {
  // Householder QR: Q orthogonal, and Q^T G upper triangular with a positive diagonal
  for (int d : {2, 3, 5, 17, 128, 200}) {
    std::vector<double> g((size_t)d * d), q((size_t)d * d);
    tq::gaussian_matrix(7, 3, tq::kMatPi, d, d, g.data());
    tq::orthogonal_factor(d, g.data(), q.data());
    double worst = 0.0;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int k = 0; k < d; ++k) s += q[(size_t)k * d + i] * q[(size_t)k * d + j];
        worst = std::fmax(worst, std::fabs(s - (i == j ? 1.0 : 0.0)));
      }
    CHECK(worst < 1e-12, "Q^T Q != I at d=%d (%.3g)", d, worst);
    double below = 0.0, diag_min = 1e300;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j <= i; ++j) {
        double r = 0.0;  // R[i][j] = (Q^T G)[i][j]
        for (int k = 0; k < d; ++k) r += q[(size_t)k * d + i] * g[(size_t)k * d + j];
        if (j < i) below = std::fmax(below, std::fabs(r));
        if (j == i) diag_min = std::fmin(diag_min, r);
      }
    CHECK(below < 1e-10 && diag_min > 0.0, "R not upper triangular with diag > 0 at d=%d", d);
  }
  // Lloyd–Max: finite, ascending, symmetric, midpoint boundaries, distortion in (0, 1)
  for (int d : {2, 3, 4, 5, 8, 64, 128, 200, 1536, 4096}) {
    for (int b = 1; b <= 8; ++b) {
      const tq::Codebook cb = tq::lloyd_max(d, b);
      const int L = 1 << b;
      bool ok = (int)cb.centroids.size() == L && (int)cb.boundaries.size() == L - 1;
      for (int k = 0; ok && k < L; ++k) {
        ok = std::isfinite(cb.centroids[k]) && std::fabs(cb.centroids[k]) < 1.0 &&
             std::fabs(cb.centroids[k] + cb.centroids[L - 1 - k]) < 1e-15;
        if (k) ok = ok && cb.centroids[k] > cb.centroids[k - 1];
        if (k + 1 < L) ok = ok && cb.boundaries[k] == 0.5 * (cb.centroids[k] + cb.centroids[k + 1]);
      }
      CHECK(ok, "codebook d=%d b=%d is not finite / ascending / symmetric", d, b);
      CHECK(cb.distortion > 0.0 && cb.distortion < 1.0, "distortion d=%d b=%d = %g", d, b, cb.distortion);
      std::vector<float> t(cb.boundaries.begin(), cb.boundaries.end());
      tq::CellTable cells;
      CHECK(tq::build_cell_table(t, 127, cells), "cell table d=%d b=%d", d, b);
      // every cell holds at most one boundary: the count below a cell never
      // drops as the cell number grows, and rises by at most one plus the
      // boundary inside the previous cell
      for (size_t r = 1; r < cells.words.size() / 2; ++r)
        CHECK(cells.words[2 * r + 1] >= cells.words[2 * r - 1], "cell counts fall at d=%d b=%d", d, b);
    }
  }
  // d = 3 is the uniform law: its quantizer is the uniform one
  const tq::Codebook u = tq::lloyd_max(3, 3);
  for (int k = 0; k < 8; ++k) CHECK(std::fabs(u.centroids[k] - ((2 * k + 1) / 8.0 - 1.0)) < 1e-14, "uniform law");
  // incomplete beta at its symmetric point and edges
  CHECK(std::fabs(tq::incomplete_beta(0.5, 2.5, 2.5) - 0.5) < 1e-14, "I_0.5(a, a) != 1/2");
  CHECK(tq::incomplete_beta(0.0, 0.5, 3.0) == 0.0 && tq::incomplete_beta(1.0, 0.5, 3.0) == 1.0, "beta edges");
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
