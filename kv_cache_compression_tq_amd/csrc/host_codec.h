// Host-side construction of a TurboQuant codec's tables (float64, once per
// codec; never on the hot path).
#pragma once
#include <cstdint>
#include <vector>

namespace tq {

constexpr int kMatPi = 0;
constexpr int kMatS = 1;

// Standard normal number `elem` of the counter-based stream (seed, group, mat):
// SplitMix64 finaliser keyed by (seed, group, mat, elem) -> two uniforms ->
// Box–Muller.
double gaussian(uint64_t seed, uint64_t group, int mat, uint64_t elem);

// rows x cols Gaussian matrix, row-major, entry (i,j) = element i*cols+j.
void gaussian_matrix(uint64_t seed, uint64_t group, int mat, int rows, int cols, double *out);

// Orthogonal factor Q of A = QR (A: n x n row-major) with diag(R) > 0, by
// Householder reflections.  Q is written row-major into q.
void orthogonal_factor(int n, const double *a, double *q);

// Regularised incomplete beta I_x(a, b).
double incomplete_beta(double x, double a, double b);

struct Codebook {
  std::vector<double> centroids;   // ascending, 2^bits
  std::vector<double> boundaries;  // midpoints, 2^bits - 1
  double distortion = 0.0;         // d * E[(X - Q(X))^2]
  int iterations = 0;
};

// Lloyd–Max quantizer for the post-rotation coordinate density
// f_d(x) ∝ (1 - x^2)^((d-3)/2) on [-1, 1] with 2^bits levels (d >= 2; d = 2
// is the arcsine law).
Codebook lloyd_max(int d, int bits);

// Table for a branch-free boundary search over a normalised coordinate u in
// [-1, 1].  Cell r (r = round(u * scale), |r| <= radius) covers
// u in [(r - 0.5 - m) / scale, (r + 0.5 + m) / scale] with a margin m = 1/16;
// scale is chosen so that no cell holds more than one boundary.  Entry
// r + radius is two words: the float bits of the boundary inside the cell
// (1e30f if none) and the number of boundaries below it.  The index of u is
// then that count, plus one when u is above the cell's boundary.
struct CellTable {
  float scale = 1.f;
  int radius = 0;
  std::vector<uint32_t> words;
};

// Builds the table for ascending float32 boundaries with a radius of at least
// min_radius cells; false if the boundaries are not strictly ascending.
bool build_cell_table(const std::vector<float> &bounds, int min_radius, CellTable &out);

}  // namespace tq
