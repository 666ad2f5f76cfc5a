// Host-side construction of the operand images used by the d = 128 MFMA
// kernels (fast128.hip).  Built once per codec at init.
#pragma once
#include <cstddef>
#include <cstdint>

namespace tq {

// True when the d = 128 kernels handle this configuration.
bool fast128_supported(int d, int mse_bits, int variant);

// 32-bit words of one rotation (or QJL) image per group.
size_t fast128_rotation_words(int d);

// Image of a d x d float64 matrix (row-major, out = mat * in) as the
// bf16 hi/lo MFMA A-operand fragments, rows permuted so that each lane ends up
// holding 32 consecutive output coordinates.  k_order 0: the contraction index
// follows the input-vector load order (rotation of x); k_order 1: it follows
// the lane-chunk order of register-resident rotated coordinates (QJL
// projection of the residual, dequantization).  f16: split into f16 hi/lo
// parts instead of bf16 (operands multiplied with f16 decode tables).
// natural_rows: output rows in natural order instead (each lane then holds
// coordinates 16 m + 4 g .. + 3 of row tile m; the dequantize images).
void fast128_build_rotation_image(const double *mat, int k_order, uint32_t *out, bool f16 = false,
                                  bool natural_rows = false);

// Image of the fused mixed-precision rotation (d = 128 split 64 + 64): pi_o and
// pi_r are the parts' 64 x 64 rotations (row-major float64), perm the 128
// channels (the 64 outlier channels, then the rest).  Output coordinates are
// ordered so that row tiles 0..3 of the MFMA give each lane group 16
// coordinates of the outlier part and tiles 4..7 16 of the regular part.
// mask (4 words): bit c set for the outlier channels.
void fast128_build_mixed_image(const double *pi_o, const double *pi_r, const int32_t *perm, uint32_t *out,
                               uint32_t *mask);

// Words of the logits decode tables for `mse_bits` (pair LUT + sign LUT).
// The pair LUT holds f16 values of alpha * c, with alpha > 0 chosen so that
// every scaled centroid rounds to f16 with the smallest relative error; the
// kernel divides the rotated query by alpha instead.  Returns 1 / alpha.
size_t fast128_lut_words(int mse_bits);
float fast128_build_logit_lut(const float *centroids, int mse_bits, uint32_t *out);

}  // namespace tq
