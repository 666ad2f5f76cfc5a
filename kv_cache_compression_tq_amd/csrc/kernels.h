// Launchers of the HIP kernels (device code lives in *.hip).  Plain C++
// signatures: device pointers, sizes and a stream.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace tq {

// Device tables of one codec (all groups concatenated, group stride d*d).
struct DeviceTables {
  int d = 0, groups = 0, variant = 0, mse_bits = 0;
  int64_t code_row = 0, sign_row = 0;
  const float *Pi = nullptr;   // [G][d][d] row-major: y = Pi x
  const float *PiT = nullptr;  // [G][d][d] = Pi^T
  const float *S = nullptr;    // [G][d][d] QJL projection (prod)
  const float *ST = nullptr;   // [G][d][d] = S^T
  const float *MT = nullptr;   // [G][d][d] = (S Pi^T)^T (prod)
  const float *cent = nullptr; // [2^mse_bits]
  const float *bnd = nullptr;  // [2^mse_bits - 1]
  // boundary-search cell table (host_codec.h CellTable): 2 words per cell
  const uint32_t *cells = nullptr;
  int cell_radius = 0;
  float cell_scale = 1.f;
  // d == 128 fast path: MFMA operand images (see quant128.hip)
  const uint32_t *pi_frag = nullptr;  // [G][...] bf16 hi/lo pairs, permuted rows
  const uint32_t *m_frag = nullptr;   // [G][...] same for M (prod)
  const uint32_t *dq_pi_frag = nullptr;  // [G][...] f16 hi/lo image of Pi^T (dequantize)
  const uint32_t *dq_s_frag = nullptr;   // [G][...] f16 hi/lo image of S^T (dequantize, prod)
  // any d (multiple of 8) != 128: 128 x 128 blocks of Pi ([G][panel][chunk]) and,
  // for prod, of S then M ([G][panel][2 chunks]); images as pi_frag
  const uint32_t *tiled_rot = nullptr;
  const uint32_t *tiled_sign = nullptr;
  const uint32_t *logit_lut = nullptr; // packed f16 decode tables for logits128
  float lut_inv_scale = 1.f;           // 1 / alpha of the f16 centroid table
  // positive halves of the codebook (host values, passed as launch arguments)
  float pos_bnd[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // t_{L/2} .. t_{L-2}
  float pos_cent[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // c_{L/2} .. c_{L-1}
};

constexpr float kQjlScale = 1.2533141373155003f;  // sqrt(pi/2)
// Radius of the boundary-search cell table the d = 128 kernels are built for
// (255 cells; wider tables send a shape to the generic kernels).
constexpr int kCellRadius = 127;

// The library's fixed device workspace (scratch.hip), for the entry points
// that allocate nothing.  static_scratch_setup(device) looks up the array's
// address on `device`, which must be current; it is done once per device.
// static_scratch(device) returns that address (nullptr before the set-up).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch_setup(int device);
void *static_scratch(int device);

// Dense baseline: logits of float16 (f32_keys = 0) or float32 keys stored
// unquantized, [n_sets][n_keys][128]; hipErrorNotSupported past 32-bit offsets.
hipError_t launch_dense_logits128(const float *q, int64_t nq, const void *keys, int f32_keys, int64_t n_sets,
                                  int64_t n_keys, float *out, hipStream_t st);
// Measurement probes (probes.hip).  kind: 0 copy, 1 read/write 4:1, 2 read/write
// 9:2, 3 read only, 4 the 9:2 mix with the logits kernel's store pattern.
int64_t probe_stream_tiles(int kind, int64_t in_bytes);
int64_t probe_stream_out_bytes(int kind, int64_t tiles);
hipError_t launch_probe_stream(int kind, const void *in, void *out, int64_t tiles, int grid, hipStream_t st);
hipError_t launch_probe_issue(int mode, int waves_per_simd, int64_t iters, int grid, uint32_t *out,
                              hipStream_t st);
hipError_t launch_probe_mfma(int f16, int64_t iters, int grid, float *out, hipStream_t st);

hipError_t launch_quant_generic(const DeviceTables &t, const void *x, int dtype, int64_t n_sets,
                                int64_t n, uint8_t *codes, uint8_t *signs, float *norms,
                                float *rnorms, hipStream_t st);
hipError_t launch_dequant_generic(const DeviceTables &t, const uint8_t *codes, const uint8_t *signs,
                                  const float *norms, const float *rnorms, int64_t n_sets, int64_t n,
                                  float *out, hipStream_t st);
hipError_t launch_logits_generic(const DeviceTables &t, const float *q, int64_t nq,
                                 const uint8_t *codes, const uint8_t *signs, const float *norms,
                                 const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
                                 hipStream_t st);
// Decode attention, any d: logits into `logits` [n_sets][nq][n_keys] (then
// softmax weights in place), value partial sums into `part`
// [attention_generic_chunks(n_keys)][n_sets][nq][2][d], result into `out`.
int64_t attention_generic_chunks(int64_t n_keys);
hipError_t launch_attention_generic(const DeviceTables &tk, const DeviceTables &tv, const float *q, int64_t nq,
                                    const uint8_t *k_codes, const uint8_t *k_signs, const float *k_norms,
                                    const float *k_rnorms, const uint8_t *v_codes, const uint8_t *v_signs,
                                    const float *v_norms, const float *v_rnorms, int64_t n_sets, int64_t n_keys,
                                    float scale, float *logits, float *part, float *out, hipStream_t st);
// One vector per set into row rows[s] of the cache arrays (rows outside
// [0, cache_rows) are skipped).
hipError_t launch_append(const DeviceTables &t, const void *x, int dtype, int64_t n_sets, const int64_t *rows,
                         int64_t cache_rows, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                         hipStream_t st);
// Outlier-channel split: gather x rows into the two parts (dtype 0 f32, 1
// bf16), scatter f32 parts back, and out += in.
hipError_t launch_gather_parts(const void *x, int dtype, int64_t rows, int64_t n, int groups, int d, int n_out,
                               const int32_t *perm, void *xo, void *xr, hipStream_t st);
hipError_t launch_scatter_parts(const float *xo, const float *xr, int64_t rows, int64_t n, int groups, int d,
                                int n_out, const int32_t *perm, float *out, hipStream_t st);
hipError_t launch_add_inplace(float *out, const float *in, int64_t count, hipStream_t st);
hipError_t launch_pack(const uint8_t *idx, int bits, int64_t rows, int count, int64_t row_bytes,
                       uint8_t *out, hipStream_t st);
hipError_t launch_unpack(const uint8_t *in, int bits, int64_t rows, int count, int64_t row_bytes,
                         uint8_t *idx, hipStream_t st);

// d == 128 fast paths (return hipErrorNotSupported when a shape is outside
// what they handle, so the caller can use the generic kernels).
hipError_t launch_quant128(const DeviceTables &t, const void *x, int dtype, int64_t n_sets,
                           int64_t n, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                           hipStream_t st);
// Fused mixed-precision quantize (d = 128, 64 outlier + 64 regular channels,
// TurboQuant_mse, bf16 input): img / masks from fast128_build_mixed_image per
// group; `to` / `tr` the part codecs' tables.
hipError_t launch_quant128_mixed(const DeviceTables &to, const DeviceTables &tr, const uint32_t *img,
                                 const uint32_t *masks, const void *x, int64_t n_sets, int64_t n, int groups,
                                 uint8_t *codes_o, float *norms_o, uint8_t *codes_r, float *norms_r,
                                 hipStream_t st);
hipError_t launch_quant_tiled(const DeviceTables &t, const void *x, int dtype, int64_t n_sets, int64_t n,
                              uint8_t *codes, uint8_t *signs, float *norms, float *rnorms, hipStream_t st);
hipError_t launch_dequant128(const DeviceTables &t, const uint8_t *codes, const uint8_t *signs,
                             const float *norms, const float *rnorms, int64_t n_sets, int64_t n,
                             float *out, hipStream_t st);
hipError_t launch_logits128(const DeviceTables &t, const float *q, int64_t nq,
                            const uint8_t *codes, const uint8_t *signs, const float *norms,
                            const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
                            hipStream_t st);
// Logits on mixed-precision keys (d = 128, 64 + 64, TurboQuant_mse parts):
// RT = [groups][128][128], the transpose of the block matrix whose rows 0..63
// are Pi_o on the outlier channels and 64..127 Pi_r on the others.
hipError_t launch_logits128_mixed(const DeviceTables &to, const DeviceTables &tr, const float *RT, const float *q,
                                  int64_t nq, const uint8_t *codes_o, const uint8_t *codes_r, const float *norms_o,
                                  const float *norms_r, int64_t n_sets, int64_t n_keys, int groups, float *out,
                                  hipStream_t st);

// Fused decode attention, d = 128, keys of any variant with <= 4 mse bits and
// TurboQuant_mse values with 1..4 bits.  attention128_workspace returns the
// bytes of `part` it needs (0 when it does not handle the codecs).
size_t attention128_workspace(const DeviceTables &tk, const DeviceTables &tv, int64_t nq, int64_t n_sets,
                              int64_t n_keys);
hipError_t launch_attention128(const DeviceTables &tk, const DeviceTables &tv, const float *q, int64_t nq,
                               const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
                               const float *krnorms, const uint8_t *vcodes, const float *vnorms, int64_t n_sets,
                               int64_t n_keys, float scale, float *part, float *out, hipStream_t st);

// Top-k maximum inner product search over one set of keys: the fused scan
// for d <= 256 and mse bits <= 4, else score-then-select through the logits
// kernels.  topk_workspace returns the bytes of `ws`.  out_idx is int32.
size_t topk_workspace(const DeviceTables &t, int64_t nq, int64_t n_keys, int k);
hipError_t launch_topk(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes, const uint8_t *signs,
                       const float *norms, const float *rnorms, int64_t n_keys, int k, void *ws, float *out_scores,
                       int32_t *out_idx, hipStream_t st);

}  // namespace tq
