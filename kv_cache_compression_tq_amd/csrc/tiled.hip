// Quantize for any dimension d (a multiple of 8) on gfx950 matrix cores.
//
// The rotation Y = Pi X is cut into 128 x 128 blocks: output panel p holds
// coordinates [128 p, 128 p + 128), contraction chunk c the input elements
// [128 c, 128 c + 128) (both zero-padded past d).  Every block is stored as
// the same bf16 hi/lo MFMA operand image the d = 128 kernels use (rows
// permuted so that each lane ends up with 32 consecutive coordinates of its
// vector).  A workgroup computes two output panels (256 coordinates) for 128
// vectors, so that each float32 input element split into bf16 hi/lo on the
// vector ALU feeds twice the MFMAs of a one-panel workgroup.  The contraction
// runs one K step (32 elements) at a time: the step's fragments of both
// panels' blocks fill one 32 KB half of a 64 KB LDS buffer (direct
// global-to-LDS loads) while the MFMAs of the previous step read the other
// half, the inputs come one step ahead through registers, and two workgroups
// share a CU.  Steps wholly past d are skipped.  After the last step each
// panel's codes are searched and packed exactly as at d = 128.  Launches too
// small to fill the chip with pairs keep one panel per workgroup.
//
// TurboQuant_prod adds a second pass.  The QJL signs need the residual of the
// whole vector, so they are taken as sign(S x - nu M c[idx]) = sign(S r)
// (nu > 0; M = S Pi^T, c[idx] decoded from the codes the first pass wrote),
// a GEMM over 2 d contraction elements with images of S and M: M c[idx]
// first, its B operands read from a table of code pairs, then each column
// scaled by -nu and S x added.  The residual norm is gathered across panels
// in fixed point (integer atomics, exact and order-independent) and finished
// by panel 0 of the second pass.
//   [ttakun] TurboQuant_mse / TurboQuant_prod; [tqnet] 实现步骤草图;
//   [admirer] 第二步 (QJL signs of the residual).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tq {
namespace {

constexpr int kTiledThreads = 256;     // 4 waves x 32 vectors
constexpr int kTiledVectors = 128;     // vectors per workgroup
constexpr int kTiledWaves = kTiledThreads / 64;
constexpr int kUnitFrags = 64;         // fragments of one unit: 16 row tiles x 2 K steps x hi/lo
constexpr uint32_t kUnitBytes = kUnitFrags * kFragVec * 16;  // 64 KB
constexpr float kFix = 268435456.f;    // 2^28: fixed-point scale of the residual norm squared

struct TiledArgs {
  int64_t n;             // vectors per set
  int d, chunks, groups;
  int pair;              // output panels per workgroup: 2, or 1 for launches too small to fill the chip
  int64_t code_row, sign_row;
  float cell_scale;      // cells per unit, times 2^-22
  float cell_magic;      // 2 + radius 2^-22
  uint32_t cell_last;    // float bits of the last cell
  int cell_words;
};

// #{k : t_k < y / nu} through the cell table at LDS byte address tab (runtime radius).
__device__ __forceinline__ uint32_t cell_index_rt(uint32_t tab, float y, float nu, float sv, const TiledArgs &a) {
  uint32_t g = __float_as_uint(fmaf(y, sv, a.cell_magic));
  g = min(max(g, 0x40000000u), a.cell_last);
  const u32x2 e = *(lds_u32x2 *)(uintptr_t)((g << 3) + tab);
  const float dd = fmaf(nu, __uint_as_float(e[0]), -y);
  return e[1] + (__float_as_uint(dd) >> 31);
}

// One unit (K steps 2 kh, 2 kh + 1 of contraction chunk c) of the blocks of
// output panels 2 pp and 2 pp + 1 into LDS by direct global-to-LDS loads:
// buffer fragment 4 m + 2 kk + hl (row tile m = 0..15; tiles 8..15 are the
// second panel's) is fragment 2 (4 (m % 8) + 2 kh + kk) + hl of that panel's
// block.  blk0 / blk1: the two panels' blocks of chunk c (blk1 unused when
// the pair has one panel).  Each wave moves 16 fragments of 1 KB.
__device__ __forceinline__ void stage_unit(const u32x4 *blk0, const u32x4 *blk1, bool two, int kh, u32x4 *dst,
                                           int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kUnitFrags / kTiledWaves; ++i) {
    const int fi = wave * (kUnitFrags / kTiledWaves) + i, m = fi >> 2, q = fi & 3;
    if (m >= 8 && !two) continue;  // wave-uniform
    const u32x4 *blk = m < 8 ? blk0 : blk1;
    __builtin_amdgcn_global_load_lds((const void *)(blk + ((m & 7) * 4 + 2 * kh) * 2 * kFragVec + q * kFragVec + lane),
                                     (__attribute__((address_space(3))) void *)(dst + fi * kFragVec), 16, 0, 0);
  }
}

// One K step (k = 0..3 of contraction chunk c) of the blocks of both panels
// into a 32 KB half of the unit buffer: buffer fragment 2 m + hl (row tile
// m = 0..15; tiles 8..15 are the second panel's) is fragment 2 (4 (m % 8) +
// k) + hl of that panel's block.  Each wave moves 8 fragments of 1 KB.
__device__ __forceinline__ void stage_step(const u32x4 *blk0, const u32x4 *blk1, bool two, int k, u32x4 *dst,
                                           int wave, int lane) {
  constexpr int kStepFrags = kUnitFrags / 2;
#pragma unroll
  for (int i = 0; i < kStepFrags / kTiledWaves; ++i) {
    const int fi = wave * (kStepFrags / kTiledWaves) + i, m = fi >> 1, hl = fi & 1;
    if (m >= 8 && !two) continue;  // wave-uniform
    const u32x4 *blk = m < 8 ? blk0 : blk1;
    __builtin_amdgcn_global_load_lds((const void *)(blk + (2 * ((m & 7) * 4 + k) + hl) * kFragVec + lane),
                                     (__attribute__((address_space(3))) void *)(dst + fi * kFragVec), 16, 0, 0);
  }
}

// Input fragments of one K step for the lane's two vectors: elements e_step +
// 8 grp .. + 8 (zero past d).
template <bool F32IN>
struct XStep {
  u32x4 v[2][F32IN ? 2 : 1];
};

template <bool F32IN>
__device__ __forceinline__ void load_step(XStep<F32IN> &r, const void *xin, const int64_t (&row)[2], int e_step, int d,
                                          int grp) {
  const int e0 = e_step + 8 * grp;  // d is a multiple of 8: groups are all in or all out
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (e0 < d) {
      if constexpr (F32IN) {
        const u32x4 *p = (const u32x4 *)((const float *)xin + row[t] * d + e0);
        r.v[t][0] = p[0];
        r.v[t][1] = p[1];
      } else {
        r.v[t][0] = *(const u32x4 *)((const uint16_t *)xin + row[t] * d + e0);
      }
    } else {
#pragma unroll
      for (int h = 0; h < (F32IN ? 2 : 1); ++h) r.v[t][h] = u32x4{0, 0, 0, 0};
    }
  }
}

// acc[t][m] += one staged K step x the step's B operands (split into bf16
// hi/lo for float32 input), in four groups of eight fragments, each group
// read before its MFMAs; also ||x||^2 of the elements when NSQ.
template <bool F32IN, bool NSQ>
__device__ __forceinline__ void mma_step(const XStep<F32IN> &x, const u32x4 *buf, int frag_lane, bool two,
                                         f32x4 (&acc)[2][16], float (&nsq)[2]) {
  u32x4 bh[2], bl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (F32IN) {
      const f32x4 a = __builtin_bit_cast(f32x4, x.v[t][0]);
      const f32x4 b = __builtin_bit_cast(f32x4, x.v[t][1]);
      const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      split8(f, bh[t], bl[t]);
      if constexpr (NSQ) {
#pragma unroll
        for (int i = 0; i < 8; ++i) nsq[t] = fmaf(f[i], f[i], nsq[t]);
      }
    } else {
      bh[t] = x.v[t][0];
      bl[t] = bh[t];
      if constexpr (NSQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_lo(bh[t][i]), hi = bf16_hi(bh[t][i]);
          nsq[t] = fmaf(lo, lo, fmaf(hi, hi, nsq[t]));
        }
      }
    }
  }
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    if (gq >= 2 && !two) break;  // wave-uniform: the pair's second panel is absent
    u32x4 fh[4], fl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = 2 * (4 * gq + i);
      fh[i] = buf[f * kFragVec + frag_lane];
      fl[i] = buf[(f + 1) * kFragVec + frag_lane];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the group's 8 LDS reads
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 &c = acc[t][4 * gq + i];
        c = mfma_bf16(fh[i], bh[t], c);
        c = mfma_bf16(fl[i], bh[t], c);
        if constexpr (F32IN) c = mfma_bf16(fh[i], bl[t], c);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 8 * (F32IN ? 3 : 2), 0);  // then their MFMAs
  }
}

// acc[t][m] += unit (LDS) x B operands, for row tiles m < 8 (one panel) or
// m < 16 (two); `operands(kk, bh, bl)` gives the bf16 hi (and lo) B operands
// of K step kk for the two column tiles.  Per K step the fragments go in four
// groups of eight (four row tiles, hi and lo), each group read before its
// MFMAs.
template <bool LO, typename Operands>
__device__ __forceinline__ void mma_unit_ops(const u32x4 *buf, int frag_lane, bool two, f32x4 (&acc)[2][16],
                                             Operands operands) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 bh[2], bl[2];
    operands(kk, bh, bl);
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      if (gq >= 2 && !two) break;  // wave-uniform: the pair's second panel is absent
      u32x4 fh[4], fl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = (4 * gq + i) * 4 + 2 * kk;
        fh[i] = buf[f * kFragVec + frag_lane];
        fl[i] = buf[(f + 1) * kFragVec + frag_lane];
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the group's 8 LDS reads
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 &c = acc[t][4 * gq + i];
          c = mfma_bf16(fh[i], bh[t], c);
          c = mfma_bf16(fl[i], bh[t], c);
          if constexpr (LO) c = mfma_bf16(fh[i], bl[t], c);
        }
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * (LO ? 3 : 2), 0);  // then their MFMAs
    }
  }
}

// Rotation (or projection) of the workgroup's 128 vectors for the panel pair,
// over the input chunks, one K step (32 contraction elements) at a time: the
// step's fragments of both panels' blocks are staged by direct global-to-LDS
// loads into one 32 KB half of the unit buffer while the MFMAs of the step
// before run from the other half, and the step's inputs come one step ahead
// through registers.  One barrier per step: after it every wave's share of
// the step has landed and every wave is done with the half the next stage
// overwrites.  Steps wholly past d are skipped.
template <bool F32IN, bool NSQ>
__device__ __forceinline__ void rotate_pair(const void *xin, const u32x4 *img0, const u32x4 *img1, bool two,
                                            u32x4 *buf, const TiledArgs &a, const int64_t (&row)[2], int wave,
                                            int lane, int grp, f32x4 (&acc)[2][16], float (&nsq)[2]) {
  const int steps = (a.d + 31) / 32;
  u32x4 *const h0 = buf, *const h1 = buf + (kUnitFrags / 2) * kFragVec;
  XStep<F32IN> x0, x1;
  // step ks: wait for its stage and inputs, then stage step ks + 1 into the
  // other half and run step ks (the loop is unrolled by two so that every
  // register and buffer choice is static)
  auto step = [&](int ks, const XStep<F32IN> &xc, XStep<F32IN> &xn, const u32x4 *hc, u32x4 *hn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of step ks (and its inputs)
    __syncthreads();
    if (ks + 1 < steps) {
      const int c = (ks + 1) >> 2, k = (ks + 1) & 3;
      stage_step(img0 + (size_t)c * kImageVec, img1 + (size_t)c * kImageVec, two, k, hn, wave, lane);
      load_step<F32IN>(xn, xin, row, 32 * (ks + 1), a.d, grp);
    }
    int frag_lane = lane;
    asm volatile("" : "+v"(frag_lane));
    mma_step<F32IN, NSQ>(xc, hc, frag_lane, two, acc, nsq);
  };
  stage_step(img0, img1, two, 0, h0, wave, lane);
  load_step<F32IN>(x0, xin, row, 0, a.d, grp);
  for (int ks = 0; ks < steps; ks += 2) {
    step(ks, x0, x1, h0, h1);
    if (ks + 1 < steps) step(ks + 1, x1, x0, h1, h0);
  }
}

// Search and pack of one panel's 32 coordinates of column tile t (lane's
// vector v); prod: the squared residual partial.
template <int MB, bool PROD>
__device__ __forceinline__ float search_pack(const f32x4 *acc, int p, int grp, float nu, float inv, float sv,
                                             uint32_t tab_addr, uint32_t cent_addr, const TiledArgs &a,
                                             uint8_t *crow, bool live) {
  uint32_t w[MB > 0 ? MB : 1];
#pragma unroll
  for (int i = 0; i < (MB > 0 ? MB : 1); ++i) w[i] = 0;
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int coord = 128 * p + 32 * grp + j;  // coordinate of acc[j >> 2][j & 3]
    const float y = acc[j >> 2][j & 3];
    if (coord < a.d) {
      float cv = 0.f;
      if constexpr (MB > 0) {
        const uint32_t idx = cell_index_rt(tab_addr, y, nu, sv, a);
        put_field<MB>(w, j, idx);
        if constexpr (PROD) cv = *(lds_f32 *)(uintptr_t)(cent_addr + 4 * idx);
      }
      if constexpr (PROD) {
        const float r = fmaf(y, inv, -cv);
        part = fmaf(r, r, part);
      }
    }
  }
  if constexpr (MB > 0) {
    // the lane's 4 MB bytes at offset 16 p MB + 4 grp MB of the code row; whole
    // words past the row (padding of the last panel) are not stored
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int64_t off = (int64_t)16 * p * MB + 4 * grp * MB + 4 * i;
      if (live && off < a.code_row) *(uint32_t *)(crow + off) = w[i];
    }
  }
  return part;
}

// Pass 1: rotation of a panel pair, norms, search and pack; prod: residual norm partials.
template <int MB, bool PROD, bool F32IN>
__global__ __launch_bounds__(kTiledThreads, 2) void k_tiled_rot(const void *__restrict__ xin, TiledArgs a,
                                                                const u32x4 *__restrict__ img_all,
                                                                const uint32_t *__restrict__ cells,
                                                                const float *__restrict__ cent,
                                                                uint8_t *__restrict__ codes, float *__restrict__ norms,
                                                                int *__restrict__ rn_fix) {
  extern __shared__ u32x4 dyn_lds[];
  u32x4 *buf = dyn_lds;  // the unit buffer, then the cell table, then the codebook
  uint32_t *tab = (uint32_t *)((char *)dyn_lds + kUnitBytes);
  float *cent_lds = (float *)(tab + a.cell_words);
  const int pp = blockIdx.x, s = blockIdx.z, g = s % a.groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int panels = a.chunks;  // square blocks: as many output panels as contraction chunks
  const int p0 = a.pair * pp;
  const bool two = a.pair == 2 && p0 + 1 < panels;
  const u32x4 *img0 = img_all + ((size_t)g * panels + p0) * (size_t)a.chunks * kImageVec;
  const u32x4 *img1 = two ? img0 + (size_t)a.chunks * kImageVec : img0;

  for (int i = tid; i < a.cell_words; i += kTiledThreads) tab[i] = cells[i];
  if (PROD && MB > 0)
    for (int i = tid; i < (1 << MB); i += kTiledThreads) cent_lds[i] = cent[i];

  const int64_t set_row0 = (int64_t)s * a.n;
  int64_t v[2], row[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v[t] = (int64_t)blockIdx.y * kTiledVectors + 32 * wave + 16 * t + col;
    row[t] = set_row0 + (v[t] < a.n ? v[t] : a.n - 1);  // ragged tail: a valid row, results discarded
  }
  f32x4 acc[2][16];
  float nsq[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[t][m] = f32x4{0, 0, 0, 0};
  rotate_pair<F32IN, true>(xin, img0, img1, two, buf, a, row, wave, lane, grp, acc, nsq);

  const uint32_t tab_addr = lds_addr(tab);
  const uint32_t cent_addr = lds_addr(cent_lds);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float q2 = nsq[t];
    q2 += __shfl_xor(q2, 16);
    q2 += __shfl_xor(q2, 32);
    const float nu = __builtin_amdgcn_sqrtf(q2);
    const float inv = __builtin_amdgcn_rcpf(nu > 0.f ? nu : 1.f);
    const float sv = a.cell_scale * inv;
    const bool live = v[t] < a.n;
    uint8_t *crow = codes + (set_row0 + v[t]) * a.code_row;
    if (live && pp == 0 && grp == 0) norms[set_row0 + v[t]] = nu;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !two) break;
      float part = search_pack<MB, PROD>(&acc[t][8 * h], p0 + h, grp, nu, inv, sv, tab_addr, cent_addr, a, crow, live);
      if constexpr (PROD) {  // each panel's share in fixed point, so the sum does not depend on the order
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (live && grp == 0 && nu > 0.f) atomicAdd(rn_fix + set_row0 + v[t], (int)rintf(part * kFix));
      }
    }
  }
}

// Pass 2 (prod): signs of S x - nu M c[idx] for a pair of projection panels,
// K = d (codes) then d (x); pair 0 also turns the fixed-point residual norms
// into float32.
template <int MB, bool F32IN>
__global__ __launch_bounds__(kTiledThreads, 2) void k_tiled_sign(const void *__restrict__ xin, TiledArgs a,
                                                                 const u32x4 *__restrict__ img_all,
                                                                 const float *__restrict__ cent,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const float *__restrict__ norms,
                                                                 uint8_t *__restrict__ signs, float *__restrict__ rnorms) {
  extern __shared__ u32x4 dyn_lds[];
  u32x4 *buf = dyn_lds;  // the unit buffer, then the code-pair table
  u32x2 *lut = (u32x2 *)((char *)dyn_lds + kUnitBytes);
  const int pp = blockIdx.x, s = blockIdx.z, g = s % a.groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int panels = a.chunks;
  const int p0 = a.pair * pp;
  const bool two = a.pair == 2 && p0 + 1 < panels;
  // per panel: the S blocks of the chunks, then the M blocks
  const u32x4 *img0 = img_all + ((size_t)g * panels + p0) * (size_t)(2 * a.chunks) * kImageVec;
  const u32x4 *img1 = two ? img0 + (size_t)(2 * a.chunks) * kImageVec : img0;

  // code pair e (codes e % 2^MB, e / 2^MB) -> (bf16 hi parts, bf16 lo parts) of their centroids
  if (MB > 0)
    for (int e = tid; e < (1 << (2 * MB)); e += kTiledThreads) {
      const float c0 = cent[e & ((1 << MB) - 1)], c1 = cent[e >> MB];
      const uint32_t h = bf16x2(c0, c1);
      lut[e] = u32x2{h, bf16x2(c0 - bf16_lo(h), c1 - bf16_hi(h))};
    }

  const int64_t set_row0 = (int64_t)s * a.n;
  int64_t v[2], row[2];
  float nu[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v[t] = (int64_t)blockIdx.y * kTiledVectors + 32 * wave + 16 * t + col;
    row[t] = set_row0 + (v[t] < a.n ? v[t] : a.n - 1);
    nu[t] = norms[row[t]];
  }
  f32x4 acc[2][16];
  float dummy[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[t][m] = f32x4{0, 0, 0, 0};

  // M c[idx] over the code chunks, with B = c for coordinates 128 cc + 32 grp
  // + 8 k + e (the lane's 32 codes of the chunk): a table read per code pair
  // gives both elements' hi and lo parts.  Coordinates past d meet zero
  // columns; every K step of a code chunk holds coordinates of all four lane
  // groups, so no unit is skipped.  Each lane then scales its column (its
  // vector) by -nu, and S x accumulates on top.
  if constexpr (MB > 0) {
    const uint32_t lut_addr = lds_addr(lut);
    const u32x4 *cimg0 = img0 + (size_t)a.chunks * kImageVec, *cimg1 = img1 + (size_t)a.chunks * kImageVec;
    uint32_t cw[2][MB];
    for (int u = 0; u < 2 * a.chunks; ++u) {
      const int cc = u >> 1, kh = u & 1;
      if (u > 0) __syncthreads();  // every wave is done with the previous unit
      stage_unit(cimg0 + (size_t)cc * kImageVec, cimg1 + (size_t)cc * kImageVec, two, kh, buf, wave, lane);
      if (kh == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int64_t off = (int64_t)16 * cc * MB + 4 * grp * MB;
          const uint8_t *crow = codes + row[t] * a.code_row;
#pragma unroll
          for (int i = 0; i < MB; ++i)
            cw[t][i] = off + 4 * i < a.code_row ? *(const uint32_t *)(crow + off + 4 * i) : 0u;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // also orders the table writes before the first reads
      int frag_lane = lane;
      asm volatile("" : "+v"(frag_lane));
      mma_unit_ops<true>(buf, frag_lane, two, acc, [&](int kk, u32x4(&bh)[2], u32x4(&bl)[2]) {
        const int k = 2 * kh + kk;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // elements 2 i, 2 i + 1: codes 8 k + 2 i and 8 k + 2 i + 1
            const int bit = (8 * k + 2 * i) * MB, wi = bit >> 5, sh = bit & 31;
            uint32_t pi = cw[t][wi] >> sh;
            if (sh + 2 * MB > 32) pi |= cw[t][wi + 1] << (32 - sh);
            pi &= (1u << (2 * MB)) - 1;
            const u32x2 e = *(lds_u32x2 *)(uintptr_t)(lut_addr + 8 * pi);
            bh[t][i] = e[0];
            bl[t][i] = e[1];
          }
      });
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 16; ++m) acc[t][m] *= -nu[t];
    __syncthreads();  // every wave is done with the last code unit
  }
  // S x over the input chunks
  rotate_pair<F32IN, false>(xin, img0, img1, two, buf, a, row, wave, lane, grp, acc, dummy);

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool live = v[t] < a.n;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !two) break;
      const int p = p0 + h;
      uint32_t bits = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int proj = 128 * p + 32 * grp + j;
        if (proj < a.d && acc[t][8 * h + (j >> 2)][j & 3] >= 0.f) bits |= 1u << j;
      }
      const int64_t off = (int64_t)16 * p + 4 * grp;
      if (live && off < a.sign_row) *(uint32_t *)(signs + (set_row0 + v[t]) * a.sign_row + off) = bits;
    }
    if (live && pp == 0 && grp == 0) {
      const int fx = *(volatile int *)(rnorms + set_row0 + v[t]);  // written by pass 1 as fixed point
      rnorms[set_row0 + v[t]] = nu[t] > 0.f ? __builtin_amdgcn_sqrtf((float)fx / kFix) : 0.f;
    }
  }
}

__global__ void k_zero_words(int *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int MB, bool PROD, bool F32IN>
hipError_t run_tiled(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n, uint8_t *codes,
                     uint8_t *signs, float *norms, float *rnorms, hipStream_t st) {
  TiledArgs a;
  a.n = n;
  a.d = t.d;
  a.chunks = (t.d + 127) / 128;
  a.groups = t.groups;
  a.code_row = t.code_row;
  a.sign_row = t.sign_row;
  a.cell_scale = t.cell_scale * 0x1p-22f;
  a.cell_magic = 2.f + (float)t.cell_radius * 0x1p-22f;
  a.cell_last = 0x40000000u + 2u * (uint32_t)t.cell_radius;
  a.cell_words = MB > 0 ? 2 * (2 * t.cell_radius + 1) : 0;
  const int panels = a.chunks;
  const int64_t tiles = (n + kTiledVectors - 1) / kTiledVectors;
  // pairs of panels per workgroup halve the split work per MFMA; a launch with
  // fewer than about four rounds of workgroups keeps one panel each
  a.pair = (panels + 1) / 2 * tiles * n_sets >= 2048 ? 2 : 1;
  const dim3 grid((unsigned)((panels + a.pair - 1) / a.pair), (unsigned)tiles, (unsigned)n_sets);
  const size_t cent_bytes = 4 * (size_t)(1 << MB) > 64 ? 4 * (size_t)(1 << MB) : 64;  // the codebook
  const size_t lds1 = kUnitBytes + 4 * (size_t)a.cell_words + cent_bytes;
  hipError_t e = hipFuncSetAttribute((const void *)k_tiled_rot<MB, PROD, F32IN>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  if (e != hipSuccess) return e;
  if constexpr (PROD) {
    const int64_t cnt = n_sets * n;
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, (int *)rnorms, cnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_tiled_rot<MB, PROD, F32IN>), grid, dim3(kTiledThreads), lds1, st, x, a,
                     (const u32x4 *)t.tiled_rot, t.cells, t.cent, codes, norms, (int *)rnorms);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (PROD) {
    const size_t lds2 = kUnitBytes + (MB > 0 ? ((size_t)8 << (2 * MB)) : 0) + 64;  // the code-pair table
    e = hipFuncSetAttribute((const void *)k_tiled_sign<MB, F32IN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds2);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_tiled_sign<MB, F32IN>), grid, dim3(kTiledThreads), lds2, st, x, a,
                       (const u32x4 *)t.tiled_sign, t.cent, codes, norms, signs, rnorms);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_quant_tiled(const DeviceTables &t, const void *x, int dtype, int64_t n_sets, int64_t n,
                              uint8_t *codes, uint8_t *signs, float *norms, float *rnorms, hipStream_t st) {
  if (!t.tiled_rot || (t.variant == 1 && !t.tiled_sign) || t.d % 8 != 0 || t.mse_bits > 4 ||
      ((uintptr_t)x & 15u) || ((uintptr_t)codes & 3u) || ((uintptr_t)signs & 3u) ||
      (n + kTiledVectors - 1) / kTiledVectors > 65535 || n_sets > 65535)
    return hipErrorNotSupported;
  if (t.mse_bits > 0 && 2 * (2 * t.cell_radius + 1) * 4 > 48 * 1024) return hipErrorNotSupported;
  const bool prod = t.variant == 1, f32 = dtype == 0;
#define TQ_T(MB, P, F) \
  if (t.mse_bits == MB && prod == P && f32 == F) \
    return run_tiled<MB, P, F>(t, x, n_sets, n, codes, signs, norms, rnorms, st);
  TQ_T(0, true, false) TQ_T(0, true, true)
  TQ_T(1, false, false) TQ_T(1, false, true) TQ_T(1, true, false) TQ_T(1, true, true)
  TQ_T(2, false, false) TQ_T(2, false, true) TQ_T(2, true, false) TQ_T(2, true, true)
  TQ_T(3, false, false) TQ_T(3, false, true) TQ_T(3, true, false) TQ_T(3, true, true)
  TQ_T(4, false, false) TQ_T(4, false, true) TQ_T(4, true, false) TQ_T(4, true, true)
#undef TQ_T
  return hipErrorNotSupported;
}

}  // namespace tq
