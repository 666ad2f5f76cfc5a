// d = 128 kernels on gfx950 matrix cores.
//
// k_quant128: rotation y = Pi x as bf16 MFMA (Pi split into hi + lo bf16
//   parts, float32 accumulation; float32 inputs are split the same way), then
//   in registers: norm, branch-free boundary search against ||x|| t_k, bit
//   packing, and for TurboQuant_prod the residual y - ||x|| c[idx], its norm
//   and the signs of M r with M = S Pi^T (a second split-bf16 MFMA).
//   [ttakun] TurboQuant_mse / TurboQuant_prod; [tqnet] 实现步骤草图 (quant).
// k_logits128: scores float32 queries against packed keys.  Each workgroup
//   rotates/projects its queries once (Pi q, S q), keeps them as f16 hi/lo MFMA
//   B operands in registers, and streams keys: 3-bit (or 1..4-bit) code pairs
//   and sign nibbles are decoded through small LDS tables straight into f16 A
//   operands, and one f16 MFMA per 32 coordinates accumulates all query heads
//   of the set at once.  [admirer] 第二步; [tmdm] 双剑合璧 (QJL estimator).
//
// Lane layouts (16x16x32 MFMA, wave64): A operand lane l holds row l%16 and
// 8 contraction elements of group l/16; B operand lane l holds column l%16 and
// the same 8 contraction elements; the accumulator lane l holds column l%16,
// rows 4*(l/16) .. 4*(l/16)+3.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "device_common.h"
#include "fast128.h"
#include "kernels.h"

namespace tq {
namespace {


constexpr int D = 128;


struct QuantParams {
  float cell_scale;  // cells per unit of the normalised coordinate, times 2^-22
  int cell_words;    // words of the cell table: 2 (2 kCellRadius + 1)
};

constexpr uint32_t kCellCap = 2048;  // LDS bytes reserved for the cell table
// Adding 2 + kCellRadius 2^-22 to u * scale 2^-22 lands in [2, 4), where one
// float step is 2^-22: the float bits are those of 2.0 plus the cell number
// r + kCellRadius.  Shifted left by 3 the bits of 2.0 wrap to zero, so the
// bits times 8 plus the table offset are the entry's LDS address.
constexpr float kCellStep = 0x1p-22f;
constexpr float kCellMagic = 2.f + kCellRadius * kCellStep;
constexpr uint32_t kCellFirst = 0x40000000u;
constexpr uint32_t kCellLast = kCellFirst + 2 * kCellRadius;
static_assert((kCellFirst << 3) == 0u, "cell base must vanish in the address");


// Index #{k : t_k < u} of the rotated coordinate y = nu u by the cell table
// at LDS byte address `tab` (sv = scale 2^-22 / nu): round u * scale to a
// cell, read that cell's (boundary, count below) pair, and add one when
// y > nu t.  The clamp keeps any input, even a non-finite one, in the table.
__device__ __forceinline__ uint32_t cell_index(uint32_t tab, float y, float nu, float sv) {
  uint32_t g = __float_as_uint(fmaf(y, sv, kCellMagic));
  g = min(max(g, kCellFirst), kCellLast);  // one v_med3_u32
  const u32x2 e = *(lds_u32x2 *)(uintptr_t)((g << 3) + tab);
  const float dd = fmaf(nu, __uint_as_float(e[0]), -y);
  return e[1] + (__float_as_uint(dd) >> 31);
}

// Codebook entry c[idx] staged in LDS at byte address `cent`.
__device__ __forceinline__ float lds_centroid(uint32_t cent, uint32_t idx) {
  return *(lds_f32 *)(uintptr_t)(cent + 4 * idx);
}



template <int MB>
__device__ __forceinline__ void store_codes(uint8_t *p, const uint32_t *w) {
  if constexpr (MB == 1) {
    *(uint32_t *)p = w[0];
  } else if constexpr (MB == 2) {
    *(u32x2 *)p = u32x2{w[0], w[1]};
  } else if constexpr (MB == 3) {
    *(u32x3 *)p = u32x3{w[0], w[1], w[2]};
  } else if constexpr (MB == 4) {
    *(u32x4 *)p = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Input fragments of one 32-vector tile: lane (col, grp) holds vectors col and
// 16 + col, elements 32 k + 8 grp .. + 8 for K steps k (bf16 pairs, or raw
// float32 for float32 input).
template <bool F32IN>
struct XRegs {
  u32x4 v[2][4][F32IN ? 2 : 1];
};

template <bool F32IN>
__device__ __forceinline__ void load_x(XRegs<F32IN> &r, const void *xin, int64_t set_row0, int64_t n,
                                       int64_t v0, int col, int grp) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int64_t v = v0 + 16 * t + col;
    v = v < n ? v : n - 1;  // ragged tail: a valid row, results discarded
    const int64_t row = set_row0 + v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (!F32IN) {
        r.v[t][k][0] = *(const u32x4 *)((const uint16_t *)xin + row * D + 32 * k + 8 * grp);
      } else {
        const u32x4 *p = (const u32x4 *)((const float *)xin + row * D + 32 * k + 8 * grp);
        r.v[t][k][0] = p[0];
        r.v[t][k][1] = p[1];
      }
    }
  }
}

// Rotation of one 32-vector tile: acc[t][m] = rows 16 m .. 16 m + 15 of the
// permuted Pi (hi and lo bf16 fragments read from LDS) times column tile t.
// K steps outermost so that 16 independent accumulator chains interleave.
// Also returns ||x||^2 of the lane's two vectors from the Gram matrices of the
// same fragments (the A and B layouts coincide, so one fragment serves as both
// operands; the diagonal holds the squared norms).
template <bool F32IN>
__device__ __forceinline__ void rotate_tile(const XRegs<F32IN> &xr, const u32x4 *img, int frag_lane,
                                            f32x4 (&acc)[2][8], float (&nsq)[2], int col) {
  u32x4 bh[2][4], bl[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (!F32IN) {
        bh[t][k] = xr.v[t][k][0];
      } else {
        const f32x4 a = __builtin_bit_cast(f32x4, xr.v[t][k][0]);
        const f32x4 b = __builtin_bit_cast(f32x4, xr.v[t][k][1]);
        const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(f, bh[t][k], bl[t][k]);
      }
    }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0, 0, 0, 0};
  // Sixteen groups (K step k, row tiles 2 h, 2 h + 1) of four fragments; the
  // reads of group g + 1 are issued before the MFMAs of group g, so one LDS
  // round trip hides behind each group's MFMAs.
  u32x4 fa[2][4];
  auto read_group = [&](int buf, int g) {
    const int k = g >> 2, h = g & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = ((2 * h + i) * 4 + k) * 2;
      fa[buf][2 * i] = img[f * kFragVec + frag_lane];
      fa[buf][2 * i + 1] = img[(f + 1) * kFragVec + frag_lane];
    }
  };
  read_group(0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    if (g + 1 < 16) {
      read_group((g + 1) & 1, g + 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    const int k = g >> 2, h = g & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = 2 * h + i;
      const u32x4 ah = fa[g & 1][2 * i], al = fa[g & 1][2 * i + 1];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t][m] = mfma_bf16(ah, bh[t][k], acc[t][m]);
        acc[t][m] = mfma_bf16(al, bh[t][k], acc[t][m]);
        if constexpr (F32IN) acc[t][m] = mfma_bf16(ah, bl[t][k], acc[t][m]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, F32IN ? 12 : 8, 0);
  }
  // G[v][v] sits in lane 16 (v/4) + v, register v%4 (selected without branches)
  const int32_t m0 = -(col & 1), m1 = -((col >> 1) & 1);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 gm = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      gm = mfma_bf16(bh[t][k], bh[t][k], gm);
      if constexpr (F32IN) {
        gm = mfma_bf16(bh[t][k], bl[t][k], gm);
        gm = mfma_bf16(bl[t][k], bh[t][k], gm);
      }
    }
    const float mine = fsel(m1, fsel(m0, gm[3], gm[2]), fsel(m0, gm[1], gm[0]));
    nsq[t] = __shfl(mine, ((col >> 2) << 4) + col);
  }
}

#ifndef TQ_MSE3_TU
// One wave quantizes 32 vectors per iteration (two 16-column tiles) and
// prefetches the next tile's input; a workgroup of 8 waves shares the rotation
// image (and the QJL image) staged in LDS.
// 8 waves share the rotation image (and for prod the QJL image): 64 / 128 KB
// of LDS, 2 waves/SIMD.
template <bool PROD>
constexpr int quant_threads() { return 512; }

template <int MB, bool PROD, bool F32IN>
__global__ __launch_bounds__(quant_threads<PROD>(), 2) void k_quant128(
    const void *__restrict__ xin, int64_t n, int groups, const uint32_t *__restrict__ pi_img,
    const uint32_t *__restrict__ m_img, const uint32_t *__restrict__ cells,
    const float *__restrict__ cent, QuantParams qp,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ signs, float *__restrict__ norms,
    float *__restrict__ rnorms) {
  extern __shared__ u32x4 lds[];
  constexpr int kQuantThreads = quant_threads<PROD>();
  // LDS: rotation image, [QJL image], cell table, [codebook]
  constexpr uint32_t kTab = (PROD ? 2 : 1) * kImageVec * 16;
  const uint32_t tab_addr = lds_addr(lds) + kTab, cent_addr = tab_addr + kCellCap;
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int col = lane & 15, grp = lane >> 4;

  {
    const u32x4 *src = (const u32x4 *)(pi_img + (size_t)g * kImageWords);
    for (int i = tid; i < kImageVec; i += kQuantThreads) lds[i] = src[i];
    if constexpr (PROD) {
      const u32x4 *srcm = (const u32x4 *)(m_img + (size_t)g * kImageWords);
      for (int i = tid; i < kImageVec; i += kQuantThreads) lds[kImageVec + i] = srcm[i];
    }
    uint32_t *tab = (uint32_t *)((char *)lds + kTab);
    for (int i = tid; i < qp.cell_words; i += kQuantThreads) tab[i] = cells[i];
    if constexpr (PROD && MB > 0) {
      float *cl = (float *)((char *)lds + kTab + kCellCap);
      if (tid < (1 << MB)) cl[tid] = cent[tid];
    }
  }
  __syncthreads();

  const int64_t ntiles = (n + 31) / 32;
  const int64_t set_row0 = (int64_t)s * n;
  constexpr int kWaves = kQuantThreads / 64;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  int64_t tile = (int64_t)blockIdx.x * kWaves + wave;
  if (tile >= ntiles) return;  // no barrier follows

  // guard: some vectors of the tile may lie past n (only the last tile of a
  // set); full tiles store without a branch, which keeps the wait-count pass
  // from waiting for every store before the next tile's loads are used
  auto process = [&](const XRegs<F32IN> &xr, int64_t v0, bool guard) {
    // The images are re-read from LDS for every tile (an opaque offset keeps
    // the reads inside the loop; hoisted, 64 KB of fragments would not fit in
    // registers).
    int frag_lane = lane;
    asm volatile("" : "+v"(frag_lane));
    u32x4 rh[2][4], rl[2][4];
    float gam2[2], nus[2];
    f32x4 acc2[2][8];
    float nsq2[2];
    rotate_tile<F32IN>(xr, lds, frag_lane, acc2, nsq2, col);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4(&acc)[8] = acc2[t];
      const int64_t v = v0 + 16 * t + col;
      const float nu = __builtin_amdgcn_sqrtf(nsq2[t]);
      // a zero vector has y = 0, which every cell scale maps to the middle
      const float sv = qp.cell_scale * __builtin_amdgcn_rcpf(nu > 0.f ? nu : 1.f);
      uint32_t w[MB > 0 ? MB : 1];
#pragma unroll
      for (int i = 0; i < (MB > 0 ? MB : 1); ++i) w[i] = 0;
      float res[32];
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {  // coordinate 32 grp + j of the lane's vector
        const float y = acc[j >> 2][j & 3];
        if constexpr (MB > 0) {
          const uint32_t idx = cell_index(tab_addr, y, nu, sv);
          put_field<MB>(w, j, idx);
          if constexpr (PROD) res[j] = fmaf(-nu, lds_centroid(cent_addr, idx), y);
        } else {
          res[j] = y;
        }
        if constexpr (PROD) rs = fmaf(res[j], res[j], rs);
      }
      if (!guard || v < n) {
        const int64_t row = set_row0 + v;
        if constexpr (MB > 0) store_codes<MB>(codes + row * (16 * MB) + grp * (4 * MB), w);
        if (grp == 0) norms[row] = nu;
      }
      if constexpr (PROD) {
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        gam2[t] = rs;
        nus[t] = nu;
#pragma unroll
        for (int k = 0; k < 4; ++k) split8(&res[8 * k], rh[t][k], rl[t][k]);
      }
    }
    if constexpr (PROD) {
      // QJL: p = M r (rows permuted like the rotation, K in lane-chunk order).
      // Each M fragment is read once for both column tiles; the M image has
      // its own base so every read's offset fits the instruction's immediate.
      // Sign bits go into a shift register (one alignbit per projection,
      // projections 31 .. 0), holding 1 for p < 0.
      int mfl = lane + kImageVec;
      asm volatile("" : "+v"(mfl));
      uint32_t neg[2] = {0u, 0u};
      u32x4 fm[2][8];
      f32x4 pa[2][2];
      auto read_tile = [&](int buf, int m) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int f = (m * 4 + k) * 2;
          fm[buf][2 * k] = lds[f * kFragVec + mfl];
          fm[buf][2 * k + 1] = lds[(f + 1) * kFragVec + mfl];
        }
      };
      read_tile(0, 7);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i <= 8; ++i) {
        if (i < 8) {  // row tile m = 7 - i
          if (i + 1 < 8) {
            read_tile((i + 1) & 1, 6 - i);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          }
          f32x4(&p)[2] = pa[i & 1];
          p[0] = f32x4{0, 0, 0, 0};
          p[1] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const u32x4 ah = fm[i & 1][2 * k], al = fm[i & 1][2 * k + 1];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              p[t] = mfma_bf16(ah, rh[t][k], p[t]);
              p[t] = mfma_bf16(ah, rl[t][k], p[t]);
              p[t] = mfma_bf16(al, rh[t][k], p[t]);
            }
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
        }
        if (i > 0) {  // signs of row tile 8 - i, whose MFMAs were issued one step earlier
          const f32x4(&p)[2] = pa[(i - 1) & 1];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int q = 3; q >= 0; --q) neg[t] = __builtin_amdgcn_alignbit(neg[t], __float_as_uint(p[t][q]), 31);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t v = v0 + 16 * t + col;
        if (!guard || v < n) {
          const int64_t row = set_row0 + v;
          ((uint32_t *)(signs + row * 16))[grp] = ~neg[t];
          if (grp == 0) rnorms[row] = nus[t] > 0.f ? sqrtf(gam2[t]) / nus[t] : 0.f;
        }
      }
    }
  };

  const int64_t nfull = n / 32;  // tiles whose 32 vectors all exist
  if constexpr (F32IN) {
    // float32 input (not the bandwidth-critical path): no prefetch
    XRegs<F32IN> xr;
    for (; tile < nfull; tile += stride) {
      load_x<F32IN>(xr, xin, set_row0, n, tile * 32, col, grp);
      process(xr, tile * 32, false);
    }
  } else if (tile < nfull) {
    // the next tile's input is loaded unconditionally (past the last full
    // tile it re-reads the current one) so no branch sits between load and use
    XRegs<F32IN> xa, xb;
    load_x<F32IN>(xa, xin, set_row0, n, tile * 32, col, grp);
    while (true) {
      int64_t nxt = tile + stride;
      bool more = nxt < nfull;
      load_x<F32IN>(xb, xin, set_row0, n, (more ? nxt : tile) * 32, col, grp);
      process(xa, tile * 32, false);
      tile = nxt;
      if (!more) break;
      nxt = tile + stride;
      more = nxt < nfull;
      load_x<F32IN>(xa, xin, set_row0, n, (more ? nxt : tile) * 32, col, grp);
      process(xb, tile * 32, false);
      tile = nxt;
      if (!more) break;
    }
  }
  if (tile == nfull && tile < ntiles) {  // the set's partial last tile, if this wave has it
    XRegs<F32IN> xr;
    load_x<F32IN>(xr, xin, set_row0, n, tile * 32, col, grp);
    process(xr, tile * 32, true);
  }
}


#endif  // TQ_MSE3_TU

// TurboQuant_mse of bfloat16 input with the rotation held in registers.  One
// wave per SIMD (a 256-thread workgroup per CU) leaves each wave 512
// registers: all 64 hi/lo fragments of Pi live in its 256 AGPRs, which the
// MFMAs read directly, so LDS carries only the 2 KB cell table.  Each wave
// runs a software pipeline over 16-vector stages: while the MFMAs rotate
// stage i+1, the vector ALU searches and packs stage i, and the inputs of
// stages i+2 .. i+kMseDepth-1 are in flight.
constexpr int kMseThreads = 256;
constexpr int kMseDepth = 4;  // input stages held in registers

// Input fragments of one 16-vector stage: lane (col, grp) holds vector col,
// elements 32 k + 8 grp .. + 8 (bf16 pairs) for K steps k.
struct XStage {
  u32x4 v[4];
};

__device__ __forceinline__ void load_stage(XStage &r, const uint16_t *xin, int64_t set_row0, int64_t n,
                                           int64_t v0, int col, int grp) {
  int64_t v = v0 + col;
  v = v < n ? v : n - 1;  // ragged tail or a padding stage: a valid row, results discarded
  const uint16_t *p = xin + (set_row0 + v) * D + 8 * grp;
#pragma unroll
  for (int k = 0; k < 4; ++k) r.v[k] = *(const u32x4 *)(p + 32 * k);
}

// acc[m] = rows 16 m .. 16 m + 15 of the permuted Pi times the stage; nsq =
// ||x||^2 of the lane's vector from the Gram diagonal.
__device__ __forceinline__ void rotate_stage(const XStage &x, const u32x4 (&im)[64], f32x4 (&acc)[8],
                                             float &nsq, int col) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      acc[m] = mfma_bf16(im[(m * 4 + k) * 2], x.v[k], acc[m]);
      acc[m] = mfma_bf16(im[(m * 4 + k) * 2 + 1], x.v[k], acc[m]);
    }
  f32x4 gm = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k) gm = mfma_bf16(x.v[k], x.v[k], gm);
  const int32_t m0 = -(col & 1), m1 = -((col >> 1) & 1);
  const float mine = fsel(m1, fsel(m0, gm[3], gm[2]), fsel(m0, gm[1], gm[0]));
  nsq = __shfl(mine, ((col >> 2) << 4) + col);
}


// The search of one stage in two halves, so that the MFMAs of the next stage
// run between them and cover the LDS latency: first the 32 cell reads, then
// the comparisons, packing and stores.
struct StageCells {
  u32x2 e[32];
  float nu, sv;
};

__device__ __forceinline__ void lookup_stage(const f32x4 (&acc)[8], float nsq, uint32_t tab_addr,
                                             float cell_scale, StageCells &c) {
  c.nu = __builtin_amdgcn_sqrtf(nsq);
  c.sv = cell_scale * __builtin_amdgcn_rcpf(c.nu > 0.f ? c.nu : 1.f);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    uint32_t g = __float_as_uint(fmaf(acc[j >> 2][j & 3], c.sv, kCellMagic));
    g = min(max(g, kCellFirst), kCellLast);
    c.e[j] = *(lds_u32x2 *)(uintptr_t)((g << 3) + tab_addr);
  }
}

template <int MB>
__device__ __forceinline__ void pack_stage(const f32x4 (&acc)[8], const StageCells &c, int64_t v,
                                           int64_t n, int grp, __amdgpu_buffer_rsrc_t rc,
                                           __amdgpu_buffer_rsrc_t rn) {
  uint32_t w[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) w[i] = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float y = acc[j >> 2][j & 3];
    const float dd = fmaf(c.nu, __uint_as_float(c.e[j][0]), -y);
    put_field<MB>(w, j, c.e[j][1] + (__float_as_uint(dd) >> 31));
  }
  const uint32_t off = v < n ? (uint32_t)v * (16 * MB) + grp * (4 * MB) : kDropped;
  if constexpr (MB == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rc, off, 0, 0);
  } else if constexpr (MB == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rc, off, 0, 0);
  } else if constexpr (MB == 3) {
    __builtin_amdgcn_raw_buffer_store_b96(u32x3{w[0], w[1], w[2]}, rc, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rc, off, 0, 0);
  }
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c.nu), rn,
                                        v < n && grp == 0 ? (uint32_t)v * 4 : kDropped, 0, 0);
}

template <int MB>
__global__ __launch_bounds__(kMseThreads, 1) void k_quant128_mse(
    const uint16_t *__restrict__ xin, int64_t n, int groups, const u32x4 *__restrict__ pi_img,
    const uint32_t *__restrict__ cells, float cell_scale, uint8_t *__restrict__ codes,
    float *__restrict__ norms) {
  constexpr int kCellWords = 2 * (2 * kCellRadius + 1);
  __shared__ uint32_t tab[kCellWords];
  __shared__ u32x4 img[kImageVec];  // staging: each CU reads the image from L2 once
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  for (int i = tid; i < kCellWords; i += kMseThreads) tab[i] = cells[i];

  // stages of this wave: tile0 + k stride, k = 0 .. count - 1 (32-bit: the
  // host guarantees n_sets n < 2^31); all of it is wave-uniform scalar work
  const int ntiles = (int)((n + 15) / 16);
  const int64_t set_row0 = (int64_t)s * n;
  constexpr int kWaves = kMseThreads / 64;
  const int stride = (int)gridDim.x * kWaves;
  const int tile0 = (int)blockIdx.x * kWaves + wave;
  const int count = __builtin_amdgcn_readfirstlane(tile0 < ntiles ? (ntiles - tile0 + stride - 1) / stride : 0);
  // first row of stage k; stages past the end read the last stage again and
  // store nothing
  auto row0 = [&](int k) { return (int64_t)(tile0 + min(k, count - 1) * stride) * 16; };
  auto valid_row0 = [&](int k) { return k < count ? (int64_t)(tile0 + k * stride) * 16 : n; };

  // the image first (every stage needs all of it), then the first inputs
  {
    const u32x4 *src = pi_img + (size_t)g * kImageVec;
    u32x4 t[kImageVec / kMseThreads];
#pragma unroll
    for (int i = 0; i < kImageVec / kMseThreads; ++i) t[i] = src[i * kMseThreads + tid];
#pragma unroll
    for (int i = 0; i < kImageVec / kMseThreads; ++i) img[i * kMseThreads + tid] = t[i];
  }
  XStage xs[kMseDepth];
#pragma unroll
  for (int j = 0; j + 1 < kMseDepth; ++j) load_stage(xs[j], xin, set_row0, n, row0(j), col, grp);
  __syncthreads();
  u32x4 im[64];
#pragma unroll
  for (int f = 0; f < 64; ++f) {
    im[f] = img[f * kFragVec + lane];
    asm volatile("" : "+a"(im[f]));  // keep the fragment in an AGPR
  }
  if (count == 0) return;  // no barrier follows
  const uint32_t tab_addr = lds_addr(tab);

  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(codes + set_row0 * (16 * MB), 0, (int)(n * (16 * MB)), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rn =
      __builtin_amdgcn_make_buffer_rsrc(norms + set_row0, 0, (int)(n * 4), kBufferFlags);
  f32x4 acc[2][8];
  float nsq[2];
  rotate_stage(xs[0], im, acc[0], nsq[0], col);
  for (int k0 = 0; k0 < count; k0 += kMseDepth) {
#pragma unroll
    for (int j = 0; j < kMseDepth; ++j) {
      const int k = k0 + j;
      // refill the buffer that stage k used; look up stage k's cells; rotate
      // stage k + 1; finish stage k
      load_stage(xs[(j + kMseDepth - 1) % kMseDepth], xin, set_row0, n, row0(k + kMseDepth - 1), col, grp);
      StageCells cells;
      lookup_stage(acc[j & 1], nsq[j & 1], tab_addr, cell_scale, cells);
      rotate_stage(xs[(j + 1) % kMseDepth], im, acc[(j + 1) & 1], nsq[(j + 1) & 1], col);
      pack_stage<MB>(acc[j & 1], cells, valid_row0(k) + col, n, grp, rc, rn);
    }
  }
}

#ifndef TQ_MSE3_TU
// ------------------------------------------------ mixed precision, d = 128 --
// Outlier-channel mixed precision with a 64 + 64 channel split, TurboQuant_mse
// of bf16 input in one pass.  [tqnet] 从工程视角看 TurboQuant 到底改变了什么
// (outlier channels kept at a higher bit width); [tqnet] 数据就是论据 › KV
// Cache 压缩基准 (2.5 and 3.5 bits per channel).  The channel split and both
// parts' rotations form one 128 x 128 image per group -- rows of Pi_o on the
// outlier channels and of Pi_r on the others, zero elsewhere -- ordered so
// that row tiles 0..3 give lane group g the outlier part's coordinates 16 g ..
// 16 g + 15 and tiles 4..7 the regular part's.  The parts' norms are the
// diagonals of two Gram products with the input masked to each part's
// channels; each part is searched in its own cell table and packed at its own
// width.  The pipeline is that of k_quant128_mse.
struct MixCells {
  u32x2 e[32];  // cells of the outlier part's 16 coordinates, then the regular part's
  float nu[2], sv[2];
};

// acc[m] = rows 16 m .. 16 m + 15 of the mixed image times the stage; nsq[p]
// = squared norm of part p of the lane's vector (mo: outlier-channel masks of
// the B-operand elements).
__device__ __forceinline__ void rotate_mixed(const XStage &x, const u32x4 (&im)[64], const u32x4 (&mo)[4],
                                             f32x4 (&acc)[8], float (&nsq)[2], int col) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      acc[m] = mfma_bf16(im[(m * 4 + k) * 2], x.v[k], acc[m]);
      acc[m] = mfma_bf16(im[(m * 4 + k) * 2 + 1], x.v[k], acc[m]);
    }
  f32x4 go = {0, 0, 0, 0}, gr = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    go = mfma_bf16(x.v[k] & mo[k], x.v[k], go);
    gr = mfma_bf16(x.v[k] & ~mo[k], x.v[k], gr);
  }
  const int32_t m0 = -(col & 1), m1 = -((col >> 1) & 1);
  const int src = ((col >> 2) << 4) + col;
  nsq[0] = __shfl(fsel(m1, fsel(m0, go[3], go[2]), fsel(m0, go[1], go[0])), src);
  nsq[1] = __shfl(fsel(m1, fsel(m0, gr[3], gr[2]), fsel(m0, gr[1], gr[0])), src);
}

__device__ __forceinline__ void lookup_mixed(const f32x4 (&acc)[8], const float (&nsq)[2], uint32_t tab_o,
                                             uint32_t tab_r, float scale_o, float scale_r, MixCells &c) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    c.nu[p] = __builtin_amdgcn_sqrtf(nsq[p]);
    c.sv[p] = (p == 0 ? scale_o : scale_r) * __builtin_amdgcn_rcpf(c.nu[p] > 0.f ? c.nu[p] : 1.f);
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int p = j >> 4, jj = j & 15;
    uint32_t g = __float_as_uint(fmaf(acc[4 * p + (jj >> 2)][jj & 3], c.sv[p], kCellMagic));
    g = min(max(g, kCellFirst), kCellLast);
    c.e[j] = *(lds_u32x2 *)(uintptr_t)((g << 3) + (p == 0 ? tab_o : tab_r));
  }
}

// Part p of the lane's vector: the 16 decisions, packed at MB bits into bytes
// 2 MB grp .. of the part's row (row bytes per vector; a row longer than 8 MB
// bytes has 8 bytes of padding, written as zero by lane group 0), and the
// part's norm.
template <int MB>
__device__ __forceinline__ void pack_mixed(const f32x4 (&acc)[8], int p, const MixCells &c, int64_t v, int64_t n,
                                           int grp, int64_t row, __amdgpu_buffer_rsrc_t rc,
                                           __amdgpu_buffer_rsrc_t rn) {
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float y = acc[4 * p + (jj >> 2)][jj & 3];
    const float dd = fmaf(c.nu[p], __uint_as_float(c.e[16 * p + jj][0]), -y);
    put_field<MB>(w, jj, c.e[16 * p + jj][1] + (__float_as_uint(dd) >> 31));
  }
  const bool ok = v < n;
  const uint32_t base = ok ? (uint32_t)(v * row) : kDropped;  // kDropped + a few bytes is still past the set
  const uint32_t at = base + 2 * MB * grp;
  if constexpr (MB == 1) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w[0], rc, at, 0, 0);
  } else if constexpr (MB == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rc, at, 0, 0);
  } else if constexpr (MB == 3) {
    // 6 bytes at 6 grp: 4 + 2 (grp even) or 2 + 4 (grp odd), so every store is aligned
    const bool even = (grp & 1) == 0;
    const uint32_t a = even ? w[0] : (w[0] & 0xFFFFu);
    const uint32_t b = even ? (w[1] & 0xFFFFu) : ((w[0] >> 16) | (w[1] << 16));
    if (even) {
      __builtin_amdgcn_raw_buffer_store_b32(a, rc, at, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b, rc, at + 4, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)a, rc, at, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(b, rc, at + 2, 0, 0);
    }
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rc, at, 0, 0);
  }
  if (row > 8 * MB)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rc, ok && grp == 0 ? base + 8 * MB : kDropped, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c.nu[p]), rn, ok && grp == 0 ? (uint32_t)v * 4 : kDropped,
                                        0, 0);
}

template <int MBO, int MBR>
__global__ __launch_bounds__(kMseThreads, 1) void k_quant128_mixed(
    const uint16_t *__restrict__ xin, int64_t n, int groups, const u32x4 *__restrict__ img_all,
    const uint32_t *__restrict__ masks, const uint32_t *__restrict__ cells_o, float scale_o,  // scales times 2^-22
    const uint32_t *__restrict__ cells_r, float scale_r, uint8_t *__restrict__ codes_o, int64_t row_o,
    uint8_t *__restrict__ codes_r, int64_t row_r, float *__restrict__ norms_o, float *__restrict__ norms_r) {
  constexpr int kCellWords = 2 * (2 * kCellRadius + 1);
  __shared__ uint32_t tab[2][kCellWords];
  __shared__ u32x4 img[kImageVec];  // staging: each CU reads the image from L2 once
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  for (int i = tid; i < kCellWords; i += kMseThreads) {
    tab[0][i] = cells_o[i];
    tab[1][i] = cells_r[i];
  }
  const int ntiles = (int)((n + 15) / 16);
  const int64_t set_row0 = (int64_t)s * n;
  constexpr int kWaves = kMseThreads / 64;
  const int stride = (int)gridDim.x * kWaves;
  const int tile0 = (int)blockIdx.x * kWaves + wave;
  const int count = __builtin_amdgcn_readfirstlane(tile0 < ntiles ? (ntiles - tile0 + stride - 1) / stride : 0);
  auto row0 = [&](int k) { return (int64_t)(tile0 + min(k, count - 1) * stride) * 16; };
  auto valid_row0 = [&](int k) { return k < count ? (int64_t)(tile0 + k * stride) * 16 : n; };
  {
    const u32x4 *src = img_all + (size_t)g * kImageVec;
    u32x4 t[kImageVec / kMseThreads];
#pragma unroll
    for (int i = 0; i < kImageVec / kMseThreads; ++i) t[i] = src[i * kMseThreads + tid];
#pragma unroll
    for (int i = 0; i < kImageVec / kMseThreads; ++i) img[i * kMseThreads + tid] = t[i];
  }
  XStage xs[kMseDepth];
#pragma unroll
  for (int j = 0; j + 1 < kMseDepth; ++j) load_stage(xs[j], xin, set_row0, n, row0(j), col, grp);
  // outlier-channel masks of the lane's B-operand elements 32 k + 8 grp + e
  u32x4 mo[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t word = masks[4 * g + k] >> (8 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mo[k][i] = ((word >> (2 * i)) & 1u ? 0x0000FFFFu : 0u) | ((word >> (2 * i + 1)) & 1u ? 0xFFFF0000u : 0u);
  }
  __syncthreads();
  u32x4 im[64];
#pragma unroll
  for (int f = 0; f < 64; ++f) {
    im[f] = img[f * kFragVec + lane];
    asm volatile("" : "+a"(im[f]));  // keep the fragment in an AGPR
  }
  if (count == 0) return;  // no barrier follows
  const uint32_t tab_o = lds_addr(tab[0]), tab_r = lds_addr(tab[1]);
  const __amdgpu_buffer_rsrc_t rco =
      __builtin_amdgcn_make_buffer_rsrc(codes_o + set_row0 * row_o, 0, (int)(n * row_o), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rcr =
      __builtin_amdgcn_make_buffer_rsrc(codes_r + set_row0 * row_r, 0, (int)(n * row_r), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rno =
      __builtin_amdgcn_make_buffer_rsrc(norms_o + set_row0, 0, (int)(n * 4), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rnr =
      __builtin_amdgcn_make_buffer_rsrc(norms_r + set_row0, 0, (int)(n * 4), kBufferFlags);
  f32x4 acc[2][8];
  float nsq[2][2];
  rotate_mixed(xs[0], im, mo, acc[0], nsq[0], col);
  for (int k0 = 0; k0 < count; k0 += kMseDepth) {
#pragma unroll
    for (int j = 0; j < kMseDepth; ++j) {
      const int k = k0 + j;
      load_stage(xs[(j + kMseDepth - 1) % kMseDepth], xin, set_row0, n, row0(k + kMseDepth - 1), col, grp);
      MixCells cells;
      lookup_mixed(acc[j & 1], nsq[j & 1], tab_o, tab_r, scale_o, scale_r, cells);
      rotate_mixed(xs[(j + 1) % kMseDepth], im, mo, acc[(j + 1) & 1], nsq[(j + 1) & 1], col);
      const int64_t v = valid_row0(k) + col;
      pack_mixed<MBO>(acc[j & 1], 0, cells, v, n, grp, row_o, rco, rno);
      pack_mixed<MBR>(acc[j & 1], 1, cells, v, n, grp, row_r, rcr, rnr);
    }
  }
}

// ---------------------------------------------------------------- logits --
constexpr int kLogitTiles = 4;     // 16-key tiles per wave iteration
constexpr int kLogitThreads = 1024;  // 16 waves share one set of decode tables
constexpr int kLogitWaves = kLogitThreads / 64;

// Per-wave registers of KT 16-key tiles: lane (col, grp) holds key col of each
// tile -- the code words of its coordinates 32 grp .. 32 grp + 31, the sign
// word of the same projections, and the key's norm and residual norm.
template <int CW>
struct KeyRegs {
  uint32_t cw[kLogitTiles][CW > 0 ? CW : 1];
  uint32_t sw[kLogitTiles];
  float nv[kLogitTiles], gv[kLogitTiles];
};

// Largest key count one launch of the fused kernels addresses: every byte
// offset into a key array (key index times at most 64 bytes per row) stays
// below 2^31.  The logits take longer sets in chunks of this many keys.
constexpr int64_t kFusedMaxKeys = int64_t(1) << 25;

// Heads per logits launch: the output rows of a set's heads h0 .. h0 + hp -
// 1 are addressed with 32-bit byte offsets, so hp n_keys 4 < 2^31 (8, the
// kernel's head slots, below 2^26 keys; fewer above).  0: too many keys.
static int logit_heads_per_launch(int64_t n_keys) {
  int hp = 8;
  while (hp > 0 && hp * n_keys * 4 >= (int64_t)kDropped) hp >>= 1;
  return hp;
}

// Key ranges per workgroup for a launch over n keys of n_sets sets: about
// one workgroup per CU overall, a whole number of iterations `unit` each.
static int64_t logit_grid_x(int64_t n_sets, int64_t n, int64_t unit, int64_t *kpw) {
  int64_t gx = (256 + n_sets - 1) / n_sets;
  const int64_t max_gx = (n + unit - 1) / unit;
  if (gx > max_gx) gx = max_gx;
  if (gx < 1) gx = 1;
  int64_t k = (n + gx - 1) / gx;
  k = (k + unit - 1) / unit * unit;
  *kpw = k;
  return (n + k - 1) / k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t set_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferFlags);
}

// Buffer resources of one set's key arrays and the lane's fixed byte offsets
// (lane (col, grp): codes and signs of key col, coordinates 32 grp .. 32 grp
// + 31; the norms of key col).
struct KeyRsrc {
  __amdgpu_buffer_rsrc_t c, s, n, g;
  uint32_t oc, os, on;
};

template <int CW>
__device__ __forceinline__ void buffer_codes(uint32_t *w, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t so) {
  if constexpr (CW == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, so, 0);
  } else if constexpr (CW == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, so, 0);
    w[0] = v[0];
    w[1] = v[1];
  } else if constexpr (CW == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, so, 0);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
  } else if constexpr (CW == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, so, 0);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
}

// Keys t0 + 16 u + col (t0 wave-uniform, an index into the set): the lane's
// offsets plus constants, t0 times the row size as the scalar offset.  TAIL:
// keys at or past kend are replaced by key t0 (always valid).
template <int CW, bool PROD, int KT, bool TAIL>
__device__ __forceinline__ void load_keys(KeyRegs<CW> &r, int64_t t0, int64_t kend, int col, const KeyRsrc &k) {
  const uint32_t k0 = (uint32_t)t0;
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const bool ok = !TAIL || t0 + 16 * u + col < kend;
    const uint32_t du = ok ? (uint32_t)(16 * u) : 0u, cu = ok ? 0u : (uint32_t)col;
    if constexpr (CW > 0) buffer_codes<CW>(r.cw[u], k.c, k.oc + du * (16 * CW) - cu * (16 * CW), k0 * (16 * CW));
    if constexpr (PROD) r.sw[u] = __builtin_amdgcn_raw_buffer_load_b32(k.s, k.os + du * 16 - cu * 16, k0 * 16, 0);
    const uint32_t noff = k.on + du * 4 - cu * 4;
    r.nv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(k.n, noff, k0 * 4, 0));
    if constexpr (PROD) r.gv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(k.g, noff, k0 * 4, 0));
  }
}

// ---------------------------------------------------------- dequantize --
// x = nu Pi^T c[idx] (mse) and x = nu (Pi^T c[idx] + sqrt(pi/2)/d gamma S^T z)
// (prod) as f16 MFMAs: the A operands are f16 hi/lo images of Pi^T and S^T
// staged in LDS (output coordinates in natural order, contraction in
// lane-chunk order), the B operands the decoded codes (alpha c, two per table
// read) and signs (+1/-1, eight per read) of 16 vectors.  Lane (vector, g)
// ends with coordinates 16 m + 4 g .. + 3 of row tiles m = 0..7 and writes
// them as eight 16-byte stores: per instruction the four lanes of a vector
// cover one contiguous 64-byte run.  [tqnet] 实现步骤草图 (dequant: inverse rotation of
// the centroids); [ttakun] TurboQuant_prod (residual reconstruction).
constexpr int kDqThreads = 512;
constexpr int kDqCodeCopies = 16;  // u32 entries; the copy is the low lane bits
constexpr int kDqSignCopies = 4;   // u32x4 entries

template <int MB>
struct DqGeom {
  static constexpr int W = 2 * MB;                               // two codes per read
  static constexpr int SHIFT = 6;                                // log2(4 kDqCodeCopies)
  static constexpr uint32_t CODE_BYTES = MB > 0 ? (1u << W) * kDqCodeCopies * 4 : 0;
  static constexpr uint32_t SIGN_OFF = CODE_BYTES;
  static constexpr uint32_t SIGN_BYTES = 256 * kDqSignCopies * 16;
  static constexpr uint32_t IMG_OFF = SIGN_OFF + SIGN_BYTES;
};

template <int MB, bool PROD>
__global__ __launch_bounds__(kDqThreads, 1) void k_dequant128(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ signs, const float *__restrict__ norms,
    const float *__restrict__ rnorms, int64_t n, int groups, const u32x4 *__restrict__ pi_img,
    const u32x4 *__restrict__ s_img, const uint32_t *__restrict__ lut, float inv_alpha, float *__restrict__ out) {
  using GQ = DqGeom<MB>;
  constexpr int CW = MB;
  extern __shared__ u32x4 dyn_lds[];  // the kernel's only LDS: starts at address 0
  uint32_t *t_code = (uint32_t *)dyn_lds;
  u32x4 *t_sg = (u32x4 *)((char *)dyn_lds + GQ::SIGN_OFF);
  u32x4 *img = (u32x4 *)((char *)dyn_lds + GQ::IMG_OFF);
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;

  if constexpr (MB > 0)
    for (int e = tid; e < (1 << GQ::W) * kDqCodeCopies; e += kDqThreads) t_code[e] = lut[e / kDqCodeCopies];
  if constexpr (PROD)
    for (int e = tid; e < 256 * kDqSignCopies; e += kDqThreads)
      t_sg[e] = ((const u32x4 *)(lut + (MB > 0 ? (1 << GQ::W) : 0)))[e / kDqSignCopies];
  if constexpr (MB > 0)
    for (int i = tid; i < kImageVec; i += kDqThreads) img[i] = pi_img[(size_t)g * kImageVec + i];
  if constexpr (PROD)
    for (int i = tid; i < kImageVec; i += kDqThreads)
      img[(MB > 0 ? kImageVec : 0) + i] = s_img[(size_t)g * kImageVec + i];
  __syncthreads();

  const int64_t ntiles = (n + 31) / 32;
  const int64_t set_row0 = (int64_t)s * n;
  constexpr int kWaves = kDqThreads / 64;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(out + set_row0 * D, 0, (int)(n * D * 4), kBufferFlags);
  const uint32_t code_base = 4 * (lane & (kDqCodeCopies - 1));
  const uint32_t sign_base = 16 * (lane & (kDqSignCopies - 1));
  const float qjl = kQjlScale / (float)D;

  // codes, signs and norms through buffer resources (vectors past n read
  // zeros; their stores are dropped), one tile ahead in a ping-pong pair of
  // register sets
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(MB > 0 ? codes + set_row0 * (16 * CW) : codes), 0, MB > 0 ? (int)(n * (16 * CW)) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(PROD ? signs + set_row0 * 16 : signs), 0, PROD ? (int)(n * 16) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rn =
      __builtin_amdgcn_make_buffer_rsrc((void *)(norms + set_row0), 0, (int)(n * 4), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(PROD ? rnorms + set_row0 : rnorms), 0, PROD ? (int)(n * 4) : 0, kBufferFlags);
  struct DqRegs {
    uint32_t cw[2][CW > 0 ? CW : 1], sw[2];
    float nu[2], ga[2];
  };
  auto dq_load = [&](DqRegs &r, int64_t tile) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t v = (uint32_t)(tile * 32 + 16 * t + col);
      if constexpr (MB > 0) {
        const uint32_t off = v * (16 * CW) + grp * (4 * CW);
        if constexpr (CW == 1) {
          r.cw[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0);
        } else if constexpr (CW == 2) {
          const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
          r.cw[t][0] = w[0];
          r.cw[t][1] = w[1];
        } else if constexpr (CW == 3) {
          const u32x3 w = __builtin_amdgcn_raw_buffer_load_b96(rc, off, 0, 0);
          r.cw[t][0] = w[0];
          r.cw[t][1] = w[1];
          r.cw[t][2] = w[2];
        } else {
          const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
          r.cw[t][0] = w[0];
          r.cw[t][1] = w[1];
          r.cw[t][2] = w[2];
          r.cw[t][3] = w[3];
        }
      }
      if constexpr (PROD) r.sw[t] = __builtin_amdgcn_raw_buffer_load_b32(rs, v * 16 + grp * 4, 0, 0);
      r.nu[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, v * 4, 0, 0));
      r.ga[t] = PROD ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, v * 4, 0, 0)) : 0.f;
    }
  };
  auto dq_tile = [&](const DqRegs &r, int64_t tile) __attribute__((always_inline)) {
    int frag_lane = lane;
    asm volatile("" : "+v"(frag_lane));
    f32x4 acc[2][8];
    float scale_c[2], scale_s[2];
    const auto &cw = r.cw;
    const auto &sw = r.sw;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      scale_c[t] = r.nu[t] * inv_alpha;
      scale_s[t] = PROD ? r.nu[t] * qjl * r.ga[t] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0, 0, 0, 0};
    }
    if constexpr (MB > 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4 bc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * k + jj;  // code pair j of the lane's 32 coordinates
            const int bit = j * GQ::W, wi = bit >> 5, sh = bit & 31;
            uint32_t x;
            if (sh + GQ::W > 32)
              x = __builtin_amdgcn_alignbit(cw[t][wi + 1], cw[t][wi], sh - GQ::SHIFT);
            else if (sh >= GQ::SHIFT)
              x = cw[t][wi] >> (sh - GQ::SHIFT);
            else
              x = cw[t][wi] << (GQ::SHIFT - sh);
            const uint32_t addr = (x & (uint32_t)(((1 << GQ::W) - 1) << GQ::SHIFT)) | code_base;
            bc[t][jj] = *(__attribute__((address_space(3))) const uint32_t *)(uintptr_t)addr;
          }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int f = (m * 4 + k) * 2;
          const u32x4 ah = img[f * kFragVec + frag_lane];
          const u32x4 al = img[(f + 1) * kFragVec + frag_lane];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            acc[t][m] = mfma_f16(ah, bc[t], acc[t][m]);
            acc[t][m] = mfma_f16(al, bc[t], acc[t][m]);
          }
        }
      }
    }
    // the code part is scaled now, so the sign part accumulates on top of it
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[t][m] *= scale_c[t];
    if constexpr (PROD) {
      f32x4 as[2][8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 8; ++m) as[t][m] = f32x4{0, 0, 0, 0};
      constexpr int SIMG = MB > 0 ? kImageVec : 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u32x4 bs[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // sign byte k times the entry stride (64 bytes), OR the lane's copy
          const uint32_t x = k == 0 ? sw[t] << 6 : sw[t] >> (8 * k - 6);
          const uint32_t addr = (x & 0x3FC0u) | sign_base;
          bs[t] = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(addr + GQ::SIGN_OFF);
        }
        // S^T takes two f16 passes (hi and lo parts), so its rounding adds
        // about 2^-22 of the QJL term instead of 2^-12 with the hi part alone.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int f = (m * 4 + k) * 2;
          const u32x4 ah = img[SIMG + f * kFragVec + frag_lane];
          const u32x4 al = img[SIMG + (f + 1) * kFragVec + frag_lane];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            as[t][m] = mfma_f16(ah, bs[t], as[t][m]);
            as[t][m] = mfma_f16(al, bs[t], as[t][m]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[t][m] += as[t][m] * scale_s[t];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t v = tile * 32 + 16 * t + col;
      // coordinates 16 m + 4 grp + q of vector v are acc[t][m][q] (the images'
      // output rows are in natural order): each store instruction writes one
      // contiguous 64-byte run per vector
      const uint32_t base = v < n ? (uint32_t)(v * D + 4 * grp) * 4 : kDropped;
#pragma unroll
      for (int m = 0; m < 8; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[t][m]), ro, base + 64 * m, 0, 0);
    }
  };
  int64_t tile = (int64_t)blockIdx.x * kWaves + wave;
  if (tile < ntiles) {
    DqRegs ra, rb;
    dq_load(ra, tile);
    while (true) {
      int64_t nxt = tile + stride;
      bool more = nxt < ntiles;
      dq_load(rb, more ? nxt : tile);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch issues before the tile's work
      dq_tile(ra, tile);
      tile = nxt;
      if (!more) break;
      nxt = tile + stride;
      more = nxt < ntiles;
      dq_load(ra, more ? nxt : tile);
      __builtin_amdgcn_sched_barrier(0);
      dq_tile(rb, tile);
      tile = nxt;
      if (!more) break;
    }
    // both register sets are read on the way out, so that neither prefetch is
    // moved below the tile worked on after it
    uint32_t keep = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (MB > 0)
#pragma unroll
        for (int i = 0; i < CW; ++i) keep ^= ra.cw[t][i] ^ rb.cw[t][i];
      keep ^= ra.sw[t] ^ rb.sw[t] ^ __float_as_uint(ra.nu[t]) ^ __float_as_uint(rb.nu[t]) ^
              __float_as_uint(ra.ga[t]) ^ __float_as_uint(rb.ga[t]);
    }
    asm volatile("" ::"v"(keep));
  }
}

// Decode tables (the host builds one copy): one u32 per pair of codes (two
// f16 values alpha c[i0], alpha c[i1]) and one u32x4 per sign byte (eight f16
// +1 / -1).  In LDS every entry is replicated so that each lane reads its own
// copy: the copy index is the low lane bits, which puts the lanes served in
// one LDS cycle on distinct banks whatever codes they hold.
template <int MB>
struct LutGeom {
  static constexpr int W = 2 * MB;                       // index bits (two codes)
  static constexpr int ENTRIES = MB > 0 ? 1 << W : 1;
  static constexpr int COPIES = MB == 4 ? 32 : 64;        // u32 entries
  static constexpr int SHIFT = MB == 4 ? 7 : 8;           // log2(4 COPIES): entry stride in bytes
  static constexpr int WORDS = MB > 0 ? ENTRIES : 1;      // host table
  // dynamic LDS: replicated code table at byte 0 (so an entry address is the
  // index shifted left by SHIFT, OR the lane's copy), sign table, query buffers
  static constexpr uint32_t CODE_BYTES = MB > 0 ? ENTRIES * COPIES * 4 : 0;
};
// Sign table: 16 copies of each 16-byte entry, entries 256 bytes apart.  A
// 16-byte LDS read serves 16 lanes per cycle from 64 four-byte banks, so the
// 16 lanes of a group must read 16 distinct 16-byte bank slots: with the copy
// index lane & 15 they do whatever bytes they look up (8 copies at a 128-byte
// stride measured about four conflict cycles per read).
constexpr int kSignCopies = 16;                    // u32x4 entries
constexpr uint32_t kSignBytes = 256 * kSignCopies * 16;
constexpr uint32_t kQueryBytes = 3 * 8 * D * 4;    // qs, qt, pp

// Score one 16-key tile.  Each LDS lookup decodes two codes (or eight signs)
// straight into f16 operand registers of the lane's key; the queries are the
// A operand (row 2h + part: head h, hi or lo f16 part) and the decoded keys the
// B operand (column = key), one MFMA per 32 coordinates of codes and one per
// 32 signs.  The accumulator then holds, in lane (key, grp), rows 4 grp .. 4
// grp + 3: the hi and lo parts of heads 2 grp and 2 grp + 1 for its own key.
// Returns those two logits (norm applied).  The QJL scale sqrt(pi/2)/d is
// folded into the projected query.
template <int MB, bool PROD>
__device__ __forceinline__ void score_tile(const KeyRegs<MB> &r, int u, const u32x4 *bq,
                                           const u32x4 *bp, uint32_t code_base, uint32_t sign_base,
                                           float &o0, float &o1) {
  using GM = LutGeom<MB>;
  constexpr int W = GM::W;
  f32x4 cm = {0, 0, 0, 0}, cq = {0, 0, 0, 0};
  if constexpr (MB > 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4 bk;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * k + jj;  // code pair j of the lane's 32 coordinates
        const int bit = j * W, wi = bit >> 5, sh = bit & 31;
        // the field moved to bit SHIFT: the entry's byte offset
        uint32_t x;
        if (sh + W > 32)
          x = __builtin_amdgcn_alignbit(r.cw[u][wi + 1], r.cw[u][wi], sh - GM::SHIFT);
        else if (sh >= GM::SHIFT)
          x = r.cw[u][wi] >> (sh - GM::SHIFT);
        else
          x = r.cw[u][wi] << (GM::SHIFT - sh);
        const uint32_t addr = (x & (uint32_t)(((1 << W) - 1) << GM::SHIFT)) | code_base;
        bk[jj] = *(__attribute__((address_space(3))) const uint32_t *)(uintptr_t)addr;
      }
      cm = mfma_f16(bq[k], bk, cm);
    }
  }
  if constexpr (PROD) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // sign byte k times the entry stride (256 bytes), OR the lane's copy
      const uint32_t x = k == 0 ? r.sw[u] << 8 : r.sw[u] >> (8 * k - 8);
      const uint32_t addr = (x & 0xFF00u) | sign_base;
      const u32x4 sg = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(addr + GM::CODE_BYTES);
      cq = mfma_f16(bp[k], sg, cq);
    }
  }
  float v0 = cm[0] + cm[1], v1 = cm[2] + cm[3];
  if constexpr (PROD) {
    v0 = fmaf(r.gv[u], cq[0] + cq[1], v0);
    v1 = fmaf(r.gv[u], cq[2] + cq[3], v1);
  }
  o0 = v0 * r.nv[u];
  o1 = v1 * r.nv[u];
}

// Workgroup layout: one 1024-thread workgroup per CU (16 waves, 4 per SIMD)
// scores one contiguous key range of one set.  Waves take 64-key blocks from
// a counter in LDS, so faster waves (the scheduler favours older ones) take
// more blocks and every wave finishes at about the same time.
template <int MB, bool PROD>
__global__ __launch_bounds__(kLogitThreads, 1) void k_logits128(
    const float *__restrict__ q, int nq, int h0, int hc, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ signs, const float *__restrict__ norms,
    const float *__restrict__ rnorms, int64_t n_keys, int64_t set_keys, int groups, const float *__restrict__ PiT,
    const float *__restrict__ ST, const uint32_t *__restrict__ lut, float lut_inv_scale,
    int64_t keys_per_wg, float *__restrict__ out) {
  constexpr int CW = MB;  // code words per lane (32 coordinates)
  using GM = LutGeom<MB>;
  extern __shared__ u32x4 dyn_lds[];  // the kernel's only LDS: starts at address 0
  uint32_t *t_code = (uint32_t *)dyn_lds;
  u32x4 *t_sg = (u32x4 *)((char *)dyn_lds + GM::CODE_BYTES);
  float *qs = (float *)((char *)dyn_lds + GM::CODE_BYTES + kSignBytes);
  float *qt = qs + 8 * D;
  float *pp = qt + 8 * D;
  float *scratch = pp + 8 * D;                 // [2][4][8][D] partial sums
  uint32_t *counter = (uint32_t *)(scratch + 2 * 4 * 8 * D);

  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t kbeg = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t kend = kbeg + keys_per_wg < n_keys ? kbeg + keys_per_wg : n_keys;
  const int64_t srow = (int64_t)s * set_keys;
  KeyRsrc kr;  // the set's arrays and the lane's offsets
  kr.c = set_rsrc(MB > 0 ? codes + srow * (16 * CW) : codes, MB > 0 ? n_keys * (16 * CW) : 0);
  kr.s = set_rsrc(PROD ? signs + srow * 16 : signs, PROD ? n_keys * 16 : 0);
  kr.n = set_rsrc(norms + srow, n_keys * 4);
  kr.g = set_rsrc(PROD ? rnorms + srow : rnorms, PROD ? n_keys * 4 : 0);
  kr.oc = (uint32_t)(col * (16 * CW) + grp * (4 * CW));
  kr.os = (uint32_t)(col * 16 + grp * 4);
  kr.on = (uint32_t)(col * 4);
  constexpr int KT = kLogitTiles;
  constexpr int W = 16 * KT;  // keys per block
  const int nfull = (int)((kend - kbeg) / W);
  const bool ragged = kbeg + (int64_t)nfull * W < kend;

  // 1. every global load of the set-up at once: this wave's first key block
  // (wave w starts with block w; later blocks come from the counter), the
  // query, the columns of Pi^T / S^T this thread contracts, the tables
  KeyRegs<CW> ra, rb;  // ping-pong: one block is scored while the next loads
  int b = wave;
  if (b < nfull) load_keys<CW, PROD, KT, false>(ra, kbeg + (int64_t)b * W, kend, col, kr);
  const int mat = tid >> 9, slice = (tid >> 7) & 3, jj = tid & 127;
  float w[32];
  {
    const float *Wm = (mat == 0 ? PiT : (PROD ? ST : PiT)) + (size_t)g * D * D + (size_t)(32 * slice) * D + jj;
#pragma unroll
    for (int k = 0; k < 32; ++k) w[k] = Wm[(size_t)k * D];
  }
  {
    const int h = tid / D;
    qs[tid] = h < hc ? q[((int64_t)s * nq + h0 + h) * D + (tid % D)] : 0.f;  // 8 D == threads
  }
  if constexpr (MB > 0)
    for (int e = tid; e < GM::ENTRIES * GM::COPIES; e += kLogitThreads) t_code[e] = lut[e / GM::COPIES];
  if constexpr (PROD)
    for (int e = tid; e < 256 * kSignCopies; e += kLogitThreads)
      t_sg[e] = ((const u32x4 *)(lut + (MB > 0 ? GM::WORDS : 0)))[e / kSignCopies];
  if (tid < 64) counter[tid] = kLogitWaves;
  __syncthreads();
  // 2. rotate (Pi q) and project (S q) every head: thread (mat, slice, j)
  // sums 32 contraction steps for output coordinate j
  if (mat == 0 || PROD) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 32; ++k)
#pragma unroll
      for (int h = 0; h < 8; ++h) a[h] = fmaf(w[k], qs[h * D + 32 * slice + k], a[h]);
#pragma unroll
    for (int h = 0; h < 8; ++h) scratch[((mat * 4 + slice) * 8 + h) * D + jj] = a[h];
  }
  __syncthreads();
  // 3. reduce the four slices
  for (int e = tid; e < (PROD ? 2 : 1) * 8 * D; e += kLogitThreads) {
    const int m = e / (8 * D), hj = e % (8 * D);
    float v = 0.f;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) v += scratch[(m * 4 + sl) * 8 * D + hj];
    (m == 0 ? qt : pp)[hj] = v;
  }
  __syncthreads();
  // 4. query operands (MFMA A): row col = (head col >> 1, part col & 1);
  // contraction element e of K step k is coordinate 32 grp + 8 k + e.
  u32x4 bq[4], bp[4];
  {
    const int h = col >> 1, part = col & 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * grp + 8 * k + 2 * i;
        // the centroid table holds alpha * c; the QJL scale sqrt(pi/2)/d
        // multiplies every sign term
        float a0 = qt[h * D + c] * lut_inv_scale, a1 = qt[h * D + c + 1] * lut_inv_scale;
        float p0 = pp[h * D + c] * kQjlScale / (float)D, p1 = pp[h * D + c + 1] * kQjlScale / (float)D;
        if (part) {
          a0 -= (float)(_Float16)a0;
          a1 -= (float)(_Float16)a1;
          p0 -= (float)(_Float16)p0;
          p1 -= (float)(_Float16)p1;
        }
        bq[k][i] = f16x2(a0, a1);
        bp[k][i] = f16x2(p0, p1);
      }
    }
  }

  const int hA = 2 * grp, hB = 2 * grp + 1;  // heads held by this lane
  // logits of this set's heads h0 .. h0 + hc - 1 through a buffer resource
  // (rows set_keys apart; out points at this launch's first key): lanes
  // without a head, and keys past the end, get an offset past num_records
  // and store nothing
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(out + ((int64_t)s * nq + h0) * set_keys, 0, (int)(hc * set_keys * 4),
                                        kBufferFlags);
  const uint32_t rowA = hA < hc ? (uint32_t)(hA * set_keys) * 4 : kDropped;
  const uint32_t rowB = hB < hc ? (uint32_t)(hB * set_keys) * 4 : kDropped;
  // each lane reads its own copy of every table entry (the tables start at
  // LDS address 0 and CODE_BYTES, so the copy offset is OR-ed in)
  const uint32_t code_base = 4 * (lane & (GM::COPIES - 1));
  const uint32_t sign_base = 16 * (lane & (kSignCopies - 1));
  // next block of this workgroup's range (wave-uniform): every lane adds one
  // to its own counter word (distinct banks, no branch on the lane); lane 0's
  // word is the atomic block counter, the other 63 keep the instruction uniform
  auto grab = [&]() {
    const uint32_t v = atomicAdd(counter + lane, 1u);
    return (int)__builtin_amdgcn_readfirstlane(v);
  };
  // A full block's logits go through this wave's 2 KB of the (now free)
  // prologue scratch, [8 heads][64 keys], and leave as 16-byte stores: each
  // instruction writes 256 contiguous bytes of four head rows.  Only this
  // wave touches its region; lanes read what other lanes wrote, so
  // wavefront-scope fences keep the compiler from moving a read above the
  // writes it needs (or the next block's writes above the reads).
  static_assert(W == 64 && kLogitWaves * 8 * W <= 2 * 4 * 8 * D, "staging fits the scratch");
  float *stage = scratch + wave * 8 * W;
  const int sh = lane >> 4, sk = 4 * (lane & 15);  // store lane: head sh (and sh + 4), keys sk .. sk + 3
  const uint32_t rowS0 = sh < hc ? (uint32_t)(sh * set_keys) * 4 : kDropped;
  const uint32_t rowS1 = sh + 4 < hc ? (uint32_t)((sh + 4) * set_keys) * 4 : kDropped;
  auto score_store = [&](const KeyRegs<CW> &r, int64_t tb) {
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      float o0, o1;
      score_tile<MB, PROD>(r, u, bq, bp, code_base, sign_base, o0, o1);
      stage[hA * W + 16 * u + col] = o0;
      stage[hB * W + 16 * u + col] = o1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v0 = *(const u32x4 *)(stage + sh * W + sk);
    const u32x4 v1 = *(const u32x4 *)(stage + (sh + 4) * W + sk);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t key4 = (uint32_t)(tb + sk) * 4;
    __builtin_amdgcn_raw_buffer_store_b128(v0, ro, rowS0 + key4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(v1, ro, rowS1 + key4, 0, 0);
  };
  if (b < nfull) {  // ra holds block b
    while (true) {
      // The prefetch is unconditional (a branch around it would make the
      // wait-count pass wait for it): past the end it re-reads block b.
      int b2 = grab();
      bool more = b2 < nfull;
      load_keys<CW, PROD, KT, false>(rb, kbeg + (int64_t)(more ? b2 : b) * W, kend, col, kr);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch issues before the block's work
      score_store(ra, kbeg + (int64_t)b * W);
      b = b2;
      if (!more) break;
      b2 = grab();
      more = b2 < nfull;
      load_keys<CW, PROD, KT, false>(ra, kbeg + (int64_t)(more ? b2 : b) * W, kend, col, kr);
      __builtin_amdgcn_sched_barrier(0);
      score_store(rb, kbeg + (int64_t)b * W);
      b = b2;
      if (!more) break;
    }
    // both buffers are read on the way out, so that neither prefetch is moved
    // below the block scored after it (into the one successor that uses it)
    uint32_t keep = 0;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      if constexpr (CW > 0)
#pragma unroll
        for (int i = 0; i < CW; ++i) keep ^= ra.cw[u][i] ^ rb.cw[u][i];
      if constexpr (PROD) keep ^= ra.sw[u] ^ rb.sw[u] ^ __float_as_uint(ra.gv[u]) ^ __float_as_uint(rb.gv[u]);
      keep ^= __float_as_uint(ra.nv[u]) ^ __float_as_uint(rb.nv[u]);
    }
    asm volatile("" ::"v"(keep));
  }
  if (b == nfull && ragged) {  // the one wave that holds the partial block: guarded loads and stores
    const int64_t t0 = kbeg + (int64_t)nfull * W;
    load_keys<CW, PROD, KT, true>(ra, t0, kend, col, kr);
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      float o0, o1;
      score_tile<MB, PROD>(ra, u, bq, bp, code_base, sign_base, o0, o1);
      const int64_t key = t0 + 16 * u + col;
      const uint32_t key4 = (uint32_t)key * 4;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o0), ro, key < kend ? rowA + key4 : kDropped, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o1), ro, key < kend ? rowB + key4 : kDropped, 0, 0);
    }
  }
}

// Decode logits on mixed-precision keys: d = 128 split 64 + 64, TurboQuant_mse
// in both parts (the layout tq_mixed_quantize writes).  [tqnet] 实现步骤草图 ›
// 集成到 attention (logits straight from the codes); [tqnet] 从工程视角看
// TurboQuant 到底改变了什么 (outlier channels at b + 1 bits).  The kernel is
// k_logits128's, with one change of layout: lane (key, grp) takes coordinates
// 16 grp .. 16 grp + 15 of each part, so contraction steps 0, 1 cover the
// outlier part and 2, 3 the regular part.  Each part decodes through its own
// code-pair table, accumulates on its own and is scaled by its own norm:
// <q, x_hat> = nu_o <Pi_o q_o, c_o> + nu_r <Pi_r q_r, c_r>.

// Code words of the lane's 16 codes of one part (2 MB bytes at bit 16 grp MB
// of the row): the one or two aligned 32-bit words that hold them.
template <int MB>
__device__ __forceinline__ void mixed_key_words(uint32_t (&w)[2], __amdgpu_buffer_rsrc_t r, uint32_t off,
                                                uint32_t so) {
  if constexpr (MB <= 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, so, 0);
    w[1] = 0u;
  } else {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, so, 0);
    w[0] = v[0];
    w[1] = v[1];
  }
}

struct MixKeyRegs {
  uint32_t o[kLogitTiles][2], r[kLogitTiles][2];
  float no[kLogitTiles], nr[kLogitTiles];
};

struct MixKeyRsrc {
  __amdgpu_buffer_rsrc_t co, cr, no, nr;
  uint32_t oo, orr, on;   // lane offsets: outlier / regular code words of key col, norm of key col
  uint32_t row_o, row_r;  // bytes per key
};

template <int MBO, int MBR, bool TAIL>
__device__ __forceinline__ void load_mixed_keys(MixKeyRegs &r, int64_t t0, int64_t kend, int col,
                                                const MixKeyRsrc &k) {
  const uint32_t k0 = (uint32_t)t0;
#pragma unroll
  for (int u = 0; u < kLogitTiles; ++u) {
    const bool ok = !TAIL || t0 + 16 * u + col < kend;
    const uint32_t du = ok ? (uint32_t)(16 * u) : 0u, cu = ok ? 0u : (uint32_t)col;  // back to key t0
    mixed_key_words<MBO>(r.o[u], k.co, k.oo + (du - cu) * k.row_o, k0 * k.row_o);
    mixed_key_words<MBR>(r.r[u], k.cr, k.orr + (du - cu) * k.row_r, k0 * k.row_r);
    const uint32_t noff = k.on + du * 4 - cu * 4;
    r.no[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(k.no, noff, k0 * 4, 0));
    r.nr[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(k.nr, noff, k0 * 4, 0));
  }
}

// Two contraction steps of one part: the lane's 16 codes (words w, first code
// at bit sh of w[0]) as 8 code-pair table reads per step pair.
template <int MB>
__device__ __forceinline__ f32x4 mixed_part(const uint32_t (&w)[2], uint32_t sh, const u32x4 *bq,
                                            uint32_t base, uint32_t table) {
  using GM = LutGeom<MB>;
  constexpr int W = GM::W;
  // the 16 codes from bit 0: two words (fields of a pair never straddle the
  // end of a 32-bit window for W <= 8 once aligned like this)
  const uint32_t n0 = MB <= 2 ? w[0] >> sh : __builtin_amdgcn_alignbit(w[1], w[0], sh);
  const uint32_t n1 = MB <= 2 ? 0u : w[1] >> sh;
  const uint32_t cw[2] = {n0, n1};
  f32x4 c = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    u32x4 bk;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * k + jj, bit = j * W, wi = bit >> 5, sh2 = bit & 31;
      uint32_t x;
      if (sh2 + W > 32)
        x = __builtin_amdgcn_alignbit(cw[wi + 1], cw[wi], sh2 - GM::SHIFT);
      else if (sh2 >= GM::SHIFT)
        x = cw[wi] >> (sh2 - GM::SHIFT);
      else
        x = cw[wi] << (GM::SHIFT - sh2);
      const uint32_t addr = ((x & (uint32_t)(((1 << W) - 1) << GM::SHIFT)) | base) + table;
      bk[jj] = *(__attribute__((address_space(3))) const uint32_t *)(uintptr_t)addr;
    }
    c = mfma_f16(bq[k], bk, c);
  }
  return c;
}

template <int MBO, int MBR>
__global__ __launch_bounds__(kLogitThreads, 1) void k_logits128_mixed(
    const float *__restrict__ q, int nq, int h0, int hc, const uint8_t *__restrict__ codes_o, int64_t row_o,
    const uint8_t *__restrict__ codes_r, int64_t row_r, const float *__restrict__ norms_o,
    const float *__restrict__ norms_r, int64_t n_keys, int64_t set_keys, int groups, const float *__restrict__ RT,
    const uint32_t *__restrict__ lut_o, float inv_o, const uint32_t *__restrict__ lut_r, float inv_r,
    int64_t keys_per_wg, float *__restrict__ out) {
  using GO = LutGeom<MBO>;
  using GR = LutGeom<MBR>;
  extern __shared__ u32x4 dyn_lds[];  // the kernel's only LDS: starts at address 0
  uint32_t *t_o = (uint32_t *)dyn_lds;
  uint32_t *t_r = (uint32_t *)((char *)dyn_lds + GO::CODE_BYTES);
  float *qs = (float *)((char *)dyn_lds + GO::CODE_BYTES + GR::CODE_BYTES);
  float *qt = qs + 8 * D;
  float *scratch = qt + 8 * D;                 // [4][8][D] partial sums, later the stores' staging
  uint32_t *counter = (uint32_t *)(scratch + 8 * 8 * D);

  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t kbeg = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t kend = kbeg + keys_per_wg < n_keys ? kbeg + keys_per_wg : n_keys;
  const int64_t srow = (int64_t)s * set_keys;
  MixKeyRsrc kr;
  kr.co = set_rsrc(codes_o + srow * row_o, n_keys * row_o);
  kr.cr = set_rsrc(codes_r + srow * row_r, n_keys * row_r);
  kr.no = set_rsrc(norms_o + srow, n_keys * 4);
  kr.nr = set_rsrc(norms_r + srow, n_keys * 4);
  kr.row_o = (uint32_t)row_o;
  kr.row_r = (uint32_t)row_r;
  kr.oo = (uint32_t)(col * row_o) + 4u * (uint32_t)((16 * grp * MBO) >> 5);
  kr.orr = (uint32_t)(col * row_r) + 4u * (uint32_t)((16 * grp * MBR) >> 5);
  kr.on = (uint32_t)(col * 4);
  const uint32_t sh_o = (uint32_t)((16 * grp * MBO) & 31), sh_r = (uint32_t)((16 * grp * MBR) & 31);
  constexpr int KT = kLogitTiles;
  constexpr int W = 16 * KT;  // keys per block
  const int nfull = (int)((kend - kbeg) / W);
  const bool ragged = kbeg + (int64_t)nfull * W < kend;

  // 1. set-up loads: this wave's first block, the query, the columns of R^T
  // this thread contracts, the tables
  MixKeyRegs ra, rb;
  int b = wave;
  if (b < nfull) load_mixed_keys<MBO, MBR, false>(ra, kbeg + (int64_t)b * W, kend, col, kr);
  const int slice = (tid >> 7) & 3, jj = tid & 127;
  float w[32];
  {
    const float *Wm = RT + (size_t)g * D * D + (size_t)(32 * slice) * D + jj;
#pragma unroll
    for (int k = 0; k < 32; ++k) w[k] = Wm[(size_t)k * D];
  }
  {
    const int h = tid / D;
    qs[tid] = h < hc ? q[((int64_t)s * nq + h0 + h) * D + (tid % D)] : 0.f;  // 8 D == threads
  }
  for (int e = tid; e < GO::ENTRIES * GO::COPIES; e += kLogitThreads) t_o[e] = lut_o[e / GO::COPIES];
  for (int e = tid; e < GR::ENTRIES * GR::COPIES; e += kLogitThreads) t_r[e] = lut_r[e / GR::COPIES];
  if (tid < 64) counter[tid] = kLogitWaves;
  __syncthreads();
  // 2. rotate every head (coordinates 0..63: Pi_o q_o, 64..127: Pi_r q_r):
  // threads of slices 0..3 (the first 512) sum 32 contraction steps each
  if (tid < 4 * D) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 32; ++k)
#pragma unroll
      for (int h = 0; h < 8; ++h) a[h] = fmaf(w[k], qs[h * D + 32 * slice + k], a[h]);
#pragma unroll
    for (int h = 0; h < 8; ++h) scratch[(slice * 8 + h) * D + jj] = a[h];
  }
  __syncthreads();
  for (int e = tid; e < 8 * D; e += kLogitThreads) {
    float v = 0.f;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) v += scratch[sl * 8 * D + e];
    qt[e] = v;
  }
  __syncthreads();
  // 3. query operands: row col = (head col >> 1, part col & 1); element e of
  // step k is coordinate 16 grp + 8 (k & 1) + e of the outlier part (k < 2) or
  // of the regular part (k >= 2), divided by that part's table scale
  u32x4 bq[4];
  {
    const int h = col >> 1, part = col & 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c0 = (k < 2 ? 0 : 64) + 16 * grp + 8 * (k & 1);
      const float sc = k < 2 ? inv_o : inv_r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a0 = qt[h * D + c0 + 2 * i] * sc, a1 = qt[h * D + c0 + 2 * i + 1] * sc;
        if (part) {
          a0 -= (float)(_Float16)a0;
          a1 -= (float)(_Float16)a1;
        }
        bq[k][i] = f16x2(a0, a1);
      }
    }
  }

  const int hA = 2 * grp, hB = 2 * grp + 1;  // heads held by this lane
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(out + ((int64_t)s * nq + h0) * set_keys, 0, (int)(hc * set_keys * 4),
                                        kBufferFlags);
  const uint32_t rowA = hA < hc ? (uint32_t)(hA * set_keys) * 4 : kDropped;
  const uint32_t rowB = hB < hc ? (uint32_t)(hB * set_keys) * 4 : kDropped;
  const uint32_t base_o = 4 * (lane & (GO::COPIES - 1)), base_r = 4 * (lane & (GR::COPIES - 1));
  auto grab = [&]() {
    const uint32_t v = atomicAdd(counter + lane, 1u);  // lane 0's word is the block counter
    return (int)__builtin_amdgcn_readfirstlane(v);
  };
  auto score = [&](const MixKeyRegs &r, int u, float &o0, float &o1) {
    const f32x4 co = mixed_part<MBO>(r.o[u], sh_o, bq, base_o, 0u);
    const f32x4 cr = mixed_part<MBR>(r.r[u], sh_r, bq + 2, base_r, GO::CODE_BYTES);
    o0 = fmaf(co[0] + co[1], r.no[u], (cr[0] + cr[1]) * r.nr[u]);
    o1 = fmaf(co[2] + co[3], r.no[u], (cr[2] + cr[3]) * r.nr[u]);
  };
  // full blocks leave through this wave's 2 KB of the scratch as 16-byte
  // stores, as in k_logits128
  static_assert(W == 64 && kLogitWaves * 8 * W <= 8 * 8 * D, "staging fits the scratch");
  float *stage = scratch + wave * 8 * W;
  const int sh = lane >> 4, sk = 4 * (lane & 15);
  const uint32_t rowS0 = sh < hc ? (uint32_t)(sh * set_keys) * 4 : kDropped;
  const uint32_t rowS1 = sh + 4 < hc ? (uint32_t)((sh + 4) * set_keys) * 4 : kDropped;
  auto score_store = [&](const MixKeyRegs &r, int64_t tb) {
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      float o0, o1;
      score(r, u, o0, o1);
      stage[hA * W + 16 * u + col] = o0;
      stage[hB * W + 16 * u + col] = o1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 v0 = *(const u32x4 *)(stage + sh * W + sk);
    const u32x4 v1 = *(const u32x4 *)(stage + (sh + 4) * W + sk);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t key4 = (uint32_t)(tb + sk) * 4;
    __builtin_amdgcn_raw_buffer_store_b128(v0, ro, rowS0 + key4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(v1, ro, rowS1 + key4, 0, 0);
  };
  if (b < nfull) {  // ra holds block b
    while (true) {
      int b2 = grab();
      bool more = b2 < nfull;
      load_mixed_keys<MBO, MBR, false>(rb, kbeg + (int64_t)(more ? b2 : b) * W, kend, col, kr);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch issues before the block's work
      score_store(ra, kbeg + (int64_t)b * W);
      b = b2;
      if (!more) break;
      b2 = grab();
      more = b2 < nfull;
      load_mixed_keys<MBO, MBR, false>(ra, kbeg + (int64_t)(more ? b2 : b) * W, kend, col, kr);
      __builtin_amdgcn_sched_barrier(0);
      score_store(rb, kbeg + (int64_t)b * W);
      b = b2;
      if (!more) break;
    }
    // both buffers are read on the way out, so that neither prefetch is moved
    // below the block scored after it
    uint32_t keep = 0;
#pragma unroll
    for (int u = 0; u < KT; ++u)
      keep ^= ra.o[u][0] ^ ra.o[u][1] ^ ra.r[u][0] ^ ra.r[u][1] ^ rb.o[u][0] ^ rb.o[u][1] ^ rb.r[u][0] ^
              rb.r[u][1] ^ __float_as_uint(ra.no[u]) ^ __float_as_uint(ra.nr[u]) ^ __float_as_uint(rb.no[u]) ^
              __float_as_uint(rb.nr[u]);
    asm volatile("" ::"v"(keep));
  }
  if (b == nfull && ragged) {  // the one wave that holds the partial block: guarded loads and stores
    const int64_t t0 = kbeg + (int64_t)nfull * W;
    load_mixed_keys<MBO, MBR, true>(ra, t0, kend, col, kr);
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      float o0, o1;
      score(ra, u, o0, o1);
      const int64_t key = t0 + 16 * u + col;
      const uint32_t key4 = (uint32_t)key * 4;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o0), ro, key < kend ? rowA + key4 : kDropped, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o1), ro, key < kend ? rowB + key4 : kDropped, 0, 0);
    }
  }
}

// ------------------------------------------------------------ attention --
// Fused decode attention over quantized keys and values, d = 128: for every
// query head h of a set, out_h = sum_t softmax_t(scale <q_h, k_hat_t>) v_hat_t
// with v_hat_t = nu_t Pi^T c[idx_t] (TurboQuant_mse values).  [tqnet]
// 实现步骤草图 › 集成到 attention (K and V both stored quantized, attention on
// the QJL-coded keys); the softmax of scaled scores is scaled dot-product
// attention, kept online (running maximum and sum) so that every key is read
// once.
//
// Each workgroup takes one key range of one set and up to four heads.  Per
// 16-key tile a wave (1) scores the keys exactly as k_logits128 does (keys are
// the MFMA B operand: lane (key, grp) gets heads 2 grp and 2 grp + 1),
// (2) turns the scores into weights w = exp(s - m) nu_V (f16 hi + lo parts)
// and passes them through a small per-wave LDS buffer into the A operand of
// (3) a second f16 MFMA that adds w alpha c[idx] in the rotated domain.  Its
// rows are (head, coordinate parity, hi/lo part): a lane's value-code pair
// lookup yields the two coordinates 2p, 2p + 1 of one key, and the parity row
// picks one of them, so the decoded pairs go into the B operand as they are.
// Lane (col, grp) of the accumulators ends with head grp, coordinates
// 8 col .. 8 col + 7.  A per-set combine kernel merges the workgroups'
// (max, sum, vector) partials and applies Pi^T once per head.
constexpr int kAttnThreads = 768;            // 12 waves: three per SIMD
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnTiles = 2;                // 16-key tiles per block
constexpr int kAttnHeads = 4;                // query heads per pass
constexpr int kAttnPart = 132;               // floats per partial: m, l, pad, pad, a[128]
constexpr uint32_t kAttnVTab = 98304;        // LDS byte offset of the value decode table
constexpr uint32_t kAttnQOff = 131072;       // query buffers (qs, qt, pp)
constexpr uint32_t kAttnWBuf = kAttnQOff + 3 * kAttnHeads * D * 4;
// per-wave weight buffer: 8 head rows x 16 kAttnTiles keys (u32 hi|lo), rows
// 40 words apart so that the two rows written at once (heads 2 grp of lanes
// 0-31) fall on different banks and the four rows read at once (16-byte
// reads, 16 lanes a cycle) on different 16-byte bank slots
constexpr uint32_t kAttnWRow = 160;
static_assert(kAttnWRow >= 16 * kAttnTiles * 4, "weight row");
constexpr uint32_t kAttnWBytes = 8 * kAttnWRow;
constexpr uint32_t kAttnCounter = kAttnWBuf + kAttnWaves * kAttnWBytes;
constexpr uint32_t kAttnLds = kAttnCounter + 64 * 4;  // one counter word per lane
// the value-table region is free before the tables are filled (rotation
// scratch of the prologue) and after the main loop (merge of the waves)
constexpr uint32_t kAttnScratch = kAttnVTab;
static_assert(2 * 4 * kAttnHeads * D * 4 <= kAttnQOff - kAttnVTab, "prologue scratch");
static_assert(kAttnWaves * kAttnHeads * (D + 2) * 4 <= kAttnQOff - kAttnVTab, "merge buffer");
static_assert(kAttnLds <= 160 * 1024, "LDS budget");

constexpr float kLog2e = 1.4426950408889634f;

// Value codes of one block: lane (col, grp) holds, for keys grp + 4 j of each
// tile, the MBV-bit codes of coordinates 8 col .. 8 col + 7 (3-bit codes: the
// two words holding them, aligned when decoded); and the value norm of key col.
template <int MBV>
struct VRegs {
  static constexpr int VW = MBV == 3 ? 2 : 1;
  uint32_t w[kAttnTiles][4][VW];
  float n[kAttnTiles];
};

// Lane offsets (bytes) of the attention loads, fixed for the kernel.
struct AttnOffsets {
  uint32_t kc, ks, kn, v, v2;  // key codes / signs / norms of key col; value codes of key grp (two words)
};

// Buffer resources of one set's key and value arrays (wave-uniform).
struct AttnRsrc {
  __amdgpu_buffer_rsrc_t kc, ks, kn, kg, vc, vn;
};

// One block of keys t0 .. t0 + 16 kAttnTiles - 1 (wave-uniform t0, an index
// into the set): the key data in the logits layout (lane (col, grp): key col
// of each tile) and the value codes in the layout of the value MFMA (lane
// (col, grp): keys grp + 4 j, so that load j of a tile reads four consecutive
// rows, whole cache lines).  Every load is a buffer load: the set's resource,
// the lane's fixed offset (plus a constant) and t0 times the row size as the
// scalar offset, so no vector address arithmetic runs per block.  TAIL: keys
// at or past kend are replaced by key t0 (always valid).
template <int CW, bool PROD, int MBV, bool TAIL>
__device__ __forceinline__ void attn_load(KeyRegs<CW> &rk, VRegs<MBV> &rv, int64_t t0, int64_t kend, int col,
                                          int grp, const AttnOffsets &o, const AttnRsrc &r) {
  constexpr int ROWV = 16 * MBV;
  const uint32_t k0 = (uint32_t)t0;
  const int lim = TAIL ? (int)(kend - t0) : 64;  // keys of this block that exist
#pragma unroll
  for (int u = 0; u < kAttnTiles; ++u) {
    // key col of tile u (logits layout)
    const bool ok = !TAIL || 16 * u + col < lim;
    const uint32_t du = ok ? (uint32_t)(16 * u) : 0u, cu = ok ? 0u : (uint32_t)col;  // back to key t0
    if constexpr (CW > 0) {
      const uint32_t off = o.kc + du * (16 * CW) - cu * (16 * CW);
      const uint32_t so = k0 * (16 * CW);
      if constexpr (CW == 1) {
        rk.cw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(r.kc, off, so, 0);
      } else if constexpr (CW == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r.kc, off, so, 0);
        rk.cw[u][0] = v[0];
        rk.cw[u][1] = v[1];
      } else if constexpr (CW == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r.kc, off, so, 0);
        rk.cw[u][0] = v[0];
        rk.cw[u][1] = v[1];
        rk.cw[u][2] = v[2];
      } else {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r.kc, off, so, 0);
        rk.cw[u][0] = v[0];
        rk.cw[u][1] = v[1];
        rk.cw[u][2] = v[2];
        rk.cw[u][3] = v[3];
      }
    }
    if constexpr (PROD) rk.sw[u] = __builtin_amdgcn_raw_buffer_load_b32(r.ks, o.ks + du * 16 - cu * 16, k0 * 16, 0);
    const uint32_t noff = o.kn + du * 4 - cu * 4;
    rk.nv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.kn, noff, k0 * 4, 0));
    if constexpr (PROD) rk.gv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.kg, noff, k0 * 4, 0));
    rv.n[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r.vn, noff, k0 * 4, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // key grp + 4 j of tile u (value layout)
      const bool okv = !TAIL || 16 * u + grp + 4 * j < lim;
      const uint32_t dv = okv ? (uint32_t)((16 * u + 4 * j) * ROWV) : 0u - (uint32_t)(grp * ROWV);
      const uint32_t so = k0 * ROWV;
      if constexpr (MBV == 1) {
        rv.w[u][j][0] = __builtin_amdgcn_raw_buffer_load_b8(r.vc, o.v + dv, so, 0);
      } else if constexpr (MBV == 2) {
        rv.w[u][j][0] = __builtin_amdgcn_raw_buffer_load_b16(r.vc, o.v + dv, so, 0);
      } else if constexpr (MBV == 4) {
        rv.w[u][j][0] = __builtin_amdgcn_raw_buffer_load_b32(r.vc, o.v + dv, so, 0);
      } else {
        // 3-bit codes: the chunk starts at byte 3 col; o.v points at its
        // aligned word, o.v2 at the next one (the row's last word for col 15)
        rv.w[u][j][0] = __builtin_amdgcn_raw_buffer_load_b32(r.vc, o.v + dv, so, 0);
        rv.w[u][j][1] = __builtin_amdgcn_raw_buffer_load_b32(r.vc, o.v2 + dv, so, 0);
      }
    }
  }
}

__device__ __forceinline__ float dpp_f(float x, int ctrl) {
  switch (ctrl) {  // the control must be a constant: one instantiation per use
    case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
    case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
    case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));
  }
}
// Maximum / sum over the 16 lanes of a row (pairs, quads, half rows, rows).
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_f(x, 0xB1));
  x = fmaxf(x, dpp_f(x, 0x4E));
  x = fmaxf(x, dpp_f(x, 0x141));
  return fmaxf(x, dpp_f(x, 0x140));
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f(x, 0xB1);
  x += dpp_f(x, 0x4E);
  x += dpp_f(x, 0x141);
  return x + dpp_f(x, 0x140);
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float sel4(int i, float a, float b, float c, float d) {
  return i == 0 ? a : i == 1 ? b : i == 2 ? c : d;
}

// Online-softmax state of one wave: running maximum of the (log2-scaled)
// scores of each head (wave-uniform), the lane's partial sums of the weights
// of heads 2 grp, 2 grp + 1, and the value accumulators (head grp).
struct AttnState {
  float m[kAttnHeads];
  float lA, lB;
  f32x4 acc[4];
};

template <int MBK, bool PRODK, int MBV>
__device__ __forceinline__ void attn_block(AttnState &st, const KeyRegs<MBK> &rk, const VRegs<MBV> &rv,
                                           int64_t tb, int64_t kend, bool tail, const u32x4 *bq,
                                           const u32x4 *bp, uint32_t code_base, uint32_t sign_base,
                                           uint32_t vbase, float sl2e, uint32_t wrow, uint32_t wread,
                                           uint32_t psel, int col, int grp) {
  using GV = LutGeom<MBV>;
  constexpr int KT = kAttnTiles;
  // 1. scores (log2 domain) of heads 2 grp, 2 grp + 1 for key col of each tile
  float s0[KT], s1[KT];
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    float o0, o1;
    score_tile<MBK, PRODK>(rk, u, bq, bp, code_base, sign_base, o0, o1);
    s0[u] = o0 * sl2e;
    s1[u] = o1 * sl2e;
    if (tail && tb + 16 * u + col >= kend) s0[u] = s1[u] = -INFINITY;
  }
  // 2. new running maxima: row maxima, then the four heads as uniform values
  float x0 = s0[0], x1 = s1[0];
#pragma unroll
  for (int u = 1; u < KT; ++u) {
    x0 = fmaxf(x0, s0[u]);
    x1 = fmaxf(x1, s1[u]);
  }
  x0 = row_max(x0);
  x1 = row_max(x1);
  float alpha[kAttnHeads];
  {
    const float bm[kAttnHeads] = {lane_f(x0, 0), lane_f(x1, 0), lane_f(x0, 16), lane_f(x1, 16)};
#pragma unroll
    for (int h = 0; h < kAttnHeads; ++h) {
      const float mn = fmaxf(st.m[h], bm[h]);
      alpha[h] = __builtin_amdgcn_exp2f(st.m[h] - mn);
      st.m[h] = mn;
    }
  }
  const bool lo_rows = grp < 2;
  const float mA = lo_rows ? (grp == 0 ? st.m[0] : st.m[2]) : 0.f;
  const float mB = lo_rows ? (grp == 0 ? st.m[1] : st.m[3]) : 0.f;
  const float aA = lo_rows ? (grp == 0 ? alpha[0] : alpha[2]) : 1.f;
  const float aB = lo_rows ? (grp == 0 ? alpha[1] : alpha[3]) : 1.f;
  // 3. weights: p = 2^(s - m), the running sums, and w = p nu_V as f16 hi|lo
  // into this wave's buffer (row = head, column = key of the block)
  float lA = st.lA * aA, lB = st.lB * aB;
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const float pA = __builtin_amdgcn_exp2f(s0[u] - mA), pB = __builtin_amdgcn_exp2f(s1[u] - mB);
    lA += pA;
    lB += pB;
    const float wA = pA * rv.n[u], wB = pB * rv.n[u];
    const _Float16 hA = (_Float16)wA, hB = (_Float16)wB;
    const uint32_t vA = f16x2((float)hA, wA - (float)hA), vB = f16x2((float)hB, wB - (float)hB);
    *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(wrow + 4 * (16 * u)) = vA;
    *(__attribute__((address_space(3))) uint32_t *)(uintptr_t)(wrow + kAttnWRow + 4 * (16 * u)) = vB;
  }
  st.lA = lA;
  st.lB = lB;
  // 4. rescale the value accumulators (head grp) when a maximum moved
  if (alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f) {
    const float a = sel4(grp, alpha[0], alpha[1], alpha[2], alpha[3]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) st.acc[nt] *= a;
  }
  // 5. value MFMAs: A = this lane's weight part of keys grp + 4 j at parity
  // p, B = decoded code pairs 4 col + nt of the same keys
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const u32x4 wv = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(wread + 4 * (16 * u));
    u32x4 a;
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = __builtin_amdgcn_perm(wv[j], wv[j], psel);
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MBV == 3)
        c[j] = __builtin_amdgcn_alignbit(rv.w[u][j][1], rv.w[u][j][0], 8 * ((3 * col) & 3));
      else
        c[j] = rv.w[u][j][0];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      constexpr int W = GV::W;
      u32x4 b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sh = W * nt;
        const uint32_t x = sh >= GV::SHIFT ? c[j] >> (sh - GV::SHIFT) : c[j] << (GV::SHIFT - sh);
        const uint32_t addr = (x & (uint32_t)(((1 << W) - 1) << GV::SHIFT)) | vbase;
        b[j] = *(__attribute__((address_space(3))) const uint32_t *)(uintptr_t)addr;
      }
      st.acc[nt] = mfma_f16(a, b, st.acc[nt]);
    }
  }
}

template <int MBK, bool PRODK, int MBV>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn128(
    const float *__restrict__ q, int nq, int h0, int hc, const uint8_t *__restrict__ kcodes,
    const uint8_t *__restrict__ ksigns, const float *__restrict__ knorms, const float *__restrict__ krnorms,
    const uint8_t *__restrict__ vcodes, const float *__restrict__ vnorms, int64_t n_keys, int kgroups,
    const float *__restrict__ PiT, const float *__restrict__ ST, const uint32_t *__restrict__ klut,
    float k_inv_scale, const uint32_t *__restrict__ vlut, float sl2e, int64_t keys_per_wg,
    float *__restrict__ part) {
  constexpr int CW = MBK;
  using GK = LutGeom<MBK>;
  using GV = LutGeom<MBV>;
  static_assert(GK::CODE_BYTES + kSignBytes <= kAttnVTab && GV::CODE_BYTES <= kAttnQOff - kAttnVTab &&
                    (kAttnVTab & (GV::CODE_BYTES - 1)) == 0,
                "LDS map");
  extern __shared__ u32x4 dyn_lds[];  // the kernel's only LDS: starts at address 0
  char *lds = (char *)dyn_lds;
  uint32_t *t_code = (uint32_t *)lds;
  u32x4 *t_sg = (u32x4 *)(lds + GK::CODE_BYTES);
  uint32_t *t_val = (uint32_t *)(lds + kAttnVTab);
  float *qs = (float *)(lds + kAttnQOff);
  float *qt = qs + kAttnHeads * D;
  float *pp = qt + kAttnHeads * D;
  float *scratch = (float *)(lds + kAttnScratch);
  uint32_t *counter = (uint32_t *)(lds + kAttnCounter);

  const int s = blockIdx.y;
  const int g = s % kgroups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t kbeg = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t kend = kbeg + keys_per_wg < n_keys ? kbeg + keys_per_wg : n_keys;
  const int64_t srow = (int64_t)s * n_keys;
  // the set's arrays (wave-uniform resources) and the lane's fixed offsets
  AttnRsrc rs;
  rs.kc = set_rsrc(MBK > 0 ? kcodes + srow * (16 * CW) : kcodes, MBK > 0 ? n_keys * (16 * CW) : 0);
  rs.ks = set_rsrc(PRODK ? ksigns + srow * 16 : ksigns, PRODK ? n_keys * 16 : 0);
  rs.kn = set_rsrc(knorms + srow, n_keys * 4);
  rs.kg = set_rsrc(PRODK ? krnorms + srow : krnorms, PRODK ? n_keys * 4 : 0);
  rs.vc = set_rsrc(vcodes + srow * (16 * MBV), n_keys * (16 * MBV));
  rs.vn = set_rsrc(vnorms + srow, n_keys * 4);
  AttnOffsets ofs;
  ofs.kc = (uint32_t)(col * (16 * CW) + grp * (4 * CW));
  ofs.ks = (uint32_t)(col * 16 + grp * 4);
  ofs.kn = (uint32_t)(col * 4);
  ofs.v = (uint32_t)(grp * (16 * MBV) + (MBV == 3 ? 4 * ((3 * col) >> 2) : col * MBV));
  ofs.v2 = ofs.v + (col == 15 ? 0u : 4u);
  constexpr int KT = kAttnTiles;
  constexpr int W = 16 * KT;  // keys per block
  const int nfull = (int)((kend - kbeg) / W);
  const bool ragged = kbeg + (int64_t)nfull * W < kend;

  // 1. set-up loads: this wave's first block, the query, the columns of Pi^T /
  // S^T this thread contracts, the decode tables
  KeyRegs<CW> ka, kb;
  VRegs<MBV> va, vb;
  // Blocks are taken in an order rotated by a per-workgroup amount, so that
  // workgroups that advance in step do not read the same offsets of their
  // sets (equal strides) at the same time.
  const int rot = nfull > 0 ? (int)(((uint32_t)s * 2654435761u + (uint32_t)blockIdx.x * 40503u) % (uint32_t)nfull) : 0;
  auto rotb = [&](int x) { return x + rot >= nfull ? x + rot - nfull : x + rot; };
  int b = wave;
  if (b < nfull)
    attn_load<CW, PRODK, MBV, false>(ka, va, kbeg + (int64_t)rotb(b) * W, kend, col, grp, ofs, rs);
  const int slice = (tid >> 7) & 3, jj = tid & 127;
  for (int e = tid; e < kAttnHeads * D; e += kAttnThreads) {
    const int h = e >> 7;
    qs[e] = h < hc ? q[((int64_t)s * nq + h0 + h) * D + (e & 127)] : 0.f;
  }
  if (tid < 64) counter[tid] = kAttnWaves;
  __syncthreads();
  // 2. rotate (Pi q) and project (S q) the heads: thread (slice, j) sums 32
  // contraction steps of output coordinate j (scratch: the value-table region)
  if (tid < 4 * D) {
#pragma unroll
    for (int mat = 0; mat < (PRODK ? 2 : 1); ++mat) {
      const float *Wm = (mat == 0 ? PiT : ST) + (size_t)g * D * D + (size_t)(32 * slice) * D + jj;
      float a[kAttnHeads] = {0, 0, 0, 0};
#pragma unroll 8
      for (int k = 0; k < 32; ++k) {
        const float wk = Wm[(size_t)k * D];
#pragma unroll
        for (int h = 0; h < kAttnHeads; ++h) a[h] = fmaf(wk, qs[h * D + 32 * slice + k], a[h]);
      }
#pragma unroll
      for (int h = 0; h < kAttnHeads; ++h) scratch[((mat * 4 + slice) * kAttnHeads + h) * D + jj] = a[h];
    }
  }
  __syncthreads();
  for (int e = tid; e < (PRODK ? 2 : 1) * kAttnHeads * D; e += kAttnThreads) {
    const int m = e / (kAttnHeads * D), hj = e % (kAttnHeads * D);
    float v = 0.f;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) v += scratch[(m * 4 + sl) * kAttnHeads * D + hj];
    (m == 0 ? qt : pp)[hj] = v;
  }
  __syncthreads();
  // the decode tables (the value table overwrites the scratch)
  if constexpr (MBK > 0)
    for (int e = tid; e < GK::ENTRIES * GK::COPIES; e += kAttnThreads) t_code[e] = klut[e / GK::COPIES];
  if constexpr (PRODK)
    for (int e = tid; e < 256 * kSignCopies; e += kAttnThreads)
      t_sg[e] = ((const u32x4 *)(klut + (MBK > 0 ? GK::WORDS : 0)))[e / kSignCopies];
  for (int e = tid; e < GV::ENTRIES * GV::COPIES; e += kAttnThreads) t_val[e] = vlut[e / GV::COPIES];
  __syncthreads();
  // 3. query operands (MFMA A of the scores): row col = (head col >> 1, part col & 1)
  u32x4 bq[4], bp[4];
  {
    const int h = col >> 1, part = col & 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * grp + 8 * k + 2 * i;
        float a0 = 0.f, a1 = 0.f, p0 = 0.f, p1 = 0.f;
        if (h < kAttnHeads) {
          a0 = qt[h * D + c] * k_inv_scale;
          a1 = qt[h * D + c + 1] * k_inv_scale;
          p0 = pp[h * D + c] * kQjlScale / (float)D;
          p1 = pp[h * D + c + 1] * kQjlScale / (float)D;
        }
        if (part) {
          a0 -= (float)(_Float16)a0;
          a1 -= (float)(_Float16)a1;
          p0 -= (float)(_Float16)p0;
          p1 -= (float)(_Float16)p1;
        }
        bq[k][i] = f16x2(a0, a1);
        bp[k][i] = f16x2(p0, p1);
      }
    }
  }

  const uint32_t code_base = 4 * (lane & (GK::COPIES - 1));
  const uint32_t sign_base = 16 * (lane & (kSignCopies - 1));
  const uint32_t vbase = kAttnVTab | (4 * (lane & (GV::COPIES - 1)));
  // weight buffer of this wave: writer lane (col, grp) owns rows 2 grp, 2 grp + 1
  // (heads), column col of each tile; reader lane (n = col, grp) takes head
  // n >> 2, keys grp + 4 j of each tile, half n & 1 at parity (n >> 1) & 1
  const uint32_t wb = kAttnWBuf + wave * kAttnWBytes;
  // (key k of a tile is stored at position 4 (k & 3) + (k >> 2): the reader's
  // four consecutive words are keys grp + 4 j, the keys of its value codes)
  const uint32_t wrow = wb + (2 * grp) * kAttnWRow + 4 * (4 * (col & 3) + (col >> 2));
  const uint32_t wread = wb + (col >> 2) * kAttnWRow + 16 * grp;
  const int wpart = col & 1, wpar = (col >> 1) & 1;
  const uint32_t psel = wpart == 0 ? (wpar == 0 ? 0x0C0C0100u : 0x01000C0Cu) : (wpar == 0 ? 0x0C0C0302u : 0x03020C0Cu);

  AttnState stt;
#pragma unroll
  for (int h = 0; h < kAttnHeads; ++h) stt.m[h] = -1e30f;
  stt.lA = stt.lB = 0.f;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) stt.acc[nt] = f32x4{0, 0, 0, 0};

  // next block of this workgroup's range: every lane adds one to its own
  // counter word (distinct banks, no branch on the lane); lane 0's word is the
  // atomic block counter, the other 63 only keep the instruction uniform
  auto grab = [&]() {
    const uint32_t v = atomicAdd(counter + lane, 1u);
    return (int)__builtin_amdgcn_readfirstlane(v);
  };
  if (b < nfull) {
    while (true) {
      int b2 = grab();
      bool more = b2 < nfull;
      int64_t nb = kbeg + (int64_t)rotb(more ? b2 : b) * W;
      attn_load<CW, PRODK, MBV, false>(kb, vb, nb, kend, col, grp, ofs, rs);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch issues before the block's work
      attn_block<MBK, PRODK, MBV>(stt, ka, va, kbeg + (int64_t)rotb(b) * W, kend, false, bq, bp, code_base,
                                  sign_base, vbase, sl2e, wrow, wread, psel, col, grp);
      b = b2;
      if (!more) break;
      b2 = grab();
      more = b2 < nfull;
      nb = kbeg + (int64_t)rotb(more ? b2 : b) * W;
      attn_load<CW, PRODK, MBV, false>(ka, va, nb, kend, col, grp, ofs, rs);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch issues before the block's work
      attn_block<MBK, PRODK, MBV>(stt, kb, vb, kbeg + (int64_t)rotb(b) * W, kend, false, bq, bp, code_base,
                                  sign_base, vbase, sl2e, wrow, wread, psel, col, grp);
      b = b2;
      if (!more) break;
    }
    // both buffers are read on the way out, so that neither prefetch is moved
    // below the block scored after it (into the one successor that uses it)
    uint32_t keep = 0;
#pragma unroll
    for (int u = 0; u < kAttnTiles; ++u) {
      if constexpr (CW > 0)
#pragma unroll
        for (int i = 0; i < CW; ++i) keep ^= ka.cw[u][i] ^ kb.cw[u][i];
      if constexpr (PRODK) keep ^= ka.sw[u] ^ kb.sw[u] ^ __float_as_uint(ka.gv[u]) ^ __float_as_uint(kb.gv[u]);
      keep ^= __float_as_uint(ka.nv[u]) ^ __float_as_uint(kb.nv[u]) ^ __float_as_uint(va.n[u]) ^
              __float_as_uint(vb.n[u]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < VRegs<MBV>::VW; ++i) keep ^= va.w[u][j][i] ^ vb.w[u][j][i];
    }
    asm volatile("" ::"v"(keep));
  }
  if (b == nfull && ragged) {  // the one wave that holds the partial block
    const int64_t t0 = kbeg + (int64_t)nfull * W;
    attn_load<CW, PRODK, MBV, true>(ka, va, t0, kend, col, grp, ofs, rs);
    attn_block<MBK, PRODK, MBV>(stt, ka, va, t0, kend, true, bq, bp, code_base, sign_base, vbase, sl2e, wrow,
                                wread, psel, col, grp);
  }

  // 4. merge the waves: each writes its maxima, sums and vectors; then thread
  // (head, coordinate) combines them and writes the workgroup's partial
  __syncthreads();  // the value table is free from here on
  float *mv = (float *)(lds + kAttnVTab);                       // [wave][head][D]
  float *ml = mv + kAttnWaves * kAttnHeads * D;                 // [wave][head][2]
  {
    const float lA = row_sum(stt.lA), lB = row_sum(stt.lB);
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < kAttnHeads; ++h) ml[(wave * kAttnHeads + h) * 2] = stt.m[h];
      ml[(wave * kAttnHeads + 0) * 2 + 1] = lA;
      ml[(wave * kAttnHeads + 1) * 2 + 1] = lB;
    }
    if (lane == 16) {
      ml[(wave * kAttnHeads + 2) * 2 + 1] = lA;
      ml[(wave * kAttnHeads + 3) * 2 + 1] = lB;
    }
    float v[8];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      v[2 * nt] = stt.acc[nt][0] + stt.acc[nt][1];
      v[2 * nt + 1] = stt.acc[nt][2] + stt.acc[nt][3];
    }
    float *dst = mv + (wave * kAttnHeads + grp) * D + 8 * col;
    *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4 *)(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  __syncthreads();
  {
    const int h = tid >> 7, j = tid & 127;
    if (h < hc) {
      float M = -1e30f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml[(w * kAttnHeads + h) * 2]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(ml[(w * kAttnHeads + h) * 2] - M);
        L = fmaf(ml[(w * kAttnHeads + h) * 2 + 1], f, L);
        A = fmaf(mv[(w * kAttnHeads + h) * D + j], f, A);
      }
      float *o = part + (((int64_t)s * nq + h0 + h) * gridDim.x + blockIdx.x) * kAttnPart;
      o[4 + j] = A;
      if (j == 0) {
        o[0] = M;
        o[1] = L;
      }
    }
  }
}

// Merge the workgroups' partials of every head of one set and map back to
// the original coordinates: out_h = Pi^T (a_h / (alpha l_h)).  512 threads:
// thread (slice, j) sums contraction steps 32 slice .. 32 slice + 31 of
// output coordinate j for up to 8 heads; Pi is read once per set.
constexpr int kCombineHeads = 8;
constexpr int kCombineThreads = 4 * D;
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine128(const float *__restrict__ part, int nq,
                                                                     int parts, int vgroups,
                                                                     const float *__restrict__ Pi,
                                                                     float v_inv_scale, float *__restrict__ out) {
  __shared__ float av[kCombineHeads][D];
  __shared__ float red[4][kCombineHeads][D];
  const int s = blockIdx.x, tid = threadIdx.x, slice = tid >> 7, j = tid & 127;
  const float *P = Pi + (size_t)(s % vgroups) * D * D;
  for (int h0 = 0; h0 < nq; h0 += kCombineHeads) {
    const int hc = nq - h0 < kCombineHeads ? nq - h0 : kCombineHeads;
    for (int h = slice; h < hc; h += 4) {
      const float *p = part + ((int64_t)s * nq + h0 + h) * parts * kAttnPart;
      float M = -1e30f;
      for (int w = 0; w < parts; ++w) M = fmaxf(M, p[w * kAttnPart]);
      float L = 0.f, A = 0.f;
      for (int w = 0; w < parts; ++w) {
        const float f = __builtin_amdgcn_exp2f(p[w * kAttnPart] - M);
        L = fmaf(p[w * kAttnPart + 1], f, L);
        A = fmaf(p[w * kAttnPart + 4 + j], f, A);
      }
      av[h][j] = A * (v_inv_scale / L);
    }
    __syncthreads();
    float o[kCombineHeads] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int k = 32 * slice; k < 32 * slice + 32; ++k) {
      const float pk = P[(size_t)k * D + j];  // (Pi^T a)_j = sum_k Pi[k][j] a_k
#pragma unroll
      for (int h = 0; h < kCombineHeads; ++h) o[h] = fmaf(pk, av[h][k], o[h]);
    }
#pragma unroll
    for (int h = 0; h < kCombineHeads; ++h) red[slice][h][j] = o[h];
    __syncthreads();
    for (int h = slice; h < hc; h += 4)
      out[((int64_t)s * nq + h0 + h) * D + j] = red[0][h][j] + red[1][h][j] + red[2][h][j] + red[3][h][j];
    __syncthreads();
  }
}

template <int MB, bool PROD>
hipError_t run_dequant(const DeviceTables &t, const uint8_t *codes, const uint8_t *signs, const float *norms,
                       const float *rnorms, int64_t n_sets, int64_t n, float *out, hipStream_t st) {
  using GQ = DqGeom<MB>;
  if (n * D * 4 >= (int64_t)kDropped) return hipErrorNotSupported;
  const size_t lds = GQ::IMG_OFF + ((MB > 0 ? 1 : 0) + (PROD ? 1 : 0)) * (size_t)kImageVec * 16;
  hipError_t e = hipFuncSetAttribute((const void *)k_dequant128<MB, PROD>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (n + 31) / 32;
  constexpr int waves = kDqThreads / 64;
  const int64_t per_set_max = (ntiles + waves - 1) / waves;
  int64_t gx = (256 + n_sets - 1) / n_sets;  // one workgroup per CU
  if (gx > per_set_max) gx = per_set_max;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_dequant128<MB, PROD>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kDqThreads), lds, st,
                     codes, signs, norms, rnorms, n, t.groups, (const u32x4 *)t.dq_pi_frag,
                     (const u32x4 *)t.dq_s_frag, t.logit_lut, t.lut_inv_scale, out);
  return hipGetLastError();
}

#endif  // TQ_MSE3_TU

template <int MB>
hipError_t run_quant_mse(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n,
                         uint8_t *codes, float *norms, hipStream_t st) {
  // per-set byte offsets of codes and norms stay below the dropped-store offset
  if (t.cell_radius != kCellRadius || n * (16 * MB) >= (int64_t)kDropped) return hipErrorNotSupported;
  const int64_t ntiles = (n + 15) / 16;
  constexpr int waves = kMseThreads / 64;
  const int64_t per_set_max = (ntiles + waves - 1) / waves;  // >= 1 stage per wave
  const int64_t target = 256;                               // one workgroup per CU
  int64_t gx = (target + n_sets - 1) / n_sets;
  if (gx > per_set_max) gx = per_set_max;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_quant128_mse<MB>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kMseThreads), 0,
                     st, (const uint16_t *)x, n, t.groups, (const u32x4 *)t.pi_frag, t.cells,
                     t.cell_scale * kCellStep, codes, norms);
  return hipGetLastError();
}

#ifndef TQ_MSE3_TU
template <int MBO, int MBR>
hipError_t run_quant_mixed(const DeviceTables &to, const DeviceTables &tr, const uint32_t *img,
                           const uint32_t *masks, const void *x, int64_t n_sets, int64_t n, int groups,
                           uint8_t *codes_o, float *norms_o, uint8_t *codes_r, float *norms_r, hipStream_t st) {
  const int64_t ntiles = (n + 15) / 16;
  constexpr int waves = kMseThreads / 64;
  const int64_t per_set_max = (ntiles + waves - 1) / waves;
  int64_t gx = (256 + n_sets - 1) / n_sets;  // one workgroup per CU
  if (gx > per_set_max) gx = per_set_max;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_quant128_mixed<MBO, MBR>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kMseThreads), 0, st,
                     (const uint16_t *)x, n, groups, (const u32x4 *)img, masks, to.cells,
                     to.cell_scale * kCellStep, tr.cells, tr.cell_scale * kCellStep, codes_o, to.code_row, codes_r,
                     tr.code_row, norms_o, norms_r);
  return hipGetLastError();
}

template <int MB, bool PROD, bool F32IN>
hipError_t run_quant(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n, uint8_t *codes,
                     uint8_t *signs, float *norms, float *rnorms, hipStream_t st) {
  QuantParams qp;
  if (MB > 0 && t.cell_radius != kCellRadius) return hipErrorNotSupported;
  qp.cell_scale = t.cell_scale * kCellStep;
  qp.cell_words = MB > 0 ? 2 * (2 * kCellRadius + 1) : 0;
  static_assert(2 * (2 * kCellRadius + 1) * 4 <= kCellCap, "cell table exceeds its LDS slot");
  const size_t lds = (PROD ? 2 : 1) * (size_t)kImageVec * sizeof(u32x4) + kCellCap + 64;
  hipError_t e = hipFuncSetAttribute((const void *)k_quant128<MB, PROD, F32IN>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (n + 31) / 32;
  constexpr int threads = quant_threads<PROD>();
  const int64_t per_set_max = (ntiles + threads / 64 - 1) / (threads / 64);  // >= 1 tile per wave
  const int64_t target = 512;  // about two workgroup rounds
  int64_t gx = (target + n_sets - 1) / n_sets;
  if (gx > per_set_max) gx = per_set_max;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_quant128<MB, PROD, F32IN>), dim3((unsigned)gx, (unsigned)n_sets), dim3(threads),
                     lds, st, x, n, t.groups, t.pi_frag, t.m_frag, t.cells, t.cent, qp, codes, signs, norms,
                     rnorms);
  return hipGetLastError();
}

// Sets longer than kFusedMaxKeys keys run as several launches, one per
// chunk of keys (the key arrays and the output advanced to the chunk, with
// the set stride n_keys passed alongside); each launch scores up to
// logit_heads_per_launch(n_keys) heads.
template <int MB, bool PROD>
hipError_t run_logits(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes,
                      const uint8_t *signs, const float *norms, const float *rnorms, int64_t n_sets,
                      int64_t n_keys, float *out, hipStream_t st) {
  const int64_t unit = kLogitWaves * 16 * kLogitTiles;  // keys per workgroup iteration
  const int hp = logit_heads_per_launch(n_keys);
  if (hp == 0) return hipErrorNotSupported;
  const size_t lds = LutGeom<MB>::CODE_BYTES + kSignBytes + kQueryBytes + 2 * 4 * 8 * D * 4 + 64 * 4;
  hipError_t e0 = hipFuncSetAttribute((const void *)k_logits128<MB, PROD>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e0 != hipSuccess) return e0;
  for (int64_t k0 = 0; k0 < n_keys; k0 += kFusedMaxKeys) {
    const int64_t n = n_keys - k0 < kFusedMaxKeys ? n_keys - k0 : kFusedMaxKeys;
    int64_t kpw;
    const int64_t gx = logit_grid_x(n_sets, n, unit, &kpw);
    const uint8_t *ck = MB > 0 ? codes + k0 * (16 * MB) : codes;
    const uint8_t *sk = PROD ? signs + k0 * 16 : signs;
    const float *gk = PROD ? rnorms + k0 : rnorms;
    for (int64_t h0 = 0; h0 < nq; h0 += hp) {
      const int hc = (int)(nq - h0 < hp ? nq - h0 : hp);
      hipLaunchKernelGGL((k_logits128<MB, PROD>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kLogitThreads), lds,
                         st, q, (int)nq, (int)h0, hc, ck, sk, norms + k0, gk, n, n_keys, t.groups, t.PiT, t.ST,
                         t.logit_lut, t.lut_inv_scale, kpw, out + k0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

template <int MBO, int MBR>
hipError_t run_logits_mixed(const DeviceTables &to, const DeviceTables &tr, const float *RT, const float *q,
                            int64_t nq, const uint8_t *codes_o, const uint8_t *codes_r, const float *norms_o,
                            const float *norms_r, int64_t n_sets, int64_t n_keys, int groups, float *out,
                            hipStream_t st) {
  const int64_t unit = kLogitWaves * 16 * kLogitTiles;  // keys per workgroup iteration
  const int64_t rmax = to.code_row > tr.code_row ? to.code_row : tr.code_row;
  const int hp = logit_heads_per_launch(n_keys);
  if (hp == 0 || rmax > 64) return hipErrorNotSupported;
  const size_t lds = LutGeom<MBO>::CODE_BYTES + LutGeom<MBR>::CODE_BYTES + 2 * 8 * D * 4 + 8 * 8 * D * 4 + 64 * 4;
  hipError_t e0 = hipFuncSetAttribute((const void *)k_logits128_mixed<MBO, MBR>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e0 != hipSuccess) return e0;
  for (int64_t k0 = 0; k0 < n_keys; k0 += kFusedMaxKeys) {  // chunks as in run_logits
    const int64_t n = n_keys - k0 < kFusedMaxKeys ? n_keys - k0 : kFusedMaxKeys;
    int64_t kpw;
    const int64_t gx = logit_grid_x(n_sets, n, unit, &kpw);
    for (int64_t h0 = 0; h0 < nq; h0 += hp) {
      const int hc = (int)(nq - h0 < hp ? nq - h0 : hp);
      hipLaunchKernelGGL((k_logits128_mixed<MBO, MBR>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kLogitThreads),
                         lds, st, q, (int)nq, (int)h0, hc, codes_o + k0 * to.code_row, to.code_row,
                         codes_r + k0 * tr.code_row, tr.code_row, norms_o + k0, norms_r + k0, n, n_keys, groups, RT,
                         to.logit_lut, to.lut_inv_scale, tr.logit_lut, tr.lut_inv_scale, kpw, out + k0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Workgroups per set of the fused attention (about one per CU overall) and
// the keys each takes (a multiple of one block per wave).
int64_t attn_grid_x(int64_t n_sets, int64_t n_keys, int64_t *kpw) {
  const int64_t unit = kAttnWaves * 16 * kAttnTiles;
  int64_t gx = (256 + n_sets - 1) / n_sets;
  const int64_t max_gx = (n_keys + unit - 1) / unit;
  if (gx > max_gx) gx = max_gx;
  if (gx < 1) gx = 1;
  int64_t k = (n_keys + gx - 1) / gx;
  k = (k + unit - 1) / unit * unit;
  *kpw = k;
  return (n_keys + k - 1) / k;
}

template <int MBK, bool PRODK, int MBV>
hipError_t run_attention(const DeviceTables &tk, const DeviceTables &tv, const float *q, int64_t nq,
                         const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms, const float *krnorms,
                         const uint8_t *vcodes, const float *vnorms, int64_t n_sets, int64_t n_keys, float scale,
                         float *part, float *out, hipStream_t st) {
  int64_t kpw = 0;
  const int64_t gx = attn_grid_x(n_sets, n_keys, &kpw);
  hipError_t e = hipFuncSetAttribute((const void *)k_attn128<MBK, PRODK, MBV>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kAttnLds);
  if (e != hipSuccess) return e;
  const float sl2e = scale * kLog2e;
  for (int64_t h0 = 0; h0 < nq; h0 += kAttnHeads) {
    const int hc = (int)(nq - h0 < kAttnHeads ? nq - h0 : kAttnHeads);
    hipLaunchKernelGGL((k_attn128<MBK, PRODK, MBV>), dim3((unsigned)gx, (unsigned)n_sets), dim3(kAttnThreads),
                       kAttnLds, st, q, (int)nq, (int)h0, hc, kcodes, ksigns, knorms, krnorms, vcodes, vnorms,
                       n_keys, tk.groups, tk.PiT, tk.ST, tk.logit_lut, tk.lut_inv_scale, tv.logit_lut, sl2e, kpw,
                       part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_attn_combine128, dim3((unsigned)n_sets), dim3(kCombineThreads), 0, st, part, (int)nq,
                     (int)gx, tv.groups, tv.Pi, tv.lut_inv_scale, out);
  return hipGetLastError();
}

#endif  // TQ_MSE3_TU

}  // namespace

#ifdef TQ_MSE3_TU
// This file is compiled a second time with TQ_MSE3_TU defined and LLVM's
// max-ilp scheduling strategy, holding only the bf16 TurboQuant_mse kernel;
// that schedule runs its 3-bit form about 6% faster (the other widths are
// not faster under it, so they stay in the main build).
hipError_t launch_quant128_mse3(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n, uint8_t *codes,
                                float *norms, hipStream_t st) {
  return run_quant_mse<3>(t, x, n_sets, n, codes, norms, st);
}
#else
// -------------------------------------------------------------- host side --
bool fast128_supported(int d, int mse_bits, int variant) {
  (void)variant;
  return d == D && mse_bits >= 0 && mse_bits <= 4;
}

size_t fast128_rotation_words(int d) { return d == D ? (size_t)kImageWords : 0; }

static uint16_t host_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float host_bf16_to_f(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t host_f16(float f) {
  const _Float16 h = (_Float16)f;
  uint16_t u;
  memcpy(&u, &h, 2);
  return u;
}

void fast128_build_rotation_image(const double *mat, int k_order, uint32_t *out, bool f16, bool natural_rows) {
  memset(out, 0, (size_t)kImageWords * 4);
  for (int m = 0; m < 8; ++m)
    for (int k = 0; k < 4; ++k)
      for (int part = 0; part < 2; ++part) {
        const int f = (m * 4 + k) * 2 + part;
        for (int lane = 0; lane < 64; ++lane) {
          const int rho = lane & 15, grp = lane >> 4;
          const int orow = natural_rows ? 16 * m + rho : 32 * (rho >> 2) + 4 * m + (rho & 3);
          for (int e = 0; e < 8; ++e) {
            const int kin = k_order == 0 ? 32 * k + 8 * grp + e : 32 * grp + 8 * k + e;
            const float v = (float)mat[(size_t)orow * D + kin];
            uint16_t val;
            if (f16) {
              const uint16_t hi = host_f16(v);
              val = part == 0 ? hi : host_f16(v - (float)(_Float16)v);
            } else {
              const uint16_t hi = host_bf16(v);
              val = part == 0 ? hi : host_bf16(v - host_bf16_to_f(hi));
            }
            out[((size_t)f * 64 + lane) * 4 + e / 2] |= (uint32_t)val << (16 * (e & 1));
          }
        }
      }
}

void fast128_build_mixed_image(const double *pi_o, const double *pi_r, const int32_t *perm, uint32_t *out,
                               uint32_t *mask) {
  std::vector<double> mat((size_t)D * D, 0.0);
  for (int orow = 0; orow < D; ++orow) {
    // the lane group, row tile and row of the MFMA output that holds image row orow
    const int grp = orow / 32, m = (orow % 32) / 4, q = orow % 4;
    const int part = m / 4, coord = 16 * grp + 4 * (m % 4) + q;
    const double *src = (part == 0 ? pi_o : pi_r) + (size_t)coord * 64;
    for (int j = 0; j < 64; ++j) mat[(size_t)orow * D + perm[64 * part + j]] = src[j];
  }
  fast128_build_rotation_image(mat.data(), 0, out);
  for (int w = 0; w < 4; ++w) mask[w] = 0;
  for (int j = 0; j < 64; ++j) mask[perm[j] >> 5] |= 1u << (perm[j] & 31);
}

// Decode-table geometry: one lookup turns G codes of `mse_bits` bits (one
// index of G * mse_bits <= 12 bits) into G f16 values.
size_t fast128_lut_words(int mse_bits) {
  const size_t code_words = mse_bits > 0 ? (size_t)1 << (2 * mse_bits) : 0;  // code pair -> 2 x f16
  return code_words + 256 * 4;  // + sign table: byte -> 8 x (+1 / -1)
}

float fast128_build_logit_lut(const float *cent, int mse_bits, uint32_t *out) {
  const int L = mse_bits > 0 ? 1 << mse_bits : 0;
  auto h16 = [](float f) {
    _Float16 h = (_Float16)f;
    uint16_t u;
    memcpy(&u, &h, 2);
    return u;
  };
  // alpha in [1, 2): minimise the largest relative f16 rounding error of
  // alpha * |c_k| (the codebook is symmetric: the positive half suffices)
  float alpha = 1.f;
  if (L > 0) {
    double best = 1e30;
    for (int i = 0; i < (1 << 18); ++i) {
      const float a = 1.f + (float)i / (float)(1 << 18);
      double worst = 0.0;
      for (int k = L / 2; k < L; ++k) {
        const float v = a * cent[k];
        const double e = std::fabs((double)(float)(_Float16)v - (double)v) / (double)v;
        if (e > worst) worst = e;
      }
      if (worst < best) {
        best = worst;
        alpha = a;
      }
    }
  }
  size_t w = 0;
  if (mse_bits > 0) {
    for (int e = 0; e < (1 << (2 * mse_bits)); ++e) {
      const int i0 = e & (L - 1), i1 = (e >> mse_bits) & (L - 1);
      out[w++] = (uint32_t)h16(alpha * cent[i0]) | ((uint32_t)h16(alpha * cent[i1]) << 16);
    }
  }
  for (int byte = 0; byte < 256; ++byte)
    for (int h = 0; h < 8; h += 2) {
      uint32_t v = 0;
      for (int half = 0; half < 2; ++half) {
        const uint16_t x = ((byte >> (h + half)) & 1) ? 0x3C00u : 0xBC00u;  // +1 / -1
        v |= (uint32_t)x << (16 * half);
      }
      out[w++] = v;
    }
  return 1.f / alpha;
}

// the 3-bit bf16 TurboQuant_mse launcher, from this file's second compilation
hipError_t launch_quant128_mse3(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n, uint8_t *codes,
                                float *norms, hipStream_t st);

hipError_t launch_quant128(const DeviceTables &t, const void *x, int dtype, int64_t n_sets,
                           int64_t n, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                           hipStream_t st) {
  if (t.d != D || !t.pi_frag || t.mse_bits > 4 || ((uintptr_t)x & 15u)) return hipErrorNotSupported;
  const bool prod = t.variant == 1, f32 = dtype == 0;
  if (!prod && !f32 && t.mse_bits >= 1) {
    switch (t.mse_bits) {
      case 1: return run_quant_mse<1>(t, x, n_sets, n, codes, norms, st);
      case 2: return run_quant_mse<2>(t, x, n_sets, n, codes, norms, st);
      case 3: return launch_quant128_mse3(t, x, n_sets, n, codes, norms, st);
      case 4: return run_quant_mse<4>(t, x, n_sets, n, codes, norms, st);
    }
  }
#define TQ_Q(MB, P, F) \
  if (t.mse_bits == MB && prod == P && f32 == F) \
    return run_quant<MB, P, F>(t, x, n_sets, n, codes, signs, norms, rnorms, st);
  TQ_Q(0, true, false) TQ_Q(0, true, true)
  TQ_Q(1, false, false) TQ_Q(1, false, true) TQ_Q(1, true, false) TQ_Q(1, true, true)
  TQ_Q(2, false, false) TQ_Q(2, false, true) TQ_Q(2, true, false) TQ_Q(2, true, true)
  TQ_Q(3, false, false) TQ_Q(3, false, true) TQ_Q(3, true, false) TQ_Q(3, true, true)
  TQ_Q(4, false, false) TQ_Q(4, false, true) TQ_Q(4, true, false) TQ_Q(4, true, true)
#undef TQ_Q
  return hipErrorNotSupported;
}

hipError_t launch_quant128_mixed(const DeviceTables &to, const DeviceTables &tr, const uint32_t *img,
                                 const uint32_t *masks, const void *x, int64_t n_sets, int64_t n, int groups,
                                 uint8_t *codes_o, float *norms_o, uint8_t *codes_r, float *norms_r,
                                 hipStream_t st) {
  if (to.d != 64 || tr.d != 64 || to.variant != 0 || tr.variant != 0 || !img || !masks ||
      to.cell_radius != kCellRadius || tr.cell_radius != kCellRadius || ((uintptr_t)x & 15u))
    return hipErrorNotSupported;
  // per-set byte offsets of codes and norms stay below the dropped-store offset
  if (n * (to.code_row > tr.code_row ? to.code_row : tr.code_row) >= (int64_t)kDropped / 2) return hipErrorNotSupported;
#define TQ_M(O, R) \
  if (to.mse_bits == O && tr.mse_bits == R) \
    return run_quant_mixed<O, R>(to, tr, img, masks, x, n_sets, n, groups, codes_o, norms_o, codes_r, norms_r, st);
  TQ_M(2, 1) TQ_M(3, 2) TQ_M(4, 3)
#undef TQ_M
  return hipErrorNotSupported;
}

hipError_t launch_dequant128(const DeviceTables &t, const uint8_t *codes, const uint8_t *signs,
                             const float *norms, const float *rnorms, int64_t n_sets, int64_t n,
                             float *out, hipStream_t st) {
  if (t.d != D || !t.dq_pi_frag || t.mse_bits > 4 || ((uintptr_t)out & 15u)) return hipErrorNotSupported;
  const bool prod = t.variant == 1;
#define TQ_DQ(MB, P) \
  if (t.mse_bits == MB && prod == P) return run_dequant<MB, P>(t, codes, signs, norms, rnorms, n_sets, n, out, st);
  TQ_DQ(0, true) TQ_DQ(1, false) TQ_DQ(1, true) TQ_DQ(2, false) TQ_DQ(2, true)
  TQ_DQ(3, false) TQ_DQ(3, true) TQ_DQ(4, false) TQ_DQ(4, true)
#undef TQ_DQ
  return hipErrorNotSupported;
}

hipError_t launch_logits128(const DeviceTables &t, const float *q, int64_t nq,
                            const uint8_t *codes, const uint8_t *signs, const float *norms,
                            const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
                            hipStream_t st) {
  if (t.d != D || !t.logit_lut || t.mse_bits > 4) return hipErrorNotSupported;
  const bool prod = t.variant == 1;
#define TQ_L(MB, P) \
  if (t.mse_bits == MB && prod == P) \
    return run_logits<MB, P>(t, q, nq, codes, signs, norms, rnorms, n_sets, n_keys, out, st);
  TQ_L(0, true) TQ_L(1, false) TQ_L(1, true) TQ_L(2, false) TQ_L(2, true)
  TQ_L(3, false) TQ_L(3, true) TQ_L(4, false) TQ_L(4, true)
#undef TQ_L
  return hipErrorNotSupported;
}

hipError_t launch_logits128_mixed(const DeviceTables &to, const DeviceTables &tr, const float *RT, const float *q,
                                  int64_t nq, const uint8_t *codes_o, const uint8_t *codes_r, const float *norms_o,
                                  const float *norms_r, int64_t n_sets, int64_t n_keys, int groups, float *out,
                                  hipStream_t st) {
  if (to.d != 64 || tr.d != 64 || to.variant != 0 || tr.variant != 0 || !RT || !to.logit_lut || !tr.logit_lut)
    return hipErrorNotSupported;
#define TQ_M(O, R) \
  if (to.mse_bits == O && tr.mse_bits == R) \
    return run_logits_mixed<O, R>(to, tr, RT, q, nq, codes_o, codes_r, norms_o, norms_r, n_sets, n_keys, groups, out, st);
  TQ_M(2, 1) TQ_M(3, 2) TQ_M(4, 3)
#undef TQ_M
  return hipErrorNotSupported;
}

static bool attention128_handles(const DeviceTables &tk, const DeviceTables &tv) {
  return tk.d == D && tv.d == D && tk.logit_lut && tv.logit_lut && tk.mse_bits <= 4 && tv.variant == 0 &&
         tv.mse_bits >= 1 && tv.mse_bits <= 4;
}

size_t attention128_workspace(const DeviceTables &tk, const DeviceTables &tv, int64_t nq, int64_t n_sets,
                              int64_t n_keys) {
  if (!attention128_handles(tk, tv) || n_sets < 1 || n_keys < 1 || n_keys > kFusedMaxKeys) return 0;
  int64_t kpw = 0;
  const int64_t gx = attn_grid_x(n_sets, n_keys, &kpw);
  return (size_t)(n_sets * nq * gx) * kAttnPart * sizeof(float);
}

hipError_t launch_attention128(const DeviceTables &tk, const DeviceTables &tv, const float *q, int64_t nq,
                               const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
                               const float *krnorms, const uint8_t *vcodes, const float *vnorms, int64_t n_sets,
                               int64_t n_keys, float scale, float *part, float *out, hipStream_t st) {
  if (!attention128_handles(tk, tv) || n_keys > kFusedMaxKeys) return hipErrorNotSupported;
  const bool prod = tk.variant == 1;
#define TQ_A(MBK, P, MBV)                                                                                 \
  if (tk.mse_bits == MBK && prod == P && tv.mse_bits == MBV)                                              \
    return run_attention<MBK, P, MBV>(tk, tv, q, nq, kcodes, ksigns, knorms, krnorms, vcodes, vnorms, n_sets, \
                                      n_keys, scale, part, out, st);
#define TQ_AV(MBV) \
  TQ_A(0, true, MBV) TQ_A(1, false, MBV) TQ_A(1, true, MBV) TQ_A(2, false, MBV) TQ_A(2, true, MBV) \
  TQ_A(3, false, MBV) TQ_A(3, true, MBV) TQ_A(4, false, MBV) TQ_A(4, true, MBV)
  TQ_AV(1) TQ_AV(2) TQ_AV(3) TQ_AV(4)
#undef TQ_AV
#undef TQ_A
  return hipErrorNotSupported;
}

#endif  // TQ_MSE3_TU

}  // namespace tq
