// Quantize for any dimension d (a multiple of 8) on gfx950 matrix cores.
//
// The rotation Y = Pi X is cut into 128 x 128 blocks: output panel p holds
// coordinates [128 p, 128 p + 128), contraction chunk c the input elements
// [128 c, 128 c + 128) (both zero-padded past d).  Every block is stored as
// the same bf16 hi/lo MFMA operand image the d = 128 kernels use (rows
// permuted so that each lane ends up with 32 consecutive coordinates of its
// vector).  A workgroup computes one panel for 128 vectors: the images of the
// chunks go through one LDS buffer (direct global-to-LDS loads), the inputs
// through registers; two workgroups share a CU, so one's MFMAs run while the
// other waits for its next chunk.  After the last chunk the panel's codes
// are searched and packed exactly as at d = 128.
//
// TurboQuant_prod adds a second pass.  The QJL signs need the residual of the
// whole vector, so they are taken as sign(S x - nu M c[idx]) = sign(S r)
// (nu > 0; M = S Pi^T, c[idx] decoded from the codes the first pass wrote),
// a GEMM over 2 d contraction elements with images of S and M.  The residual
// norm is gathered across panels in fixed point (integer atomics, exact and
// order-independent) and finished by panel 0 of the second pass.
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
constexpr uint32_t kImgBytes = kImageVec * 16;
constexpr float kFix = 268435456.f;    // 2^28: fixed-point scale of the residual norm squared

struct TiledArgs {
  int64_t n;             // vectors per set
  int d, chunks, groups;
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

// Direct global-to-LDS copy of one 64 KB image block by the whole workgroup
// (each wave moves 16 KB in 1 KB steps; lane data lands in lane order).
__device__ __forceinline__ void stage_image(const u32x4 *src, u32x4 *dst, int wave, int lane) {
  constexpr int kSteps = kImageVec / 64 / kTiledWaves;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int off = (wave * kSteps + i) * 64;  // u32x4 index of this 1 KB step
    __builtin_amdgcn_global_load_lds((const void *)(src + off + lane),
                                     (__attribute__((address_space(3))) void *)(dst + off), 16, 0, 0);
  }
}

// Input fragments of one chunk for the lane's two vectors: elements
// 128 c + 32 k + 8 grp .. + 8 (bf16 pairs, or raw float32).
template <bool F32IN>
struct XChunk {
  u32x4 v[2][4][F32IN ? 2 : 1];
};

template <bool F32IN>
__device__ __forceinline__ void load_chunk(XChunk<F32IN> &r, const void *xin, const int64_t (&row)[2], int c,
                                           int d, int grp) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = 128 * c + 32 * k + 8 * grp;  // d is a multiple of 8: groups are all in or all out
      if (e0 < d) {
        if constexpr (F32IN) {
          const u32x4 *p = (const u32x4 *)((const float *)xin + row[t] * d + e0);
          r.v[t][k][0] = p[0];
          r.v[t][k][1] = p[1];
        } else {
          r.v[t][k][0] = *(const u32x4 *)((const uint16_t *)xin + row[t] * d + e0);
        }
      } else {
#pragma unroll
        for (int h = 0; h < (F32IN ? 2 : 1); ++h) r.v[t][k][h] = u32x4{0, 0, 0, 0};
      }
    }
}

// acc[t][m] += image block (LDS) x chunk; also ||x||^2 of the chunk's elements.
// Per K step the 16 A fragments (8 row tiles, hi and lo) are read from LDS
// together before that step's MFMAs, so one LDS round trip serves 32 or 48
// MFMAs; the scheduling-group barriers keep the reads in one group.
template <bool F32IN>
__device__ __forceinline__ void mma_chunk(const XChunk<F32IN> &x, const u32x4 *img, int frag_lane,
                                          f32x4 (&acc)[2][8], float (&nsq)[2]) {
  u32x4 bh[2][4], bl[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (F32IN) {
        const f32x4 a = __builtin_bit_cast(f32x4, x.v[t][k][0]);
        const f32x4 b = __builtin_bit_cast(f32x4, x.v[t][k][1]);
        const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(f, bh[t][k], bl[t][k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) nsq[t] = fmaf(f[i], f[i], nsq[t]);
      } else {
        bh[t][k] = x.v[t][k][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_lo(bh[t][k][i]), hi = bf16_hi(bh[t][k][i]);
          nsq[t] = fmaf(lo, lo, fmaf(hi, hi, nsq[t]));
        }
      }
    }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 ah[8], al[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int f = (m * 4 + k) * 2;
      ah[m] = img[f * kFragVec + frag_lane];
      al[m] = img[(f + 1) * kFragVec + frag_lane];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // the 16 LDS reads
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t][m] = mfma_bf16(ah[m], bh[t][k], acc[t][m]);
        acc[t][m] = mfma_bf16(al[m], bh[t][k], acc[t][m]);
        if constexpr (F32IN) acc[t][m] = mfma_bf16(ah[m], bl[t][k], acc[t][m]);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, F32IN ? 48 : 32, 0);  // then the step's MFMAs
  }
}

// Pass 1: rotation panel, norms, search and pack; prod: residual norm partials.
template <int MB, bool PROD, bool F32IN>
__global__ __launch_bounds__(kTiledThreads, 2) void k_tiled_rot(const void *__restrict__ xin, TiledArgs a,
                                                                const u32x4 *__restrict__ img_all,
                                                                const uint32_t *__restrict__ cells,
                                                                const float *__restrict__ cent,
                                                                uint8_t *__restrict__ codes, float *__restrict__ norms,
                                                                int *__restrict__ rn_fix) {
  extern __shared__ u32x4 dyn_lds[];
  u32x4 *buf = dyn_lds;  // the image buffer, then the cell table, then the codebook
  uint32_t *tab = (uint32_t *)((char *)dyn_lds + kImgBytes);
  float *cent_lds = (float *)(tab + a.cell_words);
  const int p = blockIdx.x, s = blockIdx.z, g = s % a.groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int panels = a.chunks;  // square blocks: as many output panels as contraction chunks
  const u32x4 *img = img_all + ((size_t)g * panels + p) * (size_t)a.chunks * kImageVec;

  for (int i = tid; i < a.cell_words; i += kTiledThreads) tab[i] = cells[i];
  if (PROD && MB > 0 && tid < (1 << MB)) cent_lds[tid] = cent[tid];

  const int64_t set_row0 = (int64_t)s * a.n;
  int64_t v[2], row[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v[t] = (int64_t)blockIdx.y * kTiledVectors + 32 * wave + 16 * t + col;
    row[t] = set_row0 + (v[t] < a.n ? v[t] : a.n - 1);  // ragged tail: a valid row, results discarded
  }
  XChunk<F32IN> xa;
  f32x4 acc[2][8];
  float nsq[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0, 0, 0, 0};

  // One image buffer per workgroup and two workgroups per CU: while one waits
  // for its chunk's image and inputs, the other one's MFMAs run.
  for (int c = 0; c < a.chunks; ++c) {
    if (c > 0) __syncthreads();  // every wave is done with the previous image
    stage_image(img + (size_t)c * kImageVec, buf, wave, lane);
    load_chunk<F32IN>(xa, xin, row, c, a.d, grp);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int frag_lane = lane;
    asm volatile("" : "+v"(frag_lane));
    mma_chunk<F32IN>(xa, buf, frag_lane, acc, nsq);
  }

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
    uint32_t w[MB > 0 ? MB : 1];
#pragma unroll
    for (int i = 0; i < (MB > 0 ? MB : 1); ++i) w[i] = 0;
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int coord = 128 * p + 32 * grp + j;  // coordinate of acc[t][j >> 2][j & 3]
      const float y = acc[t][j >> 2][j & 3];
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
    const bool live = v[t] < a.n;
    if constexpr (MB > 0) {
      // the lane's 4 MB bytes at offset 16 p MB + 4 grp MB of the code row; whole
      // words past the row (padding of the last panel) are not stored
      uint8_t *crow = codes + (set_row0 + v[t]) * a.code_row;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int64_t off = (int64_t)16 * p * MB + 4 * grp * MB + 4 * i;
        if (live && off < a.code_row) *(uint32_t *)(crow + off) = w[i];
      }
    }
    if (live && p == 0 && grp == 0) norms[set_row0 + v[t]] = nu;
    if constexpr (PROD) {
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (live && grp == 0 && nu > 0.f) atomicAdd(rn_fix + set_row0 + v[t], (int)rintf(part * kFix));
    }
  }
}

// Pass 2 (prod): signs of S x - nu M c[idx], K = d (x) then d (codes);
// panel 0 also turns the fixed-point residual norms into float32.
template <int MB, bool F32IN>
__global__ __launch_bounds__(kTiledThreads, 2) void k_tiled_sign(const void *__restrict__ xin, TiledArgs a,
                                                                 const u32x4 *__restrict__ img_all,
                                                                 const float *__restrict__ cent,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const float *__restrict__ norms,
                                                                 uint8_t *__restrict__ signs, float *__restrict__ rnorms) {
  extern __shared__ u32x4 dyn_lds[];
  u32x4 *buf = dyn_lds;  // the image buffer, then the codebook
  float *cent_lds = (float *)((char *)dyn_lds + kImgBytes);
  const int p = blockIdx.x, s = blockIdx.z, g = s % a.groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int panels = a.chunks;
  const int kchunks = (MB > 0 ? 2 : 1) * a.chunks;
  const u32x4 *img = img_all + ((size_t)g * panels + p) * (size_t)(2 * a.chunks) * kImageVec;

  if (MB > 0 && tid < (1 << MB)) cent_lds[tid] = cent[tid];

  const int64_t set_row0 = (int64_t)s * a.n;
  int64_t v[2], row[2];
  float nu[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v[t] = (int64_t)blockIdx.y * kTiledVectors + 32 * wave + 16 * t + col;
    row[t] = set_row0 + (v[t] < a.n ? v[t] : a.n - 1);
    nu[t] = norms[row[t]];
  }
  XChunk<F32IN> xa;
  f32x4 acc[2][8];
  float dummy[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0, 0, 0, 0};
  const uint32_t cent_addr = lds_addr(cent_lds);

  // S x over the input chunks (one image buffer, as in pass 1)
  for (int c = 0; c < a.chunks; ++c) {
    if (c > 0) __syncthreads();
    stage_image(img + (size_t)c * kImageVec, buf, wave, lane);
    load_chunk<F32IN>(xa, xin, row, c, a.d, grp);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int frag_lane = lane;
    asm volatile("" : "+v"(frag_lane));
    mma_chunk<F32IN>(xa, buf, frag_lane, acc, dummy);
  }
  // - nu M c[idx] over the code chunks: B = -nu c for coordinates
  // 128 cc + 32 grp + 8 k + e (the lane's 32 codes), split into bf16 hi/lo;
  // coordinates past d meet zero columns
  if constexpr (MB > 0) {
    for (int c = a.chunks; c < kchunks; ++c) {
      __syncthreads();  // every wave is done with the previous image
      stage_image(img + (size_t)c * kImageVec, buf, wave, lane);
      const int cc = c - a.chunks;
      XChunk<true> cx;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t cw[MB];
        const int64_t off = (int64_t)16 * cc * MB + 4 * grp * MB;
        const uint8_t *crow = codes + row[t] * a.code_row;
#pragma unroll
        for (int i = 0; i < MB; ++i) cw[i] = off + 4 * i < a.code_row ? *(const uint32_t *)(crow + off + 4 * i) : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 8 * k + e, bit = j * MB, wi = bit >> 5, sh = bit & 31;
            uint32_t idx = cw[wi] >> sh;
            if (sh + MB > 32) idx |= cw[wi + 1] << (32 - sh);
            idx &= (1u << MB) - 1;
            f[e] = -nu[t] * *(lds_f32 *)(uintptr_t)(cent_addr + 4 * idx);
          }
          cx.v[t][k][0] = __builtin_bit_cast(u32x4, f32x4{f[0], f[1], f[2], f[3]});
          cx.v[t][k][1] = __builtin_bit_cast(u32x4, f32x4{f[4], f[5], f[6], f[7]});
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      int frag_lane = lane;
      asm volatile("" : "+v"(frag_lane));
      mma_chunk<true>(cx, buf, frag_lane, acc, dummy);
    }
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int proj = 128 * p + 32 * grp + j;
      if (proj < a.d && acc[t][j >> 2][j & 3] >= 0.f) bits |= 1u << j;
    }
    const bool live = v[t] < a.n;
    const int64_t off = (int64_t)16 * p + 4 * grp;
    if (live && off < a.sign_row) *(uint32_t *)(signs + (set_row0 + v[t]) * a.sign_row + off) = bits;
    if (live && p == 0 && grp == 0) {
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
  const dim3 grid((unsigned)panels, (unsigned)((n + kTiledVectors - 1) / kTiledVectors), (unsigned)n_sets);
  const size_t lds1 = kImgBytes + 4 * (size_t)a.cell_words + 64;
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
    const size_t lds2 = kImgBytes + 64;
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
