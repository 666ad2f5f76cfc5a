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

#include <cstring>

#include "fast128.h"
#include "kernels.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int kFragVec = 64;                  // u32x4 per fragment (one per lane)
constexpr int kImageVec = 8 * 4 * 2 * kFragVec;  // 8 row tiles x 4 K steps x hi/lo
constexpr int kImageWords = kImageVec * 4;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  b2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Split 8 floats into bf16 hi and lo parts (hi + lo carries 16 significant bits).
__device__ __forceinline__ void split8(const float *f, u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = bf16x2(f[2 * i], f[2 * i + 1]);
    hi[i] = h;
    lo[i] = bf16x2(f[2 * i] - bf16_lo(h), f[2 * i + 1] - bf16_hi(h));
  }
}

struct QuantParams {
  float pos_bnd[8];   // positive boundaries t_{L/2}, ..., t_{L-2}
  float pos_cent[8];  // positive centroids c_{L/2}, ..., c_{L-1}
};

// #{k : T_k < a} over the L/2 - 1 positive scaled boundaries (sorted), by a
// branch-free binary search.
template <int MB>
__device__ __forceinline__ int count_below(float a, const float *T) {
  if constexpr (MB <= 1) {
    return 0;
  } else if constexpr (MB == 2) {
    return T[0] < a ? 1 : 0;
  } else if constexpr (MB == 3) {
    const int b1 = T[1] < a;
    const int b0 = (b1 ? T[2] : T[0]) < a;
    return 2 * b1 + b0;
  } else {
    const int b2 = T[3] < a;
    const int b1 = (b2 ? T[5] : T[1]) < a;
    const float t = b2 ? (b1 ? T[6] : T[4]) : (b1 ? T[2] : T[0]);
    const int b0 = t < a;
    return 4 * b2 + 2 * b1 + b0;
  }
}

template <int MB>
__device__ __forceinline__ float pos_centroid(int cnt, const float *C) {
  if constexpr (MB <= 1) {
    return C[0];
  } else if constexpr (MB == 2) {
    return cnt ? C[1] : C[0];
  } else if constexpr (MB == 3) {
    const float lo = (cnt & 1) ? C[1] : C[0], hi = (cnt & 1) ? C[3] : C[2];
    return (cnt & 2) ? hi : lo;
  } else {
    const float a = (cnt & 1) ? C[1] : C[0], b = (cnt & 1) ? C[3] : C[2];
    const float c = (cnt & 1) ? C[5] : C[4], d = (cnt & 1) ? C[7] : C[6];
    const float ab = (cnt & 2) ? b : a, cd = (cnt & 2) ? d : c;
    return (cnt & 4) ? cd : ab;
  }
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

// One wave quantizes 32 vectors per iteration (two 16-column tiles); a
// workgroup of 4 waves shares the rotation image (and the QJL image) in LDS.
template <int MB, bool PROD, bool F32IN>
__global__ __launch_bounds__(256) void k_quant128(
    const void *__restrict__ xin, int64_t n, int groups, const uint32_t *__restrict__ pi_img,
    const uint32_t *__restrict__ m_img, QuantParams qp, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ signs, float *__restrict__ norms, float *__restrict__ rnorms) {
  extern __shared__ u32x4 lds[];
  constexpr int L = 1 << MB;
  constexpr int NB = MB > 0 ? L / 2 - 1 : 0;  // positive boundaries
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  {
    const u32x4 *src = (const u32x4 *)(pi_img + (size_t)g * kImageWords);
    for (int i = tid; i < kImageVec; i += 256) lds[i] = src[i];
    if constexpr (PROD) {
      const u32x4 *srcm = (const u32x4 *)(m_img + (size_t)g * kImageWords);
      for (int i = tid; i < kImageVec; i += 256) lds[kImageVec + i] = srcm[i];
    }
  }
  __syncthreads();

  const int64_t ntiles = (n + 31) / 32;
  const int64_t set_row0 = (int64_t)s * n;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < ntiles; tile += (int64_t)gridDim.x * 4) {
    const int64_t v0 = tile * 32;
    // prod: both images (128 KB) cannot live in registers; re-read them from LDS
    // each tile (an opaque offset keeps the reads inside the loop)
    int frag_lane = lane;
    if constexpr (PROD) asm volatile("" : "+v"(frag_lane));
    // ---- B operands: x[v][32 k + 8 grp + e], e = 0..7, for K steps k
    u32x4 bx[2][4];
    u32x4 bxl[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t v = v0 + 16 * t + col;
      const bool ok = v < n;
      const int64_t row = set_row0 + (ok ? v : 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (!F32IN) {
          const u32x4 *p = (const u32x4 *)((const uint16_t *)xin + row * D + 32 * k + 8 * grp);
          bx[t][k] = ok ? *p : u32x4{0, 0, 0, 0};
        } else {
          const f32x4 *p = (const f32x4 *)((const float *)xin + row * D + 32 * k + 8 * grp);
          f32x4 a = ok ? p[0] : f32x4{0, 0, 0, 0}, b = ok ? p[1] : f32x4{0, 0, 0, 0};
          const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          split8(f, bx[t][k], bxl[t][k]);
        }
      }
    }
    // ---- rotation: acc[m][t] = rows 16m..16m+15 of the permuted Pi times x
    f32x4 acc[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m][0] = acc[m][1] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int f = (m * 4 + k) * 2;
        const u32x4 ah = lds[f * kFragVec + frag_lane];
        const u32x4 al = lds[(f + 1) * kFragVec + frag_lane];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[m][t] = mfma_bf16(ah, bx[t][k], acc[m][t]);
          acc[m][t] = mfma_bf16(al, bx[t][k], acc[m][t]);
          if constexpr (F32IN) acc[m][t] = mfma_bf16(ah, bxl[t][k], acc[m][t]);
        }
      }
    }
    // ---- epilogue: lane holds y for coordinates 32 grp + 4 m + r of vector v
    u32x4 rh[2][4], rl[2][4];
    float gam2[2], nus[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t v = v0 + 16 * t + col;
      const bool ok = v < n;
      float ss = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss = fmaf(acc[m][t][r], acc[m][t][r], ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float nu = sqrtf(ss);
      const float nthr = nu > 0.f ? nu : 1.f;
      float T[NB > 0 ? NB : 1];
#pragma unroll
      for (int k = 0; k < NB; ++k) T[k] = nthr * qp.pos_bnd[k];
      uint32_t w[MB > 0 ? MB : 1];
#pragma unroll
      for (int i = 0; i < (MB > 0 ? MB : 1); ++i) w[i] = 0;
      float res[32];
      float rs = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 4 * m + r;
          const float y = acc[m][t][r];
          if constexpr (MB > 0) {
            const bool pos = y > 0.f;
            // non-positive y counts boundaries <= |y|: compare with the next float up
            const float a = __uint_as_float((__float_as_uint(y) & 0x7fffffffu) + (pos ? 0u : 1u));
            const int cnt = count_below<MB>(a, T);
            const uint32_t idx = (uint32_t)(cnt ^ (pos ? L / 2 : L / 2 - 1));
            const int bit = j * MB, wi = bit >> 5, sh = bit & 31;
            w[wi] |= idx << sh;
            if (sh + MB > 32) w[wi + 1] |= idx >> (32 - sh);
            if constexpr (PROD) {
              const float cv = pos_centroid<MB>(cnt, qp.pos_cent);
              res[j] = y - nu * (pos ? cv : -cv);
            }
          } else {
            res[j] = y;
          }
          if constexpr (PROD) rs = fmaf(res[j], res[j], rs);
        }
      }
      const int64_t row = set_row0 + v;
      if (ok) {
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
      // ---- QJL: p = M r (rows permuted like the rotation, K = lane chunk order)
      f32x4 pa[8][2];
#pragma unroll
      for (int m = 0; m < 8; ++m) pa[m][0] = pa[m][1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int f = (m * 4 + k) * 2;
          const u32x4 ah = lds[kImageVec + f * kFragVec + frag_lane];
          const u32x4 al = lds[kImageVec + (f + 1) * kFragVec + frag_lane];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            pa[m][t] = mfma_bf16(ah, rh[t][k], pa[m][t]);
            pa[m][t] = mfma_bf16(ah, rl[t][k], pa[m][t]);
            pa[m][t] = mfma_bf16(al, rh[t][k], pa[m][t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int64_t v = v0 + 16 * t + col;
        if (v >= n) continue;
        uint32_t bits = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) bits |= (pa[m][t][r] >= 0.f ? 1u : 0u) << (4 * m + r);
        const int64_t row = set_row0 + v;
        ((uint32_t *)(signs + row * 16))[grp] = bits;
        if (grp == 0) rnorms[row] = nus[t] > 0.f ? sqrtf(gam2[t]) / nus[t] : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------- logits --
constexpr int kLogitTiles = 4;  // 16-key tiles per wave iteration

template <int MB, bool PROD>
__global__ __launch_bounds__(256) void k_logits128(
    const float *__restrict__ q, int nq, int h0, int hc, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ signs, const float *__restrict__ norms,
    const float *__restrict__ rnorms, int64_t n_keys, int groups, const float *__restrict__ PiT,
    const float *__restrict__ ST, const uint32_t *__restrict__ lut, int64_t keys_per_wg,
    float *__restrict__ out) {
  constexpr int P = MB > 0 ? 1 << (2 * MB) : 0;  // pair-table entries
  constexpr int CW = MB;                         // code words per lane (32 coords)
  __shared__ float qs[8 * D];
  __shared__ float qt[8 * D];
  __shared__ float pp[8 * D];
  __shared__ uint32_t t_hi[P > 0 ? P : 1], t_lo[P > 0 ? P : 1];
  __shared__ u32x2 t_sg[16];

  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  for (int e = tid; e < 8 * D; e += 256) {
    const int h = e / D;
    qs[e] = h < hc ? q[((int64_t)s * nq + h0 + h) * D + (e % D)] : 0.f;
  }
  for (int e = tid; e < P; e += 256) {
    t_hi[e] = lut[e];
    t_lo[e] = lut[P + e];
  }
  if (PROD && tid < 16) t_sg[tid] = u32x2{lut[2 * P + 2 * tid], lut[2 * P + 2 * tid + 1]};
  __syncthreads();
  {
    // rotate (threads 0..127) and project (threads 128..255) every head once
    const int j = tid & 127;
    const float *W = tid < 128 ? PiT + (size_t)g * D * D : (PROD ? ST + (size_t)g * D * D : nullptr);
    if (W) {
      float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < D; ++k) {
        const float w = W[(size_t)k * D + j];
#pragma unroll
        for (int h = 0; h < 8; ++h) a[h] = fmaf(w, qs[h * D + k], a[h]);
      }
      float *dst = tid < 128 ? qt : pp;
#pragma unroll
      for (int h = 0; h < 8; ++h) dst[h * D + j] = a[h];
    }
  }
  __syncthreads();
  // B operands: column col = (head col & 7, part col >> 3); contraction
  // element e of K step k is coordinate 32 grp + 8 k + e.
  u32x4 bq[4], bp[4];
  {
    const int h = col & 7, part = col >> 3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * grp + 8 * k + 2 * i;
        float a0 = qt[h * D + c], a1 = qt[h * D + c + 1];
        float p0 = pp[h * D + c], p1 = pp[h * D + c + 1];
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
  const float kscale = kQjlScale / (float)D;
  const int64_t kbeg = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t kend = kbeg + keys_per_wg < n_keys ? kbeg + keys_per_wg : n_keys;
  const int64_t srow = (int64_t)s * n_keys;
  const bool writer = col < hc;
  float *obase = out + ((int64_t)s * nq + h0 + (col & 7)) * n_keys;

  for (int64_t t0 = kbeg + (int64_t)wave * 16 * kLogitTiles; t0 < kend; t0 += 4 * 16 * kLogitTiles) {
    uint32_t cw[kLogitTiles][CW > 0 ? CW : 1];
    uint32_t sw[kLogitTiles];
    f32x4 nv[kLogitTiles], gv[kLogitTiles];
#pragma unroll
    for (int u = 0; u < kLogitTiles; ++u) {
      const int64_t tb = t0 + 16 * u;
      const int64_t key = tb + col;
      const bool ok = key < kend;
      const int64_t row = srow + (ok ? key : kbeg);
      if constexpr (CW == 1) cw[u][0] = *(const uint32_t *)(codes + row * 16 + grp * 4);
      if constexpr (CW == 2) {
        const u32x2 v = *(const u32x2 *)(codes + row * 32 + grp * 8);
        cw[u][0] = v[0];
        cw[u][1] = v[1];
      }
      if constexpr (CW == 3) {
        const u32x3 v = *(const u32x3 *)(codes + row * 48 + grp * 12);
        cw[u][0] = v[0];
        cw[u][1] = v[1];
        cw[u][2] = v[2];
      }
      if constexpr (CW == 4) {
        const u32x4 v = *(const u32x4 *)(codes + row * 64 + grp * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[u][i] = v[i];
      }
      if constexpr (PROD) sw[u] = *(const uint32_t *)(signs + row * 16 + grp * 4);
      // norms of the accumulator rows 4 grp .. 4 grp + 3 of this tile
      const int64_t r0 = tb + 4 * grp;
      if (r0 + 3 < kend) {
        nv[u] = *(const f32x4 *)(norms + srow + r0);
        if constexpr (PROD) gv[u] = *(const f32x4 *)(rnorms + srow + r0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool okr = r0 + r < kend;
          nv[u][r] = okr ? norms[srow + r0 + r] : 0.f;
          if constexpr (PROD) gv[u][r] = okr ? rnorms[srow + r0 + r] : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kLogitTiles; ++u) {
      const int64_t tb = t0 + 16 * u;
      if (tb >= kend) break;
      f32x4 cm = {0, 0, 0, 0}, cq = {0, 0, 0, 0};
      if constexpr (MB > 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          u32x4 ah, al;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // pair 4k + i of the lane's 32 coordinates: 2 MB bits
            const int pr = 4 * k + i;
            const int bit = pr * 2 * MB, wi = bit >> 5, sh = bit & 31;
            uint32_t fld;
            if (sh + 2 * MB <= 32)
              fld = (cw[u][wi] >> sh) & (uint32_t)(P - 1);
            else
              fld = (uint32_t)((((uint64_t)cw[u][wi + 1] << 32) | cw[u][wi]) >> sh) & (uint32_t)(P - 1);
            ah[i] = t_hi[fld];
            al[i] = t_lo[fld];
          }
          cm = mfma_f16(ah, bq[k], cm);
          cm = mfma_f16(al, bq[k], cm);
        }
      }
      if constexpr (PROD) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t byte = (sw[u] >> (8 * k)) & 0xffu;
          const u32x2 lo = t_sg[byte & 15u], hi = t_sg[byte >> 4];
          const u32x4 as = {lo[0], lo[1], hi[0], hi[1]};
          cq = mfma_f16(as, bp[k], cq);
        }
      }
      // combine hi + lo columns (col, col ^ 8), scale, store
      f32x4 res;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = cm[r];
        if constexpr (PROD) v = fmaf(kscale * gv[u][r], cq[r], v);
        const float o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
        res[r] = (v + o) * nv[u][r];
      }
      const int64_t r0 = tb + 4 * grp;
      if (writer) {
        if (r0 + 3 < kend) {
          *(f32x4 *)(obase + r0) = res;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r0 + r < kend) obase[r0 + r] = res[r];
        }
      }
    }
  }
}

template <int MB, bool PROD, bool F32IN>
hipError_t run_quant(const DeviceTables &t, const void *x, int64_t n_sets, int64_t n, uint8_t *codes,
                     uint8_t *signs, float *norms, float *rnorms, hipStream_t st) {
  QuantParams qp;
  for (int k = 0; k < 8; ++k) {
    qp.pos_bnd[k] = t.pos_bnd[k];
    qp.pos_cent[k] = t.pos_cent[k];
  }
  const size_t lds = (PROD ? 2 : 1) * (size_t)kImageVec * sizeof(u32x4);
  hipError_t e = hipFuncSetAttribute((const void *)k_quant128<MB, PROD, F32IN>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (n + 31) / 32;
  const int64_t per_set_max = (ntiles + 3) / 4;  // at least one tile per wave
  const int64_t target = PROD ? 256 : 512;        // one workgroup round (LDS-limited)
  int64_t gx = (target + n_sets - 1) / n_sets;
  if (gx > per_set_max) gx = per_set_max;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_quant128<MB, PROD, F32IN>), dim3((unsigned)gx, (unsigned)n_sets), dim3(256),
                     lds, st, x, n, t.groups, t.pi_frag, t.m_frag, qp, codes, signs, norms, rnorms);
  return hipGetLastError();
}

template <int MB, bool PROD>
hipError_t run_logits(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes,
                      const uint8_t *signs, const float *norms, const float *rnorms, int64_t n_sets,
                      int64_t n_keys, float *out, hipStream_t st) {
  const int64_t unit = 4 * 16 * kLogitTiles;  // keys per workgroup iteration
  int64_t gx = (1024 + n_sets - 1) / n_sets;  // about one round of workgroups
  const int64_t max_gx = (n_keys + unit - 1) / unit;
  if (gx > max_gx) gx = max_gx;
  if (gx < 1) gx = 1;
  int64_t kpw = (n_keys + gx - 1) / gx;
  kpw = (kpw + unit - 1) / unit * unit;
  gx = (n_keys + kpw - 1) / kpw;
  for (int64_t h0 = 0; h0 < nq; h0 += 8) {
    const int hc = (int)(nq - h0 < 8 ? nq - h0 : 8);
    hipLaunchKernelGGL((k_logits128<MB, PROD>), dim3((unsigned)gx, (unsigned)n_sets), dim3(256), 0,
                       st, q, (int)nq, (int)h0, hc, codes, signs, norms, rnorms, n_keys, t.groups,
                       t.PiT, t.ST, t.logit_lut, kpw, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

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

void fast128_build_rotation_image(const double *mat, int k_order, uint32_t *out) {
  memset(out, 0, (size_t)kImageWords * 4);
  for (int m = 0; m < 8; ++m)
    for (int k = 0; k < 4; ++k)
      for (int part = 0; part < 2; ++part) {
        const int f = (m * 4 + k) * 2 + part;
        for (int lane = 0; lane < 64; ++lane) {
          const int rho = lane & 15, grp = lane >> 4;
          const int orow = 32 * (rho >> 2) + 4 * m + (rho & 3);
          for (int e = 0; e < 8; ++e) {
            const int kin = k_order == 0 ? 32 * k + 8 * grp + e : 32 * grp + 8 * k + e;
            const float v = (float)mat[(size_t)orow * D + kin];
            const uint16_t hi = host_bf16(v);
            const uint16_t val = part == 0 ? hi : host_bf16(v - host_bf16_to_f(hi));
            out[((size_t)f * 64 + lane) * 4 + e / 2] |= (uint32_t)val << (16 * (e & 1));
          }
        }
      }
}

size_t fast128_lut_words(int mse_bits) {
  const size_t P = mse_bits > 0 ? (size_t)1 << (2 * mse_bits) : 0;
  return 2 * P + 32;
}

void fast128_build_logit_lut(const float *cent, int mse_bits, uint32_t *out) {
  const int P = mse_bits > 0 ? 1 << (2 * mse_bits) : 0;
  auto h16 = [](float f) {
    _Float16 h = (_Float16)f;
    uint16_t u;
    memcpy(&u, &h, 2);
    return u;
  };
  auto f16val = [](float f) { return (float)(_Float16)f; };
  for (int e = 0; e < P; ++e) {
    const int a = e & ((1 << mse_bits) - 1), b = e >> mse_bits;
    out[e] = (uint32_t)h16(cent[a]) | ((uint32_t)h16(cent[b]) << 16);
    out[P + e] = (uint32_t)h16(cent[a] - f16val(cent[a])) |
                 ((uint32_t)h16(cent[b] - f16val(cent[b])) << 16);
  }
  for (int nib = 0; nib < 16; ++nib)
    for (int w = 0; w < 2; ++w) {
      uint32_t v = 0;
      for (int half = 0; half < 2; ++half) {
        const int e = 2 * w + half;
        const uint16_t h = ((nib >> e) & 1) ? 0x3C00u : 0xBC00u;  // +1 / -1
        v |= (uint32_t)h << (16 * half);
      }
      out[2 * P + 2 * nib + w] = v;
    }
}

hipError_t launch_quant128(const DeviceTables &t, const void *x, int dtype, int64_t n_sets,
                           int64_t n, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                           hipStream_t st) {
  if (t.d != D || !t.pi_frag || t.mse_bits > 4 || ((uintptr_t)x & 15u)) return hipErrorNotSupported;
  const bool prod = t.variant == 1, f32 = dtype == 0;
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

hipError_t launch_logits128(const DeviceTables &t, const float *q, int64_t nq,
                            const uint8_t *codes, const uint8_t *signs, const float *norms,
                            const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
                            hipStream_t st) {
  if (t.d != D || !t.logit_lut || t.mse_bits > 4 || (n_keys & 3) || ((uintptr_t)norms & 15u) ||
      ((uintptr_t)out & 15u) || (rnorms && ((uintptr_t)rnorms & 15u)))
    return hipErrorNotSupported;
  const bool prod = t.variant == 1;
#define TQ_L(MB, P) \
  if (t.mse_bits == MB && prod == P) \
    return run_logits<MB, P>(t, q, nq, codes, signs, norms, rnorms, n_sets, n_keys, out, st);
  TQ_L(0, true) TQ_L(1, false) TQ_L(1, true) TQ_L(2, false) TQ_L(2, true)
  TQ_L(3, false) TQ_L(3, true) TQ_L(4, false) TQ_L(4, true)
#undef TQ_L
  return hipErrorNotSupported;
}

}  // namespace tq
