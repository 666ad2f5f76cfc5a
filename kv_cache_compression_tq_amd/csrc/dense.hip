// Dense baseline for the decode-logits comparison: <q, k> for every query of a
// set and every key stored unquantized (float16 or float32), d = 128.  The
// pages compare the attention logits of 4-bit TurboQuant keys with those of
// unquantized keys ([admirer] 內存價格能下來嗎？: up to 8x at 4 bits against
// 32-bit keys; [tmdm] 实测数据): this kernel is that comparison on the same
// hardware.  Not part of the quantized path.
//
// Same tile as the quantized logits kernel: the queries are the MFMA A
// operand (row 2h + part: head h, hi or lo part of its float32 value), 16 keys
// are the B operand (column = key), 4 K steps of 32 coordinates.  float16 keys
// enter the f16 MFMA as loaded (products of f16 values are exact in the f32
// accumulator); float32 keys are split into bf16 hi and lo parts and take two
// bf16 MFMAs per K step, against bf16 hi/lo query rows.  Lane (key, grp) ends
// with heads 2 grp and 2 grp + 1 of its key.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tq {
namespace {

constexpr int D = 128;
constexpr int kDenseThreads = 256;  // 4 waves
constexpr int kDenseTiles = 4;      // 16-key tiles per block (64 keys)

template <bool F32K>
struct DenseRegs {
  u32x4 v[kDenseTiles][4][F32K ? 2 : 1];
};

// Keys key0 .. key0 + 63 of the set (rows past the set read zero).
template <bool F32K>
__device__ __forceinline__ void dense_load(DenseRegs<F32K> &r, __amdgpu_buffer_rsrc_t rs, int64_t key0, int col,
                                           int grp) {
  constexpr uint32_t kRow = F32K ? 4 * D : 2 * D;
#pragma unroll
  for (int u = 0; u < kDenseTiles; ++u) {
    const uint32_t base = (uint32_t)(key0 + 16 * u + col) * kRow;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (F32K) {
        const uint32_t off = base + 128 * k + 32 * grp;  // elements 32 k + 8 grp .. + 8
        r.v[u][k][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        r.v[u][k][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
      } else {
        r.v[u][k][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + 64 * k + 16 * grp, 0, 0);
      }
    }
  }
}

template <bool F32K>
__global__ __launch_bounds__(kDenseThreads) void k_dense_logits128(const float *__restrict__ q, int nq, int h0, int hc,
                                                                   const void *__restrict__ keys, int64_t n_keys,
                                                                   int64_t keys_per_wg, float *__restrict__ out) {
  constexpr uint32_t kRow = F32K ? 4 * D : 2 * D;
  constexpr int BK = 16 * kDenseTiles;
  const int s = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t kbeg = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t kend = kbeg + keys_per_wg < n_keys ? kbeg + keys_per_wg : n_keys;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>((const char *)keys + (int64_t)s * n_keys * kRow), 0, (int)(n_keys * kRow), kBufferFlags);
  const int nblk = (int)((kend - kbeg + BK - 1) / BK);
  int b = wave;
  DenseRegs<F32K> ra, rb;
  if (b < nblk) dense_load<F32K>(ra, rs, kbeg + (int64_t)b * BK, col, grp);

  // query operands: row col = (head col >> 1, part col & 1); element e of K
  // step k is coordinate 32 k + 8 grp + e
  u32x4 aq[4];
  {
    const int h = col >> 1, part = col & 1;
    const float *qh = q + ((int64_t)s * nq + h0 + (h < hc ? h : 0)) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * k + 8 * grp + 2 * i;
        float a0 = h < hc ? qh[c] : 0.f, a1 = h < hc ? qh[c + 1] : 0.f;
        if constexpr (F32K) {
          const uint32_t hi = bf16x2(a0, a1);
          aq[k][i] = part ? bf16x2(a0 - bf16_lo(hi), a1 - bf16_hi(hi)) : hi;
        } else {
          if (part) {
            a0 -= (float)(_Float16)a0;
            a1 -= (float)(_Float16)a1;
          }
          aq[k][i] = f16x2(a0, a1);
        }
      }
  }
  const int hA = 2 * grp, hB = 2 * grp + 1;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(out + (int64_t)s * nq * n_keys, 0, (int)(nq * n_keys * 4), kBufferFlags);
  const uint32_t rowA = hA < hc ? (uint32_t)((h0 + hA) * n_keys) * 4 : kDropped;
  const uint32_t rowB = hB < hc ? (uint32_t)((h0 + hB) * n_keys) * 4 : kDropped;

  auto score_store = [&](const DenseRegs<F32K> &r, int64_t key0) {
#pragma unroll
    for (int u = 0; u < kDenseTiles; ++u) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (F32K) {
          const f32x4 x0 = __builtin_bit_cast(f32x4, r.v[u][k][0]);
          const f32x4 x1 = __builtin_bit_cast(f32x4, r.v[u][k][1]);
          const float f[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          u32x4 kh, kl;
          split8(f, kh, kl);
          acc = mfma_bf16(aq[k], kh, acc);
          acc = mfma_bf16(aq[k], kl, acc);
        } else {
          acc = mfma_f16(aq[k], r.v[u][k][0], acc);
        }
      }
      // keys past the range and heads past hc store at offsets >= 2^31, past
      // the output's num_records (host-checked below 2^31): dropped
      const int64_t key = key0 + 16 * u + col;
      const uint32_t key4 = (uint32_t)key * 4;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0] + acc[1]), ro, key < kend ? rowA + key4 : kDropped,
                                            0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[2] + acc[3]), ro, key < kend ? rowB + key4 : kDropped,
                                            0, 0);
    }
  };
  // blocks wave, wave + 4, ...: the four waves read neighbouring blocks
  while (b < nblk) {
    const int b2 = b + 4 < nblk ? b + 4 : b;  // past the end: re-read block b (no branch around the load)
    dense_load<F32K>(rb, rs, kbeg + (int64_t)b2 * BK, col, grp);
    __builtin_amdgcn_sched_barrier(0);
    score_store(ra, kbeg + (int64_t)b * BK);
    if (b2 == b) break;
    b = b2;
    const int b3 = b + 4 < nblk ? b + 4 : b;
    dense_load<F32K>(ra, rs, kbeg + (int64_t)b3 * BK, col, grp);
    __builtin_amdgcn_sched_barrier(0);
    score_store(rb, kbeg + (int64_t)b * BK);
    if (b3 == b) break;
    b = b3;
  }
}

}  // namespace

hipError_t launch_dense_logits128(const float *q, int64_t nq, const void *keys, int f32_keys, int64_t n_sets,
                                  int64_t n_keys, float *out, hipStream_t st) {
  const int64_t row = f32_keys ? 4 * D : 2 * D;
  // 32-bit buffer offsets: a set's keys (plus one block of overrun) and its
  // logits (below 2^31, so that the dropped offsets lie past them)
  if (n_keys * row > 0xFFFF0000ll || nq * n_keys * 4 > 0x7FFFFFFFll) return hipErrorNotSupported;
  // about eight workgroups per CU in total, each a whole number of 64-key blocks
  const int64_t target = 2048;
  int64_t gx = (target + n_sets - 1) / n_sets;
  int64_t per = (n_keys + gx - 1) / gx;
  per = (per + 63) / 64 * 64;
  gx = (n_keys + per - 1) / per;
  for (int64_t h0 = 0; h0 < nq; h0 += 8) {
    const int hc = (int)(nq - h0 < 8 ? nq - h0 : 8);
    if (f32_keys)
      hipLaunchKernelGGL(k_dense_logits128<true>, dim3((unsigned)gx, (unsigned)n_sets), dim3(kDenseThreads), 0, st, q,
                         (int)nq, (int)h0, hc, keys, n_keys, per, out);
    else
      hipLaunchKernelGGL(k_dense_logits128<false>, dim3((unsigned)gx, (unsigned)n_sets), dim3(kDenseThreads), 0, st,
                         q, (int)nq, (int)h0, hc, keys, n_keys, per, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
