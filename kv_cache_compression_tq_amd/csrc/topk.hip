// Maximum inner product search over packed codes (d <= 256): for every
// query, the k keys with the largest estimates <q, k_hat> (the logits), best
// first, equal scores by key index.  [ttakun] 索引速度 (vector search on the
// quantized index); [admirer] 第二步 (full-precision query against the
// codes); [tmdm] 双剑合璧 (QJL inner-product estimator).
//
// k_topk_qprep: q~ = Pi q (scaled for the code table) and p = S q
//   (scaled by sqrt(pi/2)/d) per query, zero-padded to 256 coordinates.
// k_topk: a workgroup of 4 waves (one per SIMD) scans one key range; each wave holds 16
//   queries as f16 hi/lo MFMA A operands (two row tiles of 8 queries) and
//   streams 16-key tiles: lane (key, grp) decodes the codes of a quarter of
//   its key's coordinates (d rounded up to 128, 224 or 256) through LDS
//   tables (a code pair per 4-byte read, eight signs -- or eight 1-bit
//   codes -- per 16-byte read).
//   Scores above a query's current k-th best go to a small LDS buffer; a
//   full buffer is merged into the query's running list, which lives in
//   registers (lane i holds the i-th best).  Each wave writes its lists.
// k_topk_merge: one wave per query merges the key ranges' lists.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device_common.h"
#include "kernels.h"

namespace tq {
namespace {

constexpr int kTkThreads = 256;           // one wave per SIMD: 512 registers per wave
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkQ = 16;                  // queries per wave: two row tiles of 8 (hi/lo rows)
constexpr int kTkPad = 256;               // largest dimension; the query rows are zero-padded to it
// A scan with KS contraction steps of 32 coordinates covers 32 KS of them:
// lane group g holds 8 KS g .. 8 KS g + 8 KS - 1 (the dimension rounded up
// to 128, 224 or 256; coordinates past d meet zero query operands).
constexpr int tk_steps(int d) { return d <= 128 ? 4 : d <= 224 ? 7 : 8; }
constexpr int kTkRing = 4;                // tiles held in registers (three in flight)
constexpr int kTkBuf = 64;                // buffered candidates per query
constexpr int kTkMergeAt = kTkBuf - 16;   // a tile adds at most 16 per query
constexpr int kTkSignCopies = 16;         // 16-byte entries 256 bytes apart: 16 lanes a cycle, no conflicts
constexpr uint32_t kTkPairOff = 65536;    // the sign table fills LDS [0, 64 KB)
constexpr uint32_t kTkBufOff = 98304;
constexpr uint32_t kTkBufBytes = kTkQ * kTkBuf * 8 + 64 * 8;  // buffers + a merge staging row
constexpr uint32_t kTkLds = kTkBufOff + kTkWaves * kTkBufBytes;
static_assert(kTkLds <= 160 * 1024, "LDS budget");

template <int MB>
struct TkGeom {  // code-pair table: two codes -> two f16 values (alpha c)
  static constexpr int W = 2 * MB;
  static constexpr int ENTRIES = MB >= 2 ? 1 << W : 1;
  static constexpr int COPIES = MB == 4 ? 32 : 64;
  static constexpr int SHIFT = MB == 4 ? 7 : 8;
  static constexpr uint32_t BYTES = MB >= 2 ? ENTRIES * COPIES * 4 : 0;
  static_assert(BYTES <= kTkBufOff - kTkPairOff, "pair table");
};

// The key data of one 16-key tile in the lane's registers: its key's code
// and sign bits of coordinates 8 KS grp .. 8 KS grp + 8 KS - 1 (bit 0 of
// word 0 first), norm and residual norm.
template <int MB, bool PROD, int KS>
struct TkKey {
  static constexpr int CB = KS * MB, SB = KS;  // code and sign bytes of a lane group
  uint32_t c[MB > 0 ? (CB + 3) / 4 : 1];
  uint32_t s[(SB + 3) / 4];
  float nu, ga;
};

// BYTES bytes from byte offset `at` of a buffer into whole words, bit 0
// first.  Rows are 16-byte aligned, so `at` is a multiple of 4 whenever BYTES
// is; otherwise the covering aligned words are read and funnel-shifted.
template <int BYTES>
__device__ __forceinline__ void tk_load_run(uint32_t (&dst)[(BYTES + 3) / 4], __amdgpu_buffer_rsrc_t r,
                                            uint32_t at) {
  constexpr int NW = (BYTES + 3) / 4;
  if constexpr (BYTES % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b32(r, at + 4 * i, 0, 0);
  } else {
    const uint32_t a0 = at & ~3u, sh = 8 * (at & 3u);
    uint32_t w[NW + 1];
#pragma unroll
    for (int i = 0; i <= NW; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, a0 + 4 * i, 0, 0);
#pragma unroll
    for (int i = 0; i < NW; ++i) dst[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], sh);
  }
}

template <int MB, bool PROD, int KS>
__device__ __forceinline__ void tk_load(TkKey<MB, PROD, KS> &r, int64_t key, int grp,
                                        __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int64_t code_row,
                                        int64_t sign_row, __amdgpu_buffer_rsrc_t rn, __amdgpu_buffer_rsrc_t rg) {
  // codes, signs and norms through buffer resources: bytes past the arrays
  // read as zero, and code bits past d (padding, or the next key's bytes)
  // meet zero query operands; keys past the range are masked by the caller
  using K = TkKey<MB, PROD, KS>;
  if constexpr (MB > 0) tk_load_run<K::CB>(r.c, rc, (uint32_t)(key * code_row) + K::CB * grp);
  if constexpr (PROD) tk_load_run<K::SB>(r.s, rs, (uint32_t)(key * sign_row) + K::SB * grp);
  r.nu = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, (uint32_t)key * 4, 0, 0));
  r.ga = PROD ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)key * 4, 0, 0)) : 0.f;
}

// Scores of one tile for the wave's 16 queries: lane (key, grp) gets queries
// 2 grp, 2 grp + 1 of each row tile (rows 4 grp .. 4 grp + 3 = two queries x
// hi/lo).  MB == 1 decodes the 1-bit codes with the sign table (c[idx] =
// c1 (2 idx - 1); c1 is folded into the query).
// The decoded B operands of one tile: code values (or 1-bit codes as
// signs) and QJL signs of the lane's key for each contraction step.
template <int KS>
struct TkB {
  u32x4 m[KS], s[KS];
};

template <int MB, bool PROD, int KS>
__device__ __forceinline__ void tk_lookup(const TkKey<MB, PROD, KS> &r, uint32_t sbase, uint32_t pbase, TkB<KS> &b) {
  using G = TkGeom<MB>;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if constexpr (MB == 1) {
      const uint32_t byte = (r.c[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      b.m[k] = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)((byte << 8) | sbase);
    } else if constexpr (MB >= 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bit = 8 * k * MB + G::W * i, wi = bit >> 5, sh = bit & 31;
        uint32_t x;
        if (sh + G::W > 32)
          x = __builtin_amdgcn_alignbit(r.c[wi + 1], r.c[wi], sh - G::SHIFT);
        else if (sh >= G::SHIFT)
          x = r.c[wi] >> (sh - G::SHIFT);
        else
          x = r.c[wi] << (G::SHIFT - sh);
        const uint32_t addr = (x & (uint32_t)(((1 << G::W) - 1) << G::SHIFT)) | pbase;
        b.m[k][i] = *(__attribute__((address_space(3))) const uint32_t *)(uintptr_t)addr;
      }
    }
    if constexpr (PROD) {
      const uint32_t byte = (r.s[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      b.s[k] = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)((byte << 8) | sbase);
    }
  }
}

// Scores of one tile for the wave's 16 queries from its decoded operands:
// lane (key, grp) gets queries 2 grp, 2 grp + 1 of each row tile (rows 4 grp
// .. 4 grp + 3 = two queries x hi/lo).  MB == 1 decodes the 1-bit codes with
// the sign table (c[idx] = c1 (2 idx - 1); c1 is folded into the query).
template <int MB, bool PROD, int KS>
__device__ __forceinline__ void tk_mma(const TkB<KS> &b, float nu, float ga, const u32x4 (&qm)[2][KS],
                                       const u32x4 (&qq)[2][KS], float (&sc)[2][2]) {
  f32x4 am[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, aq[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if constexpr (MB > 0) {
      am[0] = mfma_f16(qm[0][k], b.m[k], am[0]);
      am[1] = mfma_f16(qm[1][k], b.m[k], am[1]);
    }
    if constexpr (PROD) {
      aq[0] = mfma_f16(qq[0][k], b.s[k], aq[0]);
      aq[1] = mfma_f16(qq[1][k], b.s[k], aq[1]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float v0 = MB > 0 ? am[rt][0] + am[rt][1] : 0.f, v1 = MB > 0 ? am[rt][2] + am[rt][3] : 0.f;
    if constexpr (PROD) {
      v0 = fmaf(ga, aq[rt][0] + aq[rt][1], v0);
      v1 = fmaf(ga, aq[rt][2] + aq[rt][3], v1);
    }
    sc[rt][0] = v0 * nu;
    sc[rt][1] = v1 * nu;
  }
}

// Float <-> int keys with the same order (for atomicMax on scores).
__device__ __forceinline__ int tk_key(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float tk_unkey(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

// (s, i) ranks before (cs, ci): a larger score, or an equal score and a
// smaller key index.
__device__ __forceinline__ bool tk_better(float s, int i, float cs, int ci) {
  return s > cs || (s == cs && i < ci);
}

// Put candidate (cs, ci) into one query's list (lane l holds its l-th
// best; lanes >= k hold entries worse than the k-th) when it beats the k-th
// best: the entries below it move down one lane.
__device__ __forceinline__ void tk_insert_one(float &ls, int &li, float cs, int ci, int lane) {
  const int pos = __popcll(__ballot(tk_better(ls, li, cs, ci)));
  const float us = __shfl_up(ls, 1);
  const int ui = __shfl_up(li, 1);
  if (lane > pos) {
    ls = us;
    li = ui;
  } else if (lane == pos) {
    ls = cs;
    li = ci;
  }
}

// Merge a sorted list held one entry per lane (vs, vi: lane c holds entry c;
// empty entries are -inf) into the running list.  Entries are taken best
// first, so the first one that does not beat the running k-th best ends it.
__device__ __forceinline__ void tk_insert_list(float &ls, int &li, float vs, int vi, int k, int lane) {
  const int n = __popcll(__ballot(vs != -INFINITY));
  for (int c = 0; c < n; ++c) {
    const float cs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vs), c));
    const int ci = __builtin_amdgcn_readlane(vi, c);
    const float ts = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), k - 1));
    const int ti = __builtin_amdgcn_readlane(li, k - 1);
    if (!tk_better(cs, ci, ts, ti)) break;
    tk_insert_one(ls, li, cs, ci, lane);
  }
}

// Merge a buffer of `cnt` <= 64 candidates (LDS, any order) into one query's
// list in one pass: candidate j lands at (list entries better than it) +
// (candidates better than it); list entry l moves down by the number of
// candidates better than it.  Entries that land at k or beyond drop out.
// `stage` is 64 float2 of LDS that only this wave uses.
__device__ __forceinline__ void tk_merge_batch(float &ls, int &li, const float2 *cand, int cnt, int k, int lane,
                                               float2 *stage) {
  float bs = -INFINITY;
  int bi = 0x7fffffff;
  if (lane < cnt) {
    const float2 e = cand[lane];
    bs = e.x;
    bi = __float_as_int(e.y);
  }
  int rank_b = 0, rank_l = 0, down = 0;  // candidates above my candidate; list above it; candidates above my entry
  for (int j = 0; j < cnt; ++j) {
    const float2 e = cand[j];  // broadcast
    const float cs = e.x;
    const int ci = __float_as_int(e.y);
    rank_b += tk_better(cs, ci, bs, bi) ? 1 : 0;
    down += tk_better(cs, ci, ls, li) ? 1 : 0;
    const int above = __popcll(__ballot(tk_better(ls, li, cs, ci)));
    rank_l = lane == j ? above : rank_l;
  }
  const int pl = lane + down, pb = rank_l + rank_b;
  if (lane < k && pl < k) stage[pl] = float2{ls, __int_as_float(li)};
  if (lane < cnt && pb < k) stage[pb] = float2{bs, __int_as_float(bi)};
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    const float2 e = stage[lane];
    ls = e.x;
    li = __float_as_int(e.y);
  } else {
    ls = -INFINITY;
    li = 0x7fffffff;
  }
  __builtin_amdgcn_wave_barrier();
}

template <int MB, bool PROD, int KS>
__global__ __launch_bounds__(kTkThreads, 1) void k_topk(
    const float *__restrict__ qprep, int nq, const uint8_t *__restrict__ codes, int64_t code_row,
    const uint8_t *__restrict__ signs, int64_t sign_row, const float *__restrict__ norms,
    const float *__restrict__ rnorms, int64_t n_keys, int k, int64_t keys_per_split, const uint32_t *__restrict__ lut,
    float2 *__restrict__ lists, int *__restrict__ gtau) {
  using G = TkGeom<MB>;
  extern __shared__ u32x4 dyn_lds[];  // the kernel's only LDS: starts at address 0
  char *lds = (char *)dyn_lds;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.y, S = gridDim.y;
  const int64_t kb = (int64_t)split * keys_per_split;
  const int64_t ke = kb + keys_per_split < n_keys ? kb + keys_per_split : n_keys;
  const int qbase = (blockIdx.x * kTkWaves + wave) * kTkQ;

  // tables: sign bytes -> eight f16 +-1 (16 copies); code pairs (MB >= 2)
  const uint32_t code_words = MB > 0 ? 1u << (2 * MB) : 0u;
  for (int e = tid; e < 256 * kTkSignCopies; e += kTkThreads)
    ((u32x4 *)lds)[e] = ((const u32x4 *)(lut + code_words))[e / kTkSignCopies];
  if constexpr (MB >= 2)
    for (int e = tid; e < G::ENTRIES * G::COPIES; e += kTkThreads)
      ((uint32_t *)(lds + kTkPairOff))[e] = lut[e / G::COPIES];
  // query operands: row col of a row tile = (query col >> 1, part col & 1);
  // element e of step k is coordinate 8 KS grp + 8 k + e
  u32x4 qm[2][KS], qq[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int q = qbase + rt * 8 + (col >> 1), part = col & 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (q < nq && (m == 0 ? MB > 0 : PROD)) {
          const f32x4 *src = (const f32x4 *)(qprep + ((int64_t)q * 2 + m) * kTkPad + 8 * KS * grp + 8 * ks);
          const f32x4 a = src[0], b = src[1];
          v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
          v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
        }
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x0 = v[2 * i], x1 = v[2 * i + 1];
          if (part) {
            x0 -= (float)(_Float16)x0;
            x1 -= (float)(_Float16)x1;
          }
          w[i] = f16x2(x0, x1);
        }
        (m == 0 ? qm : qq)[rt][ks] = w;
      }
    }
  }
  // the query operands stay in AGPRs (the MFMAs read them from there), which
  // leaves the VGPRs to the tile's table reads
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      asm volatile("" : "+a"(qm[rt][ks]));
      asm volatile("" : "+a"(qq[rt][ks]));
    }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc((void *)codes, 0, MB > 0 ? (int)(n_keys * code_row) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)signs, 0, PROD ? (int)(n_keys * sign_row) : 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc((void *)norms, 0, (int)(n_keys * 4), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rg =
      __builtin_amdgcn_make_buffer_rsrc((void *)rnorms, 0, PROD ? (int)(n_keys * 4) : 0, kBufferFlags);
  const uint32_t sbase = 16 * (lane & (kTkSignCopies - 1));
  const uint32_t pbase = kTkPairOff | (4 * (lane & (G::COPIES - 1)));
  float2 *buf = (float2 *)(lds + kTkBufOff + wave * kTkBufBytes);  // [kTkQ][kTkBuf]

  // running lists (lane l: the l-th best) and thresholds / buffer counts of
  // queries 2 grp + h of each row tile (uniform over the lane's row)
  float ls[kTkQ];
  int li[kTkQ];
#pragma unroll
  for (int i = 0; i < kTkQ; ++i) {
    ls[i] = -INFINITY;
    li[i] = 0x7fffffff;
  }
  float tau[2][2];
  int cnt[2][2] = {{0, 0}, {0, 0}};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h)  // queries past nq never take candidates
      tau[rt][h] = qbase + rt * 8 + 2 * grp + h < nq ? -INFINITY : INFINITY;
  // shared threshold of each query over all key ranges: the largest k-th
  // best score any range's full list has reached.  The final k-th best is at
  // least that, so a key below it cannot make the top k; ties are kept (>=)
  // because keys of other ranges may carry smaller indices.
  float tg[2][2] = {{-INFINITY, -INFINITY}, {-INFINITY, -INFINITY}};
  // the loads are issued two tiles before the values are applied, so that
  // no wait on them stalls the tile that issues them
  int tgn[2][2] = {{0, 0}, {0, 0}};
  auto refresh = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = qbase + rt * 8 + 2 * grp + h;
        tgn[rt][h] = __hip_atomic_load(gtau + (q < nq ? q : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  };
  auto apply = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (qbase + rt * 8 + 2 * grp + h < nq) tg[rt][h] = tk_unkey(tgn[rt][h]);
  };

  auto merge = [&]() __attribute__((always_inline)) {  // every query with buffered candidates
#pragma unroll
    for (int qi = 0; qi < kTkQ; ++qi) {
      const int rt = qi >> 3, r = qi & 7, gq = r >> 1, h = r & 1;
      const int c = __builtin_amdgcn_readlane(cnt[rt][h], 16 * gq);
      if (c > 0) {
        tk_merge_batch(ls[qi], li[qi], buf + qi * kTkBuf, c, k, lane, buf + kTkQ * kTkBuf);
        const float t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[qi]), k - 1));
        if (grp == gq) {
          tau[rt][h] = t;
          cnt[rt][h] = 0;
        }
        if (lane == 0 && t != -INFINITY && qbase + qi < nq) atomicMax(gtau + qbase + qi, tk_key(t));
      }
    }
  };

  // scores of tile t0 (decoded operands b, norms nu, ga) -> candidates
  auto step = [&](const TkB<KS> &b, float nu, float ga, int64_t t0) __attribute__((always_inline)) {
    float sc[2][2];
    tk_mma<MB, PROD, KS>(b, nu, ga, qm, qq, sc);
    const int64_t key = t0 + col;
    const bool valid = key < ke;
    bool cand[2][2];
    bool anyc = false;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        cand[rt][h] = valid && sc[rt][h] > tau[rt][h] && sc[rt][h] >= tg[rt][h];
        anyc |= cand[rt][h];
      }
    if (__ballot(anyc) == 0) return;
    const uint32_t below = (1u << col) - 1u;
    bool full = false;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint64_t m = __ballot(cand[rt][h]);
        const uint32_t row = (uint32_t)(m >> (16 * grp)) & 0xFFFFu;
        if (cand[rt][h]) {
          const int qi = rt * 8 + 2 * grp + h;
          buf[qi * kTkBuf + cnt[rt][h] + __popc(row & below)] = float2{sc[rt][h], __int_as_float((int)key)};
        }
        cnt[rt][h] += __popc(row);
        full |= cnt[rt][h] > kTkMergeAt;
      }
    if (__ballot(full) != 0) merge();
  };
  // a ring of kTkRing tiles in registers (tile i + kTkRing - 1 loads while
  // tile i is scored) and a software pipeline: while the MFMAs of tile i
  // run, the table reads of tile i + 1 are in flight (operand sets b0 / b1
  // alternate)
  const int64_t nt = (ke - kb + 15) / 16;
  TkKey<MB, PROD, KS> ring[kTkRing];
#pragma unroll
  for (int j = 0; j < kTkRing - 1; ++j)
    tk_load<MB, PROD, KS>(ring[j], kb + 16 * j + col, grp, rc, rs, code_row, sign_row, rn, rg);
  TkB<KS> b0, b1;
  tk_lookup<MB, PROD, KS>(ring[0], sbase, pbase, b0);
  float nu0 = ring[0].nu, ga0 = ring[0].ga, nu1 = 0.f, ga1 = 0.f;
  // no branch inside the loop body (a branch there makes the wait-count pass
  // wait for the newest loads): the scan runs whole groups of 8 tiles, and
  // tiles past the range hold keys that are never candidates (past the
  // arrays the buffer loads read zeros)
  for (int64_t i0 = 0; i0 < nt; i0 += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = i0 + j;
      if (j == 5) refresh();
      if (j == 7) apply();
      tk_load<MB, PROD, KS>(ring[(j + kTkRing - 1) % kTkRing], kb + 16 * (i + kTkRing - 1) + col, grp, rc, rs, code_row,
                        sign_row, rn, rg);
      TkB<KS> &bc = (j & 1) ? b1 : b0, &bn = (j & 1) ? b0 : b1;
      float &nuc = (j & 1) ? nu1 : nu0, &gac = (j & 1) ? ga1 : ga0;
      float &nun = (j & 1) ? nu0 : nu1, &gan = (j & 1) ? ga0 : ga1;
      const TkKey<MB, PROD, KS> &rk = ring[(j + 1) % kTkRing];
      tk_lookup<MB, PROD, KS>(rk, sbase, pbase, bn);
      nun = rk.nu;
      gan = rk.ga;
      step(bc, nuc, gac, kb + 16 * i);
    }
  }
  merge();
  // this range's lists
#pragma unroll
  for (int qi = 0; qi < kTkQ; ++qi) {
    const int q = qbase + qi;
    if (q < nq && lane < k) lists[((int64_t)q * S + split) * k + lane] = float2{ls[qi], __int_as_float(li[qi])};
  }
}

// One wave per query: merge the ranges' lists into the final top-k.
__global__ __launch_bounds__(64) void k_topk_merge(const float2 *__restrict__ lists, int S, int k,
                                                  float *__restrict__ out_scores, int32_t *__restrict__ out_idx) {
  const int q = blockIdx.x, lane = threadIdx.x;
  float ls = -INFINITY;
  int li = 0x7fffffff;
  for (int s = 0; s < S; ++s) {  // each list sorted, -inf entries empty
    const float2 e = lane < k ? lists[((int64_t)q * S + s) * k + lane] : float2{-INFINITY, 0.f};
    tk_insert_list(ls, li, e.x, __float_as_int(e.y), k, lane);
  }
  if (lane < k) {
    out_scores[(int64_t)q * k + lane] = ls;
    out_idx[(int64_t)q * k + lane] = li;
  }
}

// ---- score-then-select search for the codecs the fused scan does not take
// (d > 256, more than 4 mse bits, or an index past its 32-bit offsets): the
// logits kernels score a chunk of keys for a block of queries into the
// workspace, k_topk_select keeps each segment's best k, and k_topk_fold
// folds the segments' lists into the query's running list.

// One wave per (segment, query row) of a logits block [rows][n]: the best k
// of keys seg p .. of row i (key numbers offset by key0), into slot 1 + p of
// the row's `slots` lists of k entries.
__global__ __launch_bounds__(64) void k_topk_select(const float *__restrict__ logits, int64_t n, int seg, int k,
                                                    int key0, int slots, float2 *__restrict__ lists) {
  const int p = blockIdx.x, i = blockIdx.y, lane = threadIdx.x;
  const float *row = logits + (int64_t)i * n;
  const int64_t b = (int64_t)p * seg, e = b + seg < n ? b + seg : n;
  float ls = -INFINITY;
  int li = 0x7fffffff;
  float ts = -INFINITY;  // the running k-th best
  int ti = 0x7fffffff;
  for (int64_t j0 = b; j0 < e; j0 += 64) {
    const int64_t j = j0 + lane;
    const bool in = j < e;
    const float v = in ? row[j] : -INFINITY;
    const int id = key0 + (int)j;
    uint64_t m = __ballot(in && tk_better(v, id, ts, ti));
    while (m != 0) {  // candidates of this block, lowest key first
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const float cs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
      const int ci = __builtin_amdgcn_readlane(id, src);
      if (tk_better(cs, ci, ts, ti)) {
        tk_insert_one(ls, li, cs, ci, lane);
        ts = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), k - 1));
        ti = __builtin_amdgcn_readlane(li, k - 1);
      }
    }
  }
  if (lane < k) lists[((int64_t)i * slots + 1 + p) * k + lane] = float2{ls, __int_as_float(li)};
}

// One wave per query row: merge lists first .. count - 1 of the row's
// `slots`, then store the result in list 0 (out_scores null) or as the
// final top k of query q0 + i.
__global__ __launch_bounds__(64) void k_topk_fold(float2 *__restrict__ lists, int slots, int first, int count, int k,
                                                  int64_t q0, float *__restrict__ out_scores,
                                                  int32_t *__restrict__ out_idx) {
  const int i = blockIdx.x, lane = threadIdx.x;
  float ls = -INFINITY;
  int li = 0x7fffffff;
  for (int s = first; s < count; ++s) {
    const float2 e = lane < k ? lists[((int64_t)i * slots + s) * k + lane] : float2{-INFINITY, 0.f};
    tk_insert_list(ls, li, e.x, __float_as_int(e.y), k, lane);
  }
  if (lane < k) {
    if (out_scores) {
      out_scores[(q0 + i) * k + lane] = ls;
      out_idx[(q0 + i) * k + lane] = li;
    } else {
      lists[(int64_t)i * slots * k + lane] = float2{ls, __int_as_float(li)};
    }
  }
}

// q~ = Pi q and p = S q of kTkPrepQ queries per workgroup (each element of
// Pi^T and S^T read from L2 serves all of them), zero-padded to 256; q~ is
// scaled for the code table (1 / alpha, or c1 for 1-bit codes decoded as
// signs), p by sqrt(pi/2) / d.
constexpr int kTkPrepQ = 16;

__global__ __launch_bounds__(kTkPad) void k_topk_qprep(const float *__restrict__ q, int nq, int d, int prod,
                                                       int mse_bits, const float *__restrict__ PiT,
                                                       const float *__restrict__ ST, float mscale,
                                                       float *__restrict__ out, int *__restrict__ gtau) {
  __shared__ float qs[kTkPrepQ][kTkPad];
  const int r0 = blockIdx.x * kTkPrepQ, j = threadIdx.x;
  const int nr = nq - r0 < kTkPrepQ ? nq - r0 : kTkPrepQ;
  for (int r = 0; r < kTkPrepQ; ++r) qs[r][j] = r < nr && j < d ? q[(int64_t)(r0 + r) * d + j] : 0.f;
  __syncthreads();
  float a[kTkPrepQ], b[kTkPrepQ];
#pragma unroll
  for (int r = 0; r < kTkPrepQ; ++r) a[r] = b[r] = 0.f;
  if (j < d) {
    for (int kk = 0; kk < d; ++kk) {
      const float pi = mse_bits > 0 ? PiT[(size_t)kk * d + j] : 0.f;  // (Pi q)_j
      const float sj = prod ? ST[(size_t)kk * d + j] : 0.f;           // (S q)_j
#pragma unroll
      for (int r = 0; r < kTkPrepQ; ++r) {
        a[r] = fmaf(pi, qs[r][kk], a[r]);
        b[r] = fmaf(sj, qs[r][kk], b[r]);
      }
    }
  }
  for (int r = 0; r < nr; ++r) {
    out[((int64_t)(r0 + r) * 2 + 0) * kTkPad + j] = a[r] * mscale;
    out[((int64_t)(r0 + r) * 2 + 1) * kTkPad + j] = b[r] * (kQjlScale / (float)d);
    if (j == 0) gtau[r0 + r] = tk_key(-INFINITY);  // the shared threshold starts empty
  }
}

}  // namespace

// Splits of the key range for nq queries: at least about two workgroups per
// CU, and among up to three times that many the count that fills the last
// round of 256 CUs best (each range at least 1024 keys).
static int topk_splits(int64_t nq, int64_t n_keys) {
  const int64_t qg = (nq + kTkWaves * kTkQ - 1) / (kTkWaves * kTkQ);
  const int64_t smax = n_keys / 1024 > 1 ? n_keys / 1024 : 1;
  int64_t s0 = (512 + qg - 1) / qg;
  if (s0 > smax) s0 = smax;
  if (s0 < 1) s0 = 1;
  int64_t best = s0;
  double best_eff = 0.0;
  for (int64_t s = s0; s <= 3 * s0 && s <= smax; ++s) {
    const int64_t wg = qg * s, rounds = (wg + 255) / 256;
    const double eff = (double)wg / (double)(256 * rounds);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  return (int)best;
}

// Score-then-select geometry: blocks of kFbQueries queries (the logits
// kernels' head count per set), chunks of at most kFbKeys keys, segments of
// kFbSeg keys per selection wave.
constexpr int64_t kFbQueries = 64;
constexpr int64_t kFbKeys = 65536;
constexpr int kFbSeg = 2048;
constexpr int kFbSlots = 1 + (int)(kFbKeys / kFbSeg);  // the running list, then one per segment

static bool fused_topk_handles(const DeviceTables &t, int64_t n_keys) {
  // the scan's buffer offsets are 32-bit
  return t.d <= kTkPad && t.mse_bits <= 4 && t.logit_lut &&
         n_keys * (t.code_row > t.sign_row ? t.code_row : t.sign_row) < ((int64_t)1 << 31);
}

static size_t fallback_workspace(int64_t nq, int64_t n_keys, int k) {
  const int64_t qb = nq < kFbQueries ? nq : kFbQueries, c = n_keys < kFbKeys ? n_keys : kFbKeys;
  return ((size_t)qb * c * sizeof(float) + 255) / 256 * 256 + (size_t)qb * kFbSlots * k * sizeof(float2);
}

static hipError_t run_topk_fallback(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes,
                                    const uint8_t *signs, const float *norms, const float *rnorms, int64_t n_keys,
                                    int k, void *ws, float *out_scores, int32_t *out_idx, hipStream_t st) {
  const int64_t qb = nq < kFbQueries ? nq : kFbQueries, cmax = n_keys < kFbKeys ? n_keys : kFbKeys;
  float *lg = (float *)ws;
  float2 *lists = (float2 *)((char *)ws + ((size_t)qb * cmax * sizeof(float) + 255) / 256 * 256);
  const bool prod = t.variant == 1;
  for (int64_t q0 = 0; q0 < nq; q0 += kFbQueries) {
    const int64_t nb = nq - q0 < kFbQueries ? nq - q0 : kFbQueries;
    for (int64_t k0 = 0; k0 < n_keys; k0 += kFbKeys) {
      const int64_t n = n_keys - k0 < kFbKeys ? n_keys - k0 : kFbKeys;
      const uint8_t *ck = t.mse_bits > 0 ? codes + k0 * t.code_row : codes;
      const uint8_t *sk = prod ? signs + k0 * t.sign_row : signs;
      const float *gk = prod ? rnorms + k0 : rnorms;
      // the block's queries are the heads of one set; logits [nb][n]
      hipError_t e = launch_logits128(t, q + q0 * t.d, nb, ck, sk, norms + k0, gk, 1, n, lg, st);
      if (e == hipErrorNotSupported) e = launch_logits_generic(t, q + q0 * t.d, nb, ck, sk, norms + k0, gk, 1, n, lg, st);
      if (e != hipSuccess) return e;
      const int parts = (int)((n + kFbSeg - 1) / kFbSeg);
      hipLaunchKernelGGL(k_topk_select, dim3((unsigned)parts, (unsigned)nb), dim3(64), 0, st, lg, n, kFbSeg, k,
                         (int)k0, kFbSlots, lists);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      const bool last = k0 + n >= n_keys;
      hipLaunchKernelGGL(k_topk_fold, dim3((unsigned)nb), dim3(64), 0, st, lists, kFbSlots, k0 == 0 ? 1 : 0,
                         1 + parts, k, q0, last ? out_scores : nullptr, last ? out_idx : nullptr);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

size_t topk_workspace(const DeviceTables &t, int64_t nq, int64_t n_keys, int k) {
  if (!fused_topk_handles(t, n_keys)) return fallback_workspace(nq, n_keys, k);
  const size_t prep = (size_t)nq * 2 * kTkPad * sizeof(float);
  const size_t lists = (size_t)nq * topk_splits(nq, n_keys) * k * sizeof(float2);
  return (prep + 255) / 256 * 256 + (lists + 255) / 256 * 256 + (size_t)nq * sizeof(int);
}

template <int MB, bool PROD, int KS>
static hipError_t run_topk(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes,
                           const uint8_t *signs, const float *norms, const float *rnorms, int64_t n_keys, int k,
                           float *ws, float *out_scores, int32_t *out_idx, hipStream_t st) {
  const int S = topk_splits(nq, n_keys);
  float *prep = ws;
  float2 *lists = (float2 *)((char *)ws + ((size_t)nq * 2 * kTkPad * sizeof(float) + 255) / 256 * 256);
  int *gtau = (int *)((char *)lists + ((size_t)nq * S * k * sizeof(float2) + 255) / 256 * 256);
  // 1-bit codes are decoded as signs: c[idx] = c1 (2 idx - 1)
  const float mscale = MB == 1 ? t.pos_cent[0] : t.lut_inv_scale;
  hipLaunchKernelGGL(k_topk_qprep, dim3((unsigned)((nq + kTkPrepQ - 1) / kTkPrepQ)), dim3(kTkPad), 0, st, q, (int)nq,
                     t.d, PROD ? 1 : 0, MB, t.PiT, t.ST, mscale, prep, gtau);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void *)k_topk<MB, PROD, KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kTkLds);
  if (e != hipSuccess) return e;
  const int64_t kps = (n_keys + S - 1) / S;
  const dim3 grid((unsigned)((nq + kTkWaves * kTkQ - 1) / (kTkWaves * kTkQ)), (unsigned)S);
  hipLaunchKernelGGL((k_topk<MB, PROD, KS>), grid, dim3(kTkThreads), kTkLds, st, prep, (int)nq, codes, t.code_row, signs,
                     t.sign_row, norms, rnorms, n_keys, k, kps, t.logit_lut, lists, gtau);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)nq), dim3(64), 0, st, lists, S, k, out_scores, out_idx);
  return hipGetLastError();
}

hipError_t launch_topk(const DeviceTables &t, const float *q, int64_t nq, const uint8_t *codes, const uint8_t *signs,
                       const float *norms, const float *rnorms, int64_t n_keys, int k, void *ws, float *out_scores,
                       int32_t *out_idx, hipStream_t st) {
  if (!fused_topk_handles(t, n_keys))
    return run_topk_fallback(t, q, nq, codes, signs, norms, rnorms, n_keys, k, ws, out_scores, out_idx, st);
  const bool prod = t.variant == 1;
  const int ks = tk_steps(t.d);
#define TQ_T(MB, P)                                                                                               \
  if (t.mse_bits == MB && prod == P) {                                                                           \
    if (ks == 4)                                                                                                 \
      return run_topk<MB, P, 4>(t, q, nq, codes, signs, norms, rnorms, n_keys, k, (float *)ws, out_scores, out_idx, \
                                st);                                                                             \
    if (ks == 7)                                                                                                 \
      return run_topk<MB, P, 7>(t, q, nq, codes, signs, norms, rnorms, n_keys, k, (float *)ws, out_scores, out_idx, \
                                st);                                                                             \
    return run_topk<MB, P, 8>(t, q, nq, codes, signs, norms, rnorms, n_keys, k, (float *)ws, out_scores, out_idx,   \
                              st);                                                                               \
  }
  TQ_T(0, true) TQ_T(1, false) TQ_T(1, true) TQ_T(2, false) TQ_T(2, true)
  TQ_T(3, false) TQ_T(3, true) TQ_T(4, false) TQ_T(4, true)
#undef TQ_T
  return hipErrorNotSupported;
}

}  // namespace tq
