// Dimension-generic kernels (any 2 <= d <= 4096): one workgroup per vector for
// quantize/dequantize, one thread per key for logits.  Plain fp32 VALU
// arithmetic.  They serve every shape the d = 128 MFMA kernels do not.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

__device__ inline float load_x(const float *p, int64_t i) { return p[i]; }
__device__ inline float load_x(const uint16_t *p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> f32 exactly
}

__device__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

// Read field j (width mb bits) of an LSB-first bit stream.
__device__ inline int read_field(const uint8_t *row, int j, int mb) {
  const int bit = j * mb;
  const int byte = bit >> 3, sh = bit & 7;
  uint32_t w = row[byte];
  if (sh + mb > 8) w |= (uint32_t)row[byte + 1] << 8;
  return (int)((w >> sh) & ((1u << mb) - 1u));
}

// TurboQuant_mse / _prod quantize of V vectors of one set per workgroup
// (grid: chunk of V vectors x set), so that every element of Pi^T (and M^T)
// read from L2 serves V vectors.  Shared memory: x[V][d], y[V][d] (later the
// residual), idx[V][d] (int; reused for the sign bits once the codes are
// packed), then the boundaries.  The index of y is the number of k with
// nu t_k < y, found by halving over the boundaries in LDS (the products
// nu t_k are monotone in k, so this is the plain count).
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void k_quant_generic(
    const T *__restrict__ x, int d, int64_t n, int groups, int mse_bits, int prod,
    const float *__restrict__ PiT, const float *__restrict__ MT, const float *__restrict__ cent,
    const float *__restrict__ bnd, uint8_t *__restrict__ codes, int64_t code_row,
    uint8_t *__restrict__ signs, int64_t sign_row, float *__restrict__ norms,
    float *__restrict__ rnorms) {
  extern __shared__ float sm[];
  __shared__ float red[kThreads / 64];
  float *xs = sm, *ys = sm + V * d;
  int *is = (int *)(sm + 2 * V * d), *bs = is;
  float *tb = sm + 3 * V * d;
  const int s = blockIdx.y;
  const int g = s % groups;
  const int64_t i0 = (int64_t)blockIdx.x * V;
  const int nv = (int)min((int64_t)V, n - i0);  // vectors of this workgroup (the set's last one may hold fewer)
  const int64_t row0 = (int64_t)s * n + i0;
  const int tid = threadIdx.x;
  const int L = 1 << mse_bits;
  for (int k = tid; k + 1 < L; k += kThreads) tb[k] = bnd[k];

  float nu[V], nthr[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float acc = 0.f;
    for (int j = tid; j < d; j += kThreads) {
      const float e = v < nv ? load_x(x + (row0 + v) * d, j) : 0.f;
      xs[v * d + j] = e;
      acc = fmaf(e, e, acc);
    }
    nu[v] = sqrtf(block_sum(acc, red));
    nthr[v] = nu[v] > 0.f ? nu[v] : 1.f;  // a zero vector has y = 0
  }
  __syncthreads();

  // y = Pi x  (PiT[k][j] = Pi[j][k]; consecutive threads read consecutive j)
  const float *P = PiT + (size_t)g * d * d;
  for (int j = tid; j < d; j += kThreads) {
    float y[V];
#pragma unroll
    for (int v = 0; v < V; ++v) y[v] = 0.f;
    for (int k = 0; k < d; ++k) {
      const float pk = P[(size_t)k * d + j];
#pragma unroll
      for (int v = 0; v < V; ++v) y[v] = fmaf(pk, xs[v * d + k], y[v]);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      int idx = 0;
      if (mse_bits > 0)
        for (int step = L >> 1; step > 0; step >>= 1)
          if (nthr[v] * tb[idx + step - 1] < y[v]) idx += step;
      is[v * d + j] = idx;
      // prod residual in the rotated domain: Pi r * ||x|| = y - ||x|| c[idx]
      ys[v * d + j] = mse_bits > 0 ? y[v] - nu[v] * cent[idx] : y[v];
    }
  }
  __syncthreads();

  for (int v = 0; v < nv; ++v) {
    const int64_t row = row0 + v;
    if (mse_bits > 0) {
      uint8_t *crow = codes + row * code_row;
      for (int byte = tid; byte < code_row; byte += kThreads) {
        uint32_t w = 0;
        for (int q = 0; q < 8; ++q) {
          const int sb = byte * 8 + q, j = sb / mse_bits, k = sb % mse_bits;
          if (j < d) w |= (uint32_t)((is[v * d + j] >> k) & 1) << q;
        }
        crow[byte] = (uint8_t)w;
      }
    }
    if (tid == 0) norms[row] = nu[v];
  }
  if (!prod) return;

  float rn[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float r2 = 0.f;
    for (int j = tid; j < d; j += kThreads) r2 = fmaf(ys[v * d + j], ys[v * d + j], r2);
    rn[v] = sqrtf(block_sum(r2, red));  // syncs first: the codes above are packed before bs overwrites is
  }
  // sign(S r) = sign(M (Pi r)), M = S Pi^T
  const float *M = MT + (size_t)g * d * d;
  for (int i = tid; i < d; i += kThreads) {
    float pr[V];
#pragma unroll
    for (int v = 0; v < V; ++v) pr[v] = 0.f;
    for (int j = 0; j < d; ++j) {
      const float mj = M[(size_t)j * d + i];
#pragma unroll
      for (int v = 0; v < V; ++v) pr[v] = fmaf(mj, ys[v * d + j], pr[v]);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) bs[v * d + i] = pr[v] >= 0.f ? 1 : 0;
  }
  __syncthreads();
  for (int v = 0; v < nv; ++v) {
    const int64_t row = row0 + v;
    uint8_t *srow = signs + row * sign_row;
    for (int byte = tid; byte < sign_row; byte += kThreads) {
      uint32_t w = 0;
      for (int q = 0; q < 8; ++q) {
        const int i = byte * 8 + q;
        if (i < d) w |= (uint32_t)bs[v * d + i] << q;
      }
      srow[byte] = (uint8_t)w;
    }
    if (tid == 0) rnorms[row] = nu[v] > 0.f ? rn[v] / nu[v] : 0.f;
  }
}

// ------------------------------------------------------- mixed precision --
// Channel split of an outlier-channel mixed codec: perm[g] lists the outlier
// channels of group g, then the regular ones.  Row r of a set of n rows uses
// group (r / n) % groups.  One thread per element.
template <typename T>
__global__ void k_gather_parts(const T *__restrict__ x, int64_t rows, int64_t n, int groups, int d, int n_out,
                               const int32_t *__restrict__ perm, T *__restrict__ xo, T *__restrict__ xr) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * d) return;
  const int64_t row = e / d;
  const int c = (int)(e % d);
  const int g = (int)((row / n) % groups);
  const T v = x[row * d + perm[(int64_t)g * d + c]];
  if (c < n_out)
    xo[row * n_out + c] = v;
  else
    xr[row * (d - n_out) + (c - n_out)] = v;
}

__global__ void k_scatter_parts(const float *__restrict__ xo, const float *__restrict__ xr, int64_t rows, int64_t n,
                                int groups, int d, int n_out, const int32_t *__restrict__ perm,
                                float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * d) return;
  const int64_t row = e / d;
  const int c = (int)(e % d);
  const int g = (int)((row / n) % groups);
  out[row * d + perm[(int64_t)g * d + c]] = c < n_out ? xo[row * n_out + c] : xr[row * (d - n_out) + (c - n_out)];
}

__global__ void k_add_inplace(float *__restrict__ out, const float *__restrict__ in, int64_t count) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < count) out[e] += in[e];
}

// ---------------------------------------------------------------- append --
// One vector per set written straight into row rows[s] of a (paged) cache:
// the online path of the pages ([ttakun] TurboQuant_mse: no training, one
// vector at a time).  One 512-thread workgroup per set, tuned for latency:
// the d x d contractions run as nsl slices of d/nsl steps per output
// coordinate (Pi^T and M^T columns read coalesced from L2), reduced in LDS;
// codes are packed a 32-bit word per thread, signs by ballot.  A row outside
// [0, cache_rows) is skipped.
//
// DC = 128 is the compile-time form for d = 128 (4 slices of 32 steps): each
// thread loads its 32 Pi^T (and 32 M^T) entries into registers at entry,
// together with the row index and x, so the whole kernel waits on global
// memory once; a skipped row only drops the stores.
constexpr int kAppendThreads = 512;
constexpr int kAppendSpan = 32;  // contraction steps per thread for d = 128

template <typename T, int DC>
__global__ __launch_bounds__(kAppendThreads) void k_append(
    const T *__restrict__ x, int d_arg, int groups, int mse_bits, int prod, const int64_t *__restrict__ rows,
    int64_t cache_rows, const float *__restrict__ PiT, const float *__restrict__ MT, const float *__restrict__ cent,
    const float *__restrict__ bnd, uint8_t *__restrict__ codes, int64_t code_row, uint8_t *__restrict__ signs,
    int64_t sign_row, float *__restrict__ norms, float *__restrict__ rnorms) {
  static_assert(DC == 0 || DC * 4 == kAppendThreads, "the fixed form has 4 slices of d / 4 steps");
  extern __shared__ float sm[];  // xs[d], part[kAppendThreads], ys[d], idx[d]
  __shared__ float red[kAppendThreads / 64];
  const int d = DC > 0 ? DC : d_arg;
  float *xs = sm, *part = sm + d, *ys = part + kAppendThreads;
  int *is = (int *)(ys + d);
  const int s = blockIdx.x, tid = threadIdx.x;
  const int g = s % groups;
  const int64_t row = rows[s];
  float pr[DC > 0 ? kAppendSpan : 1], mr[DC > 0 ? kAppendSpan : 1];
  if constexpr (DC > 0) {
    // thread (slice, j): Pi^T[k][j] and M^T[k][j] for k in [32 slice, 32 slice + 32)
    const size_t off = (size_t)g * DC * DC + (size_t)(kAppendSpan * (tid / DC)) * DC + tid % DC;
#pragma unroll
    for (int u = 0; u < kAppendSpan; ++u) pr[u] = PiT[off + (size_t)u * DC];
    if (prod) {
#pragma unroll
      for (int u = 0; u < kAppendSpan; ++u) mr[u] = MT[off + (size_t)u * DC];
    }
  } else {
    if (row < 0 || row >= cache_rows) return;  // the whole workgroup leaves together
  }
  const bool keep = row >= 0 && row < cache_rows;
  const int nsl = d <= kAppendThreads ? kAppendThreads / d : 1;  // contraction slices per coordinate
  const int span = (d + nsl - 1) / nsl;
  const T *xv = x + (int64_t)s * d;
  __shared__ float cl[DC > 0 ? 256 : 1];  // the fixed form's codebook copy (at most 8 bits)
  float acc = 0.f;
  if constexpr (DC > 0) {
    // x and the codebook are loaded before either is stored, so the kernel's
    // loads all share one wait; the row index is forced into registers there too
    // (unconditional loads at clamped indices: the table holds at least one entry)
    const int L = mse_bits > 0 ? 1 << mse_bits : 1;
    const float cv = cent[tid < L ? tid : L - 1];
    const float v = load_x(xv, tid < DC ? tid : DC - 1);
    asm volatile("" ::"s"(row));
    if (mse_bits > 0 && tid < L) cl[tid] = cv;
    if (tid < DC) {
      xs[tid] = v;
      acc = v * v;
    }
  } else {
    for (int j = tid; j < d; j += kAppendThreads) {
      const float v = load_x(xv, j);
      xs[j] = v;
      acc = fmaf(v, v, acc);
    }
  }
  const float nu = sqrtf(block_sum(acc, red));  // block_sum syncs before it reads
  const float nthr = nu > 0.f ? nu : 1.f;
  // y = Pi x: thread (slice, j) sums its span of k (PiT[k][j] = Pi[j][k])
  auto contract_regs = [&](const float (&rg)[DC > 0 ? kAppendSpan : 1], const float *vin, float *vout) {
    const int k0 = kAppendSpan * (tid / (DC > 0 ? DC : 1));
    float p4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kAppendSpan; ++u) p4[u & 3] = fmaf(rg[u], vin[k0 + u], p4[u & 3]);
    part[tid] = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    __syncthreads();
    if (tid < DC) vout[tid] = (part[tid] + part[DC + tid]) + (part[2 * DC + tid] + part[3 * DC + tid]);
    __syncthreads();
  };
  auto contract = [&](const float *Mt, const float *vin, float *vout) {
    for (int j0 = 0; j0 < d; j0 += kAppendThreads / nsl) {
      const int j = j0 + tid % (kAppendThreads / nsl), sl = tid / (kAppendThreads / nsl);
      float a = 0.f;
      if (j < d && sl < nsl) {
        const int k0 = sl * span, k1 = min(d, k0 + span);
        // eight independent partial sums keep eight L2 loads in flight
        float p8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int k = k0;
        for (; k + 8 <= k1; k += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) p8[u] = fmaf(Mt[(size_t)(k + u) * d + j], vin[k + u], p8[u]);
        }
        for (; k < k1; ++k) p8[0] = fmaf(Mt[(size_t)k * d + j], vin[k], p8[0]);
        a = ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
      }
      __syncthreads();
      part[tid] = a;
      __syncthreads();
      if (tid < kAppendThreads / nsl && j0 + tid < d) {
        float v = 0.f;
        for (int q = 0; q < nsl; ++q) v += part[q * (kAppendThreads / nsl) + tid];
        vout[j0 + tid] = v;
      }
    }
    __syncthreads();
  };
  if constexpr (DC > 0)
    contract_regs(pr, xs, ys);
  else
    contract(PiT + (size_t)g * d * d, xs, ys);
  const int L = 1 << mse_bits;
  for (int j = tid; j < d; j += kAppendThreads) {
    const float y = ys[j];
    int idx = 0;
    if (mse_bits > 0)
      for (int k = 0; k + 1 < L; ++k) idx += fmaf(nthr, bnd[k], -y) < 0.f ? 1 : 0;  // nu t_k < y
    is[j] = idx;
    const float c = mse_bits > 0 ? (DC > 0 ? cl[idx] : cent[idx]) : 0.f;
    ys[j] = mse_bits > 0 ? y - nu * c : y;  // nu times the rotated residual
  }
  __syncthreads();
  if (mse_bits > 0 && keep) {
    uint32_t *crow = (uint32_t *)(codes + row * code_row);
    for (int w = tid; w < (int)(code_row / 4); w += kAppendThreads) {
      uint32_t v = 0;
      const int b0 = 32 * w;
      for (int j = b0 / mse_bits; j < d && j * mse_bits < b0 + 32; ++j) {
        const int sh = j * mse_bits - b0;  // may be negative for the field that straddles in
        const uint32_t f = (uint32_t)is[j];
        v |= sh >= 0 ? f << sh : f >> (-sh);
      }
      crow[w] = v;
    }
  }
  if (tid == 0 && keep) norms[row] = nu;
  if (!prod) return;
  float r2 = 0.f;
  for (int j = tid; j < d; j += kAppendThreads) r2 = fmaf(ys[j], ys[j], r2);
  const float rn = sqrtf(block_sum(r2, red));
  // sign(S r) = sign(M (Pi r)) with M = S Pi^T (MT[j][i] = M[i][j]); xs is free now
  if constexpr (DC > 0)
    contract_regs(mr, ys, xs);
  else
    contract(MT + (size_t)g * d * d, ys, xs);
  uint32_t *srow = (uint32_t *)(signs + row * sign_row);
  for (int i0 = 0; i0 < (int)(sign_row * 8); i0 += kAppendThreads) {
    const int i = i0 + tid;
    const uint64_t m = __ballot(i < d && xs[i] >= 0.f);
    if ((tid & 63) == 0 && keep) {
      const int w = i >> 5;  // lane 0 of each wave writes its 64 bits
      if (w < (int)(sign_row / 4)) srow[w] = (uint32_t)m;
      if (w + 1 < (int)(sign_row / 4)) srow[w + 1] = (uint32_t)(m >> 32);
    }
  }
  if (tid == 0 && keep) rnorms[row] = nu > 0.f ? rn / nu : 0.f;
}

// Reconstruction of V vectors of one set per workgroup (grid: chunk x set):
// out = nu (Pi^T c[idx] + sqrt(pi/2)/d * gamma * S^T z), every element of Pi
// and S read from L2 serving V vectors.
template <int V>
__global__ __launch_bounds__(kThreads) void k_dequant_generic(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ signs,
    const float *__restrict__ norms, const float *__restrict__ rnorms, int d, int64_t n,
    int groups, int mse_bits, int prod, const float *__restrict__ Pi, const float *__restrict__ S,
    const float *__restrict__ cent, int64_t code_row, int64_t sign_row, float *__restrict__ out) {
  extern __shared__ float sm[];
  float *cv = sm, *zv = sm + V * d;
  const int s = blockIdx.y;
  const int g = s % groups;
  const int64_t i0 = (int64_t)blockIdx.x * V;
  const int nv = (int)min((int64_t)V, n - i0);
  const int64_t row0 = (int64_t)s * n + i0;
  const int tid = threadIdx.x;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t row = row0 + (v < nv ? v : 0);  // rows past the set repeat the first (not stored)
    const uint8_t *crow = codes ? codes + row * code_row : nullptr;
    const uint8_t *srow = prod ? signs + row * sign_row : nullptr;
    for (int j = tid; j < d; j += kThreads) {
      cv[v * d + j] = mse_bits > 0 ? cent[read_field(crow, j, mse_bits)] : 0.f;
      if (prod) zv[v * d + j] = ((srow[j >> 3] >> (j & 7)) & 1) ? 1.f : -1.f;
    }
  }
  __syncthreads();
  float nu[V], w[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t row = row0 + (v < nv ? v : 0);
    nu[v] = norms[row];
    w[v] = prod ? kQjlScale / (float)d * rnorms[row] : 0.f;
  }
  const float *P = Pi + (size_t)g * d * d, *Sg = S ? S + (size_t)g * d * d : nullptr;
  for (int i = tid; i < d; i += kThreads) {
    float a[V], b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) a[v] = b[v] = 0.f;
    if (mse_bits > 0)
      for (int j = 0; j < d; ++j) {
        const float pj = P[(size_t)j * d + i];
#pragma unroll
        for (int v = 0; v < V; ++v) a[v] = fmaf(pj, cv[v * d + j], a[v]);
      }
    if (prod)
      for (int j = 0; j < d; ++j) {
        const float sj = Sg[(size_t)j * d + i];
#pragma unroll
        for (int v = 0; v < V; ++v) b[v] = fmaf(sj, zv[v * d + j], b[v]);
      }
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (v < nv) out[(row0 + v) * d + i] = nu[v] * fmaf(w[v], b[v], a[v]);
  }
}

// Logits: each workgroup rotates/projects the queries of its set (heads in
// chunks of up to HC) into LDS as [coordinate][HC] -- one 16-byte read gives
// four heads -- beside the codebook; then each thread scores keys one at a
// time.  A key's code row streams through a 64-bit window filled by aligned
// 32-bit loads (rows are 16-byte aligned and padded), each field indexes the
// LDS codebook, and the sign row is read a word per 32 projections.
constexpr int kMaxHeads = 8;
constexpr int kKeysPerThread = 8;

template <int HC>
__global__ __launch_bounds__(kThreads) void k_logits_generic(
    const float *__restrict__ q, int nq, int h0, int hc, const uint8_t *__restrict__ codes,
    const uint8_t *__restrict__ signs, const float *__restrict__ norms,
    const float *__restrict__ rnorms, int d, int64_t n_keys, int groups, int mse_bits, int prod,
    const float *__restrict__ PiT, const float *__restrict__ ST, const float *__restrict__ cent,
    int64_t code_row, int64_t sign_row, float *__restrict__ out) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  extern __shared__ f4 sm4[];
  float *qt = (float *)sm4, *pp = qt + HC * d, *cl = pp + HC * d;
  const int s = blockIdx.y;
  const int g = s % groups;
  const int tid = threadIdx.x;
  if (mse_bits > 0)
    for (int e = tid; e < (1 << mse_bits); e += kThreads) cl[e] = cent[e];
  // (Pi q)_j and (S q)_j of head h at [j][h]; heads past hc are zero
  const float *P = PiT + (size_t)g * d * d;
  const float *Sg = prod ? ST + (size_t)g * d * d : nullptr;
  for (int e = tid; e < HC * d; e += kThreads) {
    const int h = e / d, j = e % d;  // consecutive threads: consecutive j (coalesced PiT reads)
    float a = 0.f, b = 0.f;
    if (h < hc) {
      const float *qh = q + ((int64_t)s * nq + h0 + h) * d;
      for (int k = 0; k < d; ++k) {
        const float qk = qh[k];
        a = fmaf(P[(size_t)k * d + j], qk, a);
        if (prod) b = fmaf(Sg[(size_t)k * d + j], qk, b);
      }
    }
    qt[j * HC + h] = a;
    pp[j * HC + h] = b;
  }
  __syncthreads();
  const float ks = kQjlScale / (float)d;
  const uint32_t mask = mse_bits > 0 ? (1u << mse_bits) - 1u : 0u;
  for (int kk = 0; kk < kKeysPerThread; ++kk) {
    const int64_t t = ((int64_t)blockIdx.x * kKeysPerThread + kk) * kThreads + tid;
    if (t >= n_keys) break;
    const int64_t row = (int64_t)s * n_keys + t;
    f4 am[HC / 4], as[HC / 4];
#pragma unroll
    for (int i = 0; i < HC / 4; ++i) am[i] = as[i] = f4{0.f, 0.f, 0.f, 0.f};
    if (mse_bits > 0) {
      const uint32_t *cw = (const uint32_t *)(codes + row * code_row);
      uint64_t win = 0;
      int have = 0, wi = 0;
      for (int j = 0; j < d; ++j) {
        if (have < mse_bits) {  // the field continues in the next word
          win |= (uint64_t)cw[wi++] << have;
          have += 32;
        }
        const float c = cl[(uint32_t)win & mask];
        win >>= mse_bits;
        have -= mse_bits;
        const f4 *qv = (const f4 *)(qt + j * HC);
#pragma unroll
        for (int i = 0; i < HC / 4; ++i) am[i] += qv[i] * c;
      }
    }
    if (prod) {
      const uint32_t *sw = (const uint32_t *)(signs + row * sign_row);
      uint32_t w = 0;
      for (int j = 0; j < d; ++j) {
        if ((j & 31) == 0) w = sw[j >> 5];
        const float z = (w & 1u) ? 1.f : -1.f;
        w >>= 1;
        const f4 *pv = (const f4 *)(pp + j * HC);
#pragma unroll
        for (int i = 0; i < HC / 4; ++i) as[i] += pv[i] * z;
      }
    }
    const float nu = norms[row];
    const float wq = prod ? ks * rnorms[row] : 0.f;
#pragma unroll
    for (int h = 0; h < HC; ++h)
      if (h < hc) out[((int64_t)s * nq + h0 + h) * n_keys + t] = nu * fmaf(wq, as[h / 4][h % 4], am[h / 4][h % 4]);
  }
}

// ------------------------------------------------------------ attention --
// Decode attention over quantized keys and values, any d: the logits come
// from the logits kernels; these three kernels turn them into
// out = sum_t softmax_t(scale l_t) v_hat_t.

// One workgroup per (set, head) row: the row's logits become normalised
// softmax weights in place (max, sum of exponentials, divide).
__global__ __launch_bounds__(kThreads) void k_softmax_rows(float *__restrict__ w, int64_t n_keys, float scale) {
  __shared__ float red[kThreads / 64];
  float *row = w + (int64_t)blockIdx.x * n_keys;
  const int tid = threadIdx.x;
  float m = -INFINITY;
  for (int64_t t = tid; t < n_keys; t += kThreads) m = fmaxf(m, scale * row[t]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, red[i]);
  float sum = 0.f;
  for (int64_t t = tid; t < n_keys; t += kThreads) sum += expf(scale * row[t] - m);
  sum = block_sum(sum, red);
  const float inv = 1.f / sum;
  for (int64_t t = tid; t < n_keys; t += kThreads) row[t] = expf(scale * row[t] - m) * inv;
}

constexpr int kAttnChunk = 256;  // keys per workgroup of the value pass

// Value pass: workgroup (chunk, set) adds, for every head h and coordinate j,
//   a[h][j] = sum_t w[h][t] nu_t c[idx_tj]        (rotated domain)
//   b[h][j] = sum_t w[h][t] nu_t gamma_t z_tj     (projected domain, prod)
// over its chunk of keys, and writes them to part[chunk][set][h][2][d].
__global__ __launch_bounds__(kThreads) void k_attn_values_generic(
    const float *__restrict__ w, int nq, const uint8_t *__restrict__ codes, const uint8_t *__restrict__ signs,
    const float *__restrict__ norms, const float *__restrict__ rnorms, int d, int64_t n_keys, int mse_bits,
    int prod, const float *__restrict__ cent, int64_t code_row, int64_t sign_row, float *__restrict__ part) {
  __shared__ float ws[kMaxHeads][kAttnChunk];
  __shared__ float nv[kAttnChunk], gv[kAttnChunk];
  const int64_t chunk = blockIdx.x, n_sets = gridDim.y;
  const int s = blockIdx.y, tid = threadIdx.x;
  const int64_t t0 = chunk * kAttnChunk;
  const int tc = (int)(n_keys - t0 < kAttnChunk ? n_keys - t0 : kAttnChunk);
  const int64_t srow = (int64_t)s * n_keys;
  for (int i = tid; i < tc; i += kThreads) {
    nv[i] = norms[srow + t0 + i];
    gv[i] = prod ? rnorms[srow + t0 + i] : 0.f;
  }
  for (int h0 = 0; h0 < nq; h0 += kMaxHeads) {
    const int hc = nq - h0 < kMaxHeads ? nq - h0 : kMaxHeads;
    __syncthreads();
    for (int e = tid; e < hc * kAttnChunk; e += kThreads) {
      const int h = e / kAttnChunk, i = e % kAttnChunk;
      ws[h][i] = i < tc ? w[((int64_t)s * nq + h0 + h) * n_keys + t0 + i] * nv[i] : 0.f;
    }
    __syncthreads();
    for (int j = tid; j < d; j += kThreads) {
      float a[kMaxHeads], b[kMaxHeads];
      for (int h = 0; h < kMaxHeads; ++h) a[h] = b[h] = 0.f;
      for (int i = 0; i < tc; ++i) {
        const int64_t row = srow + t0 + i;
        const float c = mse_bits > 0 ? cent[read_field(codes + row * code_row, j, mse_bits)] : 0.f;
        float z = 0.f;
        if (prod) z = ((signs[row * sign_row + (j >> 3)] >> (j & 7)) & 1) ? gv[i] : -gv[i];
        for (int h = 0; h < kMaxHeads; ++h)
          if (h < hc) {
            a[h] = fmaf(ws[h][i], c, a[h]);
            b[h] = fmaf(ws[h][i], z, b[h]);
          }
      }
      for (int h = 0; h < hc; ++h) {
        float *o = part + (((chunk * n_sets + s) * nq + h0 + h) * 2) * (int64_t)d;
        o[j] = a[h];
        o[d + j] = b[h];
      }
    }
  }
}

// Finish: workgroup (set, head) sums the chunks in a fixed order and maps the
// result back: out = Pi^T a + sqrt(pi/2)/d S^T b.
__global__ __launch_bounds__(kThreads) void k_attn_finish_generic(
    const float *__restrict__ part, int64_t chunks, int nq, int d, int groups, int prod,
    const float *__restrict__ Pi, const float *__restrict__ S, float *__restrict__ out) {
  extern __shared__ float sm[];
  float *av = sm, *bv = sm + d;
  const int64_t n_sets = gridDim.y;
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int g = s % groups;
  for (int j = tid; j < d; j += kThreads) {
    float a = 0.f, b = 0.f;
    for (int64_t c = 0; c < chunks; ++c) {
      const float *o = part + (((c * n_sets + s) * nq + h) * 2) * (int64_t)d;
      a += o[j];
      b += o[d + j];
    }
    av[j] = a;
    bv[j] = b;
  }
  __syncthreads();
  const float *P = Pi + (size_t)g * d * d, *Sg = prod ? S + (size_t)g * d * d : nullptr;
  const float ks = kQjlScale / (float)d;
  for (int i = tid; i < d; i += kThreads) {
    float a = 0.f, b = 0.f;
    for (int j = 0; j < d; ++j) a = fmaf(P[(size_t)j * d + i], av[j], a);
    if (prod)
      for (int j = 0; j < d; ++j) b = fmaf(Sg[(size_t)j * d + i], bv[j], b);
    out[((int64_t)s * nq + h) * d + i] = fmaf(ks, b, a);
  }
}

__global__ void k_pack(const uint8_t *__restrict__ idx, int bits, int64_t rows, int count,
                       int64_t row_bytes, uint8_t *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * row_bytes) return;
  const int64_t r = e / row_bytes;
  const int byte = (int)(e % row_bytes);
  const uint8_t *ir = idx + r * count;
  uint32_t v = 0;
  for (int p = 0; p < 8; ++p) {
    const int sb = byte * 8 + p, j = sb / bits, k = sb % bits;
    if (j < count) v |= (uint32_t)((ir[j] >> k) & 1) << p;
  }
  out[e] = (uint8_t)v;
}

__global__ void k_unpack(const uint8_t *__restrict__ in, int bits, int64_t rows, int count,
                         int64_t row_bytes, uint8_t *__restrict__ idx) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * count) return;
  const int64_t r = e / count;
  const int j = (int)(e % count);
  const uint8_t *row = in + r * row_bytes;
  uint32_t v = 0;
  for (int k = 0; k < bits; ++k) {
    const int sb = j * bits + k;
    v |= (uint32_t)((row[sb >> 3] >> (sb & 7)) & 1) << k;
  }
  idx[e] = (uint8_t)v;
}

}  // namespace

// Vectors per workgroup of the generic quantize and dequantize: 8 when their
// rows fit 48 KB of LDS, else fewer (1 at d = 4096).
static int generic_batch(int d, int per_vec_floats) {
  int v = 8;
  while (v > 1 && (size_t)v * per_vec_floats * d * sizeof(float) > 48 * 1024) v >>= 1;
  return v;
}

hipError_t launch_quant_generic(const DeviceTables &t, const void *x, int dtype, int64_t n_sets,
                                int64_t n, uint8_t *codes, uint8_t *signs, float *norms,
                                float *rnorms, hipStream_t st) {
  if (n_sets == 0 || n == 0) return hipSuccess;
  const int V = generic_batch(t.d, 3);
  const size_t shmem = (size_t)3 * V * t.d * sizeof(float) + sizeof(float) * (1u << t.mse_bits);
  const int prod = t.variant == 1;
  const dim3 grid((unsigned)((n + V - 1) / V), (unsigned)n_sets);
#define TQ_QG(T, VV)                                                                                              \
  hipLaunchKernelGGL((k_quant_generic<T, VV>), grid, dim3(kThreads), shmem, st, (const T *)x, t.d, n, t.groups,   \
                     t.mse_bits, prod, t.PiT, t.MT, t.cent, t.bnd, codes, t.code_row, signs, t.sign_row, norms, rnorms)
#define TQ_QGV(T)                \
  switch (V) {                   \
    case 8: TQ_QG(T, 8); break;  \
    case 4: TQ_QG(T, 4); break;  \
    case 2: TQ_QG(T, 2); break;  \
    default: TQ_QG(T, 1); break; \
  }
  if (dtype == 0) {
    TQ_QGV(float)
  } else {
    TQ_QGV(uint16_t)
  }
#undef TQ_QGV
#undef TQ_QG
  return hipGetLastError();
}

hipError_t launch_append(const DeviceTables &t, const void *x, int dtype, int64_t n_sets, const int64_t *rows,
                         int64_t cache_rows, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                         hipStream_t st) {
  if (n_sets == 0) return hipSuccess;
  const size_t shmem = ((size_t)3 * t.d + kAppendThreads) * sizeof(float);
  const int prod = t.variant == 1;
  const bool fixed = t.d * 4 == kAppendThreads && t.mse_bits <= 8;
#define TQ_APPEND(T, DC)                                                                                         \
  hipLaunchKernelGGL((k_append<T, DC>), dim3((unsigned)n_sets), dim3(kAppendThreads), shmem, st, (const T *)x, t.d, \
                     t.groups, t.mse_bits, prod, rows, cache_rows, t.PiT, t.MT, t.cent, t.bnd, codes, t.code_row,   \
                     signs, t.sign_row, norms, rnorms)
  if (dtype == 0) {
    if (fixed)
      TQ_APPEND(float, kAppendThreads / 4);
    else
      TQ_APPEND(float, 0);
  } else {
    if (fixed)
      TQ_APPEND(uint16_t, kAppendThreads / 4);
    else
      TQ_APPEND(uint16_t, 0);
  }
#undef TQ_APPEND
  return hipGetLastError();
}

hipError_t launch_gather_parts(const void *x, int dtype, int64_t rows, int64_t n, int groups, int d, int n_out,
                               const int32_t *perm, void *xo, void *xr, hipStream_t st) {
  const int64_t total = rows * d;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == 0)
    hipLaunchKernelGGL(k_gather_parts<float>, grid, dim3(256), 0, st, (const float *)x, rows, n, groups, d, n_out,
                       perm, (float *)xo, (float *)xr);
  else
    hipLaunchKernelGGL(k_gather_parts<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)x, rows, n, groups, d,
                       n_out, perm, (uint16_t *)xo, (uint16_t *)xr);
  return hipGetLastError();
}

hipError_t launch_scatter_parts(const float *xo, const float *xr, int64_t rows, int64_t n, int groups, int d,
                                int n_out, const int32_t *perm, float *out, hipStream_t st) {
  const int64_t total = rows * d;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scatter_parts, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, xo, xr, rows, n,
                     groups, d, n_out, perm, out);
  return hipGetLastError();
}

hipError_t launch_add_inplace(float *out, const float *in, int64_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_add_inplace, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, out, in, count);
  return hipGetLastError();
}

hipError_t launch_dequant_generic(const DeviceTables &t, const uint8_t *codes, const uint8_t *signs,
                                  const float *norms, const float *rnorms, int64_t n_sets, int64_t n,
                                  float *out, hipStream_t st) {
  if (n_sets == 0 || n == 0) return hipSuccess;
  const int V = generic_batch(t.d, 2);
  const size_t shmem = (size_t)2 * V * t.d * sizeof(float);
  const dim3 grid((unsigned)((n + V - 1) / V), (unsigned)n_sets);
#define TQ_DG(VV)                                                                                                  \
  hipLaunchKernelGGL((k_dequant_generic<VV>), grid, dim3(kThreads), shmem, st, codes, signs, norms, rnorms, t.d, n, \
                     t.groups, t.mse_bits, (int)(t.variant == 1), t.Pi, t.S, t.cent, t.code_row, t.sign_row, out)
  switch (V) {
    case 8: TQ_DG(8); break;
    case 4: TQ_DG(4); break;
    case 2: TQ_DG(2); break;
    default: TQ_DG(1); break;
  }
#undef TQ_DG
  return hipGetLastError();
}

hipError_t launch_logits_generic(const DeviceTables &t, const float *q, int64_t nq,
                                 const uint8_t *codes, const uint8_t *signs, const float *norms,
                                 const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
                                 hipStream_t st) {
  if (n_sets == 0 || n_keys == 0) return hipSuccess;
  // query tables [d][HC] for the rotation and the projection, then the codebook
  const bool wide = t.d <= 1024;
  const int hc_max = wide ? 8 : 4;
  const size_t shmem = (size_t)2 * hc_max * t.d * sizeof(float) + sizeof(float) * (1u << t.mse_bits);
  const void *fn = wide ? (const void *)k_logits_generic<8> : (const void *)k_logits_generic<4>;
  if (shmem > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const int64_t per_block = (int64_t)kThreads * kKeysPerThread;
  const dim3 grid((unsigned)((n_keys + per_block - 1) / per_block), (unsigned)n_sets);
  for (int h0 = 0; h0 < nq; h0 += hc_max) {
    const int hc = (int)((nq - h0) < hc_max ? (nq - h0) : hc_max);
    if (wide)
      hipLaunchKernelGGL(k_logits_generic<8>, grid, dim3(kThreads), shmem, st, q, (int)nq, h0, hc, codes, signs,
                         norms, rnorms, t.d, n_keys, t.groups, t.mse_bits, (int)(t.variant == 1), t.PiT, t.ST, t.cent,
                         t.code_row, t.sign_row, out);
    else
      hipLaunchKernelGGL(k_logits_generic<4>, grid, dim3(kThreads), shmem, st, q, (int)nq, h0, hc, codes, signs,
                         norms, rnorms, t.d, n_keys, t.groups, t.mse_bits, (int)(t.variant == 1), t.PiT, t.ST, t.cent,
                         t.code_row, t.sign_row, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int64_t attention_generic_chunks(int64_t n_keys) { return (n_keys + kAttnChunk - 1) / kAttnChunk; }

hipError_t launch_attention_generic(const DeviceTables &tk, const DeviceTables &tv, const float *q, int64_t nq,
                                    const uint8_t *k_codes, const uint8_t *k_signs, const float *k_norms,
                                    const float *k_rnorms, const uint8_t *v_codes, const uint8_t *v_signs,
                                    const float *v_norms, const float *v_rnorms, int64_t n_sets, int64_t n_keys,
                                    float scale, float *logits, float *part, float *out, hipStream_t st) {
  hipError_t e = launch_logits128(tk, q, nq, k_codes, k_signs, k_norms, k_rnorms, n_sets, n_keys, logits, st);
  if (e == hipErrorNotSupported)
    e = launch_logits_generic(tk, q, nq, k_codes, k_signs, k_norms, k_rnorms, n_sets, n_keys, logits, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_softmax_rows, dim3((unsigned)(n_sets * nq)), dim3(kThreads), 0, st, logits, n_keys, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t chunks = attention_generic_chunks(n_keys);
  const int prod = tv.variant == 1;
  hipLaunchKernelGGL(k_attn_values_generic, dim3((unsigned)chunks, (unsigned)n_sets), dim3(kThreads), 0, st,
                     logits, (int)nq, v_codes, v_signs, v_norms, v_rnorms, tv.d, n_keys, tv.mse_bits, prod,
                     tv.cent, tv.code_row, tv.sign_row, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_finish_generic, dim3((unsigned)nq, (unsigned)n_sets), dim3(kThreads),
                     (size_t)2 * tv.d * sizeof(float), st, part, chunks, (int)nq, tv.d, tv.groups, prod, tv.Pi,
                     tv.S, out);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *idx, int bits, int64_t rows, int count, int64_t row_bytes,
                       uint8_t *out, hipStream_t st) {
  const int64_t total = rows * row_bytes;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, idx, bits,
                     rows, count, row_bytes, out);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *in, int bits, int64_t rows, int count, int64_t row_bytes,
                         uint8_t *idx, hipStream_t st) {
  const int64_t total = rows * (int64_t)count;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, in, bits,
                     rows, count, row_bytes, idx);
  return hipGetLastError();
}

}  // namespace tq
