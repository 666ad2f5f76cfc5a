// C ABI of the TurboQuant hot path: argument validation, codec construction
// (host, float64, once), device table upload and kernel dispatch.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <new>
#include <string>
#include <vector>

#include "../../include/tq.h"
#include "fast128.h"
#include "host_codec.h"
#include "kernels.h"

struct tq_codec {
  int d = 0, b = 0, variant = 0, groups = 0, mse_bits = 0;
  int device = 0;
  void *arena = nullptr;  // one device allocation holding every table
  tq::DeviceTables dev;
  // host copies (float32, as stored on the device)
  std::vector<float> h_pi, h_s, h_c, h_t;
};

namespace {

thread_local std::string g_last_error;

// TQ_LOG = 0..3 (read once): 1 logs every failure to stderr, 2 also every
// data call with its shape.
int log_level() {
  static const int level = [] {
    const char *v = std::getenv("TQ_LOG");
    return v ? std::atoi(v) : 0;
  }();
  return level;
}

int fail(int code, const std::string &msg) {
  g_last_error = msg;
  if (log_level() >= 1) std::fprintf(stderr, "tq: error %d: %s\n", code, msg.c_str());
  return code;
}

void trace_call(const char *fn, int d, int64_t n_sets, int64_t n, int64_t nq) {
  if (log_level() >= 2)
    std::fprintf(stderr, "tq: %s d=%d n_sets=%lld n=%lld nq=%lld\n", fn, d, (long long)n_sets, (long long)n,
                 (long long)nq);
}

// TQ_FAULT=launch: every data call fails as a kernel launch would, after its
// validation and before anything is enqueued (a test hook for the TQ_EHIP
// path).  Read on every call so that a test can switch it.
int launch_fault(const char *fn) {
  const char *v = std::getenv("TQ_FAULT");
  if (v && std::strcmp(v, "launch") == 0)
    return fail(TQ_EHIP, std::string(fn) + ": kernel launch failed (TQ_FAULT=launch)");
  return TQ_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(TQ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t row_bytes(int64_t count, int bits) {
  const int64_t raw = (count * bits + 7) / 8;
  return (raw + 15) / 16 * 16;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Validate (d, b, variant) and return the number of mse bits.
int check_config(int d, int b, int variant, int groups, int *mse_bits) {
  if (d < 2 || d > 4096) return fail(TQ_EINVAL, "d must be in [2, 4096]");
  if (groups < 1 || groups > 4096) return fail(TQ_EINVAL, "groups must be in [1, 4096]");
  if (variant == TQ_MSE) {
    if (b < 1 || b > 8) return fail(TQ_EINVAL, "mse needs 1 <= b <= 8");
    *mse_bits = b;
  } else if (variant == TQ_PROD) {
    if (b < 1 || b > 5) return fail(TQ_EINVAL, "prod needs 1 <= b <= 5");
    *mse_bits = b - 1;
  } else {
    return fail(TQ_EINVAL, "variant must be TQ_MSE or TQ_PROD");
  }
  return TQ_OK;
}

// Host tables of group g in float64: Pi (row-major), S, M = S Pi^T.
void group_matrices(int d, uint64_t seed, int g, bool prod, std::vector<double> &pi,
                    std::vector<double> &s, std::vector<double> &m) {
  std::vector<double> gm((size_t)d * d);
  tq::gaussian_matrix(seed, (uint64_t)g, tq::kMatPi, d, d, gm.data());
  pi.assign((size_t)d * d, 0.0);
  tq::orthogonal_factor(d, gm.data(), pi.data());
  if (!prod) return;
  s.assign((size_t)d * d, 0.0);
  tq::gaussian_matrix(seed, (uint64_t)g, tq::kMatS, d, d, s.data());
  m.assign((size_t)d * d, 0.0);
  // M[i][j] = sum_k S[i][k] Pi[j][k]
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      const double *si = &s[(size_t)i * d], *pj = &pi[(size_t)j * d];
      for (int k = 0; k < d; ++k) acc += si[k] * pj[k];
      m[(size_t)i * d + j] = acc;
    }
}

// out = transpose of the d x d row-major matrix a
void transpose(int d, const std::vector<double> &a, std::vector<double> &out) {
  out.resize((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) out[(size_t)j * d + i] = a[(size_t)i * d + j];
}

template <class T>
T *carve(char *base, size_t &off, size_t count) {
  off = (off + 255) / 256 * 256;
  T *p = reinterpret_cast<T *>(base + off);
  off += count * sizeof(T);
  return p;
}

int make_codec(int d, int b, int variant, uint64_t seed, int groups, tq_handle *out) {
  int mse_bits = 0;
  int st = check_config(d, b, variant, groups, &mse_bits);
  if (st != TQ_OK) return st;
  if (!out) return fail(TQ_EINVAL, "out is NULL");
  const bool prod = variant == TQ_PROD;
  const size_t dd = (size_t)d * d;
  const int L = mse_bits > 0 ? 1 << mse_bits : 0;

  auto *h = new (std::nothrow) tq_codec;
  if (!h) return fail(TQ_ENOMEM, "host allocation failed");
  h->d = d;
  h->b = b;
  h->variant = variant;
  h->groups = groups;
  h->mse_bits = mse_bits;

  // Codebook (shared by all groups): float64 Lloyd–Max, rounded to float32.
  if (mse_bits > 0) {
    const tq::Codebook cb = tq::lloyd_max(d, mse_bits);
    for (double c : cb.centroids) h->h_c.push_back((float)c);
    for (double t : cb.boundaries) h->h_t.push_back((float)t);
  }
  tq::CellTable cells;
  if (mse_bits > 0 && !tq::build_cell_table(h->h_t, tq::kCellRadius, cells)) {
    delete h;
    return fail(TQ_EINVAL, "codebook boundaries are not strictly ascending");
  }
  const bool fast = tq::fast128_supported(d, mse_bits, variant);
  const size_t rot_words = fast ? tq::fast128_rotation_words(d) : 0;
  // other dimensions (multiples of 8): 128 x 128 block images for the tiled
  // kernels, when all of them fit in 1 GiB
  const int nblk = (d + 127) / 128;
  const size_t blk_words = tq::fast128_rotation_words(128);
  const size_t tiled_rot_words = (size_t)groups * nblk * nblk * blk_words;
  const size_t tiled_sign_words = prod ? 2 * tiled_rot_words : 0;
  const bool tiled = !fast && d % 8 == 0 && mse_bits <= 4 && d > 8 &&
                     (tiled_rot_words + tiled_sign_words) * 4 <= ((size_t)1 << 30);
  // decode tables (code pairs, sign bytes) for every codebook of <= 4 bits:
  // the d = 128 kernels and the top-k search read them
  const size_t lut_words = mse_bits <= 4 ? tq::fast128_lut_words(mse_bits) : 0;

  // Host images of every device table.
  std::vector<float> pi_all(groups * dd), pit_all(groups * dd);
  std::vector<float> s_all, st_all, mt_all;
  std::vector<uint32_t> pi_img(groups * rot_words), m_img(prod ? groups * rot_words : 0);
  std::vector<uint32_t> dq_pi_img(groups * rot_words), dq_s_img(prod ? groups * rot_words : 0);
  std::vector<double> trans;
  std::vector<uint32_t> t_rot(tiled ? tiled_rot_words : 0), t_sign(tiled ? tiled_sign_words : 0);
  std::vector<double> blk(128 * 128);
  // image of the 128 x 128 block (rows r0.., cols c0..) of a d x d matrix, zero past d
  auto block_image = [&](const std::vector<double> &mat, int r0, int c0, int k_order, uint32_t *dst) {
    for (int i = 0; i < 128; ++i)
      for (int j = 0; j < 128; ++j)
        blk[(size_t)i * 128 + j] = (r0 + i < d && c0 + j < d) ? mat[(size_t)(r0 + i) * d + c0 + j] : 0.0;
    tq::fast128_build_rotation_image(blk.data(), k_order, dst);
  };
  if (prod) {
    s_all.resize(groups * dd);
    st_all.resize(groups * dd);
    mt_all.resize(groups * dd);
  }
  std::vector<double> pi, s, m;
  for (int g = 0; g < groups; ++g) {
    group_matrices(d, seed, g, prod, pi, s, m);
    float *P = &pi_all[g * dd], *PT = &pit_all[g * dd];
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        P[(size_t)i * d + j] = (float)pi[(size_t)i * d + j];
        PT[(size_t)j * d + i] = (float)pi[(size_t)i * d + j];
      }
    if (fast) {
      tq::fast128_build_rotation_image(pi.data(), 0, &pi_img[g * rot_words]);
      transpose(d, pi, trans);
      tq::fast128_build_rotation_image(trans.data(), 1, &dq_pi_img[g * rot_words], true, true);
    }
    if (prod) {
      float *S = &s_all[g * dd], *ST = &st_all[g * dd], *MT = &mt_all[g * dd];
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
          S[(size_t)i * d + j] = (float)s[(size_t)i * d + j];
          ST[(size_t)j * d + i] = (float)s[(size_t)i * d + j];
          MT[(size_t)j * d + i] = (float)m[(size_t)i * d + j];
        }
      if (fast) {
        tq::fast128_build_rotation_image(m.data(), 1, &m_img[g * rot_words]);
        transpose(d, s, trans);
        tq::fast128_build_rotation_image(trans.data(), 1, &dq_s_img[g * rot_words], true, true);
      }
    }
    if (tiled) {
      for (int pp = 0; pp < nblk; ++pp)
        for (int c = 0; c < nblk; ++c) {
          block_image(pi, 128 * pp, 128 * c, 0, &t_rot[(((size_t)g * nblk + pp) * nblk + c) * blk_words]);
          if (prod) {
            const size_t base = ((size_t)g * nblk + pp) * 2 * nblk;
            block_image(s, 128 * pp, 128 * c, 0, &t_sign[(base + c) * blk_words]);
            block_image(m, 128 * pp, 128 * c, 1, &t_sign[(base + nblk + c) * blk_words]);
          }
        }
    }
    if (g == 0) {
      h->h_pi.assign(P, P + dd);
      if (prod) h->h_s.assign(&s_all[0], &s_all[0] + dd);
    }
  }
  std::vector<uint32_t> lut(lut_words);
  float lut_inv_scale = 1.f;
  if (lut_words) lut_inv_scale = tq::fast128_build_logit_lut(h->h_c.data(), mse_bits, lut.data());

  // One device arena.
  size_t off = 0;
  char *const base0 = nullptr;
  auto plan = [&](char *base) {
    off = 0;
    h->dev.Pi = carve<float>(base, off, groups * dd);
    h->dev.PiT = carve<float>(base, off, groups * dd);
    if (prod) {
      h->dev.S = carve<float>(base, off, groups * dd);
      h->dev.ST = carve<float>(base, off, groups * dd);
      h->dev.MT = carve<float>(base, off, groups * dd);
    }
    h->dev.cent = carve<float>(base, off, L ? L : 1);
    h->dev.bnd = carve<float>(base, off, L > 1 ? L - 1 : 1);
    h->dev.cells = carve<uint32_t>(base, off, cells.words.empty() ? 2 : cells.words.size());
    if (tiled) {
      h->dev.tiled_rot = carve<uint32_t>(base, off, tiled_rot_words);
      if (prod) h->dev.tiled_sign = carve<uint32_t>(base, off, tiled_sign_words);
    }
    if (fast) {
      h->dev.pi_frag = carve<uint32_t>(base, off, groups * rot_words);
      if (prod) h->dev.m_frag = carve<uint32_t>(base, off, groups * rot_words);
      h->dev.dq_pi_frag = carve<uint32_t>(base, off, groups * rot_words);
      if (prod) h->dev.dq_s_frag = carve<uint32_t>(base, off, groups * rot_words);
    }
    if (lut_words) h->dev.logit_lut = carve<uint32_t>(base, off, lut_words);
    return off;
  };
  const size_t bytes = plan(base0);
  const char *env_fault = std::getenv("TQ_FAULT");
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  if (env_fault && std::strcmp(env_fault, "alloc") == 0) {
    delete h;
    return fail(TQ_ENOMEM, "device allocation failed (TQ_FAULT=alloc)");
  }
  e = hipMalloc(&h->arena, bytes);
  if (e != hipSuccess) {
    delete h;
    return e == hipErrorOutOfMemory ? fail(TQ_ENOMEM, "hipMalloc of the codec tables failed")
                                    : hip_fail(e, "hipMalloc");
  }
  plan((char *)h->arena);
  auto up = [&](const void *dst, const void *src, size_t n) {
    if (n == 0 || e != hipSuccess) return;
    e = hipMemcpy(const_cast<void *>(dst), src, n, hipMemcpyHostToDevice);
  };
  up(h->dev.Pi, pi_all.data(), pi_all.size() * 4);
  up(h->dev.PiT, pit_all.data(), pit_all.size() * 4);
  if (prod) {
    up(h->dev.S, s_all.data(), s_all.size() * 4);
    up(h->dev.ST, st_all.data(), st_all.size() * 4);
    up(h->dev.MT, mt_all.data(), mt_all.size() * 4);
  }
  up(h->dev.cent, h->h_c.data(), h->h_c.size() * 4);
  up(h->dev.bnd, h->h_t.data(), h->h_t.size() * 4);
  up(h->dev.cells, cells.words.data(), cells.words.size() * 4);
  if (tiled) {
    up(h->dev.tiled_rot, t_rot.data(), t_rot.size() * 4);
    if (prod) up(h->dev.tiled_sign, t_sign.data(), t_sign.size() * 4);
  }
  if (fast) {
    up(h->dev.pi_frag, pi_img.data(), pi_img.size() * 4);
    if (prod) up(h->dev.m_frag, m_img.data(), m_img.size() * 4);
    up(h->dev.dq_pi_frag, dq_pi_img.data(), dq_pi_img.size() * 4);
    if (prod) up(h->dev.dq_s_frag, dq_s_img.data(), dq_s_img.size() * 4);
  }
  if (lut_words) up(h->dev.logit_lut, lut.data(), lut.size() * 4);
  if (e != hipSuccess) {
    (void)hipFree(h->arena);
    delete h;
    return hip_fail(e, "hipMemcpy of the codec tables");
  }
  // address of the fixed workspace on this device (for tq_attention_static);
  // a failure here is reported by that call, which retries the lookup
  (void)tq::static_scratch_setup(h->device);
  if (mse_bits > 0 && mse_bits <= 4) {
    for (int k = 0; k < L / 2; ++k) h->dev.pos_cent[k] = h->h_c[L / 2 + k];
    for (int k = 0; k + 1 < L / 2; ++k) h->dev.pos_bnd[k] = h->h_t[L / 2 + k];
  }
  h->dev.lut_inv_scale = lut_inv_scale;
  h->dev.cell_radius = cells.radius;
  h->dev.cell_scale = cells.scale;
  h->dev.d = d;
  h->dev.groups = groups;
  h->dev.variant = variant;
  h->dev.mse_bits = mse_bits;
  h->dev.code_row = mse_bits > 0 ? row_bytes(d, mse_bits) : 0;
  h->dev.sign_row = prod ? row_bytes(d, 1) : 0;
  *out = h;
  return TQ_OK;
}

int check_handle(tq_handle h) {
  if (!h) return fail(TQ_EINVAL, "handle is NULL");
  return TQ_OK;
}

int check_rows(tq_handle h, int64_t n_sets, int64_t n) {
  if (n_sets < 0 || n < 0) return fail(TQ_EINVAL, "n_sets and n must be >= 0");
  if (n_sets > 65535) return fail(TQ_EINVAL, "n_sets must be <= 65535");
  if (n_sets * n > (int64_t)0x7fffffff) return fail(TQ_EINVAL, "n_sets * n must be < 2^31");
  (void)h;
  return TQ_OK;
}

int check_code_ptrs(tq_handle h, const void *codes, const void *signs, const void *norms,
                    const void *rnorms, bool writing) {
  const bool prod = h->variant == TQ_PROD;
  if (h->mse_bits > 0 && !codes) return fail(TQ_EINVAL, "codes is NULL");
  if (codes && !aligned16(codes)) return fail(TQ_EINVAL, "codes must be 16-byte aligned");
  if (!norms || ((uintptr_t)norms & 3u)) return fail(TQ_EINVAL, "norms NULL or misaligned");
  if (prod) {
    if (!signs || !aligned16(signs)) return fail(TQ_EINVAL, "signs NULL or not 16-byte aligned");
    if (!rnorms || ((uintptr_t)rnorms & 3u)) return fail(TQ_EINVAL, "rnorms NULL or misaligned");
  } else if (writing && (signs || rnorms)) {
    return fail(TQ_EINVAL, "signs/rnorms must be NULL for an mse codec");
  }
  return TQ_OK;
}

template <class F>
int guarded(F f) {
  try {
    return f();
  } catch (const std::bad_alloc &) {
    return fail(TQ_ENOMEM, "host allocation failed");
  } catch (const std::exception &ex) {
    return fail(TQ_EINVAL, ex.what());
  } catch (...) {
    return fail(TQ_EINVAL, "unknown error");
  }
}

}  // namespace

extern "C" {

int tq_init(int d, int b, int variant, uint64_t seed, tq_handle *out) {
  return tq_init_groups(d, b, variant, seed, 1, out);
}

int tq_init_groups(int d, int b, int variant, uint64_t seed, int groups, tq_handle *out) {
  g_last_error.clear();
  return guarded([&]() -> int { return make_codec(d, b, variant, seed, groups, out); });
}

int tq_destroy(tq_handle h) {
  if (!h) return TQ_OK;
  if (h->arena) (void)hipFree(h->arena);
  delete h;
  return TQ_OK;
}

int tq_layout(tq_handle h, int64_t *code_row_bytes, int64_t *sign_row_bytes, int *mse_bits) {
  int st = check_handle(h);
  if (st) return st;
  if (code_row_bytes) *code_row_bytes = h->dev.code_row;
  if (sign_row_bytes) *sign_row_bytes = h->dev.sign_row;
  if (mse_bits) *mse_bits = h->mse_bits;
  return TQ_OK;
}

int tq_quantize(tq_handle h, const void *x, int dtype, int64_t n_sets, int64_t n, void *codes,
                void *signs, float *norms, float *rnorms, void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if ((st = check_rows(h, n_sets, n))) return st;
  if (n_sets == 0 || n == 0) return TQ_OK;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_EINVAL, "dtype must be TQ_F32 or TQ_BF16");
  if (!x || ((uintptr_t)x & (dtype == TQ_F32 ? 3u : 1u))) return fail(TQ_EINVAL, "x NULL or misaligned");
  if ((st = check_code_ptrs(h, codes, signs, norms, rnorms, true))) return st;
  trace_call("tq_quantize", h->d, n_sets, n, 0);
  if ((st = launch_fault("tq_quantize"))) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = tq::launch_quant128(h->dev, x, dtype, n_sets, n, (uint8_t *)codes,
                                     (uint8_t *)signs, norms, rnorms, s);
  if (e == hipErrorNotSupported)
    e = tq::launch_quant_tiled(h->dev, x, dtype, n_sets, n, (uint8_t *)codes, (uint8_t *)signs, norms,
                               rnorms, s);
  if (e == hipErrorNotSupported)
    e = tq::launch_quant_generic(h->dev, x, dtype, n_sets, n, (uint8_t *)codes, (uint8_t *)signs,
                                 norms, rnorms, s);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "quantize launch");
}

int tq_append(tq_handle h, const void *x, int dtype, int64_t n_sets, const int64_t *rows, int64_t cache_rows,
              void *codes, void *signs, float *norms, float *rnorms, void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if (n_sets < 0 || n_sets > 65535) return fail(TQ_EINVAL, "n_sets must be in [0, 65535]");
  if (cache_rows < 0) return fail(TQ_EINVAL, "cache_rows must be >= 0");
  if (n_sets == 0) return TQ_OK;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_EINVAL, "dtype must be TQ_F32 or TQ_BF16");
  if (!x || ((uintptr_t)x & (dtype == TQ_F32 ? 3u : 1u))) return fail(TQ_EINVAL, "x NULL or misaligned");
  if (!rows || ((uintptr_t)rows & 7u)) return fail(TQ_EINVAL, "rows NULL or misaligned");
  if ((st = check_code_ptrs(h, codes, signs, norms, rnorms, true))) return st;
  trace_call("tq_append", h->d, n_sets, 1, 0);
  if ((st = launch_fault("tq_append"))) return st;
  hipError_t e = tq::launch_append(h->dev, x, dtype, n_sets, rows, cache_rows, (uint8_t *)codes, (uint8_t *)signs,
                                   norms, rnorms, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "append launch");
}

int tq_dequantize(tq_handle h, const void *codes, const void *signs, const float *norms,
                  const float *rnorms, int64_t n_sets, int64_t n, float *x_out, void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if ((st = check_rows(h, n_sets, n))) return st;
  if (n_sets == 0 || n == 0) return TQ_OK;
  if ((st = check_code_ptrs(h, codes, signs, norms, rnorms, false))) return st;
  if (!x_out || ((uintptr_t)x_out & 3u)) return fail(TQ_EINVAL, "x_out NULL or misaligned");
  trace_call("tq_dequantize", h->d, n_sets, n, 0);
  if ((st = launch_fault("tq_dequantize"))) return st;
  hipError_t e = tq::launch_dequant128(h->dev, (const uint8_t *)codes, (const uint8_t *)signs, norms,
                                       rnorms, n_sets, n, x_out, (hipStream_t)stream);
  if (e == hipErrorNotSupported)
    e = tq::launch_dequant_generic(h->dev, (const uint8_t *)codes, (const uint8_t *)signs, norms, rnorms,
                                   n_sets, n, x_out, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "dequantize launch");
}

int tq_logits(tq_handle h, const float *q, int64_t nq, const void *codes, const void *signs,
              const float *norms, const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
              void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if ((st = check_rows(h, n_sets, n_keys))) return st;
  if (nq < 1 || nq > 64) return fail(TQ_EINVAL, "nq must be in [1, 64]");
  if (n_sets == 0 || n_keys == 0) return TQ_OK;
  if (!q || ((uintptr_t)q & 3u)) return fail(TQ_EINVAL, "q NULL or misaligned");
  if (!out || ((uintptr_t)out & 3u)) return fail(TQ_EINVAL, "out NULL or misaligned");
  if ((st = check_code_ptrs(h, codes, signs, norms, rnorms, false))) return st;
  if (n_sets * nq * n_keys > ((int64_t)1 << 40)) return fail(TQ_EINVAL, "output too large");
  trace_call("tq_logits", h->d, n_sets, n_keys, nq);
  if ((st = launch_fault("tq_logits"))) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = tq::launch_logits128(h->dev, q, nq, (const uint8_t *)codes, (const uint8_t *)signs,
                                      norms, rnorms, n_sets, n_keys, out, s);
  if (e == hipErrorNotSupported)
    e = tq::launch_logits_generic(h->dev, q, nq, (const uint8_t *)codes, (const uint8_t *)signs,
                                  norms, rnorms, n_sets, n_keys, out, s);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "logits launch");
}

namespace {

// Which kernels serve an attention call, and the workspace they need.
struct AttnPlan {
  bool fused = false;  // the d = 128 fused kernel (else the any-d kernels)
  size_t logits_off = 0, part_off = 0, bytes = 0;
};

int check_attention(tq_handle hk, tq_handle hv, int64_t nq, int64_t n_sets, int64_t n_keys) {
  int st = check_handle(hk);
  if (st) return st;
  if ((st = check_handle(hv))) return st;
  if (hk->d != hv->d) return fail(TQ_EINVAL, "key and value codecs must have the same d");
  if (hk->device != hv->device) return fail(TQ_EINVAL, "key and value codecs live on different devices");
  if ((st = check_rows(hk, n_sets, n_keys))) return st;
  if (nq < 1 || nq > 64) return fail(TQ_EINVAL, "nq must be in [1, 64]");
  if (n_sets > 0 && n_keys < 1) return fail(TQ_EINVAL, "attention needs n_keys >= 1");
  if (n_sets * nq * n_keys > ((int64_t)1 << 40)) return fail(TQ_EINVAL, "problem too large");
  return TQ_OK;
}

AttnPlan plan_attention(tq_handle hk, tq_handle hv, int64_t nq, int64_t n_sets, int64_t n_keys) {
  AttnPlan p;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t fused = tq::attention128_workspace(hk->dev, hv->dev, nq, n_sets, n_keys);
  if (fused > 0) {
    p.fused = true;
    p.bytes = up(fused);
    return p;
  }
  p.logits_off = 0;
  p.part_off = up((size_t)(n_sets * nq * n_keys) * sizeof(float));
  p.bytes = p.part_off + up((size_t)tq::attention_generic_chunks(n_keys) * n_sets * nq * 2 * hk->d * sizeof(float));
  return p;
}

}  // namespace

int tq_attention_workspace(tq_handle hk, tq_handle hv, int64_t nq, int64_t n_sets, int64_t n_keys,
                           size_t *bytes) {
  int st = check_attention(hk, hv, nq, n_sets, n_keys);
  if (st) return st;
  if (!bytes) return fail(TQ_EINVAL, "bytes is NULL");
  *bytes = (n_sets == 0) ? 0 : plan_attention(hk, hv, nq, n_sets, n_keys).bytes;
  return TQ_OK;
}

int tq_attention(tq_handle hk, tq_handle hv, const float *q, int64_t nq, const void *k_codes,
                 const void *k_signs, const float *k_norms, const float *k_rnorms, const void *v_codes,
                 const void *v_signs, const float *v_norms, const float *v_rnorms, int64_t n_sets,
                 int64_t n_keys, float scale, float *out, void *workspace, size_t workspace_bytes,
                 void *stream) {
  int st = check_attention(hk, hv, nq, n_sets, n_keys);
  if (st) return st;
  if (n_sets == 0) return TQ_OK;
  if (!std::isfinite(scale)) return fail(TQ_EINVAL, "scale must be finite");
  if (!q || ((uintptr_t)q & 3u)) return fail(TQ_EINVAL, "q NULL or misaligned");
  if (!out || ((uintptr_t)out & 3u)) return fail(TQ_EINVAL, "out NULL or misaligned");
  if ((st = check_code_ptrs(hk, k_codes, k_signs, k_norms, k_rnorms, false))) return st;
  if ((st = check_code_ptrs(hv, v_codes, v_signs, v_norms, v_rnorms, false))) return st;
  const AttnPlan p = plan_attention(hk, hv, nq, n_sets, n_keys);
  if (!workspace || ((uintptr_t)workspace & 255u)) return fail(TQ_EINVAL, "workspace NULL or not 256-byte aligned");
  if (workspace_bytes < p.bytes) return fail(TQ_EINVAL, "workspace smaller than tq_attention_workspace reports");
  trace_call("tq_attention", hk->d, n_sets, n_keys, nq);
  if ((st = launch_fault("tq_attention"))) return st;
  char *ws = (char *)workspace;
  hipError_t e;
  if (p.fused) {
    e = tq::launch_attention128(hk->dev, hv->dev, q, nq, (const uint8_t *)k_codes, (const uint8_t *)k_signs,
                                k_norms, k_rnorms, (const uint8_t *)v_codes, v_norms, n_sets, n_keys, scale,
                                (float *)ws, out, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : hip_fail(e, "attention launch");
  }
  e = tq::launch_attention_generic(
      hk->dev, hv->dev, q, nq, (const uint8_t *)k_codes, (const uint8_t *)k_signs, k_norms, k_rnorms,
      (const uint8_t *)v_codes, (const uint8_t *)v_signs, v_norms, v_rnorms, n_sets, n_keys, scale,
      (float *)(ws + p.logits_off), (float *)(ws + p.part_off), out, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "attention launch");
}

int tq_attention_static(tq_handle hk, tq_handle hv, const float *q, int64_t nq, const void *k_codes,
                        const void *k_signs, const float *k_norms, const float *k_rnorms, const void *v_codes,
                        const void *v_signs, const float *v_norms, const float *v_rnorms, int64_t n_sets,
                        int64_t n_keys, float scale, float *out, void *stream) {
  int st = check_attention(hk, hv, nq, n_sets, n_keys);
  if (st) return st;
  if (n_sets == 0) return TQ_OK;
  const size_t need = plan_attention(hk, hv, nq, n_sets, n_keys).bytes;
  if (need > tq::kStaticScratchBytes)
    return fail(TQ_EINVAL, "this shape needs " + std::to_string(need) + " bytes of workspace, more than the " +
                               std::to_string(tq::kStaticScratchBytes) +
                               "-byte static workspace; call tq_attention with a caller workspace");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void *ws = tq::static_scratch(dev);
  if (!ws) {
    if ((e = tq::static_scratch_setup(dev)) != hipSuccess) return hip_fail(e, "static workspace address");
    ws = tq::static_scratch(dev);
  }
  return tq_attention(hk, hv, q, nq, k_codes, k_signs, k_norms, k_rnorms, v_codes, v_signs, v_norms, v_rnorms,
                      n_sets, n_keys, scale, out, ws, tq::kStaticScratchBytes, stream);
}

// ------------------------------------------------------------------ top-k --
int tq_topk_workspace(tq_handle h, int64_t nq, int64_t n_keys, int k, size_t *bytes) {
  int st = check_handle(h);
  if (st) return st;
  if (!bytes) return fail(TQ_EINVAL, "bytes is NULL");
  if (nq < 0 || nq > 65535 * 128) return fail(TQ_EINVAL, "nq out of range");
  if (k < 1 || k > 64 || n_keys < k) return fail(TQ_EINVAL, "need 1 <= k <= 64 and n_keys >= k");
  *bytes = tq::topk_workspace(h->dev, nq, n_keys, k);  // 0 when nq is 0
  return TQ_OK;
}

int tq_topk(tq_handle h, const float *q, int64_t nq, const void *codes, const void *signs, const float *norms,
            const float *rnorms, int64_t n_keys, int k, float *out_scores, int32_t *out_idx, void *workspace,
            size_t workspace_bytes, void *stream) {
  size_t need = 0;
  int st = tq_topk_workspace(h, nq, n_keys, k, &need);
  if (st) return st;
  if (nq == 0) return TQ_OK;
  if ((st = check_rows(h, 1, n_keys))) return st;
  if (!q || ((uintptr_t)q & 3u)) return fail(TQ_EINVAL, "q NULL or misaligned");
  if (!out_scores || ((uintptr_t)out_scores & 3u) || !out_idx || ((uintptr_t)out_idx & 3u))
    return fail(TQ_EINVAL, "outputs NULL or misaligned");
  if ((st = check_code_ptrs(h, codes, signs, norms, rnorms, false))) return st;
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(TQ_EINVAL, "workspace NULL, not 256-byte aligned or smaller than tq_topk_workspace reports");
  trace_call("tq_topk", h->d, 1, n_keys, nq);
  if ((st = launch_fault("tq_topk"))) return st;
  hipError_t e = tq::launch_topk(h->dev, q, nq, (const uint8_t *)codes, (const uint8_t *)signs, norms, rnorms, n_keys,
                                 k, workspace, out_scores, out_idx, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "top-k launch");
}

// ------------------------------------------------------- mixed precision --
struct tq_mixed_codec {
  int d = 0, n_out = 0, groups = 0, variant = 0;
  tq_handle parts[2] = {nullptr, nullptr};  // outlier part (n_out dims, b + 1 bits), regular part
  int32_t *perm = nullptr;                  // device [groups][d]: outlier channels, then the rest ascending
  // fused quantize (d = 128, n_out = 64, TurboQuant_mse, b + 1 <= 4): device
  // [groups] rotation images, then [groups][4] outlier-channel masks
  uint32_t *fused = nullptr;
  // fused logits (same configurations): device [groups][128][128], the
  // transpose of the block matrix (rows 0..63: Pi_o on the outlier channels,
  // 64..127: Pi_r on the others)
  float *rt = nullptr;
};

namespace {

int check_mixed(tq_mixed m) { return m ? TQ_OK : fail(TQ_EINVAL, "mixed handle is NULL"); }

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// Bytes of `rows` vectors split into the two parts, each part's block
// starting on a 256-byte boundary: [rows][n_out] then [rows][d - n_out].
size_t mixed_split_bytes(const tq_mixed_codec *m, int64_t rows, size_t elem) {
  return up256((size_t)rows * m->n_out * elem) + up256((size_t)rows * (m->d - m->n_out) * elem);
}

// Both parts' arrays, checked as the part codec's own calls check them, before
// anything is enqueued.
int check_mixed_ptrs(tq_mixed m, const void *const codes[2], const void *const signs[2], const float *const norms[2],
                     const float *const rnorms[2], bool writing) {
  for (int p = 0; p < 2; ++p) {
    const int st = check_code_ptrs(m->parts[p], codes[p], signs[p], norms[p], rnorms[p], writing);
    if (st) return fail(st, std::string(p == 0 ? "outlier part: " : "regular part: ") + g_last_error);
  }
  return TQ_OK;
}

}  // namespace

int tq_mixed_init(int d, int b, int variant, uint64_t seed, int groups, int n_out, const int32_t *out_channels,
                  tq_mixed *out) {
  g_last_error.clear();
  return guarded([&]() -> int {
    if (!out) return fail(TQ_EINVAL, "out is NULL");
    if (d < 4 || d > 4096) return fail(TQ_EINVAL, "d must be in [4, 4096]");
    if (groups < 1 || groups > 4096) return fail(TQ_EINVAL, "groups must be in [1, 4096]");
    if (n_out < 2 || n_out > d - 2) return fail(TQ_EINVAL, "n_out must be in [2, d - 2]");
    if (variant == TQ_MSE ? (b < 1 || b > 7) : variant == TQ_PROD ? (b < 1 || b > 4) : true)
      return fail(TQ_EINVAL, "mse needs 1 <= b <= 7, prod 1 <= b <= 4 (the outlier part takes b + 1 bits)");
    if (!out_channels) return fail(TQ_EINVAL, "out_channels is NULL");
    std::vector<int32_t> perm((size_t)groups * d);
    for (int g = 0; g < groups; ++g) {
      std::vector<char> used(d, 0);
      int32_t *pg = perm.data() + (size_t)g * d;
      for (int i = 0; i < n_out; ++i) {
        const int32_t c = out_channels[(size_t)g * n_out + i];
        if (c < 0 || c >= d || used[c]) return fail(TQ_EINVAL, "out_channels must be distinct channels of [0, d)");
        used[c] = 1;
        pg[i] = c;
      }
      int k = n_out;
      for (int c = 0; c < d; ++c)
        if (!used[c]) pg[k++] = c;
    }
    auto *m = new (std::nothrow) tq_mixed_codec;
    if (!m) return fail(TQ_ENOMEM, "host allocation failed");
    m->d = d;
    m->n_out = n_out;
    m->groups = groups;
    m->variant = variant;
    int st = make_codec(n_out, b + 1, variant, seed, groups, &m->parts[0]);
    if (st == TQ_OK) st = make_codec(d - n_out, b, variant, seed + 1, groups, &m->parts[1]);
    if (st == TQ_OK) {
      hipError_t e = hipMalloc((void **)&m->perm, perm.size() * sizeof(int32_t));
      if (e == hipSuccess) e = hipMemcpy(m->perm, perm.data(), perm.size() * sizeof(int32_t), hipMemcpyHostToDevice);
      if (e != hipSuccess) st = hip_fail(e, "channel map upload");
    }
    if (st == TQ_OK && d == 128 && n_out == 64 && variant == TQ_MSE && b + 1 <= 4) {
      // one image per group: both parts' rotations on their channels (the
      // parts' matrices are those of make_codec: seeds seed and seed + 1)
      const size_t rot_words = tq::fast128_rotation_words(128);
      std::vector<uint32_t> host((size_t)groups * (rot_words + 4));
      std::vector<float> rt((size_t)groups * d * d, 0.f);
      std::vector<double> pi_o, pi_r, unused_s, unused_m;
      for (int g = 0; g < groups; ++g) {
        group_matrices(64, seed, g, false, pi_o, unused_s, unused_m);
        group_matrices(64, seed + 1, g, false, pi_r, unused_s, unused_m);
        const int32_t *pg = perm.data() + (size_t)g * d;
        tq::fast128_build_mixed_image(pi_o.data(), pi_r.data(), pg, &host[(size_t)g * rot_words],
                                      &host[(size_t)groups * rot_words + 4 * g]);
        float *R = &rt[(size_t)g * d * d];  // R^T[c][j] = R[j][c]
        for (int j = 0; j < 64; ++j)
          for (int i = 0; i < 64; ++i) {
            R[(size_t)pg[i] * d + j] = (float)pi_o[(size_t)j * 64 + i];
            R[(size_t)pg[64 + i] * d + 64 + j] = (float)pi_r[(size_t)j * 64 + i];
          }
      }
      hipError_t e = hipMalloc((void **)&m->fused, host.size() * sizeof(uint32_t));
      if (e == hipSuccess) e = hipMemcpy(m->fused, host.data(), host.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
      if (e == hipSuccess) e = hipMalloc((void **)&m->rt, rt.size() * sizeof(float));
      if (e == hipSuccess) e = hipMemcpy(m->rt, rt.data(), rt.size() * sizeof(float), hipMemcpyHostToDevice);
      if (e != hipSuccess) st = hip_fail(e, "mixed rotation image upload");
    }
    if (st != TQ_OK) {
      tq_mixed_destroy(m);
      return st;
    }
    *out = m;
    return TQ_OK;
  });
}

int tq_mixed_destroy(tq_mixed m) {
  if (!m) return TQ_OK;
  tq_destroy(m->parts[0]);
  tq_destroy(m->parts[1]);
  if (m->perm) (void)hipFree(m->perm);
  if (m->fused) (void)hipFree(m->fused);
  if (m->rt) (void)hipFree(m->rt);
  delete m;
  return TQ_OK;
}

int tq_mixed_parts(tq_mixed m, tq_handle *outlier, tq_handle *regular) {
  int st = check_mixed(m);
  if (st) return st;
  if (outlier) *outlier = m->parts[0];
  if (regular) *regular = m->parts[1];
  return TQ_OK;
}

int tq_mixed_workspace(tq_mixed m, int64_t n_sets, int64_t n, int64_t nq, size_t *bytes) {
  int st = check_mixed(m);
  if (st) return st;
  if (!bytes) return fail(TQ_EINVAL, "bytes is NULL");
  if (n_sets < 0 || n < 0 || nq < 0) return fail(TQ_EINVAL, "sizes must be >= 0");
  // quantize / dequantize: the two parts' gathered inputs or reconstructions
  const size_t vec = mixed_split_bytes(m, n_sets * n, sizeof(float));
  // logits: the two parts' gathered queries, then the regular part's logits
  const size_t lg = mixed_split_bytes(m, n_sets * nq, sizeof(float)) + up256((size_t)(n_sets * nq * n) * sizeof(float));
  *bytes = vec > lg ? vec : lg;
  return TQ_OK;
}

int tq_mixed_quantize(tq_mixed m, const void *x, int dtype, int64_t n_sets, int64_t n, void *const codes[2],
                      void *const signs[2], float *const norms[2], float *const rnorms[2], void *workspace,
                      size_t workspace_bytes, void *stream) {
  int st = check_mixed(m);
  if (st) return st;
  if (!codes || !signs || !norms || !rnorms) return fail(TQ_EINVAL, "part pointer arrays must not be NULL");
  if ((st = check_rows(m->parts[0], n_sets, n))) return st;
  if (n_sets == 0 || n == 0) return TQ_OK;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_EINVAL, "dtype must be TQ_F32 or TQ_BF16");
  if (!x || ((uintptr_t)x & (dtype == TQ_F32 ? 3u : 1u))) return fail(TQ_EINVAL, "x NULL or misaligned");
  if ((st = check_mixed_ptrs(m, codes, signs, norms, rnorms, true))) return st;
  size_t need = 0;
  tq_mixed_workspace(m, n_sets, n, 0, &need);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(TQ_EINVAL, "workspace NULL, not 256-byte aligned or smaller than tq_mixed_workspace reports");
  if ((st = launch_fault("tq_mixed_quantize"))) return st;
  hipStream_t s = (hipStream_t)stream;
  if (m->fused && dtype == TQ_BF16) {
    const uint32_t *masks = m->fused + (size_t)m->groups * tq::fast128_rotation_words(128);
    const hipError_t e = tq::launch_quant128_mixed(m->parts[0]->dev, m->parts[1]->dev, m->fused, masks, x, n_sets, n,
                                                   m->groups, (uint8_t *)codes[0], norms[0], (uint8_t *)codes[1],
                                                   norms[1], s);
    if (e != hipErrorNotSupported) return e == hipSuccess ? TQ_OK : hip_fail(e, "mixed quantize launch");
  }
  const size_t es = dtype == TQ_F32 ? 4 : 2;
  char *xo = (char *)workspace;
  char *xr = xo + up256((size_t)(n_sets * n) * m->n_out * es);
  hipError_t e = tq::launch_gather_parts(x, dtype, n_sets * n, n, m->groups, m->d, m->n_out, m->perm, xo, xr, s);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  for (int p = 0; p < 2; ++p)
    if ((st = tq_quantize(m->parts[p], p == 0 ? xo : xr, dtype, n_sets, n, codes[p], signs[p], norms[p], rnorms[p],
                          stream)))
      return st;
  return TQ_OK;
}

int tq_mixed_dequantize(tq_mixed m, const void *const codes[2], const void *const signs[2],
                        const float *const norms[2], const float *const rnorms[2], int64_t n_sets, int64_t n,
                        float *x_out, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_mixed(m);
  if (st) return st;
  if (!codes || !signs || !norms || !rnorms) return fail(TQ_EINVAL, "part pointer arrays must not be NULL");
  if ((st = check_rows(m->parts[0], n_sets, n))) return st;
  if (n_sets == 0 || n == 0) return TQ_OK;
  if (!x_out || ((uintptr_t)x_out & 3u)) return fail(TQ_EINVAL, "x_out NULL or misaligned");
  if ((st = check_mixed_ptrs(m, codes, signs, norms, rnorms, false))) return st;
  size_t need = 0;
  tq_mixed_workspace(m, n_sets, n, 0, &need);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(TQ_EINVAL, "workspace NULL, not 256-byte aligned or smaller than tq_mixed_workspace reports");
  if ((st = launch_fault("tq_mixed_dequantize"))) return st;
  float *xo = (float *)workspace;
  float *xr = (float *)((char *)workspace + up256((size_t)(n_sets * n) * m->n_out * 4));
  for (int p = 0; p < 2; ++p)
    if ((st = tq_dequantize(m->parts[p], codes[p], signs[p], norms[p], rnorms[p], n_sets, n, p == 0 ? xo : xr,
                            stream)))
      return st;
  hipError_t e = tq::launch_scatter_parts(xo, xr, n_sets * n, n, m->groups, m->d, m->n_out, m->perm, x_out,
                                          (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "scatter launch");
}

int tq_mixed_logits(tq_mixed m, const float *q, int64_t nq, const void *const codes[2], const void *const signs[2],
                    const float *const norms[2], const float *const rnorms[2], int64_t n_sets, int64_t n_keys,
                    float *out, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_mixed(m);
  if (st) return st;
  if (!codes || !signs || !norms || !rnorms) return fail(TQ_EINVAL, "part pointer arrays must not be NULL");
  if ((st = check_rows(m->parts[0], n_sets, n_keys))) return st;
  if (nq < 1 || nq > 64) return fail(TQ_EINVAL, "nq must be in [1, 64]");
  if (n_sets == 0 || n_keys == 0) return TQ_OK;
  if (!q || ((uintptr_t)q & 3u)) return fail(TQ_EINVAL, "q NULL or misaligned");
  if (!out || ((uintptr_t)out & 3u)) return fail(TQ_EINVAL, "out NULL or misaligned");
  if ((st = check_mixed_ptrs(m, codes, signs, norms, rnorms, false))) return st;
  size_t need = 0;
  tq_mixed_workspace(m, n_sets, n_keys, nq, &need);
  if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
    return fail(TQ_EINVAL, "workspace NULL, not 256-byte aligned or smaller than tq_mixed_workspace reports");
  if ((st = launch_fault("tq_mixed_logits"))) return st;
  if (m->rt) {
    const hipError_t e = tq::launch_logits128_mixed(m->parts[0]->dev, m->parts[1]->dev, m->rt, q, nq,
                                                    (const uint8_t *)codes[0], (const uint8_t *)codes[1], norms[0],
                                                    norms[1], n_sets, n_keys, m->groups, out, (hipStream_t)stream);
    if (e != hipErrorNotSupported) return e == hipSuccess ? TQ_OK : hip_fail(e, "mixed logits launch");
  }
  char *ws = (char *)workspace;
  float *qo = (float *)ws;
  float *qr = (float *)(ws + up256((size_t)(n_sets * nq) * m->n_out * 4));
  float *lr = (float *)(ws + mixed_split_bytes(m, n_sets * nq, 4));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = tq::launch_gather_parts(q, TQ_F32, n_sets * nq, nq, m->groups, m->d, m->n_out, m->perm, qo, qr, s);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  if ((st = tq_logits(m->parts[0], qo, nq, codes[0], signs[0], norms[0], rnorms[0], n_sets, n_keys, out, stream)))
    return st;
  if ((st = tq_logits(m->parts[1], qr, nq, codes[1], signs[1], norms[1], rnorms[1], n_sets, n_keys, lr, stream)))
    return st;
  e = tq::launch_add_inplace(out, lr, n_sets * nq * n_keys, s);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "accumulate launch");
}

int tq_dense_logits(const float *q, int64_t nq, const void *keys, int dtype, int d, int64_t n_sets, int64_t n_keys,
                    float *out, void *stream) {
  if (d != 128) return fail(TQ_EUNSUPPORTED, "the dense baseline handles d = 128");
  if (dtype != TQ_F16 && dtype != TQ_F32) return fail(TQ_EINVAL, "dtype must be TQ_F16 or TQ_F32");
  if (n_sets < 0 || n_keys < 0 || n_sets > 65535) return fail(TQ_EINVAL, "n_sets must be in [0, 65535], n_keys >= 0");
  if (nq < 1 || nq > 64) return fail(TQ_EINVAL, "nq must be in [1, 64]");
  if (n_sets == 0 || n_keys == 0) return TQ_OK;
  if (!q || ((uintptr_t)q & 3u)) return fail(TQ_EINVAL, "q NULL or misaligned");
  if (!keys || !aligned16(keys)) return fail(TQ_EINVAL, "keys NULL or not 16-byte aligned");
  if (!out || ((uintptr_t)out & 3u)) return fail(TQ_EINVAL, "out NULL or misaligned");
  if (const int f = launch_fault("tq_dense_logits")) return f;
  const hipError_t e = tq::launch_dense_logits128(q, nq, keys, dtype == TQ_F32, n_sets, n_keys, out,
                                                  (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(TQ_EUNSUPPORTED, "set too large for 32-bit offsets");
  return e == hipSuccess ? TQ_OK : hip_fail(e, "dense logits launch");
}

int tq_probe_stream(int kind, const void *in, int64_t in_bytes, void *out, int64_t out_bytes, int grid, void *stream) {
  const int64_t tiles = tq::probe_stream_tiles(kind, in_bytes);
  if (tiles < 0) return fail(TQ_EINVAL, "kind must be in [0, 5]");
  if (tiles == 0) return TQ_OK;
  if (!in || !aligned16(in) || !out || !aligned16(out)) return fail(TQ_EINVAL, "in/out NULL or not 16-byte aligned");
  if (out_bytes < tq::probe_stream_out_bytes(kind, tiles) || out_bytes < 1024)
    return fail(TQ_EINVAL, "out smaller than the stream writes");
  if (grid < 1 || grid > (1 << 20)) return fail(TQ_EINVAL, "grid must be in [1, 2^20]");
  if (kind == 4 && tq::probe_stream_out_bytes(kind, tiles) > 0x7FFFFFFF)
    return fail(TQ_EINVAL, "kind 4 writes 32-bit offsets: in_bytes too large");
  const hipError_t e = tq::launch_probe_stream(kind, in, out, tiles, grid, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "probe launch");
}

int tq_probe_issue(int mode, int waves_per_simd, int64_t iters, int grid, uint32_t *out, void *stream) {
  if (mode < 0 || mode > 2 || waves_per_simd < 1 || waves_per_simd > 2 || iters < 0 || grid < 1 ||
      grid > 4096 || !out)
    return fail(TQ_EINVAL, "bad probe arguments");
  const hipError_t e = tq::launch_probe_issue(mode, waves_per_simd, iters, grid, out, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "probe launch");
}

int tq_probe_mfma(int f16, int64_t iters, int grid, float *out, void *stream) {
  if (iters < 0 || grid < 1 || grid > (1 << 20) || !out) return fail(TQ_EINVAL, "bad probe arguments");
  const hipError_t e = tq::launch_probe_mfma(f16 != 0, iters, grid, out, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "probe launch");
}

const char *tq_strerror(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_ENOMEM: return "out of memory";
    case TQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *tq_last_error(void) { return g_last_error.c_str(); }

int tq_get_tables(tq_handle h, int g, float *Pi, float *S, float *centroids, float *bounds) {
  int st = check_handle(h);
  if (st) return st;
  if (g < 0 || g >= h->groups) return fail(TQ_EINVAL, "group out of range");
  const size_t dd = (size_t)h->d * h->d;
  hipError_t e = hipSuccess;
  if (Pi) e = hipMemcpy(Pi, h->dev.Pi + g * dd, dd * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && S && h->variant == TQ_PROD)
    e = hipMemcpy(S, h->dev.S + g * dd, dd * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && centroids && h->mse_bits > 0)
    e = hipMemcpy(centroids, h->dev.cent, h->h_c.size() * 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && bounds && h->mse_bits > 0)
    e = hipMemcpy(bounds, h->dev.bnd, h->h_t.size() * 4, hipMemcpyDeviceToHost);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "hipMemcpy of the tables");
}

int tq_host_tables(int d, int b, int variant, uint64_t seed, int g, float *Pi, float *S,
                   float *centroids, float *bounds) {
  g_last_error.clear();
  return guarded([&]() -> int {
    int mse_bits = 0;
    int st = check_config(d, b, variant, 1, &mse_bits);
    if (st) return st;
    if (g < 0) return fail(TQ_EINVAL, "group must be >= 0");
    std::vector<double> pi, s, m;
    group_matrices(d, seed, g, variant == TQ_PROD, pi, s, m);
    const size_t dd = (size_t)d * d;
    if (Pi)
      for (size_t i = 0; i < dd; ++i) Pi[i] = (float)pi[i];
    if (S && variant == TQ_PROD)
      for (size_t i = 0; i < dd; ++i) S[i] = (float)s[i];
    if (mse_bits > 0 && (centroids || bounds)) {
      const tq::Codebook cb = tq::lloyd_max(d, mse_bits);
      if (centroids)
        for (size_t k = 0; k < cb.centroids.size(); ++k) centroids[k] = (float)cb.centroids[k];
      if (bounds)
        for (size_t k = 0; k < cb.boundaries.size(); ++k) bounds[k] = (float)cb.boundaries[k];
    }
    return TQ_OK;
  });
}

int tq_pack(tq_handle h, const uint8_t *idx, int bits, int64_t rows, void *out, void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if (bits < 1 || bits > 8) return fail(TQ_EINVAL, "bits must be in [1, 8]");
  if (rows < 0) return fail(TQ_EINVAL, "rows must be >= 0");
  if (rows == 0) return TQ_OK;
  if (!idx || !out || !aligned16(out)) return fail(TQ_EINVAL, "idx/out NULL or out misaligned");
  hipError_t e = tq::launch_pack(idx, bits, rows, h->d, row_bytes(h->d, bits), (uint8_t *)out,
                                 (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "pack launch");
}

int tq_unpack(tq_handle h, const void *in, int bits, int64_t rows, uint8_t *idx, void *stream) {
  int st = check_handle(h);
  if (st) return st;
  if (bits < 1 || bits > 8) return fail(TQ_EINVAL, "bits must be in [1, 8]");
  if (rows < 0) return fail(TQ_EINVAL, "rows must be >= 0");
  if (rows == 0) return TQ_OK;
  if (!idx || !in || !aligned16(in)) return fail(TQ_EINVAL, "in/idx NULL or in misaligned");
  hipError_t e = tq::launch_unpack((const uint8_t *)in, bits, rows, h->d, row_bytes(h->d, bits),
                                   idx, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "unpack launch");
}

}  // extern "C"
