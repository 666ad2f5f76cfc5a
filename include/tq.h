/*
 * tq.h -- C ABI of the TurboQuant hot path on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, section):
 *   [ttakun]  "KV缓存52GB瞬间爆内存？TurboQuant随机旋转+标量量化如何把LLM长上下文推理成本砍到1/16
 *             且失真逼近理论极限", sections "为什么随机旋转是整个算法的底层杠杆" and
 *             "TurboQuant_mse vs TurboQuant_prod两个变体的精确分工".
 *   [tmdm]    "谷歌悄悄扔下一颗'性能核弹'", section "双剑合璧：PolarQuant + QJL".
 *   [admirer] admirer.cn TurboQuant article, sections "第一步" and "第二步".
 *   [tqnet]   turboquant.net/zh, sections "TurboQuant 两阶段算法 › 坐标分布公式",
 *             "实现步骤草图" and "工程风险与应对".
 *
 * Conventions shared by every entry point
 *   - Status: TQ_OK (0) or a negative TQ_E* code; tq_last_error() returns a
 *     thread-local message for the last failure on the calling thread.  C++
 *     exceptions never cross this boundary.
 *   - Validation failures return before anything is enqueued.  A failed kernel
 *     launch returns TQ_EHIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation.
 *   - Data calls are asynchronous: they enqueue on `stream` (a hipStream_t,
 *     NULL = the default stream) and return.  Every data pointer is a device
 *     pointer owned by the caller; the library allocates no memory per call.
 *   - The handle owns its device tables (rotation, projection, codebook),
 *     allocated on the HIP device current at tq_init and freed by tq_destroy.
 *     A handle is immutable after init: concurrent calls on it are safe.
 *   - Identical inputs give bitwise identical outputs, with one exception:
 *     the d = 128 attention kernel (tq_attention, tq_attention_static) hands
 *     key blocks to its waves from a counter as they finish, so the order of
 *     its float32 softmax sums varies from run to run and its outputs agree
 *     to float32 rounding (about 1e-7 relative), not bit for bit.
 *
 * Stored layout (the pages leave it open)
 *   - codes : [n_sets][n][code_row_bytes] uint8.  Coordinate j's index
 *             occupies bits [j*mb, j*mb+mb) of the row's little-endian,
 *             LSB-first bit stream (stream bit k = bit k%8 of byte k/8);
 *             mb = mse bits.  Rows are zero-padded to a multiple of 16 bytes.
 *   - signs : [n_sets][n][sign_row_bytes] uint8, same layout with 1 bit per
 *             projection; bit 1 <=> sign +1 (sign(0) = +1).
 *   - norms : [n_sets][n] float32 = ||x||;  rnorms : [n_sets][n] float32 =
 *             ||r|| of the prod residual of the unit vector.
 *   - Block s of n_sets uses codec group s % groups.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tq_codec *tq_handle;

enum { TQ_MSE = 0, TQ_PROD = 1 };
enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 };  /* TQ_F16: dense baseline keys only */
enum { TQ_OK = 0, TQ_EINVAL = -1, TQ_EUNSUPPORTED = -2, TQ_ENOMEM = -3, TQ_EHIP = -4 };

/* Build a codec: d dimensions, b bits per coordinate, variant TQ_MSE or
 * TQ_PROD, deterministic from `seed`.  Equivalent to tq_init_groups(..., 1).
 * [tqnet] 实现步骤草图 (precompute the Lloyd–Max centroids once, generate the
 * rotation by QR of a Gaussian matrix); [tqnet] 工程风险与应对 (pre-generate
 * and reuse the matrix).  Valid: 2 <= d <= 4096; mse: 1 <= b <= 8;
 * prod: 1 <= b <= 5 (b-1 mse bits, b = 1 is QJL only).  *out receives the
 * handle (unchanged on failure).  Errors: TQ_EINVAL, TQ_ENOMEM, TQ_EHIP. */
int tq_init(int d, int b, int variant, uint64_t seed, tq_handle *out);

/* As tq_init with `groups` independent (Pi, S) pairs; group g draws its
 * matrices from stream (seed, g).  The codebook is shared.  1 <= groups <= 4096. */
int tq_init_groups(int d, int b, int variant, uint64_t seed, int groups, tq_handle *out);

/* Free the handle and its device tables.  NULL is a no-op. */
int tq_destroy(tq_handle h);

/* Row sizes of the stored arrays and the number of mse bits per coordinate
 * (b for mse, b-1 for prod).  Any output pointer may be NULL. */
int tq_layout(tq_handle h, int64_t *code_row_bytes, int64_t *sign_row_bytes, int *mse_bits);

/* Quantize n_sets blocks of n vectors x[n_sets][n][d] (dtype TQ_F32 or TQ_BF16).
 * mse ([ttakun] TurboQuant_mse: normalise and store ||x|| as float32, rotate,
 * index each coordinate against the precomputed codebook): writes codes and
 * norms.  prod ([ttakun] TurboQuant_prod; [admirer] 第一步/第二步: (b-1)-bit mse
 * stage, residual r, 1-bit QJL signs of S r): also writes signs and rnorms.
 * The index of coordinate j is #{k : t_k < (Pi x/||x||)_j} (ties to the lower
 * index).  A zero vector gets norm 0, rnorm 0 and all signs +1.
 * codes may be NULL only when the handle has 0 mse bits; signs/rnorms must be
 * NULL for mse and non-NULL for prod.  Pointers 16-byte aligned (x: 4-byte for
 * f32 / 2-byte for bf16; norms 4-byte).  n == 0 or n_sets == 0 is a no-op.
 * Errors: TQ_EINVAL, TQ_EHIP. */
int tq_quantize(tq_handle h, const void *x, int dtype, int64_t n_sets, int64_t n,
                void *codes, void *signs, float *norms, float *rnorms, void *stream);

/* Online append: quantize one vector per set, x[n_sets][d] (dtype TQ_F32 or
 * TQ_BF16), and write it into row rows[s] of the cache arrays codes / signs /
 * norms / rnorms, each holding cache_rows rows in the tq_quantize row layout
 * ([ttakun] TurboQuant_mse: no training or warm-up, so each new token is
 * quantized on its own as it arrives).  rows: device array of n_sets int64
 * physical row indices (a paged cache resolves its page table into them);
 * a row outside [0, cache_rows) is skipped, and two sets naming one row race.
 * Set s uses codec group s % groups.  The codes follow the same definition
 * as tq_quantize's (the contraction is plain fp32 here, split-bf16 MFMA
 * there, so a coordinate within rounding of a boundary may take the
 * neighbouring index).  Pointer and NULL rules as tq_quantize.
 * n_sets == 0 is a no-op.  Errors: TQ_EINVAL, TQ_EHIP. */
int tq_append(tq_handle h, const void *x, int dtype, int64_t n_sets, const int64_t *rows, int64_t cache_rows,
              void *codes, void *signs, float *norms, float *rnorms, void *stream);

/* Reconstruct x_out[n_sets][n][d] float32.  mse: ||x|| Pi^T c[idx] ([ttakun]
 * inverse rotation and rescale; [tqnet] dequant x = Pi.T @ centroids[idx]).
 * prod: ||x|| (Pi^T c[idx] + sqrt(pi/2)/d * ||r|| S^T z), the unbiased QJL
 * reconstruction.  Arguments as in tq_quantize.  Errors: TQ_EINVAL, TQ_EHIP. */
int tq_dequantize(tq_handle h, const void *codes, const void *signs, const float *norms,
                  const float *rnorms, int64_t n_sets, int64_t n, float *x_out, void *stream);

/* Attention logits / inner products scored directly on packed keys
 * ([admirer] 第二步: the full-precision query balanced against the 1-bit codes;
 * [tmdm] unbiased estimator at attention time).  For set s, query i and key t:
 *   out[s][i][t] = <q[s][i], k_hat[s][t]>   (no 1/sqrt(d), no softmax),
 * where k_hat is the tq_dequantize reconstruction.  q: [n_sets][nq][d] float32
 * (grouped-query attention passes the query heads of one KV head as one set).
 * The kernel rotates and projects each query once and never materialises
 * k_hat.  At d = 128 (mse bits <= 4) sets below 2^29 keys take the
 * streaming kernel, in launches of at most 2^25 keys; longer sets (and other
 * d) take the generic one, with the same results up to fp32 rounding.
 * 1 <= nq <= 64.  Errors: TQ_EINVAL, TQ_EHIP. */
int tq_logits(tq_handle h, const float *q, int64_t nq, const void *codes, const void *signs,
              const float *norms, const float *rnorms, int64_t n_sets, int64_t n_keys, float *out,
              void *stream);

/* Decode attention over quantized keys and values ([tqnet] 实现步骤草图 ›
 * 集成到 attention: keys and values are both stored in the quantized format and
 * attention reads the QJL-coded keys).  For set s and query i:
 *   out[s][i] = sum_t softmax_t(scale * <q[s][i], k_hat[s][t]>) v_hat[s][t],
 * with k_hat the tq_dequantize reconstruction of the keys under hk and v_hat
 * that of the values under hv (same d; any variants and bits).  The softmax
 * runs over the n_keys keys of set s; scale is the caller's (1/sqrt(d) for
 * standard attention) and must be finite.  Set s uses group s % groups of
 * each codec.  q: [n_sets][nq][d] float32, out: [n_sets][nq][d] float32
 * (4-byte aligned); key and value arrays as in tq_logits / tq_dequantize.
 * workspace: caller-owned device memory, 256-byte aligned, of at least the
 * size tq_attention_workspace reports for the same (hk, hv, nq, n_sets,
 * n_keys); its contents are scratch (undefined before and after), and two
 * calls in flight at once need two workspaces.  1 <= nq <= 64; n_keys >= 1
 * unless n_sets == 0 (a no-op).  Errors: TQ_EINVAL (also for a small or
 * misaligned workspace), TQ_EHIP. */
int tq_attention(tq_handle hk, tq_handle hv, const float *q, int64_t nq, const void *k_codes,
                 const void *k_signs, const float *k_norms, const float *k_rnorms, const void *v_codes,
                 const void *v_signs, const float *v_norms, const float *v_rnorms, int64_t n_sets,
                 int64_t n_keys, float scale, float *out, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Workspace bytes tq_attention needs for this shape (0 when n_sets == 0).
 * Host only; validates as tq_attention does.  Errors: TQ_EINVAL. */
int tq_attention_workspace(tq_handle hk, tq_handle hv, int64_t nq, int64_t n_sets, int64_t n_keys,
                           size_t *bytes);

/* tq_attention for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the workspace taken from a fixed device
 * array inside the library instead of an argument.  That array holds
 * TQ_STATIC_SCRATCH_BYTES (16 MiB) on every GPU the library runs on, from the
 * library's load until the process ends; its address on a device is looked
 * up at tq_init on that device (or at this call's first use there).  The call
 * allocates nothing.  A shape whose tq_attention_workspace size exceeds the
 * array fails with TQ_EINVAL (the decode shape, 128 sets x 4 heads x 131072
 * keys at d = 128, needs 0.5 MiB).  All calls on one GPU share its array:
 * calls that overlap in time on that GPU (two streams, two threads) race and
 * give undefined results; calls ordered on one stream are safe.  Arguments,
 * other rules and errors as tq_attention. */
#define TQ_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int tq_attention_static(tq_handle hk, tq_handle hv, const float *q, int64_t nq, const void *k_codes,
                        const void *k_signs, const float *k_norms, const float *k_rnorms, const void *v_codes,
                        const void *v_signs, const float *v_norms, const float *v_rnorms, int64_t n_sets,
                        int64_t n_keys, float scale, float *out, void *stream);

/* Maximum inner product search over one set of n_keys packed keys (group
 * 0): for each query q[i] (float32 [nq][d]), the k keys with the largest
 * estimates <q[i], k_hat[t]> (the tq_logits values), best first; equal
 * scores are ordered by key index.  out_scores: [nq][k] float32, out_idx:
 * [nq][k] int32.  The scan is fused with the selection: no score matrix is
 * written when d <= 256, mse bits <= 4 and the index fits 32-bit offsets.
 * Other codecs score 65536-key chunks of 64-query blocks into the
 * workspace with the tq_logits kernels and select from those (the same
 * estimates up to fp32 rounding, slower).  ([ttakun] 索引速度: the same codes serve vector search;
 * the inner-product estimator as in tq_logits.)  1 <= k <= 64, n_keys >= k.
 * workspace: caller-owned device memory, 256-byte aligned, of at least the
 * tq_topk_workspace size (0 when nq is 0); scratch.  Errors: TQ_EINVAL,
 * TQ_EHIP. */
int tq_topk_workspace(tq_handle h, int64_t nq, int64_t n_keys, int k, size_t *bytes);
int tq_topk(tq_handle h, const float *q, int64_t nq, const void *codes, const void *signs, const float *norms,
            const float *rnorms, int64_t n_keys, int k, float *out_scores, int32_t *out_idx, void *workspace,
            size_t workspace_bytes, void *stream);

/* ---- outlier-channel mixed precision ----
 * The pages keep outlier channels apart at a higher precision ([tqnet]
 * 从工程视角看 TurboQuant 到底改变了什么) and quote 2.5- and 3.5-bit KV
 * configurations ([tqnet] 数据就是论据 › KV Cache 压缩基准; [ttakun], 3.5 bits
 * per channel).  No split rule is given; this is the plainest one.  A mixed codec
 * splits the d channels of every vector into an outlier part (n_out channels
 * per group, named by the caller) and a regular part (the other d - n_out
 * channels, ascending).  Each part is an independent TurboQuant codec of its
 * own dimension: the outlier part at b + 1 bits with `seed`, the regular part
 * at b bits with `seed + 1`, same variant and groups.  n_out = d / 2 gives
 * b + 0.5 bits per channel (2.5 at b = 2, 3.5 at b = 3).  Reconstructions
 * scatter the parts back; inner products are the sum of the parts'. */
typedef struct tq_mixed_codec *tq_mixed;

/* out_channels: host array [groups][n_out] of distinct channels in [0, d)
 * per group.  Valid: 4 <= d <= 4096; 2 <= n_out <= d - 2; mse 1 <= b <= 7,
 * prod 1 <= b <= 4.  Errors: TQ_EINVAL, TQ_ENOMEM, TQ_EHIP. */
int tq_mixed_init(int d, int b, int variant, uint64_t seed, int groups, int n_out, const int32_t *out_channels,
                  tq_mixed *out);
int tq_mixed_destroy(tq_mixed m);

/* The two part codecs (owned by m: do not destroy them).  Their tq_layout
 * gives each part's row sizes; their tables are the parts' tables. */
int tq_mixed_parts(tq_mixed m, tq_handle *outlier, tq_handle *regular);

/* Workspace bytes the calls below need for n_sets x n vectors and nq
 * queries per set (pass nq = 0 when no logits call is planned). */
int tq_mixed_workspace(tq_mixed m, int64_t n_sets, int64_t n, int64_t nq, size_t *bytes);

/* Quantize x[n_sets][n][d] (TQ_F32 / TQ_BF16): every argument array of two
 * device pointers holds the outlier part's array at [0] and the regular
 * part's at [1], each in the layout of tq_quantize for that part's codec.
 * workspace: caller-owned device memory, 256-byte aligned, at least the
 * tq_mixed_workspace size; scratch.  For d = 128 with 64 outlier channels,
 * TurboQuant_mse, b <= 3 and 16-byte aligned TQ_BF16 input, one fused pass
 * does both parts (the workspace is then not touched); otherwise the channels
 * are gathered into the workspace and each part codec quantizes its share.
 * Errors: TQ_EINVAL, TQ_EHIP. */
int tq_mixed_quantize(tq_mixed m, const void *x, int dtype, int64_t n_sets, int64_t n, void *const codes[2],
                      void *const signs[2], float *const norms[2], float *const rnorms[2], void *workspace,
                      size_t workspace_bytes, void *stream);

/* Reconstruct x_out[n_sets][n][d] float32 (each part's tq_dequantize,
 * scattered back to its channels).  Arrays and workspace as above. */
int tq_mixed_dequantize(tq_mixed m, const void *const codes[2], const void *const signs[2],
                        const float *const norms[2], const float *const rnorms[2], int64_t n_sets, int64_t n,
                        float *x_out, void *workspace, size_t workspace_bytes, void *stream);

/* out[s][i][t] = <q[s][i], x_hat[s][t]> for the mixed reconstruction: the
 * outlier part's logits plus the regular part's (queries split the same
 * way).  q: [n_sets][nq][d] float32, 1 <= nq <= 64.  Arrays and workspace
 * as above (the workspace also holds one part's logits).  For d = 128 with
 * 64 outlier channels and TurboQuant_mse parts (b <= 3) one kernel reads both
 * parts' codes and the workspace is not touched. */
int tq_mixed_logits(tq_mixed m, const float *q, int64_t nq, const void *const codes[2], const void *const signs[2],
                    const float *const norms[2], const float *const rnorms[2], int64_t n_sets, int64_t n_keys,
                    float *out, void *workspace, size_t workspace_bytes, void *stream);

/* ---- dense baseline (unquantized keys; not part of the quantized path) ----
 * out[s][i][t] = <q[s][i], k[s][t]> for keys stored unquantized as float16
 * (dtype TQ_F16) or float32 (TQ_F32), keys: [n_sets][n_keys][d] (16-byte
 * aligned), q: [n_sets][nq][d] float32, out: [n_sets][nq][n_keys] float32,
 * float32 accumulation.  This is the comparison the pages draw for the
 * attention logits of 4-bit codes against unquantized keys ([admirer]
 * 內存價格能下來嗎？; [tmdm] 实测数据), run on the same GPU.  d = 128 only
 * (else TQ_EUNSUPPORTED); 1 <= nq <= 64; a set's keys must fit 32-bit byte
 * offsets (else TQ_EUNSUPPORTED).  Errors: TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP. */
int tq_dense_logits(const float *q, int64_t nq, const void *keys, int dtype, int d, int64_t n_sets, int64_t n_keys,
                    float *out, void *stream);

/* ---- measurement probes (the ceilings the kernels are compared with) ----
 * tq_probe_stream: one streaming kernel over in[in_bytes] (device, 16-byte
 * aligned): kind 0 copies (reads and writes the same bytes), 1 reads 4 bytes
 * per byte written (the d = 128 quantize's mix), 2 reads 9 per 2 written (the
 * decode logits' mix), 3 only reads, 4 is the mix of kind 2 with the logits
 * kernel's store pattern (4-byte stores into four rows), 5 writes 8 bytes per
 * byte read (the d = 128 dequantize's mix).  Whole 16 KiB / 36 KiB tiles only;
 * out must hold what the kind writes (in_bytes, in_bytes / 4, 2 in_bytes / 9,
 * 1 KiB, 2 in_bytes / 9, 8 in_bytes).  grid: workgroups of 256 threads.
 * tq_probe_mfma: `grid` workgroups of 4 waves, each running iters x 8 back-
 * to-back 16x16x32 MFMAs (bf16, or f16 when f16 != 0); out: grid x 256
 * floats.
 * tq_probe_issue: `grid` workgroups of waves_per_simd (1 or 2) x 4 waves,
 * each running iters iterations of 48 independent float32 FMAs (mode 0), 16
 * back-to-back bf16 MFMAs (mode 1), or both interleaved as one MFMA and three
 * FMAs (mode 2).  out (device): 2 uint32 per wave in launch order, the
 * wave's shader-clock cycles over the loop and its ticks of the 100 MHz real
 * time counter, so cycles / (ticks x 10 ns) is the clock it ran at; grid <=
 * 4096.  Errors: TQ_EINVAL, TQ_EHIP. */
int tq_probe_stream(int kind, const void *in, int64_t in_bytes, void *out, int64_t out_bytes, int grid, void *stream);
int tq_probe_mfma(int f16, int64_t iters, int grid, float *out, void *stream);
int tq_probe_issue(int mode, int waves_per_simd, int64_t iters, int grid, uint32_t *out, void *stream);

/* Static text for a status code. */
const char *tq_strerror(int status);
/* Thread-local detail of the last failure on this thread ("" if none). */
const char *tq_last_error(void);

/* ---- test hooks (not used by the hot path) ---- */

/* Host copies of group g's tables as the device holds them: Pi [d][d]
 * row-major (y = Pi x), S [d][d] (prod only, else ignored), centroids
 * [2^mb] ascending, boundaries [2^mb - 1].  Any pointer may be NULL.
 * Synchronous.  Errors: TQ_EINVAL, TQ_EHIP. */
int tq_get_tables(tq_handle h, int g, float *Pi, float *S, float *centroids, float *bounds);

/* The same tables computed on the host only (no device needed). */
int tq_host_tables(int d, int b, int variant, uint64_t seed, int g, float *Pi, float *S,
                   float *centroids, float *bounds);

/* Pack rows x d indices (uint8, each < 2^bits) into the stored layout with
 * h's dimension d: out[rows][row_bytes(d, bits)].  1 <= bits <= 8.
 * Errors: TQ_EINVAL, TQ_EHIP. */
int tq_pack(tq_handle h, const uint8_t *idx, int bits, int64_t rows, void *out, void *stream);
/* Inverse of tq_pack. */
int tq_unpack(tq_handle h, const void *in, int bits, int64_t rows, uint8_t *idx, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
