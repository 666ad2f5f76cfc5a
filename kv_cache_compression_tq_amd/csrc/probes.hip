// Measurement probes: the memory-system and matrix-core ceilings the hot-path
// kernels are compared with.  Not part of the hot path.
//
// k_probe_stream<R, W>: a wave takes a tile of 64 units; it reads R 16-byte
//   words per unit and writes W (R x 64 then W x 64 consecutive words, so
//   every load and store instruction moves 1 KiB of consecutive bytes).  The
//   words written are the XOR of the words read, so no load can be dropped.
//   R:W = 1:1 is a copy, 4:1 the read/write mix of the d = 128 quantize (256 B
//   read per 68 B written), 9:2 that of the decode logits (72 B per key read,
//   16 B written), 1:8 that of the d = 128 dequantize (68 B read per 512 B
//   written), 1:0 a read-only stream.
// k_probe_rows: the logits mix with the logits kernel's store pattern: per
//   16-key tile, 4-byte stores into four output rows (16 keys x 4 bytes each),
//   instead of whole 1 KiB runs.
// k_probe_mfma: back-to-back 16x16x32 bf16 (or f16) MFMAs on eight
//   independent accumulators per wave, no memory traffic.
// k_probe_issue: what one wave (or two waves sharing a SIMD) can issue: per
//   iteration 48 independent float FMAs (mode 0), 16 bf16 MFMAs (mode 1), or
//   both, one MFMA then three FMAs (mode 2).  Each wave records its shader
//   clock cycles and its real time (100 MHz counter) over the loop, which give
//   cycles per instruction and the clock the chip ran at.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace tq {
namespace {

constexpr int kProbeThreads = 256;

// U consecutive tiles per iteration, so that each lane keeps at least eight
// 16-byte loads in flight whatever R is (one load per lane per iteration
// leaves the memory system idle between a load and its dependent store).
template <int R, int W>
__global__ __launch_bounds__(kProbeThreads) void k_probe_stream(const u32x4 *__restrict__ in, u32x4 *__restrict__ out,
                                                                int64_t tiles) {
  constexpr int U = R >= 8 ? 1 : (8 + R - 1) / R;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
  u32x4 keep = {0, 0, 0, 0};
  for (int64_t t0 = wave * U; t0 < tiles; t0 += waves * U) {
    u32x4 v[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u < tiles ? t0 + u : tiles - 1;  // a short last group re-reads a tile
#pragma unroll
      for (int r = 0; r < R; ++r) v[u][r] = __builtin_nontemporal_load(in + (t * R + r) * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < R; ++r) acc ^= v[u][r];
      if constexpr (W > 0) {
        if (t0 + u < tiles) {
#pragma unroll
          for (int w = 0; w < W; ++w) out[((t0 + u) * W + w) * 64 + lane] = acc + (uint32_t)w;
        }
      } else {
        keep ^= acc;
      }
    }
  }
  if constexpr (W == 0)
    if (keep[0] == 0x9E3779B9u && keep[1] == 0x7F4A7C15u) out[lane] = keep;  // practically never
}

// Keys of 72 bytes (4.5 words) read as 9 words per pair of keys; per 16-key
// tile each lane of groups 0 and 1 stores one float into each of the rows of
// heads 2 grp and 2 grp + 1 (four rows of n_keys floats), as the logits kernel
// does for four query heads (its lanes of groups 2 and 3 hold no head).
__global__ __launch_bounds__(kProbeThreads) void k_probe_rows(const u32x4 *__restrict__ in, float *__restrict__ out,
                                                              int64_t tiles, int64_t n_keys) {
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
  // a tile is 128 keys: 9 x 64 words read; 8 x 16 keys stored into 4 rows
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)(4 * n_keys * 4), kBufferFlags);
  const uint32_t rowA = (uint32_t)(2 * grp * n_keys) * 4, rowB = (uint32_t)((2 * grp + 1) * n_keys) * 4;
  for (int64_t t = wave; t < tiles; t += waves) {
    u32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 9; ++r) acc ^= __builtin_nontemporal_load(in + (t * 9 + r) * 64 + lane);
    const float v = __uint_as_float((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) & 0x3fffffffu);
    // as in the logits kernel: lanes without a head store at an offset past
    // the buffer (dropped), with no branch that would let the compiler skip
    // their loads
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t key4 = (uint32_t)(t * 128 + 16 * u + col) * 4;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v + (float)u), ro, grp < 2 ? rowA + key4 : kDropped, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v - (float)u), ro, grp < 2 ? rowB + key4 : kDropped, 0, 0);
    }
  }
}

template <bool F16>
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int64_t iters, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 a = {(uint32_t)lane * 0x00010001u, 0x3c003c00u, 0x3c003c00u, (uint32_t)lane};
  u32x4 b = {0x3c003c00u, (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  f32x4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4{0, 0, 0, (float)i};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = F16 ? mfma_f16(a, b, c[i]) : mfma_bf16(a, b, c[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

template <int MODE>
__global__ __launch_bounds__(512) void k_probe_issue(int64_t iters, uint32_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 a = {(uint32_t)lane * 0x00010001u, 0x3c003c00u, 0x3c003c00u, (uint32_t)lane};
  const u32x4 b = {0x3c003c00u, (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  asm volatile("" : "+a"(a));  // the A operand in an AGPR, as in the quantize kernel
  f32x4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4{0, 0, 0, (float)i};
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = lane * 0.01f + i;
  const float r0 = 0.999f + lane * 1e-6f, r1 = 0.001f - lane * 1e-7f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), q0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
#pragma unroll
      for (int v = 0; v < 48; ++v) f[v & 15] = fmaf(f[v & 15], r0, r1);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        c[j & 7] = mfma_bf16(a, b, c[j & 7]);
        if constexpr (MODE == 2) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
          for (int v = 0; v < 3; ++v) f[(3 * j + v) & 15] = fmaf(f[(3 * j + v) & 15], r0, r1);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), q1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += c[i][0] + c[i][1] + c[i][2] + c[i][3];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += f[i];
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (lane == 0) {
    out[2 * wave] = (uint32_t)(t1 - t0);
    out[2 * wave + 1] = (uint32_t)(q1 - q0) | (sum == 1.2345e-30f ? 1u : 0u);  // keeps the work alive
  }
}

template <int R, int W>
hipError_t run_stream(const void *in, void *out, int64_t tiles, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_probe_stream<R, W>), dim3(grid), dim3(kProbeThreads), 0, st, (const u32x4 *)in,
                     (u32x4 *)out, tiles);
  return hipGetLastError();
}

}  // namespace

int64_t probe_stream_tiles(int kind, int64_t in_bytes) {
  static const int reads[] = {1, 4, 9, 1, 9, 1};
  if (kind < 0 || kind > 5) return -1;
  return in_bytes / (reads[kind] * 64 * 16);
}

int64_t probe_stream_out_bytes(int kind, int64_t tiles) {
  static const int writes[] = {1, 1, 2, 0, 0, 8};
  if (kind < 0 || kind > 5) return -1;
  if (kind == 4) return tiles * 128 * 4 * 4;  // 4 rows of 128 keys per tile
  return tiles * writes[kind] * 64 * 16;
}

hipError_t launch_probe_stream(int kind, const void *in, void *out, int64_t tiles, int grid, hipStream_t st) {
  switch (kind) {
    case 0: return run_stream<1, 1>(in, out, tiles, grid, st);
    case 1: return run_stream<4, 1>(in, out, tiles, grid, st);
    case 2: return run_stream<9, 2>(in, out, tiles, grid, st);
    case 3: return run_stream<1, 0>(in, out, tiles, grid, st);
    case 4:
      hipLaunchKernelGGL(k_probe_rows, dim3(grid), dim3(kProbeThreads), 0, st, (const u32x4 *)in, (float *)out,
                         tiles, tiles * 128);
      return hipGetLastError();
    case 5: return run_stream<1, 8>(in, out, tiles, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_probe_issue(int mode, int waves_per_simd, int64_t iters, int grid, uint32_t *out,
                              hipStream_t st) {
  const dim3 block((unsigned)(256 * waves_per_simd));
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_probe_issue<0>, dim3(grid), block, 0, st, iters, out); break;
    case 1: hipLaunchKernelGGL(k_probe_issue<1>, dim3(grid), block, 0, st, iters, out); break;
    case 2: hipLaunchKernelGGL(k_probe_issue<2>, dim3(grid), block, 0, st, iters, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int f16, int64_t iters, int grid, float *out, hipStream_t st) {
  if (f16)
    hipLaunchKernelGGL(k_probe_mfma<true>, dim3(grid), dim3(kProbeThreads), 0, st, iters, out);
  else
    hipLaunchKernelGGL(k_probe_mfma<false>, dim3(grid), dim3(kProbeThreads), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace tq
