// Device helpers shared by the HIP kernels: operand types, MFMA wrappers,
// bf16/f16 splitting, LDS addressing, packed-field and buffer-store helpers.
//
// Lane layouts (16x16x32 MFMA, wave64): A operand lane l holds row l%16 and
// 8 contraction elements of group l/16; B operand lane l holds column l%16 and
// the same 8 contraction elements; the accumulator lane l holds column l%16,
// rows 4*(l/16) .. 4*(l/16)+3.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One operand image block: a 128 x 128 matrix as bf16 (or f16) hi/lo MFMA A
// fragments, 8 row tiles x 4 K steps x hi/lo, one u32x4 per lane.
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

typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const float lds_f32;

// LDS byte address of a shared array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// OR the MB-bit field of coordinate j (0..31) into the lane's code words.
template <int MB>
__device__ __forceinline__ void put_field(uint32_t *w, int j, uint32_t idx) {
  const int bit = j * MB, wi = bit >> 5, sh = bit & 31;
  w[wi] |= idx << sh;
  if (sh + MB > 32) w[wi + 1] |= idx >> (32 - sh);
}

// Bitwise select m ? a : b for an all-ones / all-zeros mask m as one
// v_bitop3_b32 (truth table 0xCA); written as a compare + lane-mask select it
// would put a mask in SGPRs and a wait state before each use.
__device__ __forceinline__ float fsel(int32_t m, float a, float b) {
  return __uint_as_float(
      __builtin_amdgcn_bitop3_b32((uint32_t)m, __float_as_uint(a), __float_as_uint(b), 0xCA));
}

// Buffer resources over one set's codes and norms: stores at byte offsets at
// or past num_records are dropped by the hardware, which masks the ragged
// tail without a branch (a branch would split the MFMA / search overlap).
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 raw buffer, 32-bit data
constexpr uint32_t kDropped = 0x80000000u;      // offset past every set (host-checked)

// Code words of one lane (CW words = 32 codes of CW bits) from global memory.
template <int CW>
__device__ __forceinline__ void load_codes(uint32_t *w, const uint8_t *p) {
  if constexpr (CW == 1) {
    w[0] = *(const uint32_t *)p;
  } else if constexpr (CW == 2) {
    const u32x2 v = *(const u32x2 *)p;
    w[0] = v[0];
    w[1] = v[1];
  } else if constexpr (CW == 3) {
    const u32x3 v = *(const u32x3 *)p;
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
  } else if constexpr (CW == 4) {
    const u32x4 v = *(const u32x4 *)p;
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
}

}  // namespace tq
