// Shared device helpers for the gfx950 draft-block kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DSPARK_DEV __device__ __forceinline__

constexpr int kWave = 64;

// bf16 <-> f32. Widening is exact (the bf16 bits are the high half of the
// f32); narrowing rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
DSPARK_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
DSPARK_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
DSPARK_DEV float to_f32(float x) { return x; }
DSPARK_DEV float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename S> DSPARK_DEV S from_f32(float x);
template <> DSPARK_DEV float from_f32<float>(float x) { return x; }
template <> DSPARK_DEV bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Unpack one 16-byte vector of storage elements into floats.
// bf16: 8 values; f32: 4 values.
template <typename S> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  DSPARK_DEV static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf_lo(v[i]);
      out[2 * i + 1] = bf_hi(v[i]);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  DSPARK_DEV static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
};

DSPARK_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
DSPARK_DEV void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Wave-wide reductions (64 lanes) through cross-lane shuffles.
DSPARK_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
DSPARK_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

DSPARK_DEV int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
