// Shared device helpers for the gfx950 draft-block kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// Two floats rounded to bf16 and packed low, high into one dword.
DSPARK_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(lo)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(hi)) << 16);
}

// c + a.lo * b.lo + a.hi * b.hi for two bf16 pairs, accumulated in f32
// (v_dot2_f32_bf16; the bf16 products are exact in f32).
DSPARK_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

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

// Cross-lane moves on the vector ALUs only (no LDS): DPP within rows of 16
// lanes, and gfx950's permlane swaps across rows. The DPP patterns pair lane
// l with l^1 and l^2 (quad permutations) and with 7-l and 15-l inside each
// group of 8 and 16 (the half-row and row mirrors); every pattern pairs a lane
// with a partner whose bit 0, 1, 2 or 3 respectively is the opposite, which
// is all a butterfly needs.
constexpr int kDppXor1 = 0xB1;        // quad_perm 1,0,3,2
constexpr int kDppXor2 = 0x4E;        // quad_perm 2,3,0,1
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
DSPARK_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// Sum (or max) over each row of 16 lanes; every lane of the row gets it.
DSPARK_DEV float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}
DSPARK_DEV float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
// The two halves of a permlane swap of (x, x): across rows 2k <-> 2k+1
// (16-lane swap) or lanes l <-> l+32 (32-lane swap), each lane gets its own
// value and its partner's, in some order.
DSPARK_DEV void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
DSPARK_DEV void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Wave-wide reductions (64 lanes); every lane receives the result. The
// whole wave must be active.
DSPARK_DEV float wave_max(float v) {
  float a, b;
  v = row16_max(v);
  swap16(v, a, b);
  v = fmaxf(a, b);
  swap32(v, a, b);
  return fmaxf(a, b);
}
DSPARK_DEV float wave_sum(float v) {
  float a, b;
  v = row16_sum(v);
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

DSPARK_DEV int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
