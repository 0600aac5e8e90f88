// rssm_device.h -- device-side number formats, rounding and Philox for the
// gfx950 materialize kernels.
//
// Formats follow the state dtypes of the flashinfer page for
// flashinfer.mamba.replayssm_materialize (state_dtype, input_dtype) and the
// dtype list of the pull request "Replayssm prefix materialize" (BF16, FP16,
// INT8 and FP8 state).  Every rounding here is exact integer/power-of-two
// arithmetic on fp32 values, so a given fp32 input always yields the same
// code:
//   nearest-even   bf16/fp16 by the hardware conversions (IEEE, overflow to
//                  infinity); int8 and e4m3 in software, saturating.
//   stochastic     with lo <= |v| < hi neighbouring grid points and
//                  f = (|v| - lo) / (hi - lo), the magnitude rounds up iff the
//                  element's 32-bit Philox word u satisfies u < f * 2^32
//                  (compared exactly as u < ceil(f * 2^32)); saturating.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

enum : int { kF32 = 0, kBF16 = 1, kF16 = 2, kI8 = 3, kF8 = 4 };

template <int DT> struct Fmt;
template <> struct Fmt<kF32> { static constexpr int bytes = 4; };
template <> struct Fmt<kBF16> { static constexpr int bytes = 2; };
template <> struct Fmt<kF16> { static constexpr int bytes = 2; };
template <> struct Fmt<kI8> { static constexpr int bytes = 1; };
template <> struct Fmt<kF8> { static constexpr int bytes = 1; };

template <int DT> constexpr bool kOneByte = (DT == kI8 || DT == kF8);

// 8 consecutive elements of one row ("chunk") in raw storage: 8/4/2 dwords.
template <int DT> struct Chunk { uint32_t w[2 * Fmt<DT>::bytes]; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, typename V>
__device__ __forceinline__ V ld(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}

template <bool NT, typename V>
__device__ __forceinline__ void st(char* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = v;
}

// NT: non-temporal (streaming) access, for data read or written once.
template <int DT, bool NT = false>
__device__ __forceinline__ Chunk<DT> load_chunk(const char* p) {
  Chunk<DT> c;
  if constexpr (Fmt<DT>::bytes == 4) {
    const u32x4 a = ld<NT, u32x4>(p);
    const u32x4 b = ld<NT, u32x4>(p + 16);
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = a.z; c.w[3] = a.w;
    c.w[4] = b.x; c.w[5] = b.y; c.w[6] = b.z; c.w[7] = b.w;
  } else if constexpr (Fmt<DT>::bytes == 2) {
    const u32x4 a = ld<NT, u32x4>(p);
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = a.z; c.w[3] = a.w;
  } else {
    const u32x2 a = ld<NT, u32x2>(p);
    c.w[0] = a.x; c.w[1] = a.y;
  }
  return c;
}

template <int DT, bool NT = false>
__device__ __forceinline__ void store_chunk(char* p, const Chunk<DT>& c) {
  if constexpr (Fmt<DT>::bytes == 4) {
    st<NT>(p, u32x4{c.w[0], c.w[1], c.w[2], c.w[3]});
    st<NT>(p + 16, u32x4{c.w[4], c.w[5], c.w[6], c.w[7]});
  } else if constexpr (Fmt<DT>::bytes == 2) {
    st<NT>(p, u32x4{c.w[0], c.w[1], c.w[2], c.w[3]});
  } else {
    st<NT>(p, u32x2{c.w[0], c.w[1]});
  }
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_bits_to_float(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_float(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = (code >> 3) & 0xFu;
  const uint32_t m = code & 7u;
  if (e == 0xFu && m == 7u) return __uint_as_float(sign | 0x7FC00000u);
  const float mag = (e == 0u) ? static_cast<float>(m) * 0x1p-9f
                              : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | sign);
}

template <int DT>
__device__ __forceinline__ void decode_chunk(const Chunk<DT>& c, float (&f)[8]) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(c.w[i]);
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(c.w[i] << 16);
      f[2 * i + 1] = __uint_as_float(c.w[i] & 0xFFFF0000u);
    }
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_bits_to_float(c.w[i] & 0xFFFFu);
      f[2 * i + 1] = f16_bits_to_float(c.w[i] >> 16);
    }
  } else if constexpr (DT == kI8) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      f[i] = static_cast<float>(static_cast<int8_t>((c.w[i >> 2] >> (8 * (i & 3))) & 0xFFu));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = e4m3_to_float((c.w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  }
}

// ---------------------------------------------------------------------------
// Philox4x32-R (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): per round, the products of counter words 0 and 2 with
// two odd multipliers; new counter (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the key
// advances by the Weyl increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32(uint4 c, uint32_t k0, uint32_t k1, int rounds) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
  for (int i = 0; i < rounds; ++i) {
    const uint64_t p0 = static_cast<uint64_t>(kM0) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(kM1) * c.z;
    c = make_uint4(static_cast<uint32_t>(p1 >> 32) ^ c.y ^ k0, static_cast<uint32_t>(p1),
                   static_cast<uint32_t>(p0 >> 32) ^ c.w ^ k1, static_cast<uint32_t>(p0));
    k0 += kW0;
    k1 += kW1;
  }
  return c;
}

// Random words of the 8 elements (r, c0..c0+7) of head h, physical request b,
// layer l: counter ((r*dstate + c) / 4, h, b, l), word c mod 4.  c0 % 8 == 0.
__device__ __forceinline__ void sr_words(uint32_t (&u)[8], int r, int c0, int dstate, int h, int b,
                                         int l, uint32_t k0, uint32_t k1, int rounds) {
  const uint32_t base = static_cast<uint32_t>((static_cast<int64_t>(r) * dstate + c0) >> 2);
  const uint4 w0 = philox4x32(make_uint4(base, h, b, l), k0, k1, rounds);
  const uint4 w1 = philox4x32(make_uint4(base + 1u, h, b, l), k0, k1, rounds);
  u[0] = w0.x; u[1] = w0.y; u[2] = w0.z; u[3] = w0.w;
  u[4] = w1.x; u[5] = w1.y; u[6] = w1.z; u[7] = w1.w;
}

// ---------------------------------------------------------------------------
// Rounding onto a grid: |v| = (n + rem) * 2^qe with integer n, rem in [0, 1).
// ---------------------------------------------------------------------------
// True iff the stochastic rule rounds the magnitude up: u < ceil(rem * 2^32).
// rem * 2^32 < 2^32 and is exact in fp32, so the ceiling is an exact integer.
__device__ __forceinline__ bool sr_up(float rem, uint32_t u) {
  return u < static_cast<uint32_t>(ceilf(ldexpf(rem, 32)));
}

// Unbiased exponent of a finite positive fp32 value (fp32 subnormals: -127).
__device__ __forceinline__ int exponent_of(float a) {
  return static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;
}

__device__ __forceinline__ uint32_t bf16_round(float v, bool stochastic, uint32_t u) {
  if (!stochastic) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 16) & 0x8000u;
  const uint32_t ab = bits & 0x7FFFFFFFu;
  if (ab > 0x7F800000u) return sign | 0x7FC0u;   // NaN
  if (ab >= 0x7F7F0000u) return sign | 0x7F7Fu;  // saturate at the largest finite value
  // bf16 keeps the top 16 bits; the dropped 16 bits are f * 2^16.
  const uint32_t up = (u < ((ab & 0xFFFFu) << 16)) ? 1u : 0u;
  return sign | ((ab >> 16) + up);
}

__device__ __forceinline__ uint32_t f16_round(float v, bool stochastic, uint32_t u) {
  if (!stochastic) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  const uint32_t sign = (__float_as_uint(v) >> 16) & 0x8000u;
  if (v != v) return sign | 0x7E00u;
  const float a = fabsf(v);
  if (a >= 65504.0f) return sign | 0x7BFFu;
  const int qe = max(exponent_of(a), -14) - 10;  // grid spacing 2^qe
  const float s = ldexpf(a, -qe);
  const float n = floorf(s);
  const float m = ldexpf(n + (sr_up(s - n, u) ? 1.0f : 0.0f), qe);  // exact fp16 value
  return sign | (__builtin_bit_cast(uint16_t, static_cast<_Float16>(m)) & 0x7FFFu);
}

__device__ __forceinline__ uint32_t i8_round(float t, bool stochastic, uint32_t u) {
  if (t != t) return 0u;
  const float a = fabsf(t);
  float q;
  if (a >= 127.0f) {
    q = 127.0f;
  } else if (!stochastic) {
    q = rintf(a);  // nearest, ties to even
  } else {
    const float n = floorf(a);
    q = n + (sr_up(a - n, u) ? 1.0f : 0.0f);
  }
  const int qi = (__float_as_uint(t) >> 31) ? -static_cast<int>(q) : static_cast<int>(q);
  return static_cast<uint32_t>(qi) & 0xFFu;
}

__device__ __forceinline__ uint32_t e4m3_round(float t, bool stochastic, uint32_t u) {
  const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
  if (t != t) return sign | 0x7Fu;
  const float a = fabsf(t);
  if (a >= 448.0f) return sign | 0x7Eu;
  const int qe = max(exponent_of(a), -6) - 3;  // 3 mantissa bits, subnormals below 2^-6
  const float s = ldexpf(a, -qe);
  const float n = floorf(s);
  const float rem = s - n;
  bool up;
  if (stochastic) up = sr_up(rem, u);
  else up = rem > 0.5f || (rem == 0.5f && (static_cast<int>(n) & 1));
  const float m = ldexpf(n + (up ? 1.0f : 0.0f), qe);  // exact e4m3 value, <= 448
  uint32_t code;
  if (m < 0x1p-6f) {
    code = static_cast<uint32_t>(m * 512.0f);  // subnormal: m = code * 2^-9
  } else {
    const uint32_t mb = __float_as_uint(m);
    code = ((((mb >> 23) & 0xFFu) - 120u) << 3) | ((mb >> 20) & 7u);
  }
  return sign | code;
}

}  // namespace rssm
