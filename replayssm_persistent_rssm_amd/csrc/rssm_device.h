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

// Every pointer the kernels dereference addresses global memory, but the bases
// arrive as integers in device tables, so the compiler cannot infer it: the
// accessors below cast to the global address space, which makes them global_*
// instructions (flat ones would also count against the LDS wait counter).
#define RSSM_GLOBAL __attribute__((address_space(1)))

template <bool NT, typename V>
__device__ __forceinline__ V ld(const char* p) {
  const RSSM_GLOBAL V* g = (const RSSM_GLOBAL V*)(p);
  if constexpr (NT) return __builtin_nontemporal_load(g);
  else return *g;
}

template <bool NT, typename V>
__device__ __forceinline__ void st(char* p, V v) {
  RSSM_GLOBAL V* g = (RSSM_GLOBAL V*)(p);
  if constexpr (NT) __builtin_nontemporal_store(v, g);
  else *g = v;
}

template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const RSSM_GLOBAL T*)(p);
}

// Read of a wave-uniform address holding data the kernel never writes, through
// the scalar data cache (a constant-address-space load).  Its completion is
// tracked by the scalar/LDS wait counter, so using the value does not wait
// for the vector loads in flight (a vector load would: their counter retires
// in order).
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

template <typename T>
__device__ __forceinline__ void gstore(T* p, T v) {
  *(RSSM_GLOBAL T*)(p) = v;
}

// Buffer accesses: a 128-bit resource (base, size in bytes) held in scalar
// registers, a 32-bit per-lane offset and a wave-uniform offset.  Compared
// with 64-bit per-lane addresses this saves the address arithmetic and two
// vector registers per live address; accesses at or past the size are
// dropped (loads return 0).  The resource word 3 is the gfx9 raw-buffer
// format; aux bit 1 requests the non-temporal (streaming) policy.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

template <bool NT>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}

template <bool NT>
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)), v),
                                         r, voff, soff, NT ? 2 : 0);
}

__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

__device__ __forceinline__ void bstore_f32(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
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
    // OCP e4m3fn (sign, 4 exponent bits with bias 7, 3 mantissa bits; only
    // S.1111.111 is NaN): gfx950's fp8 conversion instructions use this format.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.w[i]), false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c.w[i]), true);
      f[4 * i + 0] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
}

// ---------------------------------------------------------------------------
// Philox4x32-R (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): per round, the products of counter words 0 and 2 with
// two odd multipliers; new counter (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the key
// advances by the Weyl increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                             uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  const uint64_t p0 = static_cast<uint64_t>(kM0) * c0;
  const uint64_t p1 = static_cast<uint64_t>(kM1) * c2;
  // Three-way XORs as one gfx950 bitop3 each (truth table 0x96 = a ^ b ^ c).
  const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
  const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
  c1 = static_cast<uint32_t>(p1);
  c3 = static_cast<uint32_t>(p0);
  c0 = n0;
  c2 = n2;
}

// Two Philox4x32-R blocks with counters (x, y, z, w) and (x + 1, y, z, w),
// interleaved for instruction-level parallelism; rounds are unrolled by two
// (fully for the common count of 10).
__device__ __forceinline__ void philox4x32_pair(uint32_t x, uint32_t y, uint32_t z, uint32_t w, uint32_t k0,
                                                uint32_t k1, int rounds, uint32_t (&u)[8]) {
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
  uint32_t a0 = x, a1 = y, a2 = z, a3 = w;
  uint32_t b0 = x + 1u, b1 = y, b2 = z, b3 = w;
  if (rounds == 10) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      philox_round(a0, a1, a2, a3, k0, k1);
      philox_round(b0, b1, b2, b3, k0, k1);
      k0 += kW0;
      k1 += kW1;
    }
    u[0] = a0; u[1] = a1; u[2] = a2; u[3] = a3;
    u[4] = b0; u[5] = b1; u[6] = b2; u[7] = b3;
    return;
  }
  int i = 0;
  for (; i + 2 <= rounds; i += 2) {
    philox_round(a0, a1, a2, a3, k0, k1);
    philox_round(b0, b1, b2, b3, k0, k1);
    k0 += kW0;
    k1 += kW1;
    philox_round(a0, a1, a2, a3, k0, k1);
    philox_round(b0, b1, b2, b3, k0, k1);
    k0 += kW0;
    k1 += kW1;
  }
  if (i < rounds) {
    philox_round(a0, a1, a2, a3, k0, k1);
    philox_round(b0, b1, b2, b3, k0, k1);
  }
  u[0] = a0; u[1] = a1; u[2] = a2; u[3] = a3;
  u[4] = b0; u[5] = b1; u[6] = b2; u[7] = b3;
}

// Random words of the 8 elements (r, c0..c0+7) of head h, physical request b,
// layer l: counter ((r*dstate + c) / 4, h, b, l), word c mod 4.  c0 % 8 == 0.
__device__ __forceinline__ void sr_words(uint32_t (&u)[8], int r, int c0, int dstate, int h, int b,
                                         int l, uint32_t k0, uint32_t k1, int rounds) {
  const uint32_t base = static_cast<uint32_t>((static_cast<int64_t>(r) * dstate + c0) >> 2);
  philox4x32_pair(base, static_cast<uint32_t>(h), static_cast<uint32_t>(b), static_cast<uint32_t>(l), k0, k1,
                  rounds, u);
}

// ---------------------------------------------------------------------------
// Byte packing.  v_perm_b32 (operands s0, s1) builds each result byte from a
// selector byte: 0-3 pick bytes 0-3 of s1, 4-7 bytes 0-3 of s0, 0x0c gives 0.
// ---------------------------------------------------------------------------
// Byte 0 of a, b, c, d as one little-endian word (three byte permutes).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// ---------------------------------------------------------------------------
// Per-row symmetric quantization parameters: scale = m / qmax and
// inv = qmax / m, both correctly rounded fp32 quotients, for a row whose
// largest magnitude is m.  A row is valid when m > 0, m is finite and inv is
// finite; an invalid row gets scale 0 (its codes are zero).
//
// For 2^-100 <= m <= 2^100 both quotients come from short fma sequences with
// a single exact-residual correction:
//   scale: s = m * c with c = RN(1/qmax), then s + (m - s*qmax) * c;
//   inv:   y = rcp(m) refined by one Newton step, q = qmax * y, then
//          q + (qmax - m*q) * y.
// Both equal the IEEE quotient for every fp32 m in that range, qmax 127 or
// 448: checked exhaustively against division (scale on the host for every
// m >= 2^-120; inv on gfx950 for all 1.68e9 values of the range).  A
// wavefront with any row outside the range uses the divisions.  All lanes of
// the wavefront must execute this.
// ---------------------------------------------------------------------------
template <int QMAX>
__device__ __forceinline__ bool row_quant(float m, float& scale, float& inv) {
  static_assert(QMAX == 127 || QMAX == 448, "qmax");
  constexpr float q = static_cast<float>(QMAX);
  constexpr float c = (QMAX == 127) ? 0x1.020408p-7f : 0x1.24924ap-9f;  // RN(1 / qmax)
  static_assert(c == 1.0f / q, "c must be the correctly rounded reciprocal of qmax");
  const bool fast = (m >= 0x1p-100f) && (m <= 0x1p100f);
  if (__builtin_expect(__ballot(!fast) == 0, 1)) {
    const float s0 = m * c;
    scale = fmaf(fmaf(-s0, q, m), c, s0);
    const float y0 = __builtin_amdgcn_rcpf(m);
    const float y1 = fmaf(fmaf(-m, y0, 1.0f), y0, y0);
    const float q0 = q * y1;
    inv = fmaf(fmaf(-m, q0, q), y1, q0);
    return true;
  }
  inv = q / m;
  const bool ok = (m > 0.0f) && !__builtin_isinf(m) && __builtin_isfinite(inv);
  scale = ok ? m / q : 0.0f;
  return ok;
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

// int8 code of t (row-scaled value): nearest-even or stochastic, saturating to
// [-127, 127]; NaN encodes as 0 (the hardware float-to-int conversion).
__device__ __forceinline__ uint32_t i8_round(float t, bool stochastic, uint32_t u) {
  int q;
  if (!stochastic) {
    q = static_cast<int>(rintf(t));
  } else {
    const float a = fminf(fabsf(t), 127.0f);
    const float n = floorf(a);
    const int m = static_cast<int>(n) + (sr_up(a - n, u) ? 1 : 0);
    q = (__float_as_uint(t) >> 31) ? -m : m;
  }
  q = min(max(q, -127), 127);
  return static_cast<uint32_t>(q) & 0xFFu;
}

// (a ^ b) + c as one gfx950 v_xad_u32 (checked on MI355X against the
// two-instruction form); the compiler does not form it from the expression
// (it emits a not, a shift and an add for the stochastic-rounding carry).
// b is wave-uniform (a constant here).
__device__ __forceinline__ uint32_t xor_add(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
  return r;
}

// Stochastic e4m3 rounding of a row-scaled value t with 2^-6 <= |t| (and t
// not NaN; callers check the range for the whole wave first), returned as
// the exactly representable fp32 value the code stands for.  |t| is first
// clamped to 448 (the saturating rule; 448's dropped bits are zero, so it
// never rounds up).  In the normal range e4m3 keeps the top 3 mantissa bits
// and the 20 dropped bits d are f * 2^20; adding (u >> 12) ^ 0xFFFFF =
// 0xFFFFF - (u >> 12) carries into bit 20 iff (u >> 12) < d, which is the
// rule u < f * 2^32, and clearing the dropped bits then leaves the rounded
// value (a carry out of the mantissa moves to the next binade).  The sign
// bit is never reached: the clamped magnitude's bits are below 2^30.
__device__ __forceinline__ float e4m3_sr_normal_value(float t, uint32_t u) {
  const float c = __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f);
  const uint32_t x = xor_add(u >> 12, 0xFFFFFu, __float_as_uint(c));
  return __uint_as_float(x & 0xFFF00000u);
}

// General e4m3 rounding (any input): nearest-even or stochastic, saturating;
// NaN keeps its sign with the NaN code.  Used where inputs are not row-scaled.
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
