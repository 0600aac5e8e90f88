/*
 * rssm_oracle.c -- plain, slow CPU oracle for ReplaySSM prefix materialize.
 *
 * TEST INFRASTRUCTURE ONLY (see rssm_oracle.h).  Written from the flashinfer
 * documentation page for flashinfer.mamba.replayssm_materialize and the
 * pull-request page "Replayssm prefix materialize" (flashinfer PR 4815).
 * Every numeric step is written the plain way: fp64 token-by-token replay,
 * then one rounding to fp32, then an encode that searches the target format's
 * code grid directly.  No blocking, fusion or reordering.
 */
#include "rssm_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats: value of a code from its sign / exponent / mantissa fields */
/* ------------------------------------------------------------------------- */

typedef struct {
  int ebits, mbits, bias, has_inf;
  uint32_t maxcode; /* largest positive finite code */
} fmt_t;

/* bfloat16: 8 exponent bits, 7 mantissa bits, bias 127, IEEE inf/NaN. */
static const fmt_t FMT_BF16 = {8, 7, 127, 1, 0x7F7Fu};
/* IEEE binary16: 5 exponent bits, 10 mantissa bits, bias 15. */
static const fmt_t FMT_F16 = {5, 10, 15, 1, 0x7BFFu};
/* OCP FP8 E4M3 ("e4m3fn"): 4 exponent bits, 3 mantissa bits, bias 7, no
 * infinities, only S.1111.111 is NaN, largest finite 448. */
static const fmt_t FMT_E4M3 = {4, 3, 7, 0, 0x7Eu};

/* Magnitude of a positive code (sign bit clear). */
static double fmt_magnitude(const fmt_t *f, uint32_t code) {
  uint32_t emask = (1u << f->ebits) - 1u;
  uint32_t mmask = (1u << f->mbits) - 1u;
  uint32_t e = (code >> f->mbits) & emask;
  uint32_t m = code & mmask;
  if (e == 0) /* subnormal: m * 2^(1 - bias - mbits) */
    return ldexp((double)m, 1 - f->bias - f->mbits);
  if (f->has_inf && e == emask) return m ? NAN : INFINITY;
  if (!f->has_inf && e == emask && m == mmask) return NAN;
  /* normal: (2^mbits + m) * 2^(e - bias - mbits) */
  return ldexp((double)((1u << f->mbits) | m), (int)e - f->bias - f->mbits);
}

static double fmt_value(const fmt_t *f, uint32_t code) {
  uint32_t sign = (code >> (f->ebits + f->mbits)) & 1u;
  double v = fmt_magnitude(f, code & ~(1u << (f->ebits + f->mbits)));
  return sign ? -v : v;
}

static const fmt_t *fmt_of(int32_t dtype) {
  switch (dtype) {
    case ORC_BF16: return &FMT_BF16;
    case ORC_F16: return &FMT_F16;
    case ORC_F8E4M3: return &FMT_E4M3;
    default: return NULL;
  }
}

double orc_decode(int32_t dtype, const void *base, int64_t index) {
  switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[index];
    case ORC_F64: return ((const double *)base)[index];
    case ORC_BF16: return fmt_value(&FMT_BF16, ((const uint16_t *)base)[index]);
    case ORC_F16: return fmt_value(&FMT_F16, ((const uint16_t *)base)[index]);
    case ORC_F8E4M3: return fmt_value(&FMT_E4M3, ((const uint8_t *)base)[index]);
    case ORC_I8: return (double)((const int8_t *)base)[index];
    default: return NAN;
  }
}

static int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F64: return 8;
    case ORC_BF16: case ORC_F16: return 2;
    case ORC_I8: case ORC_F8E4M3: return 1;
    default: return 0;
  }
}

static int is_one_byte(int32_t dtype) { return dtype == ORC_I8 || dtype == ORC_F8E4M3; }

/* ------------------------------------------------------------------------- */
/* Rounding onto a code grid                                                  */
/* ------------------------------------------------------------------------- */
/* The positive codes of every narrow format are ordered like their values, so
 * the grid point below a magnitude is found by bisection over codes, each code
 * decoded by the plain field formula above.  int8 uses the integers 0..127
 * (symmetric range; -128 is never produced). */

static uint32_t grid_maxcode(int32_t dtype) {
  if (dtype == ORC_I8) return 127u;
  return fmt_of(dtype)->maxcode;
}

static double grid_mag(int32_t dtype, uint32_t code) {
  if (dtype == ORC_I8) return (double)code;
  return fmt_magnitude(fmt_of(dtype), code);
}

/* Largest code whose magnitude is <= a, for 0 <= a < grid max. */
static uint32_t grid_floor(int32_t dtype, double a) {
  uint32_t lo = 0, hi = grid_maxcode(dtype); /* mag(lo) <= a < mag(hi) */
  while (hi - lo > 1u) {
    uint32_t mid = lo + (hi - lo) / 2u;
    if (grid_mag(dtype, mid) <= a) lo = mid; else hi = mid;
  }
  return lo;
}

/* Attach the sign to a magnitude code. */
static uint32_t grid_signed(int32_t dtype, uint32_t mag_code, int negative) {
  if (dtype == ORC_I8) {
    int32_t q = negative ? -(int32_t)mag_code : (int32_t)mag_code;
    return (uint32_t)(uint8_t)(int8_t)q;
  }
  const fmt_t *f = fmt_of(dtype);
  return negative ? (mag_code | (1u << (f->ebits + f->mbits))) : mag_code;
}

static uint32_t nan_code(int32_t dtype, int negative) {
  switch (dtype) {
    case ORC_BF16: return (negative ? 0x8000u : 0u) | 0x7FC0u;
    case ORC_F16: return (negative ? 0x8000u : 0u) | 0x7E00u;
    case ORC_F8E4M3: return (negative ? 0x80u : 0u) | 0x7Fu;
    default: return 0u; /* int8: NaN encodes as 0 */
  }
}

/* Round v (an fp32 value) onto the grid.  stochastic == 0: nearest, ties to
 * the even code; bf16/f16 overflow to infinity, e4m3/int8 saturate.
 * stochastic != 0: with lo <= |v| < hi adjacent grid points and
 * f = (|v| - lo) / (hi - lo), the magnitude rounds up iff u < f * 2^32;
 * magnitudes at or above the largest finite value saturate to it. */
uint32_t orc_round_value(int32_t dtype, float v, int32_t stochastic, uint32_t u) {
  int negative = signbit(v) ? 1 : 0;
  double a = fabs((double)v);
  uint32_t maxc = grid_maxcode(dtype);
  double maxv = grid_mag(dtype, maxc);
  if (isnan(v)) return nan_code(dtype, negative);

  if (a >= maxv) {
    if (stochastic || dtype == ORC_I8 || dtype == ORC_F8E4M3 || a == maxv)
      return grid_signed(dtype, maxc, negative);
    /* IEEE overflow for bf16 / f16: the next grid point above the largest
     * finite value is 2^(emax+1) (the infinity code); ties go to it because
     * the largest finite code is odd. */
    double ulp_top = maxv - grid_mag(dtype, maxc - 1u);
    double next = maxv + ulp_top;
    if (isinf(a) || a - maxv >= next - a) return grid_signed(dtype, maxc + 1u, negative);
    return grid_signed(dtype, maxc, negative);
  }

  uint32_t c = grid_floor(dtype, a);
  double lo = grid_mag(dtype, c);
  if (lo == a) return grid_signed(dtype, c, negative);
  double hi = grid_mag(dtype, c + 1u);
  uint32_t out;
  if (stochastic) {
    double f = (a - lo) / (hi - lo); /* exact: power-of-two spacing */
    out = ((double)u < f * 4294967296.0) ? c + 1u : c;
  } else {
    double dlo = a - lo, dhi = hi - a;
    if (dlo < dhi) out = c;
    else if (dlo > dhi) out = c + 1u;
    else out = (c % 2u == 0u) ? c : c + 1u;
  }
  return grid_signed(dtype, out, negative);
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-R (Salmon, Moraes, Dror, Shaw, SC'11)                           */
/* ------------------------------------------------------------------------- */
/* One round: two 32x32->64 products of counter words 0 and 2 with the
 * multipliers; the new counter is (hi1^c1^k0, lo1, hi0^c3^k1, lo0).  The key
 * advances by the Weyl increments between rounds. */
void orc_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int32_t rounds, uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int32_t i = 0; i < rounds; ++i) {
    if (i > 0) { k0 += W0; k1 += W1; }
    uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 32-bit random word of state element (r, c) of head h, request b
 * (physical batch index), layer l: counter ((r*dstate + c) / 4, h, b, l),
 * key (low, high) words of the seed, output word c mod 4. */
static uint32_t sr_word(const orc_params *p, int32_t l, int32_t b, int32_t h, int32_t r, int32_t c) {
  uint32_t ctr[4], key[2], o[4];
  ctr[0] = (uint32_t)(((int64_t)r * p->dstate + c) >> 2);
  ctr[1] = (uint32_t)h;
  ctr[2] = (uint32_t)b;
  ctr[3] = (uint32_t)l;
  key[0] = (uint32_t)(p->seed & 0xFFFFFFFFu);
  key[1] = (uint32_t)(p->seed >> 32);
  orc_philox4x32(ctr, key, p->philox_rounds, o);
  return o[c & 3];
}

/* ------------------------------------------------------------------------- */
/* Encode one state row                                                       */
/* ------------------------------------------------------------------------- */
static void store_code(int32_t dtype, void *codes, int64_t idx, uint32_t code) {
  if (elem_bytes(dtype) == 2) ((uint16_t *)codes)[idx] = (uint16_t)code;
  else ((uint8_t *)codes)[idx] = (uint8_t)code;
}

int orc_encode_row(const orc_params *p, const float *row, int32_t layer, int32_t request,
                   int32_t head, int32_t r, void *codes, float *scale) {
  const int32_t n = p->dstate;
  const int32_t dt = p->state_dtype;
  const int stochastic = p->philox_rounds > 0;
  if (dt == ORC_F32) {
    memcpy(codes, row, (size_t)n * sizeof(float));
    return ORC_OK;
  }
  if (dt == ORC_F64) {
    for (int32_t c = 0; c < n; ++c) ((double *)codes)[c] = (double)row[c];
    return ORC_OK;
  }
  if (dt == ORC_BF16 || dt == ORC_F16) {
    for (int32_t c = 0; c < n; ++c) {
      uint32_t u = stochastic ? sr_word(p, layer, request, head, r, c) : 0u;
      store_code(dt, codes, c, orc_round_value(dt, row[c], stochastic, u));
    }
    return ORC_OK;
  }
  if (!is_one_byte(dt)) return ORC_BAD_PARAM;

  /* Per-row symmetric quantization: rowmax = max |v| (NaN ignored),
   * scale = rowmax / qmax and inv = qmax / rowmax (fp32 IEEE divisions),
   * t = v * inv (fp32), code = round(t).  An all-zero row, or one whose inv
   * overflows, stores scale 0 and zero codes. */
  const float qmax = (dt == ORC_I8) ? 127.0f : 448.0f;
  float rowmax = 0.0f;
  for (int32_t c = 0; c < n; ++c) rowmax = fmaxf(rowmax, fabsf(row[c]));
  float inv = qmax / rowmax;
  if (!(rowmax > 0.0f) || isinf(rowmax) || !isfinite(inv)) {
    *scale = 0.0f;
    for (int32_t c = 0; c < n; ++c) store_code(dt, codes, c, 0u);
    return ORC_OK;
  }
  *scale = rowmax / qmax;
  for (int32_t c = 0; c < n; ++c) {
    float t = row[c] * inv;
    uint32_t u = stochastic ? sr_word(p, layer, request, head, r, c) : 0u;
    store_code(dt, codes, c, orc_round_value(dt, t, stochastic, u));
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* One head tile                                                              */
/* ------------------------------------------------------------------------- */
static int check_params(const orc_params *p) {
  if (p->num_layers < 1 || p->batch < 1 || p->num_heads < 1 || p->heads_per_group < 1) return ORC_BAD_PARAM;
  if (p->num_heads % p->heads_per_group != 0) return ORC_BAD_PARAM;
  if (p->dim < 1 || p->dstate < 1 || p->ring_len < 1) return ORC_BAD_PARAM;
  if (p->max_window < 1 || p->max_window > 16) return ORC_BAD_PARAM;
  if (p->philox_rounds < 0) return ORC_BAD_PARAM;
  if (p->philox_rounds > 0 && p->dstate % 4 != 0) return ORC_BAD_PARAM;
  if (elem_bytes(p->state_dtype) == 0) return ORC_BAD_PARAM;
  if (p->input_dtype != ORC_F32 && p->input_dtype != ORC_BF16 && p->input_dtype != ORC_F16) return ORC_BAD_PARAM;
  return ORC_OK;
}

int orc_tile(const orc_params *p, int32_t layer, int32_t request, int32_t head,
             int32_t ring_start, int32_t k, float A_h,
             const void *src_tile, const float *src_scale,
             const void *x_slot, const void *B_slot, const float *dt_slot,
             double *exact, double *mag, void *codes, float *scale) {
  int st = check_params(p);
  if (st != ORC_OK) return st;
  const int32_t dim = p->dim, ds = p->dstate, H = p->num_heads, R = p->ring_len;
  const int32_t G = H / p->heads_per_group;
  const int32_t g = head / p->heads_per_group; /* contiguous head groups */
  const int one_byte = is_one_byte(p->state_dtype);
  const int64_t tile_elems = (int64_t)dim * ds;
  if (k < 0 || k > p->max_window || ring_start < 0 || ring_start >= R) return ORC_BAD_METADATA;
  if (ds > 4096) return ORC_BAD_PARAM;

  if (k == 0) {
    /* A zero-length prefix is an exact byte copy of the state (and scales). */
    if (codes) memcpy(codes, src_tile, (size_t)tile_elems * (size_t)elem_bytes(p->state_dtype));
    if (one_byte && scale) memcpy(scale, src_scale, (size_t)dim * sizeof(float));
    for (int64_t idx = 0; idx < tile_elems; ++idx) {
      double s0 = orc_decode(p->state_dtype, src_tile, idx);
      if (one_byte) s0 *= (double)src_scale[idx / ds];
      if (exact) exact[idx] = s0;
      if (mag) mag[idx] = fabs(s0);
    }
    return ORC_OK;
  }

  double *S = exact ? exact : (double *)malloc((size_t)tile_elems * sizeof(double));
  if (!S) return ORC_BAD_PARAM;
  for (int32_t r = 0; r < dim; ++r) {
    for (int32_t c = 0; c < ds; ++c) {
      /* Dequantized source value: stored code times the source row scale. */
      double s = orc_decode(p->state_dtype, src_tile, (int64_t)r * ds + c);
      if (one_byte) s *= (double)src_scale[r];
      double m = fabs(s);
      /* Token by token: S <- exp(dt*A) * S + dt * x[r] * B[c]. */
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = (ring_start + j) % R; /* ring entries wrap modulo R */
        double dtv = (double)dt_slot[(int64_t)e * H + head];
        double a = exp(dtv * (double)A_h);
        double xv = orc_decode(p->input_dtype, x_slot, ((int64_t)e * H + head) * dim + r);
        double bv = orc_decode(p->input_dtype, B_slot, ((int64_t)e * G + g) * ds + c);
        s = a * s + dtv * xv * bv;
        m = a * m + dtv * fabs(xv * bv);
      }
      S[(int64_t)r * ds + c] = s;
      if (mag) mag[(int64_t)r * ds + c] = m;
    }
  }

  if (codes) {
    if (p->state_dtype == ORC_F64) {
      /* fp64 storage keeps the result unrounded. */
      memcpy(codes, S, (size_t)tile_elems * sizeof(double));
    } else {
      float rowbuf[4096];
      for (int32_t r = 0; r < dim; ++r) {
        /* One rounding, fp64 -> fp32 (nearest even), then the encode. */
        for (int32_t c = 0; c < ds; ++c) rowbuf[c] = (float)S[(int64_t)r * ds + c];
        char *row_codes = (char *)codes + (size_t)r * (size_t)ds * (size_t)elem_bytes(p->state_dtype);
        float sc = 0.0f;
        orc_encode_row(p, rowbuf, layer, request, head, r, row_codes, &sc);
        if (one_byte && scale) scale[r] = sc;
      }
    }
  }
  if (!exact) free(S);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Whole operation                                                            */
/* ------------------------------------------------------------------------- */
int orc_materialize(const orc_params *p, const orc_inputs *in, const orc_outputs *out) {
  int st = check_params(p);
  if (st != ORC_OK) return st;
  const int32_t L = p->num_layers, B = p->batch, H = p->num_heads;
  const int32_t dim = p->dim, ds = p->dstate;
  const int one_byte = is_one_byte(p->state_dtype);
  const int64_t esz = elem_bytes(p->state_dtype);
  const int64_t tile_elems = (int64_t)dim * ds;

  /* Requests are taken from the active list until its first -1. */
  for (int32_t i = 0; i < B; ++i) {
    int32_t b = in->active[i];
    if (b == -1) break;
    if (b < 0 || b >= B) return ORC_BAD_METADATA;
    for (int32_t l = 0; l < L; ++l) {
      int32_t s = in->src_slots[(int64_t)l * B + b];
      int32_t d = in->dst_slots[(int64_t)l * B + b];
      /* A (layer, request) is skipped when either slot is the pad sentinel. */
      if (s == p->pad_slot_id || d == p->pad_slot_id) continue;
      if (s < 0 || d < 0) return ORC_BAD_METADATA;
      int32_t k = in->prefix_len[b];
      int32_t r0 = in->ring_start[b];
      for (int32_t h = 0; h < H; ++h) {
        const char *src_tile = (const char *)in->state[l] + ((int64_t)s * in->state_stride[l] + h * tile_elems) * esz;
        char *dst_tile = (char *)out->state[l] + ((int64_t)d * in->state_stride[l] + h * tile_elems) * esz;
        const float *src_scale = one_byte ? in->scale[l] + (int64_t)s * in->scale_stride[l] + (int64_t)h * dim : NULL;
        float *dst_scale = one_byte ? out->scale[l] + (int64_t)d * in->scale_stride[l] + (int64_t)h * dim : NULL;
        const char *x_slot = (const char *)in->x[l] + (int64_t)s * in->x_stride[l] * elem_bytes(p->input_dtype);
        const char *B_slot = (const char *)in->Bm[l] + (int64_t)s * in->B_stride[l] * elem_bytes(p->input_dtype);
        const float *dt_slot = in->dt[l] + (int64_t)s * in->dt_stride[l];
        double *ex = out->exact ? out->exact[l] + (int64_t)d * in->state_stride[l] + h * tile_elems : NULL;
        double *mg = out->mag ? out->mag[l] + (int64_t)d * in->state_stride[l] + h * tile_elems : NULL;
        st = orc_tile(p, l, b, h, r0, k, in->A[l][h], src_tile, src_scale, x_slot, B_slot, dt_slot,
                      ex, mg, dst_tile, dst_scale);
        if (st != ORC_OK) return st;
      }
    }
  }
  return ORC_OK;
}
