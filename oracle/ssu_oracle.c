/*
 * ssu_oracle.c -- CPU oracle for the ReplaySSM decode step.
 * TEST INFRASTRUCTURE ONLY; see ssu_oracle.h for the operation and the
 * readings it takes.
 *
 * Parity status: orc_ssu_decode is pinned by the CPU tests (a unit C_t reads
 * out one column of the materialized state -- the materialize oracle's result
 * for prefix n + t + 1; C = 0 leaves D x gated by silu(z); linearity in C;
 * softplus values and ring positions of the appended entries; padded
 * requests untouched).
 */
#include "ssu_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "rssm_oracle.h" /* orc_decode and the dtype codes */

static int bytes_of(int32_t dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16:
    case ORC_F16: return 2;
    default: return 0;
  }
}

/* softplus(v) = log(1 + e^v), evaluated without overflow. */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

int orc_ssu_decode(const orc_ssu_params *p, const orc_ssu_inputs *in, const orc_ssu_outputs *out) {
  const int32_t B = p->batch, H = p->num_heads, dim = p->dim, ds = p->dstate, R = p->ring_len, T = p->tokens;
  if (B < 0 || H < 1 || p->heads_per_group < 1 || H % p->heads_per_group != 0 || dim < 1 || ds < 1 || R < 1 ||
      T < 1 || bytes_of(p->state_dtype) == 0 || bytes_of(p->input_dtype) == 0)
    return 1;
  const int32_t G = H / p->heads_per_group;
  const int ib = bytes_of(p->input_dtype);
  double *S = malloc(sizeof(double) * (size_t)dim * ds);
  double *M = malloc(sizeof(double) * (size_t)dim * ds);
  if (!S || !M) {
    free(S);
    free(M);
    return 1;
  }
  int st = 0;
  for (int32_t b = 0; b < B && st == 0; ++b) {
    const int32_t s = in->slots[b];
    if (s == p->pad_slot_id) continue;
    const int32_t n = in->num_buffered[b], r0 = in->ring_start[b];
    if (s < 0 || n < 0 || n + T > R || r0 < 0 || r0 >= R) {
      st = 2;
      break;
    }
    /* append the new tokens' inputs to the ring (bytes as given; dt after
       bias and softplus, rounded once to fp32) */
    for (int32_t t = 0; t < T; ++t) {
      const int32_t e = (r0 + n + t) % R;
      for (int32_t h = 0; h < H; ++h) {
        memcpy((char *)out->x_ring + (((int64_t)s * in->x_stride) + ((int64_t)e * H + h) * dim) * ib,
               (const char *)in->x_new + ((((int64_t)b * T + t) * H + h) * dim) * ib, (size_t)dim * ib);
        double dt = (double)in->dt_new[((int64_t)b * T + t) * H + h];
        if (in->dt_bias) dt += (double)in->dt_bias[h];
        if (p->dt_softplus) dt = softplus(dt);
        out->dt_ring[(int64_t)s * in->dt_stride + (int64_t)e * H + h] = (float)dt;
        if (out->dt_exact) out->dt_exact[((int64_t)b * T + t) * H + h] = dt;
      }
      for (int32_t g = 0; g < G; ++g)
        memcpy((char *)out->B_ring + (((int64_t)s * in->B_stride) + ((int64_t)e * G + g) * ds) * ib,
               (const char *)in->B_new + ((((int64_t)b * T + t) * G + g) * ds) * ib, (size_t)ds * ib);
    }
    for (int32_t h = 0; h < H; ++h) {
      const int32_t g = h / p->heads_per_group;
      const double A = (double)in->A[h];
      const int64_t sbase = (int64_t)s * in->state_stride + (int64_t)h * dim * ds;
      for (int64_t i = 0; i < (int64_t)dim * ds; ++i) {
        S[i] = orc_decode(p->state_dtype, in->state, sbase + i);
        M[i] = fabs(S[i]);
      }
      /* the pending ring entries, then the new tokens, one at a time */
      for (int32_t j = 0; j < n + T; ++j) {
        double dt;
        const void *xb, *Bb;
        int64_t xi, Bi;
        if (j < n) {
          const int32_t e = (r0 + j) % R;
          dt = (double)in->dt_ring[(int64_t)s * in->dt_stride + (int64_t)e * H + h];
          xb = in->x_ring;
          xi = (int64_t)s * in->x_stride + ((int64_t)e * H + h) * dim;
          Bb = in->B_ring;
          Bi = (int64_t)s * in->B_stride + ((int64_t)e * G + g) * ds;
        } else {
          const int32_t t = j - n;
          dt = (double)in->dt_new[((int64_t)b * T + t) * H + h];
          if (in->dt_bias) dt += (double)in->dt_bias[h];
          if (p->dt_softplus) dt = softplus(dt);
          xb = in->x_new;
          xi = (((int64_t)b * T + t) * H + h) * dim;
          Bb = in->B_new;
          Bi = (((int64_t)b * T + t) * G + g) * ds;
        }
        const double a = exp(dt * A);
        for (int32_t r = 0; r < dim; ++r) {
          const double xr = orc_decode(p->input_dtype, xb, xi + r);
          for (int32_t c = 0; c < ds; ++c) {
            const double bc = orc_decode(p->input_dtype, Bb, Bi + c);
            S[(int64_t)r * ds + c] = a * S[(int64_t)r * ds + c] + dt * xr * bc;
            M[(int64_t)r * ds + c] = a * M[(int64_t)r * ds + c] + fabs(dt * xr * bc);
          }
        }
        if (j < n) continue;
        /* readout of the new token */
        const int32_t t = j - n;
        const int64_t cbase = (((int64_t)b * T + t) * G + g) * ds;
        const int64_t ybase = (((int64_t)b * T + t) * H + h) * dim;
        for (int32_t r = 0; r < dim; ++r) {
          double y = 0.0, my = 0.0;
          for (int32_t c = 0; c < ds; ++c) {
            const double cc = orc_decode(p->input_dtype, in->C_new, cbase + c);
            y += S[(int64_t)r * ds + c] * cc;
            my += M[(int64_t)r * ds + c] * fabs(cc);
          }
          if (in->D) {
            const double dx = (double)in->D[h] * orc_decode(p->input_dtype, in->x_new, ybase + r);
            y += dx;
            my += fabs(dx);
          }
          if (in->z) {
            const double zv = orc_decode(p->input_dtype, in->z, ybase + r);
            const double gate = zv / (1.0 + exp(-zv));
            y *= gate;
            my *= fabs(gate);
          }
          out->y[ybase + r] = y;
          if (out->ymag) out->ymag[ybase + r] = my;
        }
      }
    }
  }
  free(S);
  free(M);
  return st;
}
