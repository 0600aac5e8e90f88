/*
 * gdn_oracle.c -- CPU oracle for the gated-delta-rule ReplaySSM commit.
 * TEST INFRASTRUCTURE ONLY; see gdn_oracle.h for the operation and its
 * source (flashinfer.gdn_decode.gated_delta_rule_replayssm_commit).
 *
 * Parity status: orc_gdn_tile and orc_gdn_commit are pinned by the CPU
 * tests (closed forms for pure decay and orthogonal keys, the delta rule's
 * S k = v property at beta = 1, key-scale invariance under normalisation,
 * head grouping, composition of two commits, no-op and tracking rules).
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32. */
static double bf16_value(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int check(const orc_gdn_params *p) {
  if (p->num_layers < 1 || p->slots < 1 || p->num_v_heads < 1 || p->num_k_heads < 1 || p->window < 1 ||
      p->batch < 0 || p->dk < 1 || p->dv < 1 || p->null_block_id < -1)
    return 1;
  if (p->num_v_heads % p->num_k_heads != 0) return 1;
  return 0;
}

int orc_gdn_tile(const orc_gdn_params *p, const float *s0, const uint16_t *k_win, const uint16_t *v_win,
                 const float *g_win, const float *b_win, int32_t n, int32_t track_step,
                 double *exact_final, double *mag_final, double *exact_track, double *mag_track) {
  if (check(p)) return 1;
  if (n < 0 || n > p->window) return 2;
  const int dk = p->dk, dv = p->dv;
  double *S = malloc(sizeof(double) * (size_t)dv * dk);
  double *M = malloc(sizeof(double) * (size_t)dv * dk);
  double *k = malloc(sizeof(double) * (size_t)dk);
  double *ka = malloc(sizeof(double) * (size_t)dk);
  double *Sk = malloc(sizeof(double) * (size_t)dv);
  double *Mk = malloc(sizeof(double) * (size_t)dv);
  if (!S || !M || !k || !ka || !Sk || !Mk) {
    free(S); free(M); free(k); free(ka); free(Sk); free(Mk);
    return 1;
  }
  for (int i = 0; i < dv * dk; ++i) {
    S[i] = (double)s0[i];
    M[i] = fabs(S[i]);
  }
  for (int t = 0; t < n; ++t) {
    /* the token's key, normalised to unit length (up to the epsilon) */
    double ss = 0.0;
    for (int j = 0; j < dk; ++j) {
      k[j] = bf16_value(k_win[(size_t)t * dk + j]);
      ss += k[j] * k[j];
    }
    if (p->use_l2norm) {
      const double nrm = sqrt(ss + 1e-6);
      for (int j = 0; j < dk; ++j) k[j] = k[j] / nrm;
    }
    for (int j = 0; j < dk; ++j) ka[j] = fabs(k[j]);
    const double alpha = exp((double)g_win[t]);
    const double beta = (double)b_win[t];
    /* decay, then the delta update toward v along k */
    for (int i = 0; i < dv * dk; ++i) S[i] *= alpha;
    for (int i = 0; i < dv; ++i) {
      double acc = 0.0, macc = 0.0;
      for (int j = 0; j < dk; ++j) {
        acc += S[(size_t)i * dk + j] * k[j];
        macc += M[(size_t)i * dk + j] * ka[j];
      }
      Sk[i] = acc;
      Mk[i] = macc;
    }
    for (int i = 0; i < dv; ++i) {
      const double v = bf16_value(v_win[(size_t)t * dv + i]);
      const double u = beta * (v - Sk[i]);
      const double mu = beta * alpha * Mk[i] + beta * fabs(v);
      for (int j = 0; j < dk; ++j) {
        S[(size_t)i * dk + j] += u * k[j];
        M[(size_t)i * dk + j] = alpha * M[(size_t)i * dk + j] + mu * ka[j];
      }
    }
    if (t == track_step) {
      if (exact_track) memcpy(exact_track, S, sizeof(double) * (size_t)dv * dk);
      if (mag_track) memcpy(mag_track, M, sizeof(double) * (size_t)dv * dk);
    }
  }
  memcpy(exact_final, S, sizeof(double) * (size_t)dv * dk);
  if (mag_final) memcpy(mag_final, M, sizeof(double) * (size_t)dv * dk);
  free(S); free(M); free(k); free(ka); free(Sk); free(Mk);
  return 0;
}

int orc_gdn_commit(const orc_gdn_params *p, const orc_gdn_inputs *in, const orc_gdn_outputs *out) {
  if (check(p)) return 1;
  const int32_t L = p->num_layers, HV = p->num_v_heads, H = p->num_k_heads, T = p->window;
  const int64_t tile = (int64_t)p->dv * p->dk;
  const int32_t group = HV / H;
  double *fin = malloc(sizeof(double) * (size_t)tile);
  double *finm = malloc(sizeof(double) * (size_t)tile);
  double *trk = malloc(sizeof(double) * (size_t)tile);
  double *trkm = malloc(sizeof(double) * (size_t)tile);
  if (!fin || !finm || !trk || !trkm) {
    free(fin); free(finm); free(trk); free(trkm);
    return 1;
  }
  int st = 0;
  for (int32_t b = 0; b < p->batch && st == 0; ++b) {
    const int32_t s = in->state_indices[b];
    const int32_t n = in->accept_lens[b];
    if (s <= p->null_block_id || n == 0) continue;     /* ignored slot; zero accepted is a no-op */
    if (s >= p->slots || n < 0 || n > T) { st = 2; break; }
    int32_t ts = -1, step = -1;
    if (p->has_track) {
      ts = in->track_state_indices[b];
      step = in->track_steps[b];
      if (ts <= p->null_block_id || step < 0 || step >= n) {
        step = -1;                                       /* outside the prefix: destination unchanged */
      } else if (ts >= p->slots) {
        st = 2;
        break;
      }
    }
    for (int32_t l = 0; l < L && st == 0; ++l) {
      for (int32_t hv = 0; hv < HV; ++hv) {
        const int64_t base = (((int64_t)l * p->slots + s) * HV + hv);
        const int64_t kbase = (((int64_t)l * p->slots + s) * H + hv / group);
        st = orc_gdn_tile(p, in->state + base * tile, in->rawk + kbase * T * p->dk, in->rawv + base * T * p->dv,
                          in->g + base * T, in->beta + base * T, n, step, fin, finm, trk, trkm);
        if (st) break;
        for (int64_t e = 0; e < tile; ++e) {
          out->state_out[base * tile + e] = (float)fin[e];
          if (out->exact) out->exact[base * tile + e] = fin[e];
          if (out->mag) out->mag[base * tile + e] = finm[e];
        }
        if (step >= 0) {
          const int64_t tb = (((int64_t)l * p->slots + ts) * HV + hv);
          for (int64_t e = 0; e < tile; ++e) {
            out->state_out[tb * tile + e] = (float)trk[e];
            if (out->exact) out->exact[tb * tile + e] = trk[e];
            if (out->mag) out->mag[tb * tile + e] = trkm[e];
          }
        }
      }
    }
  }
  free(fin); free(finm); free(trk); free(trkm);
  return st;
}
