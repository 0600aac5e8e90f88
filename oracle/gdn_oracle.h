/*
 * gdn_oracle.h -- CPU oracle for the gated-delta-rule ReplaySSM commit.
 *
 * TEST INFRASTRUCTURE ONLY, like rssm_oracle.h: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load or call it, and
 * it shares nothing with the HIP path.
 *
 * What it computes follows the flashinfer documentation page for
 * flashinfer.gdn_decode.gated_delta_rule_replayssm_commit (summary,
 * Parameters, Notes): for every request b whose pool slot s =
 * state_indices[b] is above null_block_id and whose accepted count
 * n = accept_lens[b] is positive, every layer l and every value head hv, the
 * fp32 checkpoint S = state[l][s][hv] (dv rows by dk columns, K last) takes
 * the first n tokens of the request's cached windows, in order:
 *     k = rawk[l][s][hv / (HV/H)][t]   (normalised k / sqrt(|k|^2 + 1e-6) when use_l2norm)
 *     v = rawv[l][s][hv][t],  alpha = exp(g[l][s][hv][t]),  beta = beta[l][s][hv][t]
 *     S <- alpha * S;   S <- S + beta * (v - S k) k^T
 * and is written back in place.  With tracking, the state after token
 * track_steps[b] (zero-based) is also written to slot track_state_indices[b]
 * when that step lies inside the accepted prefix and the slot is above
 * null_block_id.  A zero accepted count writes nothing, tracked or not.
 *
 * Arithmetic: fp64 throughout, token by token, rounded once to fp32 per
 * written state.  Alongside, a magnitude bound M >= |S| runs the same
 * recurrence on absolute values:
 *     M <- alpha M + beta alpha (M |k|) |k|^T + beta |v| |k|^T
 * which scales the rounding error any fp32 evaluation of the update can
 * make.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_layers;     /* L */
  int32_t slots;          /* pool slots per layer */
  int32_t num_v_heads;    /* HV */
  int32_t num_k_heads;    /* H, divides HV; value head hv reads key head hv / (HV / H) */
  int32_t window;         /* T, tokens per cached window */
  int32_t batch;          /* B */
  int32_t dk, dv;         /* state columns (key width) and rows (value width) */
  int32_t use_l2norm;     /* 1: normalise cached keys with epsilon 1e-6 */
  int32_t null_block_id;  /* slots <= this are ignored; >= -1 */
  int32_t has_track;      /* 1: track_state_indices / track_steps are given */
} orc_gdn_params;

/* Contiguous tensors, as on the page (bf16 as raw 16-bit codes). */
typedef struct {
  const float *state;          /* [L][slots][HV][dv][dk] */
  const uint16_t *rawv;        /* [L][slots][HV][T][dv] */
  const uint16_t *rawk;        /* [L][slots][H][T][dk] */
  const float *g;              /* [L][slots][HV][T], log decay */
  const float *beta;           /* [L][slots][HV][T] */
  const int32_t *state_indices;        /* [B] */
  const int32_t *accept_lens;          /* [B] in [0, T] */
  const int32_t *track_state_indices;  /* [B] or NULL */
  const int32_t *track_steps;          /* [B] or NULL */
} orc_gdn_inputs;

/* state_out must hold a copy of the input state (untouched regions keep it);
 * exact and mag (fp64, same shape, may be NULL) receive the unrounded state
 * and the magnitude bound of every written tile. */
typedef struct {
  float *state_out;
  double *exact;
  double *mag;
} orc_gdn_outputs;

/* Returns 0, 1 (bad scalar) or 2 (metadata outside the page's contract). */
int orc_gdn_commit(const orc_gdn_params *p, const orc_gdn_inputs *in, const orc_gdn_outputs *out);

/* One (layer, request, value head) tile: s0 [dv][dk]; k_win [T][dk] of the
 * tile's key head, v_win [T][dv], g_win / b_win [T].  Writes the state after
 * n tokens (exact_final, mag_final, fp64 [dv][dk]) and, when
 * 0 <= track_step < n, the state after token track_step (exact_track,
 * mag_track; may be NULL otherwise). */
int orc_gdn_tile(const orc_gdn_params *p, const float *s0, const uint16_t *k_win, const uint16_t *v_win,
                 const float *g_win, const float *b_win, int32_t n, int32_t track_step,
                 double *exact_final, double *mag_final, double *exact_track, double *mag_track);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
