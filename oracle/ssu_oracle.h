/*
 * ssu_oracle.h -- CPU oracle for the ReplaySSM decode step (the
 * checkpointing selective-state update that fills the replay ring).
 *
 * TEST INFRASTRUCTURE ONLY, like rssm_oracle.h: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load or call it, and
 * it shares nothing with the HIP path.
 *
 * The flashinfer pages reference this step (flashinfer.mamba.
 * replayssm_materialize, Summary and Parameters; the pull request "Replayssm
 * prefix materialize", Description): a kept checkpoint state plus the ring of
 * replay inputs stands for the current state, decode appends each new
 * token's inputs to the ring instead of updating the state, and the ring is
 * flushed into the state when it fills.  The pages do not spell the step
 * out; the readings taken here (one layer per call):
 *   - request b uses slot s = slots[b] for both its checkpoint state and its
 *     ring; n = num_buffered[b] ring entries starting at ring_start[b]
 *     (wrapping modulo R) are pending; the step brings T new tokens and
 *     n + T <= R (flushing is the caller's: an in-place materialize);
 *   - new token t gets dt = softplus(dt_raw + dt_bias) (dt_bias optional,
 *     softplus when dt_softplus) and is appended at ring entry
 *     (ring_start + n + t) mod R: x, B (per group) and dt;
 *   - its output is the Mamba-2 readout of the state after all pending and
 *     new tokens up to and including t:
 *         S <- exp(dt A_h) S + dt x B^T        (token by token, from the checkpoint)
 *         y_t[r] = sum_c S[r][c] C_t[c] + D_h x_t[r],   times silu(z_t[r]) when z is given;
 *   - the checkpoint state is read, never written.
 * fp64 throughout; y is returned unrounded, with a magnitude bound
 *     My = (sum_c M[r][c] |C_t[c]| + |D_h x_t[r]|) |silu(z)|
 * where M bounds |S| by the same recurrence on absolute values.
 */
#ifndef SSU_ORACLE_H
#define SSU_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch;            /* B */
  int32_t num_heads;        /* H */
  int32_t heads_per_group;  /* group of head h is h / heads_per_group */
  int32_t dim, dstate;
  int32_t ring_len;         /* R */
  int32_t tokens;           /* T new tokens per request */
  int32_t pad_slot_id;
  int32_t state_dtype;      /* ORC_F32 | ORC_BF16 | ORC_F16 (rssm_oracle.h codes) */
  int32_t input_dtype;      /* x, B, C, z: ORC_F32 | ORC_BF16 | ORC_F16 */
  int32_t dt_softplus;      /* 1: dt = softplus(dt_raw + bias) */
} orc_ssu_params;

/* One layer.  Slot-indexed pools are dense per slot with the given strides
 * (in elements); per-step inputs are dense. */
typedef struct {
  const void *state; int64_t state_stride;      /* [slots][H][dim][dstate] */
  const void *x_ring; int64_t x_stride;         /* [slots][R][H][dim] */
  const void *B_ring; int64_t B_stride;         /* [slots][R][G][dstate] */
  const float *dt_ring; int64_t dt_stride;      /* [slots][R][H] */
  const float *A;                               /* [H] */
  const float *D;                               /* [H] or NULL */
  const float *dt_bias;                         /* [H] or NULL */
  const void *x_new;                            /* [B][T][H][dim] */
  const void *B_new;                            /* [B][T][G][dstate] */
  const void *C_new;                            /* [B][T][G][dstate] */
  const float *dt_new;                          /* [B][T][H], before bias and softplus */
  const void *z;                                /* [B][T][H][dim] or NULL */
  const int32_t *slots, *ring_start, *num_buffered;   /* [B] */
} orc_ssu_inputs;

/* x_ring / B_ring / dt_ring: copies of the input rings that receive the
 * appended entries; y, ymag: [B][T][H][dim] fp64 (NaN for padded requests). */
typedef struct {
  void *x_ring;
  void *B_ring;
  float *dt_ring;
  double *y;
  double *ymag;
  double *dt_exact;   /* [B][T][H] fp64 dt of the new tokens, or NULL */
} orc_ssu_outputs;

/* Returns 0, 1 (bad scalar) or 2 (metadata outside the contract). */
int orc_ssu_decode(const orc_ssu_params *p, const orc_ssu_inputs *in, const orc_ssu_outputs *out);

#ifdef __cplusplus
}
#endif

#endif /* SSU_ORACLE_H */
