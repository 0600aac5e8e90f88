/*
 * rssm_ssu_decode.h -- C ABI of the ReplaySSM decode step in
 * librssm_materialize (MI355X, gfx950).
 *
 * The step the materialize operation serves (flashinfer page for
 * flashinfer.mamba.replayssm_materialize, Summary and Parameters; the pull
 * request "Replayssm prefix materialize", Description): a request's kept
 * checkpoint state plus its replay ring of inputs stands for its current
 * state, and a decode step appends the new tokens' inputs to the ring rather
 * than rewriting the state; materialize later flushes the ring into the
 * state.  The pages name this step without spelling it out; the reading
 * implemented here, for one layer per call:
 *
 * Request b uses slot s = slots[b] for both its checkpoint and its ring
 * (requests whose slot is pad_slot_id are skipped and their outputs left
 * untouched).  Its n = num_buffered[b] pending ring entries start at entry
 * ring_start[b] and wrap modulo R; the step brings T new tokens.  New token
 * t gets dt = softplus(dt_raw[b][t][h] + dt_bias[h]) (bias optional, softplus
 * optional) and its x, dt and B are written to ring entry
 * (ring_start + n + t) mod R of slot s.  Its output is the Mamba-2 readout
 * of the state after the n pending tokens and the new tokens up to t:
 *     S <- exp(dt A_h) S + dt x B^T           (from the checkpoint, token by token)
 *     y[b][t][h][r] = sum_c S[r][c] C[b][t][g][c] + D_h x[b][t][h][r],
 *                     times silu(z[b][t][h][r]) when z is given,
 * with g = h / heads_per_group.  The checkpoint state is read, never written.
 *
 * Plain C types only.  Every pointer is DEVICE memory owned by the caller;
 * the library allocates nothing and never synchronises.
 */
#ifndef RSSM_SSU_DECODE_H
#define RSSM_SSU_DECODE_H

#include <stdint.h>

#include "rssm_materialize.h" /* dtype codes, rssm_status, rssm_last_error */

#ifdef __cplusplus
extern "C" {
#endif

/* Most new tokens per call, and most pending + new tokens one call replays
 * (the materialize operation's max_window bound). */
#define RSSM_SSU_MAX_TOKENS 8
#define RSSM_SSU_MAX_REPLAY 16

/* Host-side scalars.
 *   batch              B >= 0 requests (0 enqueues nothing and reads no table pointer)
 *   num_heads          H >= 1
 *   heads_per_group    divides H; head h reads B and C group h / heads_per_group
 *   dim, dstate        compiled shape: (64, 128)
 *   ring_buffer_len    R >= tokens
 *   tokens             T, new tokens per request, in [1, RSSM_SSU_MAX_TOKENS]
 *   num_slots          slots of the state and ring pools (>= 1)
 *   pad_slot_id        slot sentinel to skip (the materialize page's default is -1)
 *   state_dtype        RSSM_F32 | RSSM_BF16 | RSSM_F16
 *   input_dtype        x, B, C, z and the x and B rings: RSSM_F32 | RSSM_BF16 | RSSM_F16
 *   dt_softplus        1: dt = softplus(dt_raw + bias); 0: dt = dt_raw + bias
 *   max_workgroups     0: about one (request, head) item per wavefront, at most
 *                      16 times the resident capacity; > 0: exactly this many
 *                      workgroups (results do not depend on it)
 *   *_slot_stride      distance between consecutive slots of each pool, in
 *                      ELEMENTS; at least the dense per-slot size below */
typedef struct {
  int32_t batch;
  int32_t num_heads;
  int32_t heads_per_group;
  int32_t dim;
  int32_t dstate;
  int32_t ring_buffer_len;
  int32_t tokens;
  int32_t num_slots;
  int32_t pad_slot_id;
  int32_t state_dtype;
  int32_t input_dtype;
  int32_t dt_softplus;
  int32_t max_workgroups;
  int64_t state_slot_stride;
  int64_t x_slot_stride;
  int64_t B_slot_stride;
  int64_t dt_slot_stride;
} rssm_ssu_decode_desc;

/* Device tensors (G = H / heads_per_group; layouts dense inside a slot, the
 * pools the materialize operation reads):
 *   state          [slots][H][dim][dstate]  state dtype, read only
 *   x_ring         [slots][R][H][dim]       input dtype, new entries written
 *   B_ring         [slots][R][G][dstate]    input dtype, new entries written
 *   dt_ring        [slots][R][H]            fp32 (after softplus), new entries written
 *   A              [H] fp32
 *   D, dt_bias     [H] fp32 each, or NULL (no skip term / no bias)
 *   x_new          [B][T][H][dim]           input dtype
 *   B_new, C_new   [B][T][G][dstate]        input dtype
 *   dt_new         [B][T][H] fp32, before bias and softplus
 *   z              [B][T][H][dim] input dtype, or NULL (no gate)
 *   y              [B][T][H][dim] fp32, written for live requests
 *   slots, ring_start, num_buffered   [B] int32
 * Device-metadata contract (not checked): live slots distinct and below
 * num_slots; ring_start in [0, R); num_buffered >= 0 with
 * num_buffered + T <= min(R, RSSM_SSU_MAX_REPLAY) (the caller flushes the
 * ring with an in-place materialize before it would overflow).  As a guard
 * against faults the kernel skips slots outside [0, num_slots), reduces
 * ring_start modulo R and clamps num_buffered to that bound.  Alignment:
 * state, B_ring, B_new and C_new 16 bytes, with state and B slot strides
 * times the element size multiples of 16 bytes; every other pointer the
 * size of its element. */
typedef struct {
  const void *state;
  void *x_ring;
  void *B_ring;
  float *dt_ring;
  const float *A;
  const float *D;
  const float *dt_bias;
  const void *x_new;
  const void *B_new;
  const void *C_new;
  const float *dt_new;
  const void *z;
  float *y;
  const int32_t *slots;
  const int32_t *ring_start;
  const int32_t *num_buffered;
} rssm_ssu_decode_tables;

/* Enqueue one decode step on `hip_stream`.  Host validation errors return
 * before any HIP call; RSSM_ERR_UNSUPPORTED for a shape or dtype with no
 * compiled instance; RSSM_ERR_HIP reports a failed launch.  Arithmetic:
 * fp32 throughout; a new token's dt is the fp32 softplus (log1p / exp form),
 * the same value stored in the ring and used for the output.  The output is
 * evaluated from the checkpoint as Dec (S_0 C) + sum_j w_j (B_j . C) x_j
 * + D x (the unrolled recurrence), so it differs from a token-by-token
 * evaluation by rounding only.  The x and B bytes appended are the inputs'
 * bytes.  Concurrent calls (or a materialize of the same slots) that touch
 * the same ring slots race; calls on one stream are ordered. */
rssm_status rssm_ssu_decode(const rssm_ssu_decode_desc *desc, const rssm_ssu_decode_tables *tables,
                            void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_SSU_DECODE_H */
