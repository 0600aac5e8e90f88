/*
 * rssm_gdn_commit.h -- C ABI of the gated-delta-rule ReplaySSM commit in
 * librssm_materialize (MI355X, gfx950).
 *
 * The operation is defined on the flashinfer documentation page for
 * flashinfer.gdn_decode.gated_delta_rule_replayssm_commit (summary,
 * Parameters, Notes): after a verify step has cached each request's raw
 * keys, values, log decays and betas in per-slot windows and acceptance is
 * known, one call commits the accepted prefix into every layer's fp32
 * checkpoint, in place.  For a request b with slot s = state_indices[b] above
 * null_block_id and n = accept_lens[b] > 0, every layer l and value head hv:
 *     for t < n:  k = rawk[l][s][hv / (HV/H)][t] / sqrt(|.|^2 + 1e-6)   (unnormalised if use_l2norm = 0)
 *                 S <- exp(g[l][s][hv][t]) * S
 *                 S <- S + beta[l][s][hv][t] * (rawv[l][s][hv][t] - S k) k^T
 * with S = state[l][s][hv] (128 value rows x 128 key columns, K last).  With
 * tracking, the state after token track_steps[b] (zero-based) is also
 * written to slot track_state_indices[b] when that step is inside the
 * accepted prefix and the slot is above null_block_id; otherwise that slot is
 * left unchanged.  A zero accepted count writes nothing.  The windows are
 * never modified.
 *
 * Plain C types only.  Every pointer is DEVICE memory owned by the caller;
 * the library allocates nothing and never synchronises.
 */
#ifndef RSSM_GDN_COMMIT_H
#define RSSM_GDN_COMMIT_H

#include <stdint.h>

#include "rssm_materialize.h" /* rssm_status, rssm_last_error */

#ifdef __cplusplus
extern "C" {
#endif

/* Host-side scalars.
 *   num_layers      L >= 1
 *   slots           pool slots per layer >= 1
 *   num_v_heads     HV >= 1
 *   num_k_heads     H >= 1, divides HV; value head hv reads key head hv / (HV / H)
 *   window          T, tokens per cached window, in [1, 16]
 *   batch           B >= 0 requests (0 enqueues nothing)
 *   use_l2norm      1: normalise cached keys with epsilon 1e-6 (the page's default); 0: use them as stored
 *   null_block_id   largest reserved slot, >= -1; slots <= it are ignored
 *   max_workgroups  0: occupancy-sized persistent grid; > 0: exactly this many */
typedef struct {
  int32_t num_layers;
  int32_t slots;
  int32_t num_v_heads;
  int32_t num_k_heads;
  int32_t window;
  int32_t batch;
  int32_t use_l2norm;
  int32_t null_block_id;
  int32_t max_workgroups;
} rssm_gdn_commit_desc;

/* Contiguous device tensors, as on the page (bf16 as 16-bit codes):
 *   checkpoint_state   fp32 [L][slots][HV][128][128], updated in place
 *   rawv_cache         bf16 [L][slots][HV][T][128]
 *   rawk_cache         bf16 [L][slots][H][T][128], before normalisation
 *   g_cache            fp32 [L][slots][HV][T], log decays
 *   beta_cache         fp32 [L][slots][HV][T]
 *   state_indices      int32 [B]
 *   accept_lens        int32 [B], in [0, T]
 *   track_state_indices, track_steps   int32 [B] each, or both NULL (no tracking)
 * Device-metadata contract (not checked, as on the page): live slots unique
 * and below `slots`; live track slots distinct and disjoint from every live
 * state slot.  As a guard against faults the kernel skips slots >= slots and
 * clamps accepted counts to [0, T].  checkpoint_state, rawv_cache and
 * rawk_cache must be 16-byte aligned, g_cache and beta_cache 4-byte aligned. */
typedef struct {
  float *checkpoint_state;
  const uint16_t *rawv_cache;
  const uint16_t *rawk_cache;
  const float *g_cache;
  const float *beta_cache;
  const int32_t *state_indices;
  const int32_t *accept_lens;
  const int32_t *track_state_indices;
  const int32_t *track_steps;
} rssm_gdn_commit_tables;

/* Enqueue one commit on `hip_stream`.  Host validation errors return before
 * any HIP call; RSSM_ERR_HIP reports a failed launch.  Arithmetic: fp32, one
 * token at a time in the order above (S k as fp32 sums; the decay is applied
 * to S k before the update, which is S <- exp(g) S + u k^T with
 * u = beta (v - exp(g) S k)). */
rssm_status rssm_gdn_commit(const rssm_gdn_commit_desc *desc, const rssm_gdn_commit_tables *tables,
                            void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_GDN_COMMIT_H */
