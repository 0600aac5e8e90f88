/*
 * rssm_materialize.h -- C ABI of librssm_materialize, the MI355X (gfx950)
 * implementation of ReplaySSM prefix materialize.
 *
 * The operation is defined on the flashinfer documentation page for
 * flashinfer.mamba.replayssm_materialize (Summary, Parameters, Notes) and the
 * flashinfer pull request "Replayssm prefix materialize" (Description): for
 * every selected (layer, request) the library applies replay_prefix_len[b]
 * entries of the request's replay ring, starting at ring_start[b] and wrapping
 * modulo ring_buffer_len, to the source state and writes the resulting state
 * to a separate destination slot.  One ring entry is the Mamba-2 step
 *     S_h <- exp(dt * A_h) * S_h + dt * x_h (outer) B_g(h).
 * All layers are handled by one persistent launch that pulls work from a
 * -1-terminated active-request list, so a call with nothing to do costs one
 * near-empty launch.
 *
 * Nothing here crosses the ABI but plain C types.  Every pointer inside
 * rssm_materialize_tables is DEVICE memory owned by the caller; the call
 * allocates nothing, keeps no reference after it returns, and reads no
 * device memory on the host (it never synchronises).  The caller keeps
 * every buffer alive until the enqueued work has completed on the stream.
 * (rssm_pool.h, a placement helper in a library of its own, librssm_pool,
 * outside this boundary, hands out physically contiguous device memory for
 * the pools; the operation works on any device memory.)
 */
#ifndef RSSM_MATERIALIZE_H
#define RSSM_MATERIALIZE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes (the page's state_dtype / input_dtype / matrixA_dtype). */
enum {
  RSSM_F32 = 0,
  RSSM_BF16 = 1,
  RSSM_F16 = 2,
  RSSM_I8 = 3,      /* symmetric int8 codes in [-127, 127] with per-row fp32 scales */
  RSSM_F8E4M3 = 4   /* OCP FP8 E4M3 (e4m3fn) codes with per-row fp32 scales */
};

/* Return status of every entry point. */
typedef enum {
  RSSM_OK = 0,
  RSSM_ERR_INVALID_ARGUMENT = 1, /* a host-visible argument is out of range or NULL */
  RSSM_ERR_UNSUPPORTED = 2,      /* valid, but no compiled instance (dtype / shape) */
  RSSM_ERR_HIP = 3               /* the HIP runtime reported an error (launch, device query) */
} rssm_status;

/* Host-side scalars of one call (the page's keyword parameters).
 *   num_layers       L >= 1
 *   batch            B >= 1, the physical batch (length of the per-request tables)
 *   num_heads        H >= 1 (runtime; int32 by type, so never narrowed)
 *   heads_per_group  divides H; head h reads B group h / heads_per_group
 *   dim, dstate      rows and columns of one head's state.  Compiled shapes:
 *                    (64, 128) for every dtype, (16, 16) for 2- and 4-byte state.
 *                    One-byte state requires (64, 128), as the page states.
 *   max_window       upper bound of replay_prefix_len, in [1, 16]
 *   ring_buffer_len  R >= 1, rows in every replay ring
 *   pad_slot_id      slot sentinel to skip (the page's default is -1)
 *   philox_rounds    0: round to nearest even; > 0: Philox4x32 stochastic
 *                    rounding with this many rounds (at most 64); needs rand_seed
 *   state_dtype      RSSM_F32 | RSSM_BF16 | RSSM_F16 | RSSM_I8 | RSSM_F8E4M3
 *   input_dtype      x and B ring dtype: RSSM_F32 | RSSM_BF16 | RSSM_F16
 *   a_dtype          A dtype: RSSM_F32 (dt is always fp32)
 *   max_workgroups   0: the default grid (the resident capacity; eight times
 *                    it for one-byte state with stochastic rounding, see
 *                    rssm_materialize_launch_config; the work loop is
 *                    persistent); > 0: exactly this many workgroups (results
 *                    do not depend on it) */
typedef struct {
  int32_t num_layers;
  int32_t batch;
  int32_t num_heads;
  int32_t heads_per_group;
  int32_t dim;
  int32_t dstate;
  int32_t max_window;
  int32_t ring_buffer_len;
  int32_t pad_slot_id;
  int32_t philox_rounds;
  int32_t state_dtype;
  int32_t input_dtype;
  int32_t a_dtype;
  int32_t max_workgroups;
} rssm_materialize_desc;

/* Device tables (the page's Parameters).  Per-layer tables hold L entries;
 * bases are device addresses as int64, slot strides are in ELEMENTS of the
 * pointed-to storage.  Per-slot layouts, dense inside a slot (a stride may be
 * larger than the dense size, leaving a gap the call never touches):
 *   state [H][dim][dstate]   state dtype
 *   scale [H][dim]           fp32 (one-byte state only; else the tables may be NULL)
 *   x     [R][H][dim]        input dtype
 *   B     [R][G][dstate]     input dtype, G = H / heads_per_group
 *   dt    [R][H]             fp32, stored after softplus (no bias, no limit)
 *   A     [H]                fp32, one vector per layer (no slot)
 * The ring (x, B, dt) of request b in layer l is the one stored in the SOURCE
 * slot src_slots[l][b].  src_slots and dst_slots are [L][B] row-major int32;
 * ring_start, replay_prefix_len and active_request_indices are [B] int32.
 * active_request_indices holds distinct physical indices in any order, then
 * -1; the kernel stops at the first entry that is -1 (or outside [0, B)).
 * rand_seed is a one-element int64 read on the device (graph-capturable):
 * Philox key = (low 32 bits, high 32 bits).
 *
 * Device-metadata contract (not checked, as on the page): ring_start in
 * [0, R) and replay_prefix_len in [0, max_window] for selected requests;
 * slots in range of their pools; destinations disjoint from every other
 * request's source and from each other; bases 16-byte aligned and slot
 * strides times element size multiples of 16 bytes.  A destination may be
 * the request's own source slot in that layer (an in-place flush of the
 * buffered tokens into the state, the "flush" of the pull-request page's
 * Description): each state element and row scale is read before it is
 * written, by the same wavefront.  Violations are undefined behaviour; as a
 * guard against faults the kernel clamps the prefix length to
 * [0, max_window], reduces ring_start modulo R and skips negative slots. */
typedef struct {
  const int64_t *state_ptrs, *state_slot_strides;
  const int64_t *x_ptrs, *x_slot_strides;
  const int64_t *B_ptrs, *B_slot_strides;
  const int64_t *dt_ptrs, *dt_slot_strides;
  const int64_t *A_ptrs;
  const int64_t *scale_ptrs, *scale_slot_strides;
  const int32_t *src_slots, *dst_slots;
  const int32_t *ring_start, *replay_prefix_len;
  const int32_t *active_request_indices;
  const int64_t *rand_seed;
} rssm_materialize_tables;

/* Enqueue one materialize call on `hip_stream` (a hipStream_t; NULL = the
 * default stream).  Returns RSSM_OK once the launch is enqueued.  Host
 * validation errors return before any HIP call, leaving device memory
 * untouched; RSSM_ERR_HIP reports a failed launch.  Source state, scales and
 * rings are never written.  Rounding: the state is accumulated in fp32 and
 * encoded once per call: fp32 stored as is; bf16/fp16 nearest-even, or
 * stochastic; one-byte rows get scale = rowmax / qmax (qmax 127 or 448),
 * codes = round(value * (qmax / rowmax)), nearest-even or stochastic,
 * saturating.  A zero prefix copies the state (and scale) bytes exactly. */
rssm_status rssm_materialize(const rssm_materialize_desc *desc,
                             const rssm_materialize_tables *tables,
                             void *hip_stream);

/* Most checkpoints per request of rssm_materialize_checkpoints. */
#define RSSM_MAX_CHECKPOINTS 4

/* Several checkpoints per request from one read of each source tile.  The
 * ring-buffer scheme of the flashinfer pages keeps more than one state per
 * request: a prefix cache that saves every `period` tokens needs the state at
 * a period boundary while the serving loop also flushes all buffered tokens
 * (the pull-request page's Description and the materialize page's Notes), and
 * the gated-delta-rule commit page writes an extra tracked checkpoint next to
 * its in-place commit (track_state_indices / track_steps).
 *
 * tables->dst_slots points to num_checkpoints consecutive [L][B] int32
 * tables and tables->replay_prefix_len to num_checkpoints consecutive [B]
 * int32 arrays; every other field is as for rssm_materialize.  The result is
 * that of num_checkpoints rssm_materialize calls, call c with destination
 * table c and prefix table c, all reading the state as it was before this
 * call: checkpoint c of request b in layer l is skipped when its destination
 * is pad_slot_id (the others are not), all are skipped when the source is;
 * a zero prefix copies bytes.  Prefix lengths may come in any order and may
 * repeat.  Destinations of one request are distinct; one of them may be the
 * source slot (in-place flush).
 *
 * Numerics: the fold runs once over the longest prefix and stores the fp32
 * running state at each shorter prefix, so the shortest positive checkpoint
 * is bit-identical to a rssm_materialize call with that prefix and the
 * others differ from separate calls only by fp32 rounding order; stochastic
 * rounding draws the same words as separate calls.  Compiled for
 * (dim, dstate) = (64, 128).  num_checkpoints outside
 * [1, RSSM_MAX_CHECKPOINTS] returns RSSM_ERR_INVALID_ARGUMENT; 1 is
 * exactly rssm_materialize. */
rssm_status rssm_materialize_checkpoints(const rssm_materialize_desc *desc,
                                         const rssm_materialize_tables *tables,
                                         int32_t num_checkpoints, void *hip_stream);

/* Text of the last non-OK status returned on the calling thread ("" if none):
 * which host-validation rule failed, or the HIP runtime's error string.  The
 * pull-request page ("Replayssm prefix materialize", change table) lists host
 * validation and runtime error checks as part of the operation; a C ABI
 * returns the status and keeps the text here instead of raising.  The
 * pointer stays valid until the next call on that thread; no other state is
 * kept. */
const char *rssm_last_error(void);

/* The launch the call would make for `desc` on the current device: grid and
 * block size in threads, and static LDS bytes per workgroup.  This is the
 * occupancy-based launch sizing of the pull-request page's change table
 * ("Replayssm prefix materialize"): the grid is the device's compute units
 * times the workgroups of this instance one compute unit holds (times 8 for
 * one-byte state with stochastic rounding, whose requests differ more in
 * cost), or desc->max_workgroups when that is > 0.  grid, block, lds_bytes: host
 * int32 outputs, all non-NULL.  Validates desc like rssm_materialize
 * (RSSM_ERR_INVALID_ARGUMENT / RSSM_ERR_UNSUPPORTED before any HIP call);
 * queries the device (may return RSSM_ERR_HIP).  Enqueues nothing. */
rssm_status rssm_materialize_launch_config(const rssm_materialize_desc *desc,
                                           int32_t *grid, int32_t *block, int32_t *lds_bytes);

/* Test hook: run the kernel's own encode step on caller-given fp32 rows, so
 * that rounding (nearest-even and Philox stochastic) can be compared bit for
 * bit.  The rounding is the one the materialize page's Parameters select
 * (rand_seed, philox_rounds: stochastic rounding with Philox when the round
 * count is positive) with the key and counter derivation of the pull-request
 * page's change table ("Philox seed derivation"), read as: key = the seed's
 * two 32-bit halves, counter = ((row * dstate + column) / 4, head, physical
 * request, layer), word column mod 4 per element.
 * rows: device [n][dstate] fp32; coords: device [n][4] int32 = (layer,
 * physical request, head, row) used as Philox coordinates; rand_seed: device
 * int64[1] (NULL when philox_rounds == 0); out_codes: device [n][dstate] in
 * state_dtype; out_scales: device [n] fp32 for one-byte state, else NULL.
 * Uses desc's state_dtype, dstate and philox_rounds; dstate must be 16 or 128
 * (128 for one-byte state).  n >= 0; n == 0 enqueues nothing. */
rssm_status rssm_debug_encode_rows(const rssm_materialize_desc *desc, const float *rows,
                                   const int32_t *coords, const int64_t *rand_seed,
                                   void *out_codes, float *out_scales, int32_t n,
                                   void *hip_stream);

/* Test hook: the row quantization parameters the one-byte encode uses, for
 * n given row maxima.  For a row whose largest magnitude is m (rowmax[i] =
 * m >= 0): scale[i] = m / qmax and inv[i] = qmax / m as correctly rounded
 * fp32 quotients, qmax = 127 (RSSM_I8) or 448 (RSSM_F8E4M3); a row with
 * m = 0, m infinite or qmax / m not finite gets scale 0 (inv is then the
 * IEEE quotient and unused by the encode).  This is the pull-request page's
 * per-row destination scale ("Replayssm prefix materialize", change table:
 * external decode-scale input, writes the destination scale buffer).
 * rowmax, scale, inv: device fp32 [n]; n >= 0 (0 enqueues nothing);
 * state_dtype other than RSSM_I8 / RSSM_F8E4M3 is RSSM_ERR_INVALID_ARGUMENT. */
rssm_status rssm_debug_row_scales(int32_t state_dtype, const float *rowmax, float *scale, float *inv,
                                  int32_t n, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_MATERIALIZE_H */
