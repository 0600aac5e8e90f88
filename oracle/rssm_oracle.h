/*
 * rssm_oracle.h -- CPU oracle for the ReplaySSM prefix-materialize operation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load, link or call this library.  The
 * product path (the HIP library and its binding) never does, and this code
 * shares nothing with it: no headers, kernels, helpers or tables.
 *
 * What it computes follows the flashinfer documentation page for
 * flashinfer.mamba.replayssm_materialize (Summary, Parameters, Notes):
 * for every selected (layer, request) it applies replay_prefix_len[b] ring
 * entries, starting at ring_start[b] and wrapping modulo ring_buffer_len, to
 * the source state and writes the result to the destination slot.  One ring
 * step is the Mamba-2 recurrence S <- exp(dt*A) * S + dt * x (outer) B.
 *
 * Arithmetic: every step runs in fp64, token by token, in the order the
 * pages describe.  The fp64 result is rounded once to fp32 and then encoded
 * into the state dtype.  fp64 state storage (ORC_F64) exists only in the
 * oracle, so that chained calls can be compared without any rounding.
 *
 * Parity status of each function is listed next to it.
 */
#ifndef RSSM_ORACLE_H
#define RSSM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes.  Values match the product library's enum by convention
 * only; nothing is shared. ORC_F64 is oracle-only. */
enum {
  ORC_F32 = 0,
  ORC_BF16 = 1,
  ORC_F16 = 2,
  ORC_I8 = 3,
  ORC_F8E4M3 = 4,
  ORC_F64 = 5
};

/* Status codes. */
enum {
  ORC_OK = 0,
  ORC_BAD_PARAM = 1,     /* a scalar parameter is out of range */
  ORC_BAD_METADATA = 2   /* a device-metadata value breaks the documented contract */
};

/* Scalars of one call (flashinfer.mamba.replayssm_materialize, Parameters). */
typedef struct {
  int32_t num_layers;       /* L */
  int32_t batch;            /* B, physical batch */
  int32_t num_heads;        /* H */
  int32_t heads_per_group;  /* must divide H; group of head h is h / heads_per_group */
  int32_t dim;              /* state rows per head */
  int32_t dstate;           /* state columns per head; multiple of 4 when SR is on */
  int32_t max_window;       /* replay_prefix_len upper bound, in [1, 16] */
  int32_t ring_len;         /* ring_buffer_len */
  int32_t pad_slot_id;      /* slot sentinel; default -1 */
  int32_t philox_rounds;    /* 0 = round to nearest even, >0 = stochastic rounding */
  int32_t state_dtype;      /* ORC_* */
  int32_t input_dtype;      /* x and B: ORC_F32, ORC_BF16 or ORC_F16 */
  uint64_t seed;            /* Philox key (low word, high word); used when rounds > 0 */
} orc_params;

/* Per-layer tables, all HOST memory.  Slot strides are in elements of the
 * pointed-to storage.  Per-slot layouts (dense inside a slot):
 *   state [H][dim][dstate]    scale [H][dim] fp32
 *   x     [R][H][dim]         B     [R][G][dstate]     dt [R][H] fp32
 *   A     [H] fp32, no slot
 * The ring (x, B, dt) is addressed through the SOURCE slot. */
typedef struct {
  const void *const *state;   const int64_t *state_stride;
  const float *const *scale;  const int64_t *scale_stride;   /* may be NULL unless 1-byte state */
  const void *const *x;       const int64_t *x_stride;
  const void *const *Bm;      const int64_t *B_stride;
  const float *const *dt;     const int64_t *dt_stride;
  const float *const *A;
  const int32_t *src_slots;   /* [L][B] */
  const int32_t *dst_slots;   /* [L][B] */
  const int32_t *ring_start;  /* [B] */
  const int32_t *prefix_len;  /* [B] */
  const int32_t *active;      /* [B]: distinct indices, then -1 */
} orc_inputs;

/* Output pools.  The caller passes a copy of the input state/scale pools;
 * the oracle writes only the destination tiles.  exact/mag are optional fp64
 * pools indexed like the state pool: the fp64 result and the magnitude sum
 * M = D*|S0| + sum_j w_j*|x_j[r]*B_j[c]| of each written element. */
typedef struct {
  void *const *state;
  float *const *scale;
  double *const *exact;   /* NULL or per-layer pointers */
  double *const *mag;     /* NULL or per-layer pointers */
} orc_outputs;

/* Whole operation.  Pinned by: k=0 byte copy, pad/inactive untouched,
 * read-only inputs, ring wrap vs. unrolled ring, composition (fp64 state),
 * closed forms (A=0 GEMM, x=0 decay, geometric series), unrolled sum. */
int orc_materialize(const orc_params *p, const orc_inputs *in, const orc_outputs *out);

/* One (layer, request, head) tile, for sampled checks at full size.
 * src_tile: [dim][dstate] in state dtype; src_scale: [dim] or NULL;
 * x_slot / B_slot / dt_slot: the SOURCE slot's ring (dense per-slot layout);
 * outputs: exact/mag [dim][dstate] (may be NULL), codes [dim][dstate] in the
 * state dtype (may be NULL), scale [dim] (1-byte state).  k == 0 copies. */
int orc_tile(const orc_params *p, int32_t layer, int32_t request, int32_t head,
             int32_t ring_start, int32_t k, float A_h,
             const void *src_tile, const float *src_scale,
             const void *x_slot, const void *B_slot, const float *dt_slot,
             double *exact, double *mag, void *codes, float *scale);

/* Encode one row of fp32 values (the state row r of head h) into the state
 * dtype, with the stochastic-rounding coordinates (layer, request, head, row).
 * Pinned by torch CPU casts (round to nearest even), exhaustive e4m3 round
 * trip, SR statistics. */
int orc_encode_row(const orc_params *p, const float *row, int32_t layer, int32_t request,
                   int32_t head, int32_t r, void *codes, float *scale);

/* Round one fp32 value to a narrow code: dtype in {BF16, F16, F8E4M3, I8};
 * stochastic != 0 uses the 32-bit word u.  Returns the code (sign included,
 * int8 as two's complement in the low byte). */
uint32_t orc_round_value(int32_t dtype, float v, int32_t stochastic, uint32_t u);

/* Decode one stored element to fp64. */
double orc_decode(int32_t dtype, const void *base, int64_t index);

/* Philox4x32 with `rounds` rounds (Salmon et al., SC'11).  Pinned by
 * rocRAND's independent Philox4x32-10 at rounds = 10. */
void orc_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int32_t rounds, uint32_t out[4]);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_ORACLE_H */
