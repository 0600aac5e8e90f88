// rssm_kernel.h -- persistent gfx950 kernel for ReplaySSM prefix materialize.
//
// Operation: flashinfer.mamba.replayssm_materialize (documentation page,
// Summary and Parameters).  For each request listed in the -1-terminated
// active list, each layer whose source and destination slots are not the pad
// sentinel, and each head h, with k = replay_prefix_len[b] ring entries
// e_j = (ring_start[b] + j) mod R taken from the SOURCE slot's ring:
//     S' = D * S + sum_j w_j * x_j (outer) B_j
//     a_j = exp(dt_j * A_h),  D = prod_j a_j,  w_j = dt_j * prod_{u>j} a_u
// which is the token-by-token recurrence S <- a_j S + dt_j x_j B_j^T unrolled.
// k = 0 copies the state (and scale) bytes exactly.
//
// Design (MI355X, wave64):
//  * Persistent grid; the -1-terminated active list is scanned once per
//    wavefront (ballot), so a call with no active request costs one launch in
//    which every wave does one load and exits (the pull-request page's reason
//    for persistent kernels and the active list).
//  * Work item = one (active request, layer, head) tile of dim x dstate,
//    ordered request-major, then layer, then head.  Chunks of 16 consecutive
//    items are dealt round-robin over the wavefronts (requests differ in cost),
//    and inside a chunk consecutive items share the request/layer metadata
//    and, within a head group, the B rows, which stay in registers.
//  * Decay weights come from a wavefront-level suffix-product scan over the k
//    per-token decays a_j = exp(dt_j A_h) held one per lane.
//  * Vector-ALU fold (fp32, bf16 and fp16 state; every multi-checkpoint
//    instance): w_j * x_j is staged per wavefront in LDS ([row][token],
//    fp32); each lane owns 8 columns, keeps B_j for those columns in
//    registers (16-token windows: tokens 0..3 in registers, 4..15 in the
//    wavefront's LDS), and streams its rows of the tile through registers
//    with 16-byte loads, folding k multiply-adds per element.  These paths
//    move ~4 bytes per 2k+1 flops and are bound by HBM, so no matrix cores.
//  * Matrix-core fold (one-byte state, one checkpoint; mfma_fold_heads):
//    there the per-element decode, row scale and encode make the vector ALU
//    the limit, so the fold itself moves to fp32 16x16x4 MFMA on 16-row
//    blocks and the vector ALU keeps only the decode and encode.
//  * No workgroup barriers: the four waves of a workgroup are independent.
#pragma once

#include "rssm_device.h"

namespace rssm {

constexpr int kWaves = 4;             // wavefronts per workgroup
constexpr int kMaxCheckpoints = 4;    // checkpoints per request of the multi-checkpoint instances
constexpr int kBlock = 64 * kWaves;   // threads per workgroup

struct KernelArgs {
  const int64_t* state_ptrs;
  const int64_t* state_strides;
  const int64_t* x_ptrs;
  const int64_t* x_strides;
  const int64_t* B_ptrs;
  const int64_t* B_strides;
  const int64_t* dt_ptrs;
  const int64_t* dt_strides;
  const int64_t* A_ptrs;
  const int64_t* scale_ptrs;
  const int64_t* scale_strides;
  const int32_t* src_slots;
  const int32_t* dst_slots;
  const int32_t* ring_start;
  const int32_t* prefix_len;
  const int32_t* active;
  const int64_t* rand_seed;
  int32_t L, B, H, hpg, R, W, pad, rounds;
  int32_t ncp;  // checkpoints per request (1 for the single-checkpoint operation)
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Orders this wavefront's LDS traffic: the compiler may not move LDS accesses
// across it, and it waits for outstanding LDS operations.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of requests before the first entry that is -1 (or outside [0, B)).
__device__ __forceinline__ int count_active(const int32_t* active, int B, int lane) {
  for (int base = 0; base < B; base += 256) {
    // All four loads are issued before any is used (indices past B read the
    // last entry and are then discarded), so the scan costs one round trip.
    uint64_t stop[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = base + 64 * q + lane;
      const int x = gload(active + (idx < B ? idx : B - 1));
      const int v = (idx < B) ? x : -1;
      stop[q] = __ballot(v < 0 || v >= B);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (stop[q]) return base + 64 * q + __builtin_ctzll(stop[q]);
  }
  return B;
}

// Liveness of 64 chunks of one wavefront at once, one chunk per lane: lane j
// tests chunk gw + (qb + j) * tw.  A chunk inside one (request, layer) is live
// unless the pair is skipped (a pad or negative source; for NCK = 1 a pad
// destination; for several checkpoints every destination the pad slot).  A
// chunk that spans several pairs is reported live and left to the main loop.
// Returns the ballot of live chunks; lanes past the last item are not live.
// Every entry read is in range: i < n_active, and count_active stops at the
// first entry outside [0, B).
template <int NCK>
__device__ __forceinline__ uint64_t live_chunks(const KernelArgs& a, int64_t gw, int64_t tw, int64_t qb,
                                                int64_t csz, int64_t items, int lane) {
  const int64_t it0 = (gw + (qb + lane) * tw) * csz;
  bool live = false;
  if (it0 < items) {
    const int64_t il0 = it0 / a.H;
    const int64_t il1 = (min(items, it0 + csz) - 1) / a.H;
    if (il0 != il1) {
      live = true;
    } else {
      const int i = static_cast<int>(il0 / a.L);
      const int l = static_cast<int>(il0 - static_cast<int64_t>(i) * a.L);
      const int b = gload(a.active + i);
      const int64_t lb = static_cast<int64_t>(l) * a.B + b;
      const int s = gload(a.src_slots + lb);
      bool any_dst = false;
      if constexpr (NCK == 1) {
        const int d = gload(a.dst_slots + lb);
        any_dst = d != a.pad && d >= 0;
      } else {
        const int64_t LB = static_cast<int64_t>(a.L) * a.B;
        for (int c = 0; c < a.ncp; ++c) {
          const int d = gload(a.dst_slots + c * LB + lb);
          any_dst = any_dst || (d != a.pad && d >= 0);
        }
      }
      live = s != a.pad && s >= 0 && any_dst;
    }
  }
  return __ballot(live);
}

// An fp32 row chunk held as two 4-column halves half a row apart (columns
// c..c+3 and c+64..c+67 of a 128-column row): with lane cc of a row at
// c = 4*cc, each 16-byte access instruction covers contiguous bytes across
// the lanes of the row, which streams faster on MI355X than 32 contiguous
// bytes per lane split over two instructions.  p = row start + 16*cc bytes.
template <bool NT>
__device__ __forceinline__ Chunk<kF32> load_split_f32(const char* p) {
  const u32x4 a = ld<NT, u32x4>(p), b = ld<NT, u32x4>(p + 256);
  Chunk<kF32> c;
  c.w[0] = a.x; c.w[1] = a.y; c.w[2] = a.z; c.w[3] = a.w;
  c.w[4] = b.x; c.w[5] = b.y; c.w[6] = b.z; c.w[7] = b.w;
  return c;
}

template <bool NT>
__device__ __forceinline__ void store_split_f32(char* p, const Chunk<kF32>& c) {
  st<NT>(p, u32x4{c.w[0], c.w[1], c.w[2], c.w[3]});
  st<NT>(p + 256, u32x4{c.w[4], c.w[5], c.w[6], c.w[7]});
}

// Value of lane-permuted v within each 16-lane DPP row (no LDS traffic).  The
// patterns used here have a valid source lane for every lane, so bound_ctrl
// never applies; a plain DPP move (rather than an update of an old value)
// lets the compiler fold it into the consuming add or max.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Value of lane (lane + N) within the lane's row of 16 (DPP row_shl:N), for
// the token scans: tokens sit in lanes 0..15, and a lane only uses the value
// when lane + N is a token lane of the same row.  No LDS round trip.
template <int N>
__device__ __forceinline__ float row_shl(float v) {
  static_assert(N >= 1 && N <= 15, "row_shl");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x100 + N, 0xF, 0xF, true));
}

// Inclusive suffix products over the token lanes j < seg_end (<= 16): lane j
// gets prod_{j <= u < seg_end} a_u; lanes at or past seg_end keep their value.
__device__ __forceinline__ float suffix_products(float a, int lane, int seg_end) {
  float P = a;
  float o = row_shl<1>(P);
  if (lane + 1 < seg_end) P *= o;
  o = row_shl<2>(P);
  if (lane + 2 < seg_end) P *= o;
  o = row_shl<4>(P);
  if (lane + 4 < seg_end) P *= o;
  o = row_shl<8>(P);
  if (lane + 8 < seg_end) P *= o;
  return P;
}

// Max over the 16 lanes of an aligned lane group (one state row) of values
// that are >= +0 and not NaN: swap lane pairs, then pairs of pairs
// (quad_perm), then mirror within 8 lanes and within 16 lanes.  The bit
// patterns of such values order as unsigned integers, so each step is one
// integer max with the lane exchange folded in (a float max would also
// quiet the moved value first).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float row16_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, dpp_u32<0xB1>(u));   // quad_perm [1,0,3,2]
  u = max(u, dpp_u32<0x4E>(u));   // quad_perm [2,3,0,1]
  u = max(u, dpp_u32<0x141>(u));  // row_half_mirror
  u = max(u, dpp_u32<0x140>(u));  // row_mirror
  return __uint_as_float(u);
}

// Sum over the 16 lanes of an aligned lane group, every lane receiving the
// total (the same exchange pattern as row16_max_nonneg).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Encode this lane's 8 fp32 values of one state row.  One-byte state reduces
// the row max over the row's 16 lanes (all 64 lanes must execute this) and
// returns the new row scale in `row_scale`.
template <int ST, bool SR>
__device__ __forceinline__ Chunk<ST> encode_chunk(const float (&acc)[8], const uint32_t (&u)[8],
                                                  float& row_scale) {
  Chunk<ST> out;
  if constexpr (ST == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = __float_as_uint(acc[i]);
  } else if constexpr (ST == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out.w[i] = bf16_round(acc[2 * i], SR, u[2 * i]) | (bf16_round(acc[2 * i + 1], SR, u[2 * i + 1]) << 16);
  } else if constexpr (ST == kF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out.w[i] = f16_round(acc[2 * i], SR, u[2 * i]) | (f16_round(acc[2 * i + 1], SR, u[2 * i + 1]) << 16);
  } else {
    // Per-row symmetric quantization: scale = rowmax/qmax, t = v * (qmax/rowmax),
    // both correctly rounded fp32 quotients (row_quant).  An all-zero row (or
    // one whose inverse overflows) stores scale 0 and zero codes.
    constexpr int qmax = (ST == kI8) ? 127 : 448;
    // The lane's max starts at +0 and fmaxf ignores NaN elements, so m is
    // >= +0 and never NaN.
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(acc[i]));
    m = row16_max_nonneg(m);
    float inv;
    const bool ok = row_quant<qmax>(m, row_scale, inv);
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = acc[i] * inv;
    // Whether any lane of the wavefront holds a NaN element (wave-uniform).
    auto any_nan = [&t]() {
      bool has_nan = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) has_nan |= (t[i] != t[i]);
      return __builtin_expect(__ballot(has_nan) != 0, 0);
    };
    if constexpr (ST == kI8) {
      uint32_t code[8];
      if (SR || any_nan()) {
#pragma unroll
        for (int i = 0; i < 8; ++i) code[i] = i8_round(t[i], SR, u[i]);
      } else {
        // Nearest-even.  In a valid row |t| <= 127 (1 + 2^-24)^2 < 127.5, so
        // adding 1.5 * 2^23 rounds t to an integer in [-127, 127] in one IEEE
        // rounding with no clamp, and the low byte of the sum's bits is the
        // two's-complement code.  An invalid row is zeroed below.
#pragma unroll
        for (int i = 0; i < 8; ++i) code[i] = __float_as_uint(t[i] + 12582912.0f);
      }
      out.w[0] = pack_low_bytes(code[0], code[1], code[2], code[3]);
      out.w[1] = pack_low_bytes(code[4], code[5], code[6], code[7]);
    } else {
      // |t| <= 448(1 + 2^-22) for every finite element of a valid row.
      if constexpr (SR) {
        // NaN elements (ignored by the row max) and elements below 2^-6 (where
        // the subnormal grid applies) are rare: one compare finds both, and a
        // wavefront holding any takes the general rule for all its elements.
        // The common path rounds each value onto the e4m3 grid as an fp32
        // value (e4m3_sr_normal_value) and converts it with the hardware
        // conversion, which is exact for values on the grid and places the
        // sign and the codes in their bytes.
        bool rare = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) rare |= !(fabsf(t[i]) >= 0x1p-6f);
        if (__builtin_expect(__ballot(rare) != 0, 0)) {
          uint32_t code[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) code[i] = e4m3_round(t[i], true, u[i]);
          out.w[0] = pack_low_bytes(code[0], code[1], code[2], code[3]);
          out.w[1] = pack_low_bytes(code[4], code[5], code[6], code[7]);
        } else {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            // (the high half of the first conversion's old operand is
            // overwritten by the second: any dead register serves)
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sr_normal_value(t[4 * w], u[4 * w]),
                                                     e4m3_sr_normal_value(t[4 * w + 1], u[4 * w + 1]),
                                                     static_cast<int>(u[4 * w]), false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sr_normal_value(t[4 * w + 2], u[4 * w + 2]),
                                                 e4m3_sr_normal_value(t[4 * w + 3], u[4 * w + 3]), pk, true);
            out.w[w] = static_cast<uint32_t>(pk);
          }
        }
      } else if (any_nan()) {
        // NaN elements (ignored by the row max) take the general rule.
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) code[i] = e4m3_round(t[i], false, u[i]);
        out.w[0] = pack_low_bytes(code[0], code[1], code[2], code[3]);
        out.w[1] = pack_low_bytes(code[4], code[5], code[6], code[7]);
      } else {
        // Hardware nearest-even conversion: equal to e4m3_round for |t| < 464
        // (checked on gfx950), which covers every finite row-scaled value.
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * i + 0], t[4 * i + 1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * i + 2], t[4 * i + 3], w, true);
          out.w[i] = static_cast<uint32_t>(w);
        }
      }
    }
    if (!ok) {
      out.w[0] = 0u;
      out.w[1] = 0u;
    }
  }
  return out;
}

// Address = wave-uniform base + 32-bit per-lane byte offset (the scalar-base
// addressing mode; keeps per-pass addresses out of vector registers).
template <typename T>
__device__ __forceinline__ T* at(T* uniform_base, uint32_t lane_off) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(uniform_base) + lane_off);
}

// Ring entry of token j: (r0 + j) mod R, for 0 <= r0 < R and j < 16.
__device__ __forceinline__ int ring_entry(int r0, int j, int R) {
  int e = r0 + j;
  while (e >= R) e -= R;
  return e;
}

// B_j rows held in registers: 8 columns cost 8 registers per token.  Windows
// of up to 8 tokens keep every row in registers; 16-token windows keep the
// first 4 and read the other 12 from the wavefront's LDS.  On MI355X that
// trade (LDS reads for registers) lets the 16-token instances run 4 waves per
// SIMD instead of 2: the e4m3 + Philox workload (windows up to 16) ran 19%
// faster than with all 16 rows in registers; 8 rows in registers at 3 waves
// gained 14%.  For int8 with 8-token windows, 4 rows in LDS ran 5% slower.
template <int KMAX> constexpr int kBRegs = (KMAX > 8) ? 4 : KMAX;

// int8 state, fp16 x/B, windows of up to 8, one checkpoint, vector-ALU fold
// (a tuning variant with the matrix-core fold off): B rows held as packed
// fp16 pairs and multiplied with v_fma_mix_f32, which leaves room for 5 waves
// per SIMD (4.3% faster than fp32 rows at 4 waves on MI355X; at 4 waves the
// packed rows alone ran 1% slower).
template <int ST, int IT, int KMAX, int NCK>
constexpr bool kMixB = (ST == kI8 && IT == kF16 && KMAX <= 8 && NCK == 1);

// Resident wavefronts per SIMD the register budget of the VALU fold is sized
// for (two- and four-byte state, and every multi-checkpoint instance; the
// one-byte single-checkpoint instances fold on the matrix cores at 4 waves,
// and reach the one-byte rules below only with that fold switched off).
// e4m3 state adds software decode/encode on top of the row scales: its
// 8-token instances get a 3-wave budget (168 registers) so they do not spill.
// int8 keeps 4 waves (5 with packed fp16 B rows, above).
// The multi-checkpoint instances (segment bookkeeping) get 3 waves, where
// they do not spill (with windows up to 8, 4 waves spilled 32 registers and
// the two-checkpoint large bf16 call ran 1% slower on MI355X).
// 16-token instances get 4 waves, except with fp32 x/B (16 raw 32-byte B
// chunks are held while a group's rows load): 3.
template <int KMAX, int ST, int IT, int NCK>
constexpr int kWavesPerSimd = (KMAX > 8) ? ((IT == kF32 || NCK > 1) ? 3 : 4)
                                         : ((ST == kF8 || NCK > 1) ? 3 : (kMixB<ST, IT, KMAX, NCK> ? 5 : 4));

// Knobs of the state stream.  The library's instances use the defaults; the
// alternatives exist so that streaming patterns can be compared on hardware.
// Defaults measured on MI355X, variants side by side in one process: on the
// large bf16 shape, non-temporal state loads and stores (each byte is touched
// once) with 8 dwords per lane in flight ran ~4.5% faster than cached
// accesses with 16 dwords in flight; chunks of 16 items dealt round-robin ran
// 5-10% faster than contiguous ranges on the int8 workload (a quarter of the
// requests copy) and 11% faster on the e4m3 + Philox workload (prefixes
// U[0, 16]), and within 1% on bf16.
struct DefaultTune {
  static constexpr int kInflightDwords = 8;   // state dwords per lane in flight (at least 2 passes)
  static constexpr bool kNtLoad = true;        // non-temporal state loads
  static constexpr bool kNtStore = true;       // non-temporal state stores
  static constexpr int kChunkItems = 16;       // 0: one contiguous item range per wavefront;
                                               // > 0: chunks of this many items dealt round-robin
  static constexpr int kWavesPerSimd = 0;      // register budget; 0: the rule above
  static constexpr bool kMfmaOneByte = true;   // one-byte state: fold on the matrix cores
  static constexpr bool kMfmaPrefetch = false; // matrix-core fold: request the next head's inputs early
  static constexpr bool kMfmaTranspose = true; // matrix-core fold: coalesced row blocks through LDS
};

// One-byte state with one checkpoint folds on the matrix cores (see
// mfma_fold_heads), unless a tuning variant turns it off.
template <class Tune, int ST, int NCK>
constexpr bool kMfmaFold = Tune::kMfmaOneByte && kOneByte<ST> && NCK == 1;

template <class Tune, int KMAX, int ST, int IT, int NCK>
constexpr int waves_per_simd() {
  return Tune::kWavesPerSimd > 0 ? Tune::kWavesPerSimd
                                 : (kMfmaFold<Tune, ST, NCK> ? 4 : kWavesPerSimd<KMAX, ST, IT, NCK>);
}

// Checkpoint bookkeeping of one (request, layer): kc[c] is the prefix length of
// the c-th checkpoint in ascending order (-1: skipped, its destination is the
// pad slot or it is not requested), dc[c] its destination slot.
template <int NCK>
__device__ __forceinline__ void sort_checkpoints(int (&kc)[NCK], int (&dc)[NCK]) {
#pragma unroll
  for (int i = 0; i < NCK; ++i) {
#pragma unroll
    for (int j = 0; j + 1 < NCK - i; ++j) {
      const bool sw = kc[j] > kc[j + 1];
      const int k0 = kc[j], d0 = dc[j];
      kc[j] = sw ? kc[j + 1] : k0;
      dc[j] = sw ? dc[j + 1] : d0;
      kc[j + 1] = sw ? k0 : kc[j + 1];
      dc[j + 1] = sw ? d0 : dc[j + 1];
    }
  }
}

// ---------------------------------------------------------------------------
// One-byte state: the fold on the matrix cores.
//
// With one-byte state and stochastic rounding the path is bound by VALU
// issue, not by HBM: per state element Philox-10 costs about 10
// instructions and the fold k fused multiply-adds, against about 9.8
// instructions' worth of issue time per element at HBM speed.  The fold is
// a rank-k update of the tile, U = W X^T B with k <= 16, i.e. a small dense
// contraction: these instances run it as fp32 16x16x4 MFMAs.  One MFMA does
// 1024 multiply-adds in 32 cycles, twice the rate of unpacked vector FMAs,
// and leaves the vector issue slots to Philox, row scales and encode; on
// MI355X it does not overlap that work (the fp32 matrix rate equals the
// fp32 vector rate), so the saving is the issue rate.
//
// Layout.  A tile is 4 blocks of 16 rows.  In a row block, lane L holds row
// j = L % 16 and, with q = L / 16, the 32 columns [16q, 16q + 16) and
// [64 + 16q, 64 + 16q + 16): two 16-byte loads per lane, each instruction
// covering 64 contiguous bytes of 16 rows.  Those 32 columns are the
// accumulator of 8 MFMAs (blocks bb = 0..7, 4 registers each): register v of
// block bb holds column col(q, bb, v) = 64 (bb / 4) + 16 q + 4 (bb % 4) + v,
// so block bb's 4 registers are 4 consecutive columns (one output dword,
// one Philox block) and blocks 0..3 / 4..7 fill the two 16-byte chunks in
// memory order.  For the 16x16x4 fp32 MFMA, D[i][j] sits in lane
// j + 16 (i / 4), register i % 4, and lane L supplies A[L % 16][L / 16] and
// B[L / 16][L % 16]; with D[i][j] = U[row j][col(i / 4, bb, i % 4)] the
// operands are A[i][t] = B_t[col(i / 4, bb, i % 4)] (ring B rows: fixed per
// head group and lane, held in registers) and B[t][j] = w_t x_t[row j]
// (staged per head in LDS as [token][row]).  C is the decoded source times
// its decay, so one MFMA chain per block gives D S + U.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The [token][row] LDS staging of w_t x_t: 64 floats per token, row r of
// token t stored at position r ^ (16 (t & 1)), so that the two token rows a
// half-wavefront reads (tokens 4 ks, 4 ks + 1; rows 16 rb .. 16 rb + 15)
// fall into disjoint banks.
constexpr int kWxStride = 64;
__device__ __forceinline__ int wx_pos(int t, int row) { return t * kWxStride + (row ^ (16 * (t & 1))); }

// LDS floats per wavefront of the matrix-core fold: the w_t x_t staging, and
// the A operands of k-steps 1 .. KMAX/4 - 1 as [k-step - 1][lane][block]
// (k-step 0 stays in registers).
template <int KMAX, bool TR>
constexpr int kMfmaLds = KMAX * kWxStride + (KMAX / 4 - 1) * 64 * 8 + (TR ? 512 : 0);

// Byte offset of 16-byte chunk c of row r in the 2 KiB LDS transposition
// buffer of one 16-row block: chunk positions rotated by row (c ^ (r & 7)),
// so that both the row-major writes (8 lanes per row) and the reads in the
// accumulator layout (one row per lane, 8 rows at once) hit distinct banks.
__device__ __forceinline__ uint32_t tr_pos(int r, int c) {
  return static_cast<uint32_t>(r * 128 + 16 * (c ^ (r & 7)));
}

// One element of the ring's B rows as fp32.
template <int IT>
__device__ __forceinline__ float load_elem(const char* p) {
  if constexpr (IT == kF32) {
    return gload(reinterpret_cast<const float*>(p));
  } else if constexpr (IT == kBF16) {
    return __uint_as_float(static_cast<uint32_t>(gload(reinterpret_cast<const uint16_t*>(p))) << 16);
  } else {
    return f16_bits_to_float(gload(reinterpret_cast<const uint16_t*>(p)));
  }
}

// Four one-byte codes (one dword, byte v = column v) decoded and multiplied
// by d: the source value times its decay.  int8: the bytes biased by 128 are
// converted as unsigned, and fma(u, d, -128 d) rounds (u - 128) d once, the
// same bits as code * d.
template <int ST>
__device__ __forceinline__ f32x4 decode4_scaled(uint32_t w, float d) {
  f32x4 r;
  if constexpr (ST == kI8) {
    const uint32_t u = w ^ 0x80808080u;
    const float nd = -128.0f * d;
    r[0] = fmaf(static_cast<float>(u & 0xFFu), d, nd);
    r[1] = fmaf(static_cast<float>((u >> 8) & 0xFFu), d, nd);
    r[2] = fmaf(static_cast<float>((u >> 16) & 0xFFu), d, nd);
    r[3] = fmaf(static_cast<float>(u >> 24), d, nd);
  } else {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    r[0] = lo[0] * d;
    r[1] = lo[1] * d;
    r[2] = hi[0] * d;
    r[3] = hi[1] * d;
  }
  return r;
}

// Encode one row block held in the MFMA layout: acc[bb][v] is column
// col(q, bb, v) of row r.  The row max runs over the lane's 32 values and
// then over the 4 lanes holding row r (lanes r % 16 + 16 q'); out[bb] is the
// dword of block bb's 4 codes, rs the new row scale.  Every lane of the
// wavefront must execute this.
template <int ST, bool SR>
__device__ __forceinline__ void encode_rowblock(f32x4 (&acc)[8], int r, int q, int h, int b, int l,
                                                uint32_t key0, uint32_t key1, int rounds, uint32_t (&out)[8],
                                                float& rs) {
  constexpr int qmax = (ST == kI8) ? 127 : 448;
  float m = 0.0f;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(acc[bb][v]));
  // values >= +0 and never NaN: their bits order as unsigned integers.  The
  // lanes of row r are L, L ^ 16, L ^ 32, L ^ 48: gfx950's row swaps give
  // each lane its partner's value one and two rows of 16 away.
  uint32_t mu = __float_as_uint(m);
  {
    const auto p16 = __builtin_amdgcn_permlane16_swap(mu, mu, false, false);
    mu = max(p16[0], p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(mu, mu, false, false);
    mu = max(p32[0], p32[1]);
  }
  m = __uint_as_float(mu);
  float inv;
  const bool ok = row_quant<qmax>(m, rs, inv);
  // Elements that take the general rule: NaN (all encodes), and for
  // stochastic e4m3 any |t| below 2^-6 (the subnormal grid).  The smallest
  // |t| is the smallest |S'| times inv (rounding is monotonic), and NaN is
  // found two elements per unordered compare.
  bool has_nan = false;
  float mn = fabsf(acc[0][0]);
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    has_nan |= __builtin_isunordered(acc[bb][0], acc[bb][1]) || __builtin_isunordered(acc[bb][2], acc[bb][3]);
    if constexpr (SR && ST == kF8)
#pragma unroll
      for (int v = 0; v < 4; ++v) mn = fminf(mn, fabsf(acc[bb][v]));
  }
  bool rare = false;
  if constexpr (SR && ST == kF8) rare = !(mn * inv >= 0x1p-6f);
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[bb][v] *= inv;   // t = S' * (qmax / rowmax)
  const bool general = __builtin_expect(__ballot(has_nan || rare) != 0, 0);
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    // blocks 2pb and 2pb + 1: Philox counters x and x + 1 (counter word 0 is
    // (r * dstate + c) / 4 for the block's first column c)
    uint32_t u[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if constexpr (SR) {
      const uint32_t x = static_cast<uint32_t>(32 * r + 16 * (pb >> 1) + 4 * q + 2 * (pb & 1));
      philox4x32_pair(x, static_cast<uint32_t>(h), static_cast<uint32_t>(b), static_cast<uint32_t>(l), key0, key1,
                      rounds, u);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int bb = 2 * pb + s;
      const f32x4 t = acc[bb];
      uint32_t w;
      if constexpr (ST == kI8) {
        if (SR || general) {
          w = pack_low_bytes(i8_round(t[0], SR, u[4 * s]), i8_round(t[1], SR, u[4 * s + 1]),
                             i8_round(t[2], SR, u[4 * s + 2]), i8_round(t[3], SR, u[4 * s + 3]));
        } else {
          // |t| <= 127 (1 + 2^-24)^2 < 127.5 in a valid row: one rounding to an
          // integer, the low byte of the sum's bits is the code
          w = pack_low_bytes(__float_as_uint(t[0] + 12582912.0f), __float_as_uint(t[1] + 12582912.0f),
                             __float_as_uint(t[2] + 12582912.0f), __float_as_uint(t[3] + 12582912.0f));
        }
      } else if constexpr (SR) {
        if (general) {
          w = pack_low_bytes(e4m3_round(t[0], true, u[4 * s]), e4m3_round(t[1], true, u[4 * s + 1]),
                             e4m3_round(t[2], true, u[4 * s + 2]), e4m3_round(t[3], true, u[4 * s + 3]));
        } else {
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sr_normal_value(t[0], u[4 * s]),
                                                   e4m3_sr_normal_value(t[1], u[4 * s + 1]),
                                                   static_cast<int>(u[4 * s]), false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sr_normal_value(t[2], u[4 * s + 2]),
                                               e4m3_sr_normal_value(t[3], u[4 * s + 3]), pk, true);
          w = static_cast<uint32_t>(pk);
        }
      } else {
        if (general) {
          w = pack_low_bytes(e4m3_round(t[0], false, 0u), e4m3_round(t[1], false, 0u), e4m3_round(t[2], false, 0u),
                             e4m3_round(t[3], false, 0u));
        } else {
          // hardware nearest-even conversion, equal to e4m3_round for |t| < 464
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], pk, true);
          w = static_cast<uint32_t>(pk);
        }
      }
      out[bb] = ok ? w : 0u;
    }
  }
}

// The heads [h0, h1) of one (request, layer) with k > 0 on the matrix-core
// fold (one-byte state, 64 x 128 tiles, one checkpoint).  wxT: this
// wavefront's LDS, kMfmaLds<KMAX, TR> floats.
template <int ST, int IT, int KMAX, bool SR, bool NTL, bool NTS, bool PF, bool TR>
__device__ __forceinline__ void mfma_fold_heads(const KernelArgs& a, int lane, float* wxT, int h0, int h1, int k,
                                                int r0, int b, int l, const char* src_state, char* dst_state,
                                                const float* src_scale, float* dst_scale, const char* x_slot,
                                                const char* B_slot, const float* dt_slot, const float* A,
                                                uint32_t key0, uint32_t key1) {
  constexpr int DIM = 64, DSTATE = 128;
  constexpr int IB = Fmt<IT>::bytes;
  constexpr int64_t kTile = static_cast<int64_t>(DIM) * DSTATE;   // bytes (one-byte state)
  constexpr int NKS = KMAX / 4;                                     // k-steps of 4 tokens
  constexpr int RBB = 16 * DSTATE;                                  // bytes per row block
  constexpr int XCH = DIM / 8;
  constexpr int XREP = (KMAX * XCH + 63) / 64;
  const int G = a.H / a.hpg;
  const int j = lane & 15, q = lane >> 4;
  const uint32_t loff = static_cast<uint32_t>(j * DSTATE + 16 * q);
  const int e_lane = (r0 + lane) % a.R;
  const int nks = (k + 3) >> 2;
  const int k4 = nks * 4;

  float* amL = wxT + KMAX * kWxStride;   // A operands of k-steps >= 1
  // TR: the row blocks are loaded and stored as two coalesced 1 KiB halves
  // (lane L: row L / 8 of the half, bytes 16 (L % 8) ..), and pass through a
  // 2 KiB LDS buffer between that layout and the accumulator layout.  On
  // MI355X a copy in the accumulator layout (16 rows x 64 bytes per
  // instruction) streamed at 4.7 TB/s against 6.1 TB/s coalesced.
  char* tT = reinterpret_cast<char*>(amL + (KMAX / 4 - 1) * 64 * 8);
  const uint32_t voff = TR ? static_cast<uint32_t>(lane) * 16 : loff;   // per-lane offset of a row-block access
  constexpr int HALF2 = TR ? 1024 : 64;                                  // offset of the second access
  for (int g = h0 / a.hpg; g * a.hpg < h1; ++g) {
    // A operands: lane L supplies B_t[col] for token t = 4 ks + L / 16 and
    // column col(i / 4, bb, i % 4), i = L % 16; zero for tokens at or past k.
    // k-step 0 in registers, the others in this wavefront's LDS.
    float Am[8];
    {
      float av[NKS][8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int t = 4 * ks + q;
        const int e = ring_entry(r0, t < k ? t : 0, a.R);
        const char* row = B_slot + (static_cast<int64_t>(e) * G + g) * DSTATE * IB;
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          const int col = 64 * (bb >> 2) + 16 * (j >> 2) + 4 * (bb & 3) + (j & 3);
          const float v = load_elem<IT>(row + col * IB);
          av[ks][bb] = t < k ? v : 0.0f;
        }
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) Am[bb] = av[0][bb];
      if constexpr (NKS > 1) {
        wave_lds_fence();   // the previous group's reads of amL are done
#pragma unroll
        for (int ks = 1; ks < NKS; ++ks) {
          f32x4* dst = reinterpret_cast<f32x4*>(amL + ((ks - 1) * 64 + lane) * 8);
          dst[0] = f32x4{av[ks][0], av[ks][1], av[ks][2], av[ks][3]};
          dst[1] = f32x4{av[ks][4], av[ks][5], av[ks][6], av[ks][7]};
        }
      }
    }
    const int hb = max(h0, g * a.hpg);
    const int he = min(h1, (g + 1) * a.hpg);
    // By default each head requests its first two row blocks, x rows, dt and
    // A at its start.  With PF (a tuning variant, off: on MI355X it ran the
    // int8 workload 1% slower) the x rows, dt and A come one head ahead
    // (right after the previous head has staged its own) and the first two
    // row blocks during the previous head's last two.
    Chunk<IT> xraw[XREP];
    float A_n = 0.0f, dt_n = 0.0f;
    auto issue_small = [&](int hn) __attribute__((always_inline)) {
#pragma unroll
      for (int rep = 0; rep < XREP; ++rep) {
        const int idx = lane + 64 * rep;
        const int tj = min(idx / XCH, 63);
        const int ej = ring_entry(r0, tj < k ? tj : 0, a.R);
        xraw[rep] = load_chunk<IT>(x_slot + ((static_cast<int64_t>(ej) * a.H + hn) * DIM + (idx % XCH) * 8) * IB);
      }
      A_n = gload(A + hn);
      if (lane < k) dt_n = gload(dt_slot + static_cast<int64_t>(e_lane) * a.H + hn);
    };
    const uint32_t soff = static_cast<uint32_t>(j) * 4;   // this lane's row scale in a row block
    u32x4 s0[2], s1[2];
    float ssc[2];
    {
      const rsrc_t rs_src = make_rsrc(src_state + hb * kTile, static_cast<uint32_t>(kTile));
      const rsrc_t rs_ssc = make_rsrc(src_scale + static_cast<int64_t>(hb) * DIM, DIM * 4);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        s0[p] = bload16<NTL>(rs_src, voff, p * RBB);
        s1[p] = bload16<NTL>(rs_src, voff, p * RBB + HALF2);
        ssc[p] = bload_f32(rs_ssc, soff, p * 64);
      }
    }
    issue_small(hb);
    for (int h = hb; h < he; ++h) {
      const bool more = PF && h + 1 < he;
      if (!PF && h > hb) {
        const rsrc_t rs_src = make_rsrc(src_state + h * kTile, static_cast<uint32_t>(kTile));
        const rsrc_t rs_ssc = make_rsrc(src_scale + static_cast<int64_t>(h) * DIM, DIM * 4);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          s0[p] = bload16<NTL>(rs_src, voff, p * RBB);
          s1[p] = bload16<NTL>(rs_src, voff, p * RBB + HALF2);
          ssc[p] = bload_f32(rs_ssc, soff, p * 64);
        }
        issue_small(h);
      }
      // the head's tiles and row scales (and the next head's) as buffer
      // resources in scalar registers
      const rsrc_t rs_src = make_rsrc(src_state + h * kTile, static_cast<uint32_t>(kTile));
      const rsrc_t rs_dst = make_rsrc(dst_state + h * kTile, static_cast<uint32_t>(kTile));
      const rsrc_t rs_ssc = make_rsrc(src_scale + static_cast<int64_t>(h) * DIM, DIM * 4);
      const rsrc_t rs_dsc = make_rsrc(dst_scale + static_cast<int64_t>(h) * DIM, DIM * 4);
      const rsrc_t rs_nsrc = make_rsrc(src_state + (h + 1) * kTile, more ? static_cast<uint32_t>(kTile) : 0u);
      const rsrc_t rs_nssc = make_rsrc(src_scale + static_cast<int64_t>(h + 1) * DIM, more ? DIM * 4 : 0u);
      const float A_h = A_n;
      float dtj = 0.0f, aj = 1.0f;
      if (lane < k) {
        dtj = dt_n;
        aj = expf(dtj * A_h);
      }
      // suffix products over the tokens: D = prod a_j, w_j = dt_j prod_{u>j} a_u
      const float P = suffix_products(aj, lane, 16);
      float Pn = row_shl<1>(P);
      if (lane + 1 >= 16) Pn = 1.0f;
      const float w = dtj * Pn;
      const float D = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), 0));
      // stage w_t x_t[row] as [token][row]; tokens k .. k4-1 get -0 weights
      // (with A = +0 their products are -0, which leave every accumulator,
      // including the sign of a zero, unchanged)
      wave_lds_fence();
#pragma unroll
      for (int rep = 0; rep < XREP; ++rep) {
        const int idx = lane + 64 * rep;
        const int tj = min(idx / XCH, 63);
        const float wj = __shfl(w, tj);
        if (idx < k4 * XCH) {
          const int r8 = (idx % XCH) * 8;
          float xv[8];
          decode_chunk<IT>(xraw[rep], xv);
          f32x4 lo, hi;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            lo[u] = tj < k ? wj * xv[u] : -0.0f;
            hi[u] = tj < k ? wj * xv[4 + u] : -0.0f;
          }
          *reinterpret_cast<f32x4*>(wxT + wx_pos(tj, r8)) = lo;       // 8 rows stay contiguous
          *reinterpret_cast<f32x4*>(wxT + wx_pos(tj, r8) + 4) = hi;
        }
      }
      wave_lds_fence();
      if (more) issue_small(h + 1);   // xraw is free again

      // row blocks in pairs (slot 0 and slot 1 of the two in flight); the
      // pair loop stays rolled, which keeps register pressure down
#pragma unroll 1
      for (int rp = 0; rp < DIM / 16; rp += 2)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int rb = rp + sl;
        const float d0 = ssc[sl] * D;
        u32x4 m0 = s0[sl], m1 = s1[sl];
        if constexpr (TR) {
          // row-major halves in, the lane's two chunks of row j out
          *reinterpret_cast<u32x4*>(tT + tr_pos(lane >> 3, lane & 7)) = m0;
          *reinterpret_cast<u32x4*>(tT + tr_pos(8 + (lane >> 3), lane & 7)) = m1;
          m0 = *reinterpret_cast<const u32x4*>(tT + tr_pos(j, q));
          m1 = *reinterpret_cast<const u32x4*>(tT + tr_pos(j, q + 4));
        }
        f32x4 acc[8];
        acc[0] = decode4_scaled<ST>(m0.x, d0);
        acc[1] = decode4_scaled<ST>(m0.y, d0);
        acc[2] = decode4_scaled<ST>(m0.z, d0);
        acc[3] = decode4_scaled<ST>(m0.w, d0);
        acc[4] = decode4_scaled<ST>(m1.x, d0);
        acc[5] = decode4_scaled<ST>(m1.y, d0);
        acc[6] = decode4_scaled<ST>(m1.z, d0);
        acc[7] = decode4_scaled<ST>(m1.w, d0);
        // the slot's bytes are decoded: its registers take the block two ahead
        // (kept after the decode, so that no copy of the slot is needed)
        __builtin_amdgcn_sched_barrier(0);
        if (rb + 2 < DIM / 16) {
          s0[sl] = bload16<NTL>(rs_src, voff, (rb + 2) * RBB);
          s1[sl] = bload16<NTL>(rs_src, voff, (rb + 2) * RBB + HALF2);
          ssc[sl] = bload_f32(rs_ssc, soff, (rb + 2) * 64);
        } else if (more) {
          // the next head's row blocks 0 and 1
          s0[sl] = bload16<NTL>(rs_nsrc, voff, (rb + 2 - DIM / 16) * RBB);
          s1[sl] = bload16<NTL>(rs_nsrc, voff, (rb + 2 - DIM / 16) * RBB + HALF2);
          ssc[sl] = bload_f32(rs_nssc, soff, (rb + 2 - DIM / 16) * 64);
        }
        int kk = nks;
        asm volatile("" : "+s"(kk));
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          if (ks < kk) {
            const float bm = wxT[wx_pos(4 * ks + q, 16 * rb + j)];
            float am[8];
            if (ks == 0) {
#pragma unroll
              for (int bb = 0; bb < 8; ++bb) am[bb] = Am[bb];
            } else {
              const f32x4* src = reinterpret_cast<const f32x4*>(amL + ((ks > 0 ? ks - 1 : 0) * 64 + lane) * 8);
              const f32x4 lo = src[0], hi = src[1];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                am[u] = lo[u];
                am[4 + u] = hi[u];
              }
            }
#pragma unroll
            for (int bb = 0; bb < 8; ++bb) acc[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[bb], bm, acc[bb], 0, 0, 0);
          }
        }
        uint32_t out[8];
        float rs = 0.0f;
        encode_rowblock<ST, SR>(acc, 16 * rb + j, q, h, b, l, key0, key1, a.rounds, out, rs);
        u32x4 o0{out[0], out[1], out[2], out[3]}, o1{out[4], out[5], out[6], out[7]};
        if constexpr (TR) {
          // the lane's two chunks of row j in, row-major halves out
          *reinterpret_cast<u32x4*>(tT + tr_pos(j, q)) = o0;
          *reinterpret_cast<u32x4*>(tT + tr_pos(j, q + 4)) = o1;
          o0 = *reinterpret_cast<const u32x4*>(tT + tr_pos(lane >> 3, lane & 7));
          o1 = *reinterpret_cast<const u32x4*>(tT + tr_pos(8 + (lane >> 3), lane & 7));
        }
        bstore16<NTS>(rs_dst, voff, rb * RBB, o0);
        bstore16<NTS>(rs_dst, voff, rb * RBB + HALF2, o1);
        if (q == 0) bstore_f32(rs_dsc, soff, rb * 64, rs);
        // one row block at a time: interleaving the next block's decode and
        // MFMAs into this block's encode would hold two sets of accumulators
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// NCK = 1: the operation of the materialize page.  NCK > 1: up to NCK
// checkpoints per request from one read of each source tile -- checkpoint c
// writes the state after prefix_len[c][b] ring entries to slot
// dst_slots[c][l][b].  The fold runs once over the longest prefix; the
// tokens between consecutive checkpoint lengths form segments, and after each
// segment the running fp32 state is encoded and stored.  Weights are
// relative to the end of their segment: over segment [k', k''),
// S_k'' = (prod_{k'<=u<k''} a_u) S_k' + sum_{k'<=j<k''} dt_j (prod_{j<u<k''} a_u) x_j B_j^T.
template <int ST, int IT, int DIM, int DSTATE, int KMAX, bool SR, int NCK = 1, class Tune = DefaultTune>
__global__ void __launch_bounds__(kBlock, (waves_per_simd<Tune, KMAX, ST, IT, NCK>())) materialize_kernel(const KernelArgs a) {
  constexpr int TPR = DSTATE / 8;                 // lanes per state row
  constexpr int RPP = 64 / TPR;                   // rows per pass of a wavefront
  constexpr int NPASS = (DIM + RPP - 1) / RPP;    // passes per tile
  constexpr bool kFull = (NPASS * RPP == DIM);
  constexpr int SB = Fmt<ST>::bytes;
  constexpr int IB = Fmt<IT>::bytes;
  constexpr int CW = 2 * SB;                      // dwords per 8-element chunk
  constexpr int PD0 = Tune::kInflightDwords / CW > 2 ? Tune::kInflightDwords / CW : 2;
  constexpr int PD = NPASS < PD0 ? NPASS : PD0;  // passes in flight
  constexpr bool NTL = Tune::kNtLoad, NTS = Tune::kNtStore;
  static_assert(NPASS % PD == 0, "passes must split into prefetch groups");
  constexpr int64_t kTile = static_cast<int64_t>(DIM) * DSTATE;
  constexpr int XCH = DIM / 8;                    // 8-row chunks of one x row
  constexpr bool Q = kOneByte<ST>;
  constexpr bool MULTI = NCK > 1;
  static_assert(DSTATE % 8 == 0 && 64 % TPR == 0 && DIM % 8 == 0, "unsupported tile shape");
  static_assert(!Q || TPR == 16, "one-byte state needs 16 lanes per row");
  static_assert(KMAX % 4 == 0 && KMAX <= 16, "KMAX");
  static_assert(NCK >= 1 && NCK <= 4, "NCK");

  constexpr bool MF = kMfmaFold<Tune, ST, NCK>;
  static_assert(!MF || (DIM == 64 && DSTATE == 128), "matrix-core fold: 64 x 128 tiles");
  constexpr bool TR = Tune::kMfmaTranspose && KMAX <= 8;   // (16-token instances: LDS budget)
  __shared__ __attribute__((aligned(16))) float lds_wx[kWaves][MF ? kMfmaLds<KMAX, TR> : DIM * KMAX];
  constexpr int KREG = kBRegs<KMAX>;   // B rows of tokens below KREG in registers
  constexpr int KLDS = KMAX - KREG;     // the others in this wavefront's LDS, [token - KREG][column]
  __shared__ __attribute__((aligned(16))) float lds_B[kWaves][(!MF && KLDS > 0) ? KLDS * DSTATE : 4];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
  float* wx = lds_wx[wave];
  float* bl = lds_B[wave];
  const int cc = lane % TPR;
  const int rr = lane / TPR;
  constexpr int PS = RPP * DSTATE * SB;  // bytes between passes of a tile
  const uint32_t lane_off = static_cast<uint32_t>((rr * DSTATE + cc * 8) * SB);  // this lane's chunk in a pass

  const int n_active = uniform(count_active(a.active, a.B, lane));
  const int64_t items = static_cast<int64_t>(n_active) * a.L * a.H;
  if (items == 0) return;

  // Items of this wavefront: one contiguous, balanced range (kChunkItems = 0),
  // or chunks of up to kChunkItems items dealt round-robin over the
  // wavefronts, so that requests of different cost (zero or long prefixes,
  // padded layers) spread evenly.  A call with fewer than kChunkItems items
  // per wavefront uses chunks of ceil(items / wavefronts): one per wavefront.
  const int64_t tw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  constexpr int64_t kC = Tune::kChunkItems;
  const int64_t csz = kC == 0 ? 0 : min(kC, (items + tw - 1) / tw);
  int64_t chunk = gw, it, end;
  // When some wavefront deals several chunks, each wavefront first tests its
  // next 64 chunks in parallel (live_chunks) and walks only the live ones, so
  // skipped (request, layer) pairs cost no round trips of their own: a call
  // whose listed requests are all padded costs about one near-empty launch.
  const bool filt = kC > 0 && (items + csz - 1) / csz > tw;
  int64_t qb = 0;       // position in this wavefront's chunk sequence of lane 0 of the batch
  uint64_t live = 0;    // live chunks of the batch not yet taken
  if constexpr (kC == 0) {
    const int64_t per = items / tw, rem = items % tw;
    it = gw * per + (gw < rem ? gw : rem);
    end = it + per + (gw < rem ? 1 : 0);
  } else if (filt) {
    it = end = 0;  // the first chunk comes from the filter
  } else {
    it = chunk * csz;
    end = min(items, it + csz);
  }

  uint32_t key0 = 0, key1 = 0;
  if constexpr (SR) {
    const uint64_t sd = static_cast<uint64_t>(*a.rand_seed);
    key0 = static_cast<uint32_t>(uniform(static_cast<int>(sd & 0xFFFFFFFFu)));
    key1 = static_cast<uint32_t>(uniform(static_cast<int>(sd >> 32)));
  }
  const int G = a.H / a.hpg;
  const int64_t LB = static_cast<int64_t>(a.L) * a.B;

  for (;;) {
    if (it >= end) {
      if constexpr (kC == 0) break;
      if (filt) {
        while (live == 0) {
          if ((gw + qb * tw) * csz >= items) break;
          live = live_chunks<NCK>(a, gw, tw, qb, csz, items, lane);
          if (live == 0) qb += 64;
        }
        if (live == 0) break;
        chunk = gw + (qb + __builtin_ctzll(live)) * tw;
        live &= live - 1;
        if (live == 0) qb += 64;
      } else {
        chunk += tw;
      }
      it = chunk * csz;
      if (it >= items) break;
      end = min(items, it + csz);
    }
    // One (request, layer): heads [h0, h1) of it belong to this wavefront.
    const int64_t il = it / a.H;
    const int h0 = static_cast<int>(it - il * a.H);
    const int h1 = static_cast<int>(min(static_cast<int64_t>(a.H), h0 + (end - it)));
    it += h1 - h0;

    const int i = static_cast<int>(il / a.L);
    const int l = static_cast<int>(il - static_cast<int64_t>(i) * a.L);
    // Metadata in two round trips: everything indexed by the layer together
    // with the active entry, then everything indexed by the request.
    const int b_raw = gload(a.active + i);
    const int64_t sbase_raw = gload(a.state_ptrs + l), sstride_raw = gload(a.state_strides + l);
    const int64_t x_raw = gload(a.x_ptrs + l), xs_raw = gload(a.x_strides + l);
    const int64_t B_raw = gload(a.B_ptrs + l), Bs_raw = gload(a.B_strides + l);
    const int64_t dt_raw = gload(a.dt_ptrs + l), dts_raw = gload(a.dt_strides + l);
    const int64_t A_raw = gload(a.A_ptrs + l);
    int64_t c_raw = 0, cs_raw = 0;
    if constexpr (Q) {
      c_raw = gload(a.scale_ptrs + l);
      cs_raw = gload(a.scale_strides + l);
    }
    const int b = uniform(b_raw);
    const int64_t lb = static_cast<int64_t>(l) * a.B + b;
    const int s_raw = gload(a.src_slots + lb);
    const int r_raw = gload(a.ring_start + b);
    int d_raw[NCK], k_raw[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const int cl = (c < a.ncp) ? c : 0;   // checkpoints past ncp read entry 0 and are then ignored
      d_raw[c] = gload(a.dst_slots + cl * LB + lb);
      k_raw[c] = gload(a.prefix_len + static_cast<int64_t>(cl) * a.B + b);
    }
    const int s = uniform(s_raw);
    // kc/dc: checkpoints in ascending prefix order (one entry when NCK = 1).
    int kc[NCK], dc[NCK];
    if constexpr (!MULTI) {
      const int d = uniform(d_raw[0]);
      if (s == a.pad || d == a.pad || s < 0 || d < 0) continue;  // pad slot: skipped
      kc[0] = min(max(uniform(k_raw[0]), 0), a.W);
      dc[0] = d;
    } else {
      if (s == a.pad || s < 0) continue;  // pad source: every checkpoint skipped
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        int d = a.pad, kk = -1;
        if (c < a.ncp) {
          d = uniform(d_raw[c]);
          kk = min(max(uniform(k_raw[c]), 0), a.W);
        }
        const bool on = d != a.pad && d >= 0;  // a pad destination skips this checkpoint only
        kc[c] = on ? kk : -1;
        dc[c] = on ? d : 0;
      }
      sort_checkpoints<NCK>(kc, dc);
      if (kc[NCK - 1] < 0) continue;
    }
    const int k = kc[NCK - 1];  // longest prefix
    int r0 = uniform(r_raw) % a.R;
    if (r0 < 0) r0 += a.R;

    const int64_t sbase = uniform64(sbase_raw);
    const int64_t sstride = uniform64(sstride_raw);
    const char* src_state = reinterpret_cast<const char*>(sbase) + static_cast<int64_t>(s) * sstride * SB;
    char* dst_state[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c)
      dst_state[c] = reinterpret_cast<char*>(sbase) + static_cast<int64_t>(dc[c]) * sstride * SB;
    const float* src_scale = nullptr;
    float* dst_scale[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) dst_scale[c] = nullptr;
    if constexpr (Q) {
      const int64_t cbase = uniform64(c_raw);
      const int64_t cstride = uniform64(cs_raw);
      src_scale = reinterpret_cast<const float*>(cbase) + static_cast<int64_t>(s) * cstride;
#pragma unroll
      for (int c = 0; c < NCK; ++c) dst_scale[c] = reinterpret_cast<float*>(cbase) + static_cast<int64_t>(dc[c]) * cstride;
    }

    if (k == 0) {
      // Zero prefix: exact byte copy of the heads' tiles (and row scales) to
      // every live destination.  The tiles of heads h0 .. h1-1 of one slot
      // are one contiguous range, copied as 1 KiB blocks, 16 bytes per lane
      // (one-byte tiles streamed 8 bytes per lane, in their fold layout,
      // copied at 5.3 TB/s on MI355X against 6.2 TB/s for 16 bytes per lane),
      // four blocks in flight; the row scales are one float per lane.
      constexpr int64_t kTileBytes = kTile * SB;
      if constexpr (kTileBytes % 1024 == 0) {
        constexpr int CPD = 4;
        const int64_t nblk = (h1 - h0) * (kTileBytes / 1024);
        const uint32_t boff = static_cast<uint32_t>(lane) * 16;
        const char* sblk = src_state + h0 * kTileBytes;
#pragma unroll 1
        for (int64_t i0 = 0; i0 < nblk; i0 += CPD) {
          u32x4 c[CPD];
#pragma unroll
          for (int q = 0; q < CPD; ++q)
            if (i0 + q < nblk) c[q] = ld<NTL, u32x4>(at(sblk + (i0 + q) * 1024, boff));
#pragma unroll
          for (int q = 0; q < CPD; ++q) {
            if (i0 + q < nblk) {
#pragma unroll
              for (int ck = 0; ck < NCK; ++ck)
                if (kc[ck] == 0) st<NTS>(at(dst_state[ck] + h0 * kTileBytes + (i0 + q) * 1024, boff), c[q]);
            }
          }
        }
      } else {
        for (int h = h0; h < h1; ++h) {
          const char* src_tile = src_state + h * kTileBytes;
#pragma unroll 1
          for (int p0 = 0; p0 < NPASS; p0 += PD) {
            Chunk<ST> c[PD];
#pragma unroll
            for (int q = 0; q < PD; ++q) {
              const int r = rr + (p0 + q) * RPP;
              if (kFull || r < DIM) c[q] = load_chunk<ST, NTL>(at(src_tile + (p0 + q) * PS, lane_off));
            }
#pragma unroll
            for (int q = 0; q < PD; ++q) {
              const int r = rr + (p0 + q) * RPP;
              if (kFull || r < DIM) {
#pragma unroll
                for (int ck = 0; ck < NCK; ++ck)
                  if (kc[ck] == 0) store_chunk<ST, NTS>(at(dst_state[ck] + h * kTileBytes + (p0 + q) * PS, lane_off), c[q]);
              }
            }
          }
        }
      }
      if constexpr (Q) {
        const int nsc = (h1 - h0) * DIM;
        for (int i = lane; i < nsc; i += 64) {
          const float sc = gload(src_scale + h0 * DIM + i);
#pragma unroll
          for (int ck = 0; ck < NCK; ++ck)
            if (kc[ck] == 0) gstore(dst_scale[ck] + h0 * DIM + i, sc);
        }
      }
      continue;
    }

    const char* x_slot = reinterpret_cast<const char*>(uniform64(x_raw)) +
                         static_cast<int64_t>(s) * uniform64(xs_raw) * IB;
    const char* B_slot = reinterpret_cast<const char*>(uniform64(B_raw)) +
                         static_cast<int64_t>(s) * uniform64(Bs_raw) * IB;
    const float* dt_slot = reinterpret_cast<const float*>(uniform64(dt_raw)) +
                           static_cast<int64_t>(s) * uniform64(dts_raw);
    const float* A = reinterpret_cast<const float*>(uniform64(A_raw));
    if constexpr (MF) {
      mfma_fold_heads<ST, IT, KMAX, SR, NTL, NTS, Tune::kMfmaPrefetch, TR>(a, lane, wx, h0, h1, k, r0, b, l, src_state, dst_state[0],
                                                  src_scale, dst_scale[0], x_slot, B_slot, dt_slot, A, key0, key1);
      continue;
    }
    const int e_lane = (r0 + lane) % a.R;  // ring entry of token `lane`
    // End of the segment that holds token `lane` (the shortest checkpoint
    // prefix above it); lanes at or past k hold no token.
    int seg_end = 16;
    if constexpr (MULTI) {
      if (lane < k) {
        seg_end = k;
#pragma unroll
        for (int c = 0; c < NCK; ++c)
          if (kc[c] > lane && kc[c] < seg_end) seg_end = kc[c];
      }
    }

    for (int g = h0 / a.hpg; g * a.hpg < h1; ++g) {
      // B_j for this lane's 8 columns, shared by the heads of group g: tokens
      // below KREG in registers, the others in the wavefront's LDS (written by
      // the lanes of row 0 of each pass).  All KMAX rows are requested at once
      // (tokens past k re-read entry r0 and are then zeroed), so the group
      // costs one round trip, not k.
      // int8 state with fp16 x/B and windows of up to 8 (single checkpoint):
      // the register rows stay packed fp16 pairs (word q holds columns 2q,
      // 2q+1) and the fold multiplies them with v_fma_mix_f32 (fp16 operand
      // converted exactly, one fp32 rounding: the same result as fmaf on the
      // decoded value).  That frees 32 registers for a fifth wave per SIMD.
      constexpr bool kMix = kMixB<ST, IT, KMAX, NCK>;
      float Bv[kMix ? 1 : KREG][8];
      uint32_t Bh[kMix ? KREG : 1][4];
      {
        Chunk<IT> braw[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          const int e = ring_entry(r0, j < k ? j : 0, a.R);
          braw[j] = load_chunk<IT>(B_slot + ((static_cast<int64_t>(e) * G + g) * DSTATE + cc * 8) * IB);
        }
        if constexpr (KLDS > 0) wave_lds_fence();  // the previous group's reads of bl are done
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          float v[8];
          decode_chunk<IT>(braw[j], v);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = (j < k) ? v[q] : 0.0f;
          if (j < KREG) {
            if constexpr (kMix) {
#pragma unroll
              for (int q = 0; q < 4; ++q) Bh[j < KREG ? j : 0][q] = (j < k) ? braw[j].w[q] : 0u;
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) Bv[j < KREG ? j : 0][q] = v[q];
            }
          } else if (rr == 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) bl[(j >= KREG ? j - KREG : 0) * DSTATE + cc * 8 + q] = v[q];
          }
        }
      }
      // B_j[c] of this lane's columns (j and c are compile-time after unrolling).
      auto Bat = [&](int j, int c) -> float {
        if (j >= KREG) return bl[(j >= KREG ? j - KREG : 0) * DSTATE + cc * 8 + c];
        if constexpr (kMix) {
          const uint32_t w = Bh[j < KREG ? j : 0][c >> 1];
          return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>((c & 1) ? (w >> 16) : (w & 0xFFFFu))));
        } else {
          return Bv[j < KREG ? j : 0][c];
        }
      };
      const int hb = max(h0, g * a.hpg);
      const int he = min(h1, (g + 1) * a.hpg);
      for (int h = hb; h < he; ++h) {
        const char* src_tile = src_state + h * kTile * SB;
        const float* src_sc = Q ? src_scale + static_cast<int64_t>(h) * DIM : nullptr;

        // Issue the first passes of the state stream before the ring work.
        Chunk<ST> buf[PD];
        float sbuf[PD];
#pragma unroll
        for (int p = 0; p < PD; ++p) {
          const int r = rr + p * RPP;
          if (kFull || r < DIM) {
            buf[p] = load_chunk<ST, NTL>(at(src_tile + p * PS, lane_off));
            if constexpr (Q) sbuf[p] = gload(src_sc + r);
          }
        }

        // Decay scan: lane j < k holds a_j; suffix products within each
        // segment give the segment decays and the weights w_j.
        // The head's x rows are requested together with dt and A (one round
        // trip): lane takes token j = idx / XCH, rows r8 .. r8+7.  Tokens past
        // k re-read token 0's entry; their values are never used.
        constexpr int XREP = (KMAX * XCH + 63) / 64;
        Chunk<IT> xraw[XREP];
#pragma unroll
        for (int rep = 0; rep < XREP; ++rep) {
          const int idx = lane + 64 * rep;
          const int j = min(idx / XCH, 63);
          const int ej = ring_entry(r0, j < k ? j : 0, a.R);
          xraw[rep] = load_chunk<IT>(x_slot + ((static_cast<int64_t>(ej) * a.H + h) * DIM + (idx % XCH) * 8) * IB);
        }
        const float A_h = gload(A + h);
        float dtj = 0.0f, aj = 1.0f;
        if (lane < k) {
          dtj = gload(dt_slot + static_cast<int64_t>(e_lane) * a.H + h);
          aj = expf(dtj * A_h);
        }
        const float P = suffix_products(aj, lane, seg_end);  // over lanes j .. seg_end-1
        float Pn = row_shl<1>(P);
        if (lane + 1 >= seg_end) Pn = 1.0f;
        const float w = dtj * Pn;
        // Decay of the segment that ends at kc[c] (1 when no token is new).
        float Dseg[NCK];
        {
          int prev = 0;
#pragma unroll
          for (int c = 0; c < NCK; ++c) {
            if (kc[c] > prev) {
              Dseg[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), prev));
              prev = kc[c];
            } else {
              Dseg[c] = 1.0f;
            }
          }
        }

        // Stage w_j * x_j[r] into this wave's LDS as [row][token].  Tokens
        // k..ceil4(k)-1 pad the last block of four (the single-checkpoint fold
        // takes blocks of two, the multi-checkpoint fold blocks of four) with
        // -0.0: with B_j = +0 their fused multiply-add adds -0, which leaves
        // every accumulator unchanged (including the sign of a zero).
        const int k4 = (k + 3) & ~3;
        wave_lds_fence();
#pragma unroll
        for (int rep = 0; rep < XREP; ++rep) {
          const int idx = lane + 64 * rep;
          const int j = min(idx / XCH, 63);
          const float wj = __shfl(w, j);
          if (idx < k4 * XCH) {
            const int r8 = (idx % XCH) * 8;
            if (j < k) {
              float xv[8];
              decode_chunk<IT>(xraw[rep], xv);
#pragma unroll
              for (int q = 0; q < 8; ++q) wx[(r8 + q) * KMAX + j] = wj * xv[q];
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) wx[(r8 + q) * KMAX + j] = -0.0f;
            }
          }
        }
        wave_lds_fence();

        // Stream the tile: decode, fold the prefix, encode, store.  Passes go
        // in groups of PD; while a group is folded the next group is in flight.
        // (In the gfx950 code the buffers are copied at the loop's back edge,
        // and the copies wait for every outstanding memory operation, so about
        // one pass stays in flight.  Reloading each buffer only after it is
        // consumed, with exact waits, kept two in flight but ran the full
        // batch 2% slower on MI355X: sixteen wavefronts per CU saturate HBM
        // either way, and the extra outstanding traffic cost efficiency.)
#pragma unroll 1
        for (int p0 = 0; p0 < NPASS; p0 += PD) {
#pragma unroll
          for (int q = 0; q < PD; ++q) {
            const int p = p0 + q;
            const Chunk<ST> cur = buf[q];
            const float cur_sc = Q ? sbuf[q] : 1.0f;
            if (p + PD < NPASS) {
              const int rn = rr + (p + PD) * RPP;
              if (kFull || rn < DIM) {
                buf[q] = load_chunk<ST, NTL>(at(src_tile + (p + PD) * PS, lane_off));
                if constexpr (Q) sbuf[q] = gload(src_sc + rn);
              }
            }
            const int r = rr + p * RPP;
            if (kFull || r < DIM) {
              const float* wrow = wx + r * KMAX;
              uint32_t u[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
              float acc[8];
              decode_chunk<ST>(cur, acc);
              if constexpr (!MULTI) {
                const float d0 = Q ? cur_sc * Dseg[0] : Dseg[0];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] *= d0;
                // An opaque scalar copy of k per pass: each block test is then
                // one scalar compare and branch (shared with other uses of
                // j < k, the tests become lane masks whose branches cost two
                // vector instructions each).
                int kk = k;
                asm volatile("" : "+s"(kk));
                // Packed fp16 rows: an opaque copy per pass keeps their
                // conversion inside v_fma_mix_f32 (hoisted out of the pass
                // loop, the converted rows would take the registers back).
                if constexpr (kMix) {
#pragma unroll
                  for (int j = 0; j < KREG; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(Bh[j][q]));
                }
#pragma unroll
                for (int jb = 0; jb < KMAX / 2; ++jb) {
                  if (jb * 2 < kk) {
                    const float2 w2 = *reinterpret_cast<const float2*>(wrow + jb * 2);
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                      acc[c] = fmaf(w2.x, Bat(jb * 2 + 0, c), acc[c]);
                      acc[c] = fmaf(w2.y, Bat(jb * 2 + 1, c), acc[c]);
                    }
                  }
                }
                if constexpr (SR) sr_words(u, r, cc * 8, DSTATE, h, b, l, key0, key1, a.rounds);
                float rs = 0.0f;
                const Chunk<ST> out = encode_chunk<ST, SR>(acc, u, rs);
                store_chunk<ST, NTS>(at(dst_state[0] + h * kTile * SB + p * PS, lane_off), out);
                if constexpr (Q) {
                  if (cc == 0) gstore(dst_scale[0] + static_cast<int64_t>(h) * DIM + r, rs);
                }
              } else {
                // One set of random words per element serves every checkpoint,
                // as separate calls would draw the same ones.
                if constexpr (SR) sr_words(u, r, cc * 8, DSTATE, h, b, l, key0, key1, a.rounds);
                // Zero-prefix checkpoints take the source bytes as they are.
#pragma unroll
                for (int ck = 0; ck < NCK; ++ck) {
                  if (kc[ck] == 0) {
                    store_chunk<ST, NTS>(at(dst_state[ck] + h * kTile * SB + p * PS, lane_off), cur);
                    if constexpr (Q) {
                      if (cc == 0) gstore(dst_scale[ck] + static_cast<int64_t>(h) * DIM + r, cur_sc);
                    }
                  }
                }
                Chunk<ST> out{};
                float rs = 0.0f;
                int prev = 0;
#pragma unroll
                for (int ck = 0; ck < NCK; ++ck) {
                  const int kend = kc[ck];
                  if (kend > prev) {
                    // Segment [prev, kend): decay, then its tokens.
                    const float dm = (prev == 0 && Q) ? cur_sc * Dseg[ck] : Dseg[ck];
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[c] *= dm;
#pragma unroll
                    for (int jb = 0; jb < KMAX / 4; ++jb) {
                      const int t0 = jb * 4;
                      if (t0 < kend && t0 + 4 > prev) {
                        const float4 w4 = *reinterpret_cast<const float4*>(wrow + t0);
                        if (t0 >= prev && (t0 + 4 <= kend || kend == k)) {
                          // whole block inside (tokens past k carry -0 weights)
#pragma unroll
                          for (int c = 0; c < 8; ++c) {
                            acc[c] = fmaf(w4.x, Bat(t0 + 0, c), acc[c]);
                            acc[c] = fmaf(w4.y, Bat(t0 + 1, c), acc[c]);
                            acc[c] = fmaf(w4.z, Bat(t0 + 2, c), acc[c]);
                            acc[c] = fmaf(w4.w, Bat(t0 + 3, c), acc[c]);
                          }
                        } else {
                          // block cut by a segment boundary: only its own tokens
                          const float wt[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                          for (int t = 0; t < 4; ++t) {
                            if (t0 + t >= prev && t0 + t < kend) {
#pragma unroll
                              for (int c = 0; c < 8; ++c) acc[c] = fmaf(wt[t], Bat(t0 + t, c), acc[c]);
                            }
                          }
                        }
                      }
                    }
                    out = encode_chunk<ST, SR>(acc, u, rs);
                    prev = kend;
                  }
                  if (kend > 0) {
                    store_chunk<ST, NTS>(at(dst_state[ck] + h * kTile * SB + p * PS, lane_off), out);
                    if constexpr (Q) {
                      if (cc == 0) gstore(dst_scale[ck] + static_cast<int64_t>(h) * DIM + r, rs);
                    }
                  }
                }
              }
            }
          }
        }
      }
    }
  }
}

// Test hook: the same encode step on caller-given fp32 rows.
template <int ST, int DSTATE, bool SR>
__global__ void __launch_bounds__(kBlock) encode_rows_kernel(const float* rows, const int32_t* coords,
                                                            const int64_t* rand_seed, char* out_codes,
                                                            float* out_scales, int n, int rounds) {
  constexpr int TPR = DSTATE / 8;
  constexpr int RPW = 64 / TPR;
  constexpr int SB = Fmt<ST>::bytes;
  const int lane = threadIdx.x & 63;
  const int64_t gwave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t row = gwave * RPW + lane / TPR;
  const int cc = lane % TPR;
  const bool ok = row < n;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = ok ? gload(rows + row * DSTATE + cc * 8 + q) : 0.0f;
  uint32_t u[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if constexpr (SR) {
    const uint64_t s = static_cast<uint64_t>(*rand_seed);
    const int l = ok ? coords[row * 4 + 0] : 0;
    const int b = ok ? coords[row * 4 + 1] : 0;
    const int h = ok ? coords[row * 4 + 2] : 0;
    const int r = ok ? coords[row * 4 + 3] : 0;
    sr_words(u, r, cc * 8, DSTATE, h, b, l, static_cast<uint32_t>(s), static_cast<uint32_t>(s >> 32), rounds);
  }
  float rs = 0.0f;
  const Chunk<ST> c = encode_chunk<ST, SR>(acc, u, rs);
  if (ok) {
    store_chunk<ST>(out_codes + (row * DSTATE + cc * 8) * SB, c);
    if constexpr (kOneByte<ST>) {
      if (cc == 0) gstore(out_scales + row, rs);
    }
  }
}

// Test hook: scale and inverse scale of row_quant<QMAX> for given row maxima
// (rowmax[i] >= 0), one per lane, in wavefronts of 64 consecutive rows.
template <int QMAX>
__global__ void __launch_bounds__(kBlock) row_scales_kernel(const float* rowmax, float* scale, float* inv,
                                                            int32_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const float m = (i < n) ? gload(rowmax + i) : 1.0f;
  float s, q;
  row_quant<QMAX>(m, s, q);
  if (i < n) {
    gstore(scale + i, s);
    gstore(inv + i, q);
  }
}

// Kernel registry entries, one table per state dtype (one translation unit each).
struct KernelEntry {
  int st, it, dim, dstate, kmax, sr, nck;  // nck: checkpoints per request the instance handles (max)
  const void* fn;
  const char* name;
};

struct EncodeEntry {
  int st, dstate, sr;
  const void* fn;
  const char* name;
};

}  // namespace rssm
