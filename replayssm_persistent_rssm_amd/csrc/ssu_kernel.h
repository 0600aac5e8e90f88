// ssu_kernel.h -- persistent gfx950 kernel for the ReplaySSM decode step
// (one layer per launch).
//
// The step is the one the flashinfer materialize page (Summary) and the pull
// request "Replayssm prefix materialize" (Description) build on: a kept
// checkpoint plus its replay ring stands for the current state, and decode
// appends to the ring instead of rewriting the state.  For request b with
// slot s (its checkpoint and its ring), n pending ring entries from
// ring_start and T new tokens:
//   dt_t = softplus(dt_raw_t + dt_bias), appended with x_t and B_t at ring
//          entry (ring_start + n + t) mod R;
//   y_t  = C_t . S_{n+t+1} + D x_t, times silu(z_t),
// where S_m is the checkpoint advanced by the first m pending + new tokens
// (S <- exp(dt A) S + dt x B^T).  Unrolled as in the materialize kernel:
//   S_m    = Dec_m S_0 + sum_{j<m} w_j^m x_j B_j^T,
//   Dec_m  = prod_{j<m} a_j,   w_j^m = dt_j prod_{j<u<m} a_u,   a_j = exp(dt_j A)
//   y_t[r] = Dec_m (S_0[r,:] . C_t) + sum_{j<m} w_j^m (B_j . C_t) x_j[r] + D x_t[r],  m = n + t + 1,
// so the checkpoint is streamed once, read-only, with T dot products per row,
// and the ring enters through (n + T) x T scalars per head.
//
// Design (MI355X, wave64).  Work item = one (request, head) 64 x 128 tile;
// chunks of up to 16 consecutive items (same request, consecutive heads)
// are dealt round-robin over the wavefronts.  Per item:
//  * lane j < n + T holds token j's dt and decay; one suffix-product scan per
//    new token gives Dec and the weights;
//  * per (request, group), kept across the heads of the group: C_t for the
//    lane's 8 columns in registers, and B_j . C_t for every (j, t) in LDS
//    (16 lanes per dot product, a 16-lane DPP sum);
//  * with lane = state row, the ring terms and the skip are summed and the
//    new tokens' x and dt are appended to the ring (B once per group, by the
//    wavefront that holds the group's first head);
//  * the checkpoint tile streams through registers, 16 lanes per row and 8
//    columns per lane, two passes of 4 rows in flight; each row is dotted
//    with every C_t, the sums pass through LDS to lane = row, and the outputs
//    are finished and gated.
// The ring entries written are not the pending entries read (n + T <= R), so
// wavefronts of one request never race.  Instances cover up to TMAX new
// tokens; for T < TMAX the unused token slots repeat token 0 and their
// results are dropped.
#pragma once

#include "rssm_kernel.h"

namespace rssm {

struct SsuArgs {
  const char* state;     // [slots][H][64][128] state dtype, slot stride state_stride
  char* x_ring;          // [slots][R][H][64] input dtype
  char* B_ring;          // [slots][R][G][128] input dtype
  float* dt_ring;        // [slots][R][H]
  const float* A;        // [H]
  const float* D;        // [H] (any valid [H] array when has_D = 0)
  const float* dt_bias;  // [H] (any valid [H] array when has_bias = 0)
  const char* x_new;     // [B][T][H][64]
  const char* B_new;     // [B][T][G][128]
  const char* C_new;     // [B][T][G][128]
  const float* dt_new;   // [B][T][H]
  const char* z;         // [B][T][H][64] (x_new when has_z = 0)
  float* y;              // [B][T][H][64]
  const int32_t* slots;
  const int32_t* ring_start;
  const int32_t* num_buffered;
  int64_t state_stride, x_stride, B_stride, dt_stride;  // slot strides, elements
  int32_t B, H, hpg, R, T, pad, num_slots, dt_softplus;
  int32_t has_D, has_bias, has_z;
};

constexpr int kSsuDim = 64;
constexpr int kSsuDstate = 128;
constexpr int kSsuMaxTokens = 16;   // pending + new tokens one call replays

// Register budget: C costs 8 * TMAX registers per lane.
template <int TMAX> constexpr int kSsuWavesPerSimd = (TMAX > 4) ? 3 : 4;

// One element of a row in input storage, widened to fp32.
template <int IT>
__device__ __forceinline__ float input_to_float(uint32_t raw) {
  if constexpr (IT == kF32) return __uint_as_float(raw);
  else if constexpr (IT == kBF16) return __uint_as_float(raw << 16);
  else return f16_bits_to_float(raw);
}

template <int IT>
__device__ __forceinline__ uint32_t load_elem(const char* p) {
  if constexpr (Fmt<IT>::bytes == 4) return gload(reinterpret_cast<const uint32_t*>(p));
  else return gload(reinterpret_cast<const uint16_t*>(p));
}

template <int IT>
__device__ __forceinline__ void store_elem(char* p, uint32_t v) {
  if constexpr (Fmt<IT>::bytes == 4) gstore(reinterpret_cast<uint32_t*>(p), v);
  else gstore(reinterpret_cast<uint16_t*>(p), static_cast<uint16_t>(v));
}

// dt of a new token, softplus(raw + bias) (or the plain sum), in fp32.  The
// sum is kept as an unevaluated pair hi + lo (Knuth's TwoSum) so that the
// softplus sees the exact input: rounding the sum first would cost |v| u
// relative, several ulps of a small dt.  softplus(v) = log(1 + e^v) in the
// form that neither overflows nor loses small values, with
// e^(hi + lo) = e^hi (1 + lo) to first order (|lo| <= ulp(hi) / 2).
__device__ __forceinline__ float new_token_dt(float raw, float bias, int softplus) {
  const float hi = raw + bias;
  const float bb = hi - raw;
  const float lo = (raw - (hi - bb)) + (bias - bb);
  if (!softplus) return hi;
  if (hi > 0.0f) return hi + (lo + log1pf(expf(-hi) * (1.0f - lo)));
  return log1pf(expf(hi) * (1.0f + lo));
}

// Layout of one state row across lanes.  When the state and the inputs share
// a 16-bit float format, the lane keeps C in raw pairs and takes the dot
// products with the packed dot instructions (two products and an add per
// instruction, no conversion of the state): 8 lanes per row, 16 columns each.
// Otherwise the lane widens to fp32 and uses fused multiply-adds: 16 lanes
// per row, 8 columns each.  Every 16-byte load instruction covers contiguous
// bytes across the lanes of a row (measured on MI355X for a read-only tile
// stream: 5.8 TB/s, against 4.8 TB/s when each lane reads 32 contiguous
// bytes in two instructions), so a lane's columns are
//   packed:               cc*8 + [0, 8)  and  64 + cc*8 + [0, 8)
//   2-byte state, fp32:   cc*8 + [0, 8)
//   4-byte state:         cc*4 + [0, 4)  and  64 + cc*4 + [0, 4)
// (cc = lane's position in its row): the first 16 bytes of state at byte
// cc*16 of the row, the second (if any) half a row further.
template <int ST, int IT>
struct SsuRow {
  static constexpr bool kPacked = (ST == IT) && (ST == kBF16 || ST == kF16);
  static constexpr int kLanes = kPacked ? 8 : 16;     // lanes per row
  static constexpr int kChunks = kPacked ? 2 : 1;     // 8-column state chunks per lane
  static constexpr bool kSplit = Fmt<ST>::bytes == 4; // fp32 state: two 4-column halves
  static constexpr int kHalfBytes = 64 * Fmt<ST>::bytes;
};

// The lane's state chunks of one row; p = row start + cc * 16 bytes.
template <int ST, int IT, bool NT>
__device__ __forceinline__ void load_lane_state(const char* p, Chunk<ST> (&c)[SsuRow<ST, IT>::kChunks]) {
  using Row = SsuRow<ST, IT>;
  if constexpr (Row::kSplit) {
    const u32x4 a = ld<NT, u32x4>(p), b = ld<NT, u32x4>(p + Row::kHalfBytes);
    c[0].w[0] = a.x; c[0].w[1] = a.y; c[0].w[2] = a.z; c[0].w[3] = a.w;
    c[0].w[4] = b.x; c[0].w[5] = b.y; c[0].w[6] = b.z; c[0].w[7] = b.w;
  } else {
#pragma unroll
    for (int k = 0; k < Row::kChunks; ++k) c[k] = load_chunk<ST, NT>(p + k * Row::kHalfBytes);
  }
}

// Four consecutive input elements, widened to fp32.
template <int IT>
__device__ __forceinline__ void load4(const char* p, float* f) {
  if constexpr (IT == kF32) {
    const u32x4 a = ld<false, u32x4>(p);
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  } else {
    const u32x2 a = ld<false, u32x2>(p);
    const uint32_t w[2] = {a.x, a.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (IT == kBF16) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        f[2 * i] = f16_bits_to_float(w[i] & 0xFFFFu);
        f[2 * i + 1] = f16_bits_to_float(w[i] >> 16);
      }
    }
  }
}

// Sum over the 8 lanes of an aligned lane group, every lane receiving the total.
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8
  return v;
}

template <int LANES>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (LANES == 8) return row8_sum(v);
  else return row16_sum(v);
}

// Two products of 16-bit pairs added to an fp32 accumulator.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (DT == kBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
}

// The lane's columns of one C_t (or of one B_j), in the state row's column
// order: raw pairs (packed), or fp32.
template <int ST, int IT>
struct LaneVec {
  using Row = SsuRow<ST, IT>;
  uint32_t w[8];

  // row = the vector's element 0, cc = the lane's position in its row
  __device__ __forceinline__ void load(const char* row, int cc) {
    constexpr int IB = Fmt<IT>::bytes;
    if constexpr (Row::kPacked) {
      const Chunk<IT> c0 = load_chunk<IT>(row + cc * 8 * IB), c1 = load_chunk<IT>(row + (64 + cc * 8) * IB);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = c0.w[i];
        w[4 + i] = c1.w[i];
      }
    } else if constexpr (Row::kSplit) {
      float f[8];
      load4<IT>(row + cc * 4 * IB, f);
      load4<IT>(row + (64 + cc * 4) * IB, f + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = __float_as_uint(f[i]);
    } else {
      float f[8];
      load4<IT>(row + cc * 8 * IB, f);
      load4<IT>(row + (cc * 8 + 4) * IB, f + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = __float_as_uint(f[i]);
    }
  }
};

// Lane partial of (state row) . C: the lane's state chunks against its columns of C.
template <int ST, int IT>
__device__ __forceinline__ float lane_dot(const Chunk<ST> (&s)[SsuRow<ST, IT>::kChunks], const LaneVec<ST, IT>& c) {
  float v = 0.0f;
  if constexpr (SsuRow<ST, IT>::kPacked) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v = dot2<ST>(s[0].w[i], c.w[i], v);
#pragma unroll
    for (int i = 0; i < 4; ++i) v = dot2<ST>(s[1].w[i], c.w[4 + i], v);
  } else {
    float f[8];
    decode_chunk<ST>(s[0], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) v = fmaf(f[i], __uint_as_float(c.w[i]), v);
  }
  return v;
}

// Lane partial of B . C for two lane vectors of the input format.
template <int ST, int IT>
__device__ __forceinline__ float lane_dot_vv(const LaneVec<ST, IT>& x, const LaneVec<ST, IT>& c) {
  float v = 0.0f;
  if constexpr (SsuRow<ST, IT>::kPacked) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v = dot2<IT>(x.w[i], c.w[i], v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v = fmaf(__uint_as_float(x.w[i]), __uint_as_float(c.w[i]), v);
  }
  return v;
}

template <int ST, int IT, int TMAX, int PD = 2>
__global__ void __launch_bounds__(kBlock, kSsuWavesPerSimd<TMAX>) ssu_decode_kernel(const SsuArgs a) {
  using Row = SsuRow<ST, IT>;
  using CVec = LaneVec<ST, IT>;
  constexpr int DIM = kSsuDim, DS = kSsuDstate;
  constexpr int TPR = Row::kLanes;         // lanes per state row
  constexpr int NCH = Row::kChunks;        // 8-column chunks per lane
  constexpr int RPP = 64 / TPR;            // rows per pass
  constexpr int NPASS = DIM / RPP;         // passes per tile
  constexpr int SB = Fmt<ST>::bytes;
  constexpr int IB = Fmt<IT>::bytes;
  constexpr int PS = RPP * DS * SB;        // bytes between passes
  constexpr int64_t kTile = static_cast<int64_t>(DIM) * DS;
  constexpr int MM = kSsuMaxTokens;
  constexpr int NRING = MM - 1;            // pending entries: n <= 16 - T <= 15
  constexpr int DSTRIDE = DIM + RPP;       // row sums per token in LDS, padded against bank conflicts
  static_assert(TMAX >= 1 && TMAX <= 8, "TMAX");
  static_assert(NPASS % PD == 0, "passes");
  static_assert(TMAX <= TPR, "one lane of each row stores each token's row sum");

  __shared__ float lds_beta[kWaves][MM * TMAX];     // B_j . C_t at [j][t]
  __shared__ float lds_c[kWaves][MM * TMAX];        // w_j^(n+t+1) (B_j . C_t) at [j][t]
  __shared__ float lds_dot[kWaves][TMAX * DSTRIDE]; // S_0[r,:] . C_t at [t][r]

  const int lane = threadIdx.x & 63;
  const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
  const int cc = lane % TPR;
  const int rr = lane / TPR;
  const uint32_t lane_off = static_cast<uint32_t>(rr * DS * SB + cc * 16);
  const int T = a.T;
  const int H = a.H;
  const int G = H / a.hpg;
  const int64_t rowsT = static_cast<int64_t>(T);
  float* beta = lds_beta[wave];
  float* cw = lds_c[wave];
  float* dots = lds_dot[wave];

  const int64_t items = static_cast<int64_t>(a.B) * H;
  const int64_t tw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  constexpr int64_t kC = 16;
  const int64_t csz = min(kC, (items + tw - 1) / tw);
  int64_t chunk = gw;
  int64_t it = chunk * csz, end = min(items, it + csz);

  int cur_b = -1, cur_g = -1, s = 0, n = 0;
  int ent_l = 0;   // ring entry of token `lane` of the current request
  bool live = false;
  CVec Cv[TMAX];
  while (true) {
    if (it >= end) {
      chunk += tw;
      it = chunk * csz;
      if (it >= items) break;
      end = min(items, it + csz);
    }
    const int b = uniform(static_cast<int>(it / H));
    const int h = uniform(static_cast<int>(it - static_cast<int64_t>(b) * H));
    ++it;
    if (b != cur_b) {
      cur_b = b;
      cur_g = -1;
      const int s_raw = gload(a.slots + b), r_raw = gload(a.ring_start + b), n_raw = gload(a.num_buffered + b);
      s = uniform(s_raw);
      // guards against faults; the contract keeps every value in range
      live = s != a.pad && s >= 0 && s < a.num_slots;
      n = min(max(uniform(n_raw), 0), min(MM, a.R) - T);
      int r0 = uniform(r_raw) % a.R;
      if (r0 < 0) r0 += a.R;
      ent_l = (r0 + lane) % a.R;
    }
    if (!live) continue;
    const int g = h / a.hpg;
    const int m = n + T;

    // ---- requests of the item, issued together ----------------------------
    const char* tile = a.state + (static_cast<int64_t>(s) * a.state_stride + h * kTile) * SB;
    Chunk<ST> buf[PD][NCH];
#pragma unroll
    for (int p = 0; p < PD; ++p) load_lane_state<ST, IT, true>(at(tile + p * PS, lane_off), buf[p]);
    // token `lane`: dt from the ring (pending) or from the step's inputs (new)
    const bool pend_l = lane < n;
    const int tnew_l = min(max(lane - n, 0), T - 1);
    const float* dsrc = pend_l ? a.dt_ring + static_cast<int64_t>(s) * a.dt_stride + static_cast<int64_t>(ent_l) * H + h
                               : a.dt_new + (b * rowsT + tnew_l) * H + h;
    const float dt_raw = gload(dsrc);
    const float A_h = gload(a.A + h);
    const float bias_h = gload(a.dt_bias + h);
    const float D_h = gload(a.D + h);
    // row `lane` of x_j: pending entries from the ring (32-bit offsets from
    // the slot's ring base), new tokens raw; z for the gate
    char* xslot = a.x_ring + static_cast<int64_t>(s) * a.x_stride * IB;
    const uint32_t xrow = static_cast<uint32_t>((h * DIM + lane) * IB);
    const uint32_t xent = static_cast<uint32_t>(H * DIM * IB);
    uint32_t xraw[NRING];
#pragma unroll
    for (int j = 0; j < NRING; ++j) {
      const uint32_t e = static_cast<uint32_t>(__builtin_amdgcn_readlane(ent_l, j < n ? j : 0));
      xraw[j] = load_elem<IT>(at(xslot, e * xent + xrow));
    }
    uint32_t xn[TMAX], zr[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int tt = t < T ? t : 0;
      const int64_t yi = ((b * rowsT + tt) * H + h) * DIM + lane;
      xn[t] = load_elem<IT>(a.x_new + yi * IB);
      zr[t] = load_elem<IT>(a.z + yi * IB);
    }

    // ---- per (request, group): C_t in registers, B_j . C_t in LDS ----------
    if (g != cur_g) {
      cur_g = g;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        const int tt = t < T ? t : 0;
        Cv[t].load(a.C_new + (((b * rowsT + tt) * G + g) * DS) * IB, cc);
      }
      CVec bc[MM / RPP];
#pragma unroll
      for (int q = 0; q < MM / RPP; ++q) {
        const int j = rr + RPP * q;   // token of this lane group
        const int ej = __shfl(ent_l, j);
        const int tj = min(max(j - n, 0), T - 1);
        const char* src = (j < n) ? a.B_ring + (static_cast<int64_t>(s) * a.B_stride +
                                                (static_cast<int64_t>(ej) * G + g) * DS) * IB
                                  : a.B_new + (((b * rowsT + tj) * G + g) * DS) * IB;
        bc[q].load(src, cc);
      }
      wave_lds_fence();   // the previous group's readers are done with beta
#pragma unroll
      for (int q = 0; q < MM / RPP; ++q) {
        const int j = rr + RPP * q;
        float sel = 0.0f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          const float v = row_sum<TPR>(lane_dot_vv<ST, IT>(bc[q], Cv[t]));
          if (cc == t) sel = v;
        }
        if (cc < TMAX) beta[j * TMAX + cc] = (j < m) ? sel : 0.0f;
      }
    }

    // ---- decays and weights: one suffix-product scan per new token -------
    float dt_l = dt_raw;
    if (lane >= n && lane < m) dt_l = new_token_dt(dt_raw, a.has_bias ? bias_h : 0.0f, a.dt_softplus);
    if (lane >= m) dt_l = 0.0f;
    const float a_l = (lane < m) ? expf(dt_l * A_h) : 1.0f;
    float dec[TMAX], w[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int mt = n + t + 1;
      float P = (lane < mt) ? a_l : 1.0f;   // after the scan: prod over lanes lane .. min(mt, 16)-1
#pragma unroll
      for (int off = 1; off < MM; off <<= 1) {
        const float o = __shfl_down(P, off);
        if (lane + off < MM) P *= o;
      }
      float Pn = __shfl_down(P, 1);
      if (lane + 1 >= mt) Pn = 1.0f;
      dec[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), 0));
      w[t] = (lane < mt) ? dt_l * Pn : 0.0f;
    }
    wave_lds_fence();   // beta written; the previous item's readers of cw are done
    if (lane < MM) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) cw[lane * TMAX + t] = w[t] * beta[lane * TMAX + t];
    }
    wave_lds_fence();

    // ---- the ring terms and the skip (lane = state row), then the append --
    float yp[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) yp[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < NRING; ++j) {
      const float x = (j < n) ? input_to_float<IT>(xraw[j]) : 0.0f;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) yp[t] = fmaf(cw[j * TMAX + t], x, yp[t]);
    }
#pragma unroll
    for (int u = 0; u < TMAX; ++u) {
      if (u < T) {
        const float x = input_to_float<IT>(xn[u]);
        const float* cu = cw + (n + u) * TMAX;   // zero for outputs t < u
#pragma unroll
        for (int t = 0; t < TMAX; ++t) yp[t] = fmaf(cu[t], x, yp[t]);
      }
    }
    if (a.has_D) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) yp[t] = fmaf(D_h, input_to_float<IT>(xn[t]), yp[t]);
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const int e = __builtin_amdgcn_readlane(ent_l, n + t);
        store_elem<IT>(at(xslot, static_cast<uint32_t>(e) * xent + xrow), xn[t]);
        if (lane == n + t)
          gstore(a.dt_ring + static_cast<int64_t>(s) * a.dt_stride + static_cast<int64_t>(e) * H + h, dt_l);
        if (h % a.hpg == 0) {
          const char* bs = a.B_new + (((b * rowsT + t) * G + g) * DS) * IB;
          char* bd = a.B_ring + (static_cast<int64_t>(s) * a.B_stride + (static_cast<int64_t>(e) * G + g) * DS) * IB;
#pragma unroll
          for (int q = 0; q < DS / 64; ++q)
            store_elem<IT>(bd + (lane + 64 * q) * IB, load_elem<IT>(bs + (lane + 64 * q) * IB));
        }
      }
    }

    // ---- stream the checkpoint tile: S_0[r,:] . C_t for every row and t ---
#pragma unroll 1
    for (int p0 = 0; p0 < NPASS; p0 += PD) {
#pragma unroll
      for (int q = 0; q < PD; ++q) {
        const int p = p0 + q;
        Chunk<ST> cur[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) cur[k] = buf[q][k];
        if (p + PD < NPASS) load_lane_state<ST, IT, true>(at(tile + (p + PD) * PS, lane_off), buf[q]);
        float sel = 0.0f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          const float v = row_sum<TPR>(lane_dot<ST, IT>(cur, Cv[t]));
          if (cc == t) sel = v;
        }
        if (cc < TMAX) dots[cc * DSTRIDE + rr + p * RPP] = sel;
      }
    }
    wave_lds_fence();

    // ---- outputs ------------------------------------------------------------
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float y = fmaf(dec[t], dots[t * DSTRIDE + lane], yp[t]);
        if (a.has_z) {
          const float zv = input_to_float<IT>(zr[t]);
          y *= zv / (1.0f + expf(-zv));
        }
        gstore(a.y + ((b * rowsT + t) * H + h) * DIM + lane, y);
      }
    }
  }
}

}  // namespace rssm
