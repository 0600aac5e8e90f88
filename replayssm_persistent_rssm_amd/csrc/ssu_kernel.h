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
// are dealt round-robin over the wavefronts, in a workgroup order that keeps
// the heads of one B group on one XCD's L2.  Per item:
//  * lane j < n + T holds token j's dt and decay; one suffix-product scan per
//    new token gives Dec and the weights;
//  * per (request, group), kept across the heads of the group: C_t for the
//    lane's columns in registers, and B_j . C_t for every (j, t) in LDS (one
//    lane group per dot product, a DPP sum);
//  * the checkpoint tile streams through registers, two passes of rows in
//    flight; each row is dotted with every C_t and the sums pass through LDS
//    to lane = row;
//  * with lane = state row, the ring terms and the skip are added and the
//    outputs gated; the new tokens' x and dt are appended to the ring, and B
//    once per group, from the group's registers, by the wavefront that holds
//    the group's first head.
// The library's default grid gives each wavefront about one item (up to 16
// times the resident capacity), so the tiles in flight lie close together in
// memory, which streamed 13% faster than a persistent grid on MI355X.  When a
// wavefront does get several items (a capped grid, very large batches) they
// are software-pipelined: before item i streams its tile, item i+1's small
// inputs (its ring x rows, new x and z rows) are requested straight into the
// other of two LDS buffers and its dt into a register, and the last passes
// of i's stream load the first passes of i+1's tile; the scan, ring terms
// and outputs of i then run while those loads are in flight.
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


// One element of a row in input storage, widened to fp32.
template <int IT>
__device__ __forceinline__ float input_to_float(uint32_t raw) {
  if constexpr (IT == kF32) return __uint_as_float(raw);
  else if constexpr (IT == kBF16) return __uint_as_float(raw << 16);
  else return f16_bits_to_float(raw);
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

// Resident wavefronts per SIMD the registers are budgeted for: C costs
// 8 * TMAX registers per lane, the fp32-widened layouts more; fp32 inputs
// double the LDS row buffers (55 KiB per workgroup at TMAX 4), which caps
// them at 2 anyway.
template <int ST, int IT, int TMAX>
constexpr int kSsuWavesPerSimd = SsuRow<ST, IT>::kPacked ? ((TMAX > 4) ? 3 : 4)
                                 : (Fmt<IT>::bytes == 4 || TMAX > 4) ? 2 : 3;

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

  // Write the lane's columns back in the input format (exact: the values
  // came from that format).
  __device__ __forceinline__ void store(char* row, int cc) const {
    constexpr int IB = Fmt<IT>::bytes;
    if constexpr (Row::kPacked) {
      st<false>(row + cc * 8 * IB, u32x4{w[0], w[1], w[2], w[3]});
      st<false>(row + (64 + cc * 8) * IB, u32x4{w[4], w[5], w[6], w[7]});
    } else {
      const int c0 = Row::kSplit ? cc * 4 : cc * 8;
      const int c1 = Row::kSplit ? 64 + cc * 4 : cc * 8 + 4;
      store4(row + c0 * IB, w);
      store4(row + c1 * IB, w + 4);
    }
  }

 private:
  __device__ __forceinline__ static void store4(char* p, const uint32_t* f) {
    if constexpr (IT == kF32) {
      st<false>(p, u32x4{f[0], f[1], f[2], f[3]});
    } else {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (IT == kBF16) h[i] = f[i] >> 16;
        else h[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(__uint_as_float(f[i])));
      }
      st<false>(p, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
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

// Value of lane + N within the lane's 16-lane DPP row, or 1 where lane + N
// leaves the row (row_shl with the old value kept, bound_ctrl off).
template <int N>
__device__ __forceinline__ float shl_row_or_one(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v), 0x100 + N, 0xF, 0xF,
                                                    false));
}

// Request metadata as the kernel uses it (uniform), with the fault guards of
// the contract: skip slots outside [0, num_slots) and the pad slot, reduce
// ring_start modulo R, clamp num_buffered to [0, min(16, R) - T].
struct SsuReq {
  int b, s, n, r0;
  bool live;
  int ent;   // per lane: ring entry of token `lane` (lanes 0..15), (r0 + lane) mod R
};

__device__ __forceinline__ SsuReq ssu_req(const SsuArgs& a, int b, int s_raw, int r_raw, int n_raw) {
  SsuReq q;
  q.b = b;
  q.s = uniform(s_raw);
  q.live = q.s != a.pad && q.s >= 0 && q.s < a.num_slots;
  q.n = min(max(uniform(n_raw), 0), min(kSsuMaxTokens, a.R) - a.T);
  int r0 = uniform(r_raw) % a.R;
  q.r0 = r0 < 0 ? r0 + a.R : r0;
  q.ent = (q.r0 + min(static_cast<int>(threadIdx.x & 63), kSsuMaxTokens - 1)) % a.R;
  return q;
}

template <int ST, int IT, int TMAX, int PD = 2>
__global__ void __launch_bounds__(kBlock, (kSsuWavesPerSimd<ST, IT, TMAX>)) ssu_decode_kernel(const SsuArgs a) {
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
  // rows of 64 input elements move as 16-byte pieces, one per lane
  constexpr int ROWB = DIM * IB;           // bytes per x row
  constexpr int LPX = ROWB / 16;           // lanes per x row
  constexpr int XPI = 64 / LPX;            // x rows per load instruction
  constexpr int NXI = MM / XPI;            // instructions for 16 ring rows
  constexpr int NZI = (2 * TMAX + XPI - 1) / XPI;   // instructions for T new-x rows and T z rows
  static_assert(TMAX >= 1 && TMAX <= 8, "TMAX");
  static_assert(NPASS % PD == 0, "passes");
  static_assert(TMAX <= TPR, "one lane of each row stores each token's row sum");

  __shared__ float lds_beta[kWaves][MM * TMAX];     // B_j . C_t at [j][t]
  __shared__ float lds_c[kWaves][MM * TMAX];        // w_j^(n+t+1) (B_j . C_t) at [j][t]
  __shared__ float lds_dot[kWaves][TMAX * DSTRIDE]; // S_0[r,:] . C_t at [t][r]
  __shared__ u32x4 lds_x[kWaves][2][NXI * 64];      // ring x rows j = 0..15, ROWB bytes each (two items)
  __shared__ u32x4 lds_xz[kWaves][2][NZI * 64];     // x_new rows t < T, then z rows (two items)

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
  const int xrow_l = lane / LPX;                    // row of this lane's 16-byte piece
  const uint32_t xpiece = static_cast<uint32_t>((lane % LPX) * 16);

  // ---- the wavefront's items, in order -------------------------------------
  const int64_t items = static_cast<int64_t>(a.B) * H;
  const int64_t tw = static_cast<int64_t>(gridDim.x) * kWaves;
  constexpr int64_t kC = 16;
  const int64_t csz = min(kC, (items + tw - 1) / tw);
  // Workgroups go to the eight XCDs (each with its own L2) in turn.  Within
  // every run of 64 workgroups, the eight that one XCD receives take eight
  // consecutive item ranges, so the heads of one B group (whose B and C rows
  // every wavefront of the group reads) share an L2, while the run as a whole
  // still covers one contiguous stretch of tiles.  (Measured on MI355X,
  // ssu_large: HBM reads 6.0 % above the algorithmic bytes in launch order,
  // 0.6 % with this order, and 212.9 against 214.2 us; one contiguous eighth
  // of the grid per XCD instead ran 225 us, the tiles in flight then lying
  // far apart.)
  int64_t bid = blockIdx.x;
  if (bid < static_cast<int64_t>(gridDim.x / 64) * 64) bid = (bid / 64) * 64 + (bid % 8) * 8 + (bid % 64) / 8;
  int64_t chunk = bid * kWaves + wave;
  int64_t nxt = chunk * csz;                         // next item not yet taken (-1: none)
  int64_t cend = min(items, nxt + csz);
  if (nxt >= items) nxt = -1;
  auto advance = [&]() {
    if (nxt < 0) return;
    if (++nxt >= cend) {
      chunk += tw;
      nxt = chunk * csz;
      if (nxt >= items) {
        nxt = -1;
        return;
      }
      cend = min(items, nxt + csz);
    }
  };

  // ---- loads in flight for the upcoming item --------------------------------
  float p_dt = 0.0f;           // token `lane`'s dt before bias / softplus (pending: as stored)
  Chunk<ST> buf[PD][NCH];      // the first passes of its tile
  // its ring x rows and its new x and z rows go straight to LDS (direct
  // global-to-LDS loads: lane L's 16 bytes land at the region's base + 16 L)
  auto to_lds = [&](const char* src, u32x4* region) {
    __builtin_amdgcn_global_load_lds((const RSSM_GLOBAL void*)(src), (__attribute__((address_space(3))) void*)(region),
                                     16, 0, 0);
  };
  auto issue_small = [&](const SsuReq& q, int h, int sb) {
    const int tnew = min(max(lane - q.n, 0), T - 1);
    p_dt = gload(lane < q.n ? a.dt_ring + static_cast<int64_t>(q.s) * a.dt_stride + static_cast<int64_t>(q.ent) * H + h
                            : a.dt_new + (q.b * rowsT + tnew) * H + h);
    const char* xslot = a.x_ring + (static_cast<int64_t>(q.s) * a.x_stride + h * DIM) * IB;
#pragma unroll
    for (int k = 0; k < NXI; ++k) {
      const int j = k * XPI + xrow_l;
      const int e = __shfl(q.ent, min(j, MM - 1));   // every lane takes part in the exchange
      if (k * XPI < q.n && j < q.n) to_lds(xslot + static_cast<int64_t>(e) * H * ROWB + xpiece, &lds_x[wave][sb][k * 64]);
    }
#pragma unroll
    for (int k = 0; k < NZI; ++k) {
      const int rrow = k * XPI + xrow_l;
      if (rrow < 2 * T) {
        const bool isz = rrow >= T;
        const int t = isz ? rrow - T : rrow;
        const char* base = isz ? a.z : a.x_new;
        to_lds(base + (((q.b * rowsT + t) * H + h) * DIM) * IB + xpiece, &lds_xz[wave][sb][k * 64]);
      }
    }
  };
  auto tile_of = [&](const SsuReq& q, int h) {
    return a.state + (static_cast<int64_t>(q.s) * a.state_stride + h * kTile) * SB;
  };

  SsuReq cur{-1, 0, 0, 0, false, 0}, nq{-1, 0, 0, 0, false, 0};
  int cur_g = -1, cur_gb = -1;
  int sb = 0;                  // LDS row-piece buffer of the upcoming item
  bool have = false;           // the loads above belong to item `nxt`
  CVec Cv[TMAX];
  while (true) {
    if (!have) {
      // cold start: the next live item, its request's metadata read here
      while (nxt >= 0) {
        const int b = static_cast<int>(nxt / H);
        if (b != nq.b) nq = ssu_req(a, b, sload(a.slots + b), sload(a.ring_start + b), sload(a.num_buffered + b));
        if (nq.live) break;
        advance();
      }
      if (nxt < 0) break;
      const int h0 = static_cast<int>(nxt - static_cast<int64_t>(nq.b) * H);
      const char* t0 = tile_of(nq, h0);
#pragma unroll
      for (int p = 0; p < PD; ++p) load_lane_state<ST, IT, true>(at(t0 + p * PS, lane_off), buf[p]);
      issue_small(nq, h0, sb);
    }
    // ---- take the item ------------------------------------------------------
    cur = nq;
    const int h = uniform(static_cast<int>(nxt - static_cast<int64_t>(cur.b) * H));
    const int b = cur.b, s = cur.s, n = cur.n;
    const int g = h / a.hpg;
    const int m = n + T;
    const char* tile = tile_of(cur, h);
    const int cb = sb;         // this item's row pieces
    sb ^= 1;
    const float dt_raw = p_dt;
    advance();
    // the following item's request metadata
    const int b2 = nxt >= 0 ? static_cast<int>(nxt / H) : -1;
    int s2_raw = 0, r2_raw = 0, n2_raw = 0;
    if (b2 >= 0 && b2 != b) {
      s2_raw = sload(a.slots + b2);
      r2_raw = sload(a.ring_start + b2);
      n2_raw = sload(a.num_buffered + b2);
    }
    const float A_h = sload(a.A + h);
    const float bias_h = sload(a.dt_bias + h);
    const float D_h = sload(a.D + h);

    // ---- per (request, group): C_t in registers, B_j . C_t in LDS ----------
    if (g != cur_g || b != cur_gb) {
      cur_g = g;
      cur_gb = b;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        const int tt = t < T ? t : 0;
        Cv[t].load(a.C_new + (((b * rowsT + tt) * G + g) * DS) * IB, cc);
      }
      CVec bc[MM / RPP];
#pragma unroll
      for (int q = 0; q < MM / RPP; ++q) {
        const int j = rr + RPP * q;   // token of this lane group
        const int ej = __shfl(cur.ent, j);
        const int tj = min(max(j - n, 0), T - 1);
        const char* src = (j < n) ? a.B_ring + (static_cast<int64_t>(s) * a.B_stride +
                                                (static_cast<int64_t>(ej) * G + g) * DS) * IB
                                  : a.B_new + (((b * rowsT + tj) * G + g) * DS) * IB;
        bc[q].load(src, cc);
        // the group's first head appends the new tokens' B rows from these registers
        if (h % a.hpg == 0 && j >= n && j < m)
          bc[q].store(a.B_ring + (static_cast<int64_t>(s) * a.B_stride + (static_cast<int64_t>(ej) * G + g) * DS) * IB,
                      cc);
      }
      wave_lds_fence();   // the previous item's readers of beta are done
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

    // ---- the following item: metadata, small loads (into the other row-piece
    // buffer, which no one reads now), first passes from the stream's tail ---
    have = false;
    if (nxt >= 0) {
      if (b2 != b) nq = ssu_req(a, b2, s2_raw, r2_raw, n2_raw);
      if (nq.live) have = true;
    }
    const int h2 = have ? uniform(static_cast<int>(nxt - static_cast<int64_t>(nq.b) * H)) : 0;
    const char* ntile = tile_of(nq, h2);
    if (have) issue_small(nq, h2, sb);

    // ---- stream the checkpoint tile: S_0[r,:] . C_t for every row and t ---
    // (fully unrolled: straight-line code lets each pass wait only for its own
    // loads, with the next passes still in flight)
    wave_lds_fence();   // the previous item's readers of the row sums are done
#pragma unroll
    for (int p0 = 0; p0 < NPASS; p0 += PD) {
#pragma unroll
      for (int q = 0; q < PD; ++q) {
        const int p = p0 + q;
        Chunk<ST> cur_c[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) cur_c[k] = buf[q][k];
        if (p + PD < NPASS) load_lane_state<ST, IT, true>(at(tile + (p + PD) * PS, lane_off), buf[q]);
        else if (have) load_lane_state<ST, IT, true>(at(ntile + (p + PD - NPASS) * PS, lane_off), buf[q]);
        float sel = 0.0f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          const float v = row_sum<TPR>(lane_dot<ST, IT>(cur_c, Cv[t]));
          if (cc == t) sel = v;
        }
        if (cc < TMAX) dots[cc * DSTRIDE + rr + p * RPP] = sel;
      }
    }

    // ---- after the stream (the next tile's first passes are in flight) ------
    // this item's row pieces: append the new x rows to the ring
    const char* xl = reinterpret_cast<const char*>(lds_x[wave][cb]);
    const char* xzl = reinterpret_cast<const char*>(lds_xz[wave][cb]);
#pragma unroll
    for (int k = 0; k < NZI; ++k) {
      const int t = k * XPI + xrow_l;
      const int e = __shfl(cur.ent, min(n + t, MM - 1));   // every lane takes part in the exchange
      if (t < T) {
        st<false>(a.x_ring + (static_cast<int64_t>(s) * a.x_stride + (static_cast<int64_t>(e) * H + h) * DIM) * IB +
                      xpiece,
                  lds_xz[wave][cb][k * 64 + lane]);
      }
    }
    auto xelem = [&](const char* base, int row) -> float {
      if constexpr (IB == 4) return *reinterpret_cast<const float*>(base + row * ROWB + lane * 4);
      else return input_to_float<IT>(*reinterpret_cast<const uint16_t*>(base + row * ROWB + lane * 2));
    };

    // decays and weights: one suffix-product scan per new token
    float dt_l = dt_raw;
    if (lane >= n && lane < m) dt_l = new_token_dt(dt_raw, a.has_bias ? bias_h : 0.0f, a.dt_softplus);
    if (lane >= m) dt_l = 0.0f;
    const float a_l = (lane < m) ? expf(dt_l * A_h) : 1.0f;
    float dec[TMAX], w[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int mt = n + t + 1;
      float P = (lane < mt) ? a_l : 1.0f;   // after the scan: prod over lanes lane .. min(mt, 16)-1
      // Hillis-Steele suffix products inside the first DPP row (lanes 0..15;
      // the other rows hold ones): row_shl brings lane j + off, and lanes whose
      // source leaves the row keep the old value 1
      P *= shl_row_or_one<1>(P);
      P *= shl_row_or_one<2>(P);
      P *= shl_row_or_one<4>(P);
      P *= shl_row_or_one<8>(P);
      float Pn = shl_row_or_one<1>(P);
      if (lane + 1 >= mt) Pn = 1.0f;
      dec[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), 0));
      w[t] = (lane < mt) ? dt_l * Pn : 0.0f;
    }
    wave_lds_fence();   // beta and the row sums written; the previous item's readers of cw are done
    if (lane < MM) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) cw[lane * TMAX + t] = w[t] * beta[lane * TMAX + t];
    }
    wave_lds_fence();

    // the ring terms, the skip and the outputs (lane = state row); dt append
    float yp[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) yp[t] = dec[t] * dots[t * DSTRIDE + lane];
#pragma unroll
    for (int j = 0; j < NRING; ++j) {
      if (j < n) {
        const float x = xelem(xl, j);
#pragma unroll
        for (int t = 0; t < TMAX; ++t) yp[t] = fmaf(cw[j * TMAX + t], x, yp[t]);
      }
    }
#pragma unroll
    for (int u = 0; u < TMAX; ++u) {
      if (u < T) {
        const float x = xelem(xzl, u);
        const float* cu = cw + (n + u) * TMAX;   // zero for outputs t < u
#pragma unroll
        for (int t = 0; t < TMAX; ++t) yp[t] = fmaf(cu[t], x, yp[t]);
        if (a.has_D) yp[u] = fmaf(D_h, x, yp[u]);
      }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float y = yp[t];
        if (a.has_z) {
          const float zv = xelem(xzl, T + t);
          y *= zv * __builtin_amdgcn_rcpf(1.0f + expf(-zv));   // silu, reciprocal within 1 ulp
        }
        gstore(a.y + ((b * rowsT + t) * H + h) * DIM + lane, y);
        const int e = __builtin_amdgcn_readlane(cur.ent, n + t);
        if (lane == n + t)
          gstore(a.dt_ring + static_cast<int64_t>(s) * a.dt_stride + static_cast<int64_t>(e) * H + h, dt_l);
      }
    }
  }
}

}  // namespace rssm
