// gdn_kernel.h -- persistent gfx950 kernel for the gated-delta-rule
// ReplaySSM commit.
//
// Operation: flashinfer.gdn_decode.gated_delta_rule_replayssm_commit
// (documentation page, summary and Parameters).  For every request b whose
// slot s = state_indices[b] lies above null_block_id and whose accepted count
// n = accept_lens[b] is positive, every layer l and value head hv, the fp32
// checkpoint S = state[l][s][hv] (128 value rows by 128 key columns, K last)
// takes the first n tokens of its cached windows in order,
//     k = normalise(rawk[l][s][hv / (HV/H)][t]),  v = rawv[l][s][hv][t]
//     S <- exp(g_t) S;   S <- S + beta_t (v - S k) k^T
// and is written back in place; optionally the state after token
// track_steps[b] also goes to slot track_state_indices[b].
//
// Design (MI355X, wave64):
//  * Work item = an eighth of a tile: 16 value rows x 128 key columns (8 KiB
//    contiguous) of one (request, layer, value head).  Each wavefront owns a
//    contiguous range of items (request-major, then layer, head, quarter), so
//    consecutive items share the request's metadata and often its keys.  No
//    workgroup barriers.
//  * 16 lanes per row, 8 columns per lane: a lane holds 4 rows x 8 columns
//    of S (32 registers) for the whole token loop (32 rows per item needed
//    about 200 registers and halved the resident waves); S is read once and written
//    once per commit (plus once more for a tracked step).
//  * Keys are normalised once per (request, layer, key head) into the
//    wavefront's LDS ([token][column], fp32); the item's 16 values per token go
//    to LDS as [token][row-in-pass][pass], so a lane reads its 4 rows with one
//    16-byte load.
//  * Per token and row, S k is 8 fused multiply-adds per lane and a 16-lane
//    DPP sum; the update S <- exp(g) S + u k^T with u = beta (v - exp(g) S k)
//    is 2 VALU operations per element.  fp32 throughout (the contractions are
//    matrix-vector products with a sequential dependence between tokens, and
//    the path is bound by HBM: 128 KiB of state per (request, layer, head)
//    against ~3 VALU operations per element per token).
#pragma once

#include "rssm_kernel.h"

namespace rssm {

struct GdnArgs {
  float* state;               // [L][slots][HV][128][128]
  const uint16_t* rawv;       // [L][slots][HV][T][128] bf16
  const uint16_t* rawk;       // [L][slots][H][T][128] bf16
  const float* g;             // [L][slots][HV][T]
  const float* beta;          // [L][slots][HV][T]
  const int32_t* state_indices;
  const int32_t* accept_lens;
  const int32_t* track_indices;  // NULL: no tracking
  const int32_t* track_steps;
  int32_t L, slots, HV, H, T, B, use_l2norm, null_block_id;
};

constexpr int kGdnDim = 128;   // key and value width, fixed by the page
constexpr int kGdnRows = 16;   // value rows per work item (an eighth of a tile)

// Sum over the 16 lanes of an aligned lane group (the same exchange pattern
// as row16_max).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

template <int TMAX>
__global__ void __launch_bounds__(kBlock, 4) gdn_commit_kernel(const GdnArgs a) {
  constexpr int D = kGdnDim;
  constexpr int TPR = 16;                 // lanes per row
  constexpr int RPP = 64 / TPR;           // rows per pass (4)
  constexpr int NP = kGdnRows / RPP;      // passes per item (4)
  constexpr int64_t kTile = static_cast<int64_t>(D) * D;
  constexpr int QPT = D / kGdnRows;       // items per tile (8)
  static_assert(TMAX >= 1 && TMAX <= 16, "TMAX");
  static_assert(NP % 4 == 0 && D % kGdnRows == 0, "item shape");

  __shared__ __attribute__((aligned(16))) float lds_k[kWaves][TMAX * D];
  __shared__ __attribute__((aligned(16))) float lds_v[kWaves][TMAX * kGdnRows];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
  float* kw = lds_k[wave];
  float* vw = lds_v[wave];
  const int cc = lane % TPR;
  const int rr = lane / TPR;
  const uint32_t lane_off = static_cast<uint32_t>((rr * D + cc * 8) * 4);  // bytes, in a pass
  constexpr int PS = RPP * D * 4;                                            // bytes between passes

  const int64_t per_req = static_cast<int64_t>(a.L) * a.HV * QPT;
  const int64_t items = static_cast<int64_t>(a.B) * per_req;
  const int64_t tw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t per = items / tw, rem = items % tw;
  int64_t it = gw * per + (gw < rem ? gw : rem);
  const int64_t end = it + per + (gw < rem ? 1 : 0);
  const int group = a.HV / a.H;
  int64_t staged_key = -1;  // (request, layer, key head) whose keys are in LDS

  while (it < end) {
    const int b = static_cast<int>(it / per_req);
    const int64_t in_req = it - static_cast<int64_t>(b) * per_req;
    const int s = uniform(a.state_indices[b]);
    int n = uniform(a.accept_lens[b]);
    if (s <= a.null_block_id || s >= a.slots || n <= 0) {
      it = min(end, static_cast<int64_t>(b + 1) * per_req);   // ignored slot or nothing accepted
      continue;
    }
    n = min(n, a.T);
    int ts = -1, step = -1;
    if (a.track_indices != nullptr) {
      ts = uniform(a.track_indices[b]);
      step = uniform(a.track_steps[b]);
      if (ts <= a.null_block_id || ts >= a.slots || step < 0 || step >= n) step = -1;  // not written
    }
    const int l = static_cast<int>(in_req / (static_cast<int64_t>(a.HV) * QPT));
    const int hq = static_cast<int>(in_req - static_cast<int64_t>(l) * a.HV * QPT);
    const int hv = hq / QPT;
    const int q = hq - hv * QPT;
    const int kh = hv / group;
    const int64_t vslot = (static_cast<int64_t>(l) * a.slots + s) * a.HV + hv;   // (l, s, hv)
    char* tile = reinterpret_cast<char*>(a.state + vslot * kTile + static_cast<int64_t>(q) * kGdnRows * D);

    // Issue the item's 16 x 128 fp32 block: 4 passes x 32 bytes per lane.
    Chunk<kF32> S[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) S[p] = load_chunk<kF32, true>(at(tile + p * PS, lane_off));

    // Keys of (b, l, kh), normalised, unless already staged.
    const int64_t key_id = (static_cast<int64_t>(b) * a.L + l) * a.H + kh;
    wave_lds_fence();
    if (key_id != staged_key) {
      const uint16_t* kwin = a.rawk + ((static_cast<int64_t>(l) * a.slots + s) * a.H + kh) * a.T * D;
#pragma unroll
      for (int rep = 0; rep < (TMAX * TPR + 63) / 64; ++rep) {
        const int t = rep * RPP + rr;        // 16 lanes per token
        float kv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (t < n) {
          const Chunk<kBF16> c = load_chunk<kBF16>(reinterpret_cast<const char*>(kwin + t * D + cc * 8));
          decode_chunk<kBF16>(c, kv);
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(kv[i], kv[i], ss);
        ss = row16_sum(ss);
        const float inv = a.use_l2norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
        if (t < n) {
#pragma unroll
          for (int i = 0; i < 8; ++i) kw[t * D + cc * 8 + i] = kv[i] * inv;
        }
      }
      staged_key = key_id;
    }
    // Values of this item's 16 rows: token t, row p*4 + rr -> vw[t*16 + rr*4 + p].
    {
      const uint16_t* vwin = a.rawv + vslot * a.T * D + q * kGdnRows;
#pragma unroll
      for (int rep = 0; rep < (TMAX * kGdnRows + 63) / 64; ++rep) {
        const int idx = rep * 64 + lane;
        const int t = idx / kGdnRows;
        const int row = idx % kGdnRows;
        if (t < n) {
          const float v = __uint_as_float(static_cast<uint32_t>(gload(vwin + t * D + row)) << 16);
          vw[t * kGdnRows + (row % RPP) * NP + row / RPP] = v;
        }
      }
    }
    wave_lds_fence();

    const float* gw_ = a.g + vslot * a.T;
    const float* bw_ = a.beta + vslot * a.T;
    float Sf[NP][8];
#pragma unroll
    for (int p = 0; p < NP; ++p) decode_chunk<kF32>(S[p], Sf[p]);

#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t >= n) break;
      const float alpha = expf(gload(gw_ + t));
      const float bt = gload(bw_ + t);
      const float4 k0 = *reinterpret_cast<const float4*>(kw + t * D + cc * 8);
      const float4 k1 = *reinterpret_cast<const float4*>(kw + t * D + cc * 8 + 4);
      const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      float vv[NP];
#pragma unroll
      for (int i = 0; i < NP; i += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(vw + t * kGdnRows + rr * NP + i);
        vv[i] = v4.x;
        vv[i + 1] = v4.y;
        vv[i + 2] = v4.z;
        vv[i + 3] = v4.w;
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        float d = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) d = fmaf(Sf[p][c], kv[c], d);
        d = row16_sum(d);                           // (S k)[row], before the decay
        const float u = bt * (vv[p] - alpha * d);   // beta (v - exp(g) S k)
#pragma unroll
        for (int c = 0; c < 8; ++c) Sf[p][c] = fmaf(Sf[p][c], alpha, u * kv[c]);
      }
      if (t == step) {
        char* ttile = reinterpret_cast<char*>(
            a.state + ((static_cast<int64_t>(l) * a.slots + ts) * a.HV + hv) * kTile +
            static_cast<int64_t>(q) * kGdnRows * D);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          Chunk<kF32> c;
#pragma unroll
          for (int i = 0; i < 8; ++i) c.w[i] = __float_as_uint(Sf[p][i]);
          store_chunk<kF32, true>(at(ttile + p * PS, lane_off), c);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      Chunk<kF32> c;
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = __float_as_uint(Sf[p][i]);
      store_chunk<kF32, true>(at(tile + p * PS, lane_off), c);
    }
    ++it;
  }
}

}  // namespace rssm
