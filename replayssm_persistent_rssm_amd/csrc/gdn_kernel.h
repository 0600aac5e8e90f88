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
//  * The update never mixes rows of S: row i evolves by its own dot product
//    with the token's key.  So a state tile is streamed row-wise, like the
//    materialize kernel's: 16 lanes per row, 8 key columns per lane (two
//    halves, 4*cc.. and 64 + 4*cc.., so that every 16-byte access instruction
//    is contiguous across the lanes of a row), 4 rows per wavefront pass, PD
//    passes in flight while earlier passes run their tokens.  Work item = one (request, layer, value head) tile; tiles are
//    dealt round-robin over the wavefronts, so each sees the same mix of
//    cheap (skipped), plain and tracked requests.  No workgroup barriers.
//  * The normalised keys live in registers (8 columns x up to TMAX tokens per
//    lane, normalised with a 16-lane DPP sum of squares); the tile's values go
//    to the wavefront's LDS as [row][token]; decays and betas sit one token
//    per lane and are read with readlane.
//  * Per token and row: S k is 8 fused multiply-adds per lane and a 16-lane
//    DPP sum; the update S <- exp(g) S + u k^T with u = beta (v - exp(g) S k)
//    is 2 VALU operations per element.  fp32 throughout: the contractions are
//    matrix-vector products with a sequential dependence between tokens, and
//    the path moves 128 KiB of state per tile against ~4 VALU operations per
//    element per token, so HBM bounds it.
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

// Register budget: the keys cost 8 * TMAX registers per lane.
template <int TMAX> constexpr int kGdnWavesPerSimd = (TMAX > 8) ? 2 : 3;

// Stream knobs (the library's instances use the defaults; the others exist so
// that streaming patterns can be compared on hardware).  Measured on MI355X,
// variants side by side in one process (48 layers, 256 requests, 32 value
// heads): with 4 tokens each, cached state loads and stores with 2 passes in
// flight ran 9.45 ms, non-temporal ones 10.5 ms, 4 passes in flight 10.2 ms;
// with the benchmark's mix (prefixes U[0, 8], a sixteenth null, tracked steps)
// dealing tiles round-robin ran 10.2 ms against 13.0 ms for contiguous ranges,
// and a 3-wave register budget 9.8 ms.
//   NTL / NTS  non-temporal state loads / stores
//   PD         state passes in flight per wavefront
//   WPS        waves per SIMD the registers are budgeted for (0: the rule above)
//   DEAL       work distribution (below)
//   KLDS       keys in the wavefront's LDS (read per token) instead of registers
template <int TMAX, bool NTL = false, bool NTS = false, int PD = 2, int WPS = 0, int DEAL = 1, bool KLDS = false>
__global__ void __launch_bounds__(kBlock, (WPS > 0 ? WPS : kGdnWavesPerSimd<TMAX>))
    gdn_commit_kernel(const GdnArgs a) {
  constexpr int D = kGdnDim;
  constexpr int TPR = 16;                 // lanes per row
  constexpr int RPP = 64 / TPR;           // rows per pass (4)
  constexpr int NPASS = D / RPP;          // passes per tile (32)
  constexpr int64_t kTile = static_cast<int64_t>(D) * D;
  constexpr int PS = RPP * D * 4;         // bytes between passes
  static_assert(TMAX % 4 == 0 && TMAX <= 16, "TMAX");
  static_assert(NPASS % PD == 0, "passes must split into prefetch groups");

  __shared__ __attribute__((aligned(16))) float lds_v[kWaves][D * TMAX];
  __shared__ __attribute__((aligned(16))) float lds_k[kWaves][KLDS ? TMAX * D : 4];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
  float* vw = lds_v[wave];
  const int cc = lane % TPR;
  const int rr = lane / TPR;
  const uint32_t lane_off = static_cast<uint32_t>(rr * D * 4 + cc * 16);  // bytes, in a pass

  const int64_t per_req = static_cast<int64_t>(a.L) * a.HV;
  const int64_t items = static_cast<int64_t>(a.B) * per_req;
  const int64_t tw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  // DEAL = 0: one contiguous, balanced range of tiles per wavefront.
  // DEAL = 1: tiles dealt round-robin (wavefront w takes w, w + waves, ...),
  // so that every wavefront sees the same mix of requests -- their costs
  // differ (skipped, tracked, short or long prefixes).
  int64_t it, end;
  if constexpr (DEAL == 0) {
    const int64_t per = items / tw, rem = items % tw;
    it = gw * per + (gw < rem ? gw : rem);
    end = it + per + (gw < rem ? 1 : 0);
  } else {
    it = gw;
    end = items;
  }
  constexpr int64_t kOne = 1;
  const int64_t advance = DEAL ? tw : kOne;
  const int group = a.HV / a.H;

  int cur_b = -1, s = 0, n = 0, ts = -1, step = -1;
  bool live = false;
  // Tiles dealt round-robin, several per wavefront: the wavefront first tests
  // the liveness of its next 64 tiles at once (one per lane: the request's
  // slot above null_block_id and a positive accepted count) and walks only the
  // live ones, so skipped requests cost no round trips of their own (a call
  // whose requests are all null is one near-empty launch).
  const bool filt = DEAL == 1 && items > tw;
  int64_t qb = 0;       // position in this wavefront's tile sequence of lane 0 of the batch
  uint64_t livem = 0;   // live tiles of the batch not yet taken

  for (;;) {
    if (filt) {
      while (livem == 0) {
        if (gw + qb * tw >= items) break;
        const int64_t tj = gw + (qb + lane) * tw;
        bool lv = false;
        if (tj < items) {
          const int bj = static_cast<int>(tj / per_req);
          const int sj = gload(a.state_indices + bj);
          const int nj = gload(a.accept_lens + bj);
          lv = sj > a.null_block_id && sj < a.slots && nj > 0;
        }
        livem = __ballot(lv);
        if (livem == 0) qb += 64;
      }
      if (livem == 0) break;
      it = gw + (qb + __builtin_ctzll(livem)) * tw;
      livem &= livem - 1;
      if (livem == 0) qb += 64;
    } else if (it >= end) {
      break;
    }
    const int b = static_cast<int>(it / per_req);
    if (b != cur_b) {
      // Request metadata, read when the request changes.
      cur_b = b;
      s = uniform(a.state_indices[b]);
      n = uniform(a.accept_lens[b]);
      live = s > a.null_block_id && s < a.slots && n > 0;   // else ignored slot or nothing accepted
      n = min(n, a.T);
      step = -1;
      if (live && a.track_indices != nullptr) {
        ts = uniform(a.track_indices[b]);
        step = uniform(a.track_steps[b]);
        if (ts <= a.null_block_id || ts >= a.slots || step < 0 || step >= n) step = -1;  // not written
      }
    }
    if (!live) {
      if constexpr (DEAL == 0) it = min(end, static_cast<int64_t>(b + 1) * per_req);
      else it += advance;
      continue;
    }
    const int64_t in_req = it - static_cast<int64_t>(b) * per_req;
    const int l = static_cast<int>(in_req / a.HV);
    const int hv = static_cast<int>(in_req - static_cast<int64_t>(l) * a.HV);
    const int kh = hv / group;
    it += advance;
    const int64_t vslot = (static_cast<int64_t>(l) * a.slots + s) * a.HV + hv;   // (l, s, hv)
    const char* tile = reinterpret_cast<const char*>(a.state + vslot * kTile);
    char* otile = reinterpret_cast<char*>(a.state + vslot * kTile);
    char* ttile = step >= 0 ? reinterpret_cast<char*>(a.state + ((static_cast<int64_t>(l) * a.slots + ts) * a.HV + hv) * kTile)
                            : nullptr;

    // Small inputs first, the state stream after them (a wavefront's memory
    // requests complete in order, so staging waits only for these).
    float g_l = 0.0f, beta_l = 0.0f;       // token `lane`
    if (lane < n) {
      g_l = gload(a.g + vslot * a.T + lane);
      beta_l = gload(a.beta + vslot * a.T + lane);
    }
    const uint16_t* vwin = a.rawv + vslot * a.T * D;
    uint32_t vraw[TMAX][2];                // token t, rows lane and lane + 64
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      vraw[t][0] = (t < n) ? gload(vwin + t * D + lane) : 0u;
      vraw[t][1] = (t < n) ? gload(vwin + t * D + 64 + lane) : 0u;
    }
    // The tile's keys (re-read per tile: the heads of one key head find them
    // in L2), 16 lanes per token row.
    Chunk<kBF16> kraw[TMAX];
    const uint16_t* kwin = a.rawk + ((static_cast<int64_t>(l) * a.slots + s) * a.H + kh) * a.T * D;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < n) {
        // the lane's key columns match its state columns: 4*cc.. and 64 + 4*cc..
        const u32x2 lo = ld<false, u32x2>(reinterpret_cast<const char*>(kwin + t * D + cc * 4));
        const u32x2 hi = ld<false, u32x2>(reinterpret_cast<const char*>(kwin + t * D + 64 + cc * 4));
        kraw[t].w[0] = lo.x; kraw[t].w[1] = lo.y; kraw[t].w[2] = hi.x; kraw[t].w[3] = hi.y;
      } else {
        kraw[t] = Chunk<kBF16>{};
      }
    }
    Chunk<kF32> buf[PD];
#pragma unroll
    for (int p = 0; p < PD; ++p) buf[p] = load_split_f32<NTL>(at(tile + p * PS, lane_off));

    const float alpha_l = expf(g_l);
    wave_lds_fence();
    float kv[KLDS ? 1 : TMAX][8];          // normalised keys, this lane's 8 columns
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      float k8[8];
      decode_chunk<kBF16>(kraw[t], k8);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(k8[i], k8[i], ss);
      ss = row16_sum(ss);
      const float inv = a.use_l2norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) k8[i] *= inv;
      if constexpr (KLDS) {
        if (rr == 0) {
          *reinterpret_cast<float4*>(&lds_k[wave][t * D + cc * 8]) = make_float4(k8[0], k8[1], k8[2], k8[3]);
          *reinterpret_cast<float4*>(&lds_k[wave][t * D + cc * 8 + 4]) = make_float4(k8[4], k8[5], k8[6], k8[7]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[t][i] = k8[i];
      }
    }
    // Values to LDS as [row][token].
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < n) {
        vw[lane * TMAX + t] = __uint_as_float(vraw[t][0] << 16);
        vw[(lane + 64) * TMAX + t] = __uint_as_float(vraw[t][1] << 16);
      }
    }
    wave_lds_fence();

    // Stream the tile: PD passes in flight; each pass runs the n tokens on
    // its rows and is written back (and, after the tracked token, copied).
#pragma unroll 1
    for (int p0 = 0; p0 < NPASS; p0 += PD) {
#pragma unroll
      for (int q = 0; q < PD; ++q) {
        const int p = p0 + q;
        const Chunk<kF32> cur = buf[q];
        if (p + PD < NPASS) buf[q] = load_split_f32<NTL>(at(tile + (p + PD) * PS, lane_off));
        const int r = rr + p * RPP;
        float S[8];
        decode_chunk<kF32>(cur, S);
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          if (t < n) {
            const float alpha = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha_l), t));
            const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(beta_l), t));
            float kt[8];
            if constexpr (KLDS) {
              const float4 k0 = *reinterpret_cast<const float4*>(&lds_k[wave][t * D + cc * 8]);
              const float4 k1 = *reinterpret_cast<const float4*>(&lds_k[wave][t * D + cc * 8 + 4]);
              kt[0] = k0.x; kt[1] = k0.y; kt[2] = k0.z; kt[3] = k0.w;
              kt[4] = k1.x; kt[5] = k1.y; kt[6] = k1.z; kt[7] = k1.w;
            } else {
#pragma unroll
              for (int c = 0; c < 8; ++c) kt[c] = kv[KLDS ? 0 : t][c];
            }
            float d = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) d = fmaf(S[c], kt[c], d);
            d = row16_sum(d);                           // (S k)[row], before the decay
            const float u = bt * (vw[r * TMAX + t] - alpha * d);   // beta (v - exp(g) S k)
#pragma unroll
            for (int c = 0; c < 8; ++c) S[c] = fmaf(S[c], alpha, u * kt[c]);
            if (t == step) {
              Chunk<kF32> o;
#pragma unroll
              for (int c = 0; c < 8; ++c) o.w[c] = __float_as_uint(S[c]);
              store_split_f32<NTS>(at(ttile + p * PS, lane_off), o);
            }
          }
        }
        Chunk<kF32> o;
#pragma unroll
        for (int c = 0; c < 8; ++c) o.w[c] = __float_as_uint(S[c]);
        store_split_f32<NTS>(at(otile + p * PS, lane_off), o);
      }
    }
  }
}

}  // namespace rssm
