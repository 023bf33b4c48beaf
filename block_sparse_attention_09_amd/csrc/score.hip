// Cluster-weighted block scores: the scoring half of IBCS.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques", IBCS paragraph: a key block's score is the weighted attention
// of the block's centroids to its averaged keys.
//   s_j = sum_c w_c * softmax_j(scale * mu_c . kmean_j),   j over sparse blocks.
//
// One work-group holds 256 centroid rows (256/C query blocks of one head) and
// streams that head's key means twice, 32 blocks per tile, through LDS (the
// means arrive in their scoring form, written by the key-means kernel):
//   pass 1: per-centroid running max and sum of exp2 (the softmax normaliser);
//   pass 2: p = exp2(logit + log2 w_c - lse_c), summed over the C centroids of
//           each query block and written to S.
// Two precisions of the dot products, both accumulated in fp32:
//   * bf16 problems (kF16): one fp16 MFMA per k-step.  The key means come as
//     fp16 scaled by a power of two per tile, the centroids are scaled by one
//     power of two per work-group, both so that their largest magnitude lies
//     in [2^14, 2^15): no overflow, 11 significant bits (finer than the bf16
//     keys and queries they are averaged from).  The two scales multiply the
//     logit inside the fma that already subtracts the running max (pass 1)
//     or adds the centroid's offset (pass 2).
//   * fp32 problems: both operands split into bf16 high and low parts
//     (hi*hi + hi*lo + lo*hi, three MFMAs per k-step), which keeps the logits
//     within ~2^-16 relative of fp32.
// Pass 1 uses the key means as the MFMA A operand (a lane then holds 16 keys
// of one centroid: cheap running max), pass 2 uses the centroids as A (a lane
// holds 16 centroids of one key: cheap sum over a query block's centroids).
// The operand registers are the same in both layouts.
//
// Each pass is software-pipelined: the MFMAs of tile t+1 are issued in the
// same block as the exp2 work of tile t, so the matrix core and the vector
// ALU run side by side.
#include "common.h"
#include "kernels.h"

namespace abatt {

constexpr int kScoreWaves = 8;                 // 256 centroid rows per work-group
constexpr int kScoreT = 64 * kScoreWaves;
constexpr int kScoreStages = 3;                // LDS ring of key-mean tiles

template <int D, int C, bool kF16>
__global__ __launch_bounds__(kScoreT, 1) void k_scores(const float* __restrict__ mu,
                                                       const float* __restrict__ w,
                                                       const uint16_t* __restrict__ kplanes,
                                                       const float* __restrict__ tscale,
                                                       float* __restrict__ S, int n_qb, int n_kbs,
                                                       int groups_per_head, int n_groups,
                                                       int64_t plane_elems, float scale_log2) {
  constexpr int ROWS = 32 * kScoreWaves;  // centroid rows per work-group
  constexpr int G = ROWS / C;             // query blocks per work-group
  constexpr int KS = D / 16;              // MFMA k-steps
  constexpr int ROWB = D + 8;             // LDS row stride (2-byte elements), padded: conflict-free reads
  constexpr int CH = D / 8;               // 16-byte chunks per key-mean row
  constexpr int TILE_CH = 32 * CH;        // chunks per plane per 32-key tile
  constexpr int NCH = (TILE_CH + kScoreT - 1) / kScoreT;  // per thread per plane
  constexpr int NP = kF16 ? 1 : 2;                         // planes of key means
  __shared__ __align__(16) uint16_t ring[kScoreStages][NP][32 * ROWB];
  __shared__ float tsc[kScoreStages];  // scale of the tile in each stage (kF16)
  __shared__ float red[kScoreWaves];
  __shared__ float a_lds[ROWS];

  const int gid = xcd_remap(blockIdx.x, n_groups);
  const int bh = gid / groups_per_head;
  const int qb0 = (gid % groups_per_head) * G;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63, l32 = lane & 31, hh = lane >> 5;

  // this lane's centroid row (operand layout: row l32 of the wave, dims 16s+8hh..+7)
  const int crow = 32 * wv + l32;
  const int qb = qb0 + crow / C;
  const int cc = crow % C;
  const bool rvalid = qb < n_qb;
  const int64_t prow = (int64_t)bh * n_qb + qb;
  auto mu_slice = [&](int s, float (&x)[8]) {
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
    if (rvalid) {
      const float* src = mu + (prow * C + cc) * D + 16 * s + 8 * hh;
      v0 = *reinterpret_cast<const f32x4*>(src);
      v1 = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (i < 4 ? v0[i] : v1[i - 4]) * scale_log2;
  };
  const float wc = rvalid ? w[prow * C + cc] : 0.f;

  const uint16_t* hbase = kplanes + (int64_t)bh * n_kbs * D;
  const uint16_t* lbase = hbase + plane_elems;
  const int n_tiles = (n_kbs + 31) / 32;
  const int tlast = n_tiles - 1;
  const float* tsbase = kF16 ? tscale + (int64_t)bh * n_tiles : nullptr;

  auto kop = [&](const uint16_t* base, int s) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(base + l32 * ROWB + 16 * s + 8 * hh);
  };

  // One pipelined pass over the planes p0 and p1 (p0 only with kF16, and
  // the tile's scale with it).  Tile t sits in LDS stage t%3.  Two register sets alternate (the loop is unrolled by two so
  // they stay in registers): the set holding tile t+2 goes to stage (t+2)%3
  // at the top of the half-iteration for tile t and is reloaded with tile
  // t+4, so every load has two half-iterations to land.  `mma(stage)` forms
  // a tile's logits from LDS, `fix(x, tile)` masks keys past the end (a
  // small block of its own), `epi(x, tile, stage)` consumes them; mma of tile t+1
  // runs in the half-iteration of tile t (stage (t+1)%3 was stored before the
  // previous barrier, and stage (t+2)%3 was last read one half-iteration
  // earlier still).
  auto run_pass = [&](const uint16_t* p0, const uint16_t* p1, auto&& mma, auto&& fix, auto&& epi) {
    struct Regs {
      u32x4 v[NP][NCH];
      float sc;
    };
    Regs ra, rb;
    auto load_tile = [&](Regs& r, int tile) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = i * kScoreT + t;
        int key = 32 * tile + q / CH;
        key = key < n_kbs ? key : n_kbs - 1;  // rows past the end are masked later
        const int64_t off = (int64_t)key * D + 8 * (q % CH);
        if (q < TILE_CH) {
          r.v[0][i] = *reinterpret_cast<const u32x4*>(p0 + off);
          if constexpr (NP == 2) r.v[1][i] = *reinterpret_cast<const u32x4*>(p1 + off);
        }
      }
      if constexpr (kF16) r.sc = tsbase[tile];
    };
    auto store_tile = [&](const Regs& r, int stage) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = i * kScoreT + t;
        if (q < TILE_CH) {
          const int o = (q / CH) * ROWB + 8 * (q % CH);
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) *reinterpret_cast<u32x4*>(&ring[stage][pl][o]) = r.v[pl][i];
        }
      }
      if constexpr (kF16)
        if (t == 0) tsc[stage] = r.sc;
    };
    load_tile(ra, 0);
    store_tile(ra, 0);
    load_tile(rb, min(1, tlast));
    store_tile(rb, 1);
    load_tile(ra, min(2, tlast));
    load_tile(rb, min(3, tlast));
    __syncthreads();
    f32x16 xa = mma(0), xb;
    int st = 0;  // stage of `tile`
    auto nxt = [](int s) { return s == kScoreStages - 1 ? 0 : s + 1; };
    // Each half-iteration's MFMAs and exp2 work form one branch-free block;
    // the MFMAs past the last tile read a stale stage and are discarded.
    for (int tile = 0; tile < n_tiles; tile += 2) {
      const int s1 = nxt(st), s2 = nxt(s1);
      store_tile(ra, s2);
      load_tile(ra, min(tile + 4, tlast));
      fix(xa, tile);
      xb = mma(s1);
      epi(xa, tile, st);
      __syncthreads();
      if (tile + 1 < n_tiles) {
        store_tile(rb, st);  // stage of tile + 3
        load_tile(rb, min(tile + 5, tlast));
        fix(xb, tile + 1);
        xa = mma(s2);
        epi(xb, tile + 1, s1);
        __syncthreads();
      }
      st = s2;
    }
  };

  // centroid operands: bf16 hi/lo (fp32 problems) or fp16 scaled by 2^-e_mu
  // (bf16 problems; e_mu from the work-group's largest |scale_log2 * mu|)
  constexpr int KH = kF16 ? 1 : KS;
  bf16x8 mh[KH], ml[KH];
  f16x8 m16[kF16 ? KS : 1];
  float fac_mu = 1.f;  // 2^e_mu
  if constexpr (kF16) {
    float x[KS][8];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      mu_slice(s, x[s]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[s][i]));
    }
    amax = wave_max(amax);
    if (lane == 0) red[wv] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kScoreWaves; ++i) m = fmaxf(m, red[i]);
    // m = f * 2^x with f in [0.5, 1): m * 2^-(x - 15) lies in [2^14, 2^15)
    int e = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 15 : 0;
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    fac_mu = __builtin_amdgcn_ldexpf(1.f, e);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) m16[s][i] = (_Float16)__builtin_amdgcn_ldexpf(x[s][i], -e);
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      mu_slice(s, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 hb = (__bf16)x[i];
        mh[s][i] = hb;
        ml[s][i] = (__bf16)(x[i] - (float)hb);
      }
    }
  }

  // ---------------- pass 1: softmax normaliser of every centroid ----------------
  float m_run = -INFINITY, s_run = 0.f;
  {
    auto mma1 = [&](int stage) {
      f32x16 x = {};
      if constexpr (kF16) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          x = mfma_f16_32x32x16(__builtin_bit_cast(f16x8, kop(ring[stage][0], s)), m16[s], x);
      } else {
        // one accumulation chain: the small cross terms first, then hi*hi
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kh = __builtin_bit_cast(bf16x8, kop(ring[stage][0], s));
          const bf16x8 kl = __builtin_bit_cast(bf16x8, kop(ring[stage][NP - 1], s));
          x = mfma_bf16_32x32x16(kl, mh[s], x);
          x = mfma_bf16_32x32x16(kh, ml[s], x);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
          x = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, kop(ring[stage][0], s)), mh[s], x);
      }
      return x;
    };
    auto fix1 = [&](f32x16& x, int tile) {
      // lane: centroid l32, keys 32*tile + 8*(v/4) + 4*hh + v%4; only the last
      // tile has keys past the end (clamped copies of the last block)
      if (32 * tile + 32 > n_kbs) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * tile + 8 * (v >> 2) + 4 * hh + (v & 3) >= n_kbs) x[v] = -INFINITY;
      }
    };
    auto epi1 = [&](const f32x16& x, int, int stage) {
      // logit = fac * x, fac a positive power of two (1 for split operands)
      const float fac = kF16 ? tsc[stage] * fac_mu : 1.f;
      float tmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, x[v]);
      const f32x2 tp = pair_x32(tmax);
      tmax = fmaxf(tp[0], tp[1]) * fac;  // finite: every tile has a valid key
      const float m_new = fmaxf(m_run, tmax);
      s_run *= __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int v = 0; v < 16; ++v) s_run += __builtin_amdgcn_exp2f(fmaf(x[v], fac, -m_run));
    };
    run_pass(hbase, lbase, mma1, fix1, epi1);
  }
  {
    const f32x2 sp = pair_x32(s_run);
    s_run = sp[0] + sp[1];
  }
  // log2 of (w_c / normaliser); -inf for an empty cluster
  const float a_c = log2f(wc) - (m_run + log2f(s_run));
  if (hh == 0) a_lds[crow] = a_c;
  __syncthreads();

  // ---------------- pass 2: weighted probabilities summed per query block ----------------
  float a_v[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) a_v[v] = a_lds[32 * wv + 8 * (v >> 2) + 4 * hh + (v & 3)];
  // S rows of this work-group's query blocks through a bounds-checked buffer:
  // stores past the last row are dropped, keys past the end get an offset
  // beyond the range
  const int rows_here = min(G, n_qb - qb0);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      S + ((int64_t)bh * n_qb + qb0) * n_kbs, (short)0, rows_here * n_kbs * 4, 0x00020000);
  auto put = [&](int qrel, int key, float v) {
    const uint32_t off = key < n_kbs ? (uint32_t)(qrel * n_kbs + key) * 4u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), srs, off, 0, 0);
  };
  auto mma2 = [&](int stage) {
    f32x16 x = {};
    if constexpr (kF16) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        x = mfma_f16_32x32x16(m16[s], __builtin_bit_cast(f16x8, kop(ring[stage][0], s)), x);
    } else {
      // one accumulation chain: the small cross terms first, then hi*hi
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kh = __builtin_bit_cast(bf16x8, kop(ring[stage][0], s));
        const bf16x8 kl = __builtin_bit_cast(bf16x8, kop(ring[stage][NP - 1], s));
        x = mfma_bf16_32x32x16(mh[s], kl, x);
        x = mfma_bf16_32x32x16(ml[s], kh, x);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
        x = mfma_bf16_32x32x16(mh[s], __builtin_bit_cast(bf16x8, kop(ring[stage][0], s)), x);
    }
    return x;
  };
  auto fix2 = [](f32x16&, int) {};
  auto epi2 = [&](const f32x16& x, int tile, int stage) {
    // lane: key 32*tile + l32, centroid rows 32*wv + 8*(v/4) + 4*hh + v%4
    const float fac = kF16 ? tsc[stage] * fac_mu : 1.f;
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(x[v], fac, a_v[v]));
    const int key = 32 * tile + l32;
    if constexpr (C == 8) {
      // rows 8g..8g+7 of the wave = one query block; this half holds 4 of them
      float part[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        part[g] = (p[4 * g] + p[4 * g + 1]) + (p[4 * g + 2] + p[4 * g + 3]);
      // the lower half completes blocks 2 and 3, the upper half blocks 0 and 1
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const f32x2 r = cross_x32(part[2 + gg], part[gg]);
        put(4 * wv + (hh ? gg : 2 + gg), key, r[0] + r[1]);
      }
    } else {
      // C == 16: rows 16gp..16gp+15 = one query block
      float part[2];
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        part[gp] = 0.f;
#pragma unroll
        for (int v = 8 * gp; v < 8 * gp + 8; ++v) part[gp] += p[v];
      }
      // the lower half completes block 1, the upper half block 0
      const f32x2 r = cross_x32(part[1], part[0]);
      put(2 * wv + (hh ? 0 : 1), key, r[0] + r[1]);
    }
  };
  run_pass(hbase, lbase, mma2, fix2, epi2);
}

template <int D, int C>
static hipError_t launch_scores_t(const Shape& s, const float* mu, const float* w,
                                  const uint16_t* kplanes, const float* tscale, float* S,
                                  hipStream_t st) {
  constexpr int G = 32 * kScoreWaves / C;
  const int gph = (s.n_qb + G - 1) / G;
  const int n_groups = s.B * s.H * gph;
  const int64_t plane = (int64_t)s.B * s.H * s.n_kbs * s.D;
  if (s.bf16)
    k_scores<D, C, true><<<n_groups, kScoreT, 0, st>>>(mu, w, kplanes, tscale, S, s.n_qb, s.n_kbs,
                                                       gph, n_groups, plane, s.scale * kLog2e);
  else
    k_scores<D, C, false><<<n_groups, kScoreT, 0, st>>>(mu, w, kplanes, nullptr, S, s.n_qb,
                                                        s.n_kbs, gph, n_groups, plane,
                                                        s.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_scores(const Shape& s, const float* mu, const float* w, const uint16_t* kplanes,
                         const float* tscale, float* S, hipStream_t st) {
  if (s.D == 128)
    return s.n_clusters == 8 ? launch_scores_t<128, 8>(s, mu, w, kplanes, tscale, S, st)
                             : launch_scores_t<128, 16>(s, mu, w, kplanes, tscale, S, st);
  return s.n_clusters == 8 ? launch_scores_t<64, 8>(s, mu, w, kplanes, tscale, S, st)
                           : launch_scores_t<64, 16>(s, mu, w, kplanes, tscale, S, st);
}

}  // namespace abatt
