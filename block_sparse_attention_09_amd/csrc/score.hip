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
// means arrive as bf16 hi and lo planes written by the key-means kernel):
//   pass 1: per-centroid running max and sum of exp2 (the softmax normaliser);
//   pass 2: p = exp2(logit + log2 w_c - lse_c), summed over the C centroids of
//           each query block and written to S.
// The dot products run on bf16 MFMA with both operands split into bf16 high
// and low parts (hi*hi + hi*lo + lo*hi, fp32 accumulation), which keeps the
// logits within ~2^-16 relative of fp32.  Pass 1 uses the key means as the
// MFMA A operand (a lane then holds 16 keys of one centroid: cheap running
// max), pass 2 uses the centroids as A (a lane holds 16 centroids of one key:
// cheap sum over a query block's centroids).  The operand registers are the
// same in both layouts.
#include "common.h"
#include "kernels.h"

namespace abatt {

constexpr int kScoreWaves = 8;                 // 256 centroid rows per work-group
constexpr int kScoreT = 64 * kScoreWaves;
constexpr int kScoreStages = 3;                // LDS ring of key-mean tiles

template <int D, int C>
__global__ __launch_bounds__(kScoreT, 1) void k_scores(const float* __restrict__ mu,
                                                       const float* __restrict__ w,
                                                       const uint16_t* __restrict__ kplanes,
                                                       float* __restrict__ S, int n_qb, int n_kbs,
                                                       int groups_per_head, int n_groups,
                                                       int64_t plane_elems, float scale_log2) {
  constexpr int ROWS = 32 * kScoreWaves;  // centroid rows per work-group
  constexpr int G = ROWS / C;             // query blocks per work-group
  constexpr int KS = D / 16;              // MFMA k-steps
  constexpr int ROWB = D + 8;             // LDS row stride (bf16), padded: conflict-free reads
  constexpr int CH = D / 8;               // 16-byte chunks per key-mean row
  constexpr int TILE_CH = 32 * CH;        // chunks per plane per 32-key tile
  constexpr int NCH = (TILE_CH + kScoreT - 1) / kScoreT;  // per thread per plane
  __shared__ __align__(16) uint16_t khi[kScoreStages][32 * ROWB];
  __shared__ __align__(16) uint16_t klo[kScoreStages][32 * ROWB];
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
  bf16x8 mh[KS], ml[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
    if (rvalid) {
      const float* src = mu + (prow * C + cc) * D + 16 * s + 8 * hh;
      v0 = *reinterpret_cast<const f32x4*>(src);
      v1 = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (i < 4 ? v0[i] : v1[i - 4]) * scale_log2;
      const uint32_t hb = f32_to_bf16_bits(x);
      const uint32_t lb = f32_to_bf16_bits(x - bf16_bits_to_f32(hb));
      mh[s][i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
      ml[s][i] = __builtin_bit_cast(__bf16, (uint16_t)lb);
    }
  }
  const float wc = rvalid ? w[prow * C + cc] : 0.f;

  const uint16_t* hbase = kplanes + (int64_t)bh * n_kbs * D;
  const uint16_t* lbase = hbase + plane_elems;
  const int n_tiles = (n_kbs + 31) / 32;
  const int tlast = n_tiles - 1;

  // Tile pipeline: tile t is computed from LDS stage t%3.  Two register sets
  // alternate (the loop is unrolled by two so they stay in registers): at the
  // top of iteration t the set holding tile t+2 goes to stage (t+2)%3 (last
  // read in iteration t-1, which ended with a barrier) and the same set is
  // reloaded with tile t+4, so every load has two iterations to land.
  struct Regs {
    u32x4 h[NCH], l[NCH];
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
        r.h[i] = *reinterpret_cast<const u32x4*>(hbase + off);
        r.l[i] = *reinterpret_cast<const u32x4*>(lbase + off);
      }
    }
  };
  auto store_tile = [&](const Regs& r, int stage) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = i * kScoreT + t;
      if (q < TILE_CH) {
        const int o = (q / CH) * ROWB + 8 * (q % CH);
        *reinterpret_cast<u32x4*>(&khi[stage][o]) = r.h[i];
        *reinterpret_cast<u32x4*>(&klo[stage][o]) = r.l[i];
      }
    }
  };
  auto kop = [&](const uint16_t* base, int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(base + l32 * ROWB + 16 * s + 8 * hh);
  };
  auto prologue = [&]() {
    load_tile(ra, 0);
    store_tile(ra, 0);
    load_tile(rb, min(1, tlast));
    store_tile(rb, 1 % kScoreStages);
    load_tile(ra, min(2, tlast));
    load_tile(rb, min(3, tlast));
    __syncthreads();
  };
  // one pipelined pass; `body(tile, stage)` computes a tile
  auto run_pass = [&](auto&& body) {
    prologue();
    int stage = 0;
    for (int tile = 0; tile < n_tiles; tile += 2) {
      store_tile(ra, (stage + 2) % kScoreStages);
      load_tile(ra, min(tile + 4, tlast));
      body(tile, stage);
      __syncthreads();
      stage = (stage + 1) % kScoreStages;
      if (tile + 1 < n_tiles) {
        store_tile(rb, (stage + 2) % kScoreStages);
        load_tile(rb, min(tile + 5, tlast));
        body(tile + 1, stage);
        __syncthreads();
        stage = (stage + 1) % kScoreStages;
      }
    }
  };

  // ---------------- pass 1: softmax normaliser of every centroid ----------------
  float m_run = -INFINITY, s_run = 0.f;
  run_pass([&](int tile, int stage) {
    // one accumulation chain: the small cross terms first, then hi*hi
    f32x16 x = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kh = kop(khi[stage], s), kl = kop(klo[stage], s);
      x = mfma_bf16_32x32x16(kl, mh[s], x);
      x = mfma_bf16_32x32x16(kh, ml[s], x);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) x = mfma_bf16_32x32x16(kop(khi[stage], s), mh[s], x);
    // lane: centroid l32, keys 32*tile + 8*(v/4) + 4*hh + v%4
    if (32 * tile + 32 > n_kbs) {  // only the last tile has keys past the end
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * tile + 8 * (v >> 2) + 4 * hh + (v & 3) >= n_kbs) x[v] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, x[v]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax > m_run) {
      s_run *= __builtin_amdgcn_exp2f(m_run - tmax);
      m_run = tmax;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s_run += __builtin_amdgcn_exp2f(x[v] - m_run);
  });
  s_run += __shfl_xor(s_run, 32);
  // log2 of (w_c / normaliser); -inf for an empty cluster
  const float a_c = log2f(wc) - (m_run + log2f(s_run));
  if (hh == 0) a_lds[crow] = a_c;
  __syncthreads();

  // ---------------- pass 2: weighted probabilities summed per query block ----------------
  float a_v[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) a_v[v] = a_lds[32 * wv + 8 * (v >> 2) + 4 * hh + (v & 3)];
  float* srow_base = S + ((int64_t)bh * n_qb) * n_kbs;
  run_pass([&](int tile, int stage) {
    f32x16 x = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kh = kop(khi[stage], s), kl = kop(klo[stage], s);
      x = mfma_bf16_32x32x16(mh[s], kl, x);
      x = mfma_bf16_32x32x16(ml[s], kh, x);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) x = mfma_bf16_32x32x16(mh[s], kop(khi[stage], s), x);
    // lane: key 32*tile + l32, centroid rows 32*wv + 8*(v/4) + 4*hh + v%4
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(x[v] + a_v[v]);
    const int key = 32 * tile + l32;
    if constexpr (C == 8) {
      // rows 8g..8g+7 of the wave = one query block; this half holds 4 of them
      float tot[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float part = (p[4 * g] + p[4 * g + 1]) + (p[4 * g + 2] + p[4 * g + 3]);
        tot[g] = part + __shfl_xor(part, 32);
      }
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * hh + gg;
        const int q = qb0 + 4 * wv + g;
        if (q < n_qb && key < n_kbs) srow_base[(int64_t)q * n_kbs + key] = tot[g];
      }
    } else {
      // C == 16: rows 16gp..16gp+15 = one query block
      float tot[2];
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float part = 0.f;
#pragma unroll
        for (int v = 8 * gp; v < 8 * gp + 8; ++v) part += p[v];
        tot[gp] = part + __shfl_xor(part, 32);
      }
      const int q = qb0 + 2 * wv + hh;
      if (q < n_qb && key < n_kbs) srow_base[(int64_t)q * n_kbs + key] = tot[hh];
    }
  });
}

template <int D, int C>
static hipError_t launch_scores_t(const Shape& s, const float* mu, const float* w,
                                  const uint16_t* kplanes, float* S, hipStream_t st) {
  constexpr int G = 32 * kScoreWaves / C;
  const int gph = (s.n_qb + G - 1) / G;
  const int n_groups = s.B * s.H * gph;
  const int64_t plane = (int64_t)s.B * s.H * s.n_kbs * s.D;
  k_scores<D, C><<<n_groups, kScoreT, 0, st>>>(mu, w, kplanes, S, s.n_qb, s.n_kbs, gph, n_groups,
                                           plane, s.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_scores(const Shape& s, const float* mu, const float* w, const uint16_t* kplanes,
                         float* S, hipStream_t st) {
  if (s.D == 128)
    return s.n_clusters == 8 ? launch_scores_t<128, 8>(s, mu, w, kplanes, S, st)
                             : launch_scores_t<128, 16>(s, mu, w, kplanes, S, st);
  return s.n_clusters == 8 ? launch_scores_t<64, 8>(s, mu, w, kplanes, S, st)
                           : launch_scores_t<64, 16>(s, mu, w, kplanes, S, st);
}

}  // namespace abatt
