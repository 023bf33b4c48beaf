// Cluster-weighted block scores: the scoring half of IBCS.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques", IBCS paragraph: a key block's score is the weighted attention
// of the block's centroids to its averaged keys.
//   s_j = sum_c w_c * softmax_j(scale * mu_c . kmean_j),   j over sparse blocks.
//
// One work-group holds 128 centroid rows (128/C query blocks of one head) and
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

template <int D, int C>
__global__ __launch_bounds__(256, 2) void k_scores(const float* __restrict__ mu,
                                                   const float* __restrict__ w,
                                                   const uint16_t* __restrict__ kplanes,
                                                   float* __restrict__ S, int n_qb, int n_kbs,
                                                   int groups_per_head, int n_groups,
                                                   int64_t plane_elems, float scale_log2) {
  constexpr int G = 128 / C;      // query blocks per work-group
  constexpr int KS = D / 16;      // MFMA k-steps
  constexpr int ROWB = D + 8;     // LDS row stride (bf16), padded: conflict-free operand reads
  constexpr int CH = D / 8;       // 16-byte chunks per key-mean row
  constexpr int NCH = CH / 8;     // chunks per thread per plane per 32-key tile
  __shared__ __align__(16) uint16_t khi[2][32 * ROWB];
  __shared__ __align__(16) uint16_t klo[2][32 * ROWB];
  __shared__ float a_lds[128];

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
  u32x4 rh[NCH], rl[NCH];

  // Tile pipeline (as in the attention kernel): tile t is computed from LDS
  // stage t%2 while the registers carry tile t+1; at the top of iteration t
  // the registers go to the free stage and the loads of tile t+2 are issued.
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = i * 256 + t;
      int key = 32 * tile + q / CH;
      key = key < n_kbs ? key : n_kbs - 1;  // rows past the end are masked later
      const int64_t off = (int64_t)key * D + 8 * (q % CH);
      rh[i] = *reinterpret_cast<const u32x4*>(hbase + off);
      rl[i] = *reinterpret_cast<const u32x4*>(lbase + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = i * 256 + t;
      const int o = (q / CH) * ROWB + 8 * (q % CH);
      *reinterpret_cast<u32x4*>(&khi[buf][o]) = rh[i];
      *reinterpret_cast<u32x4*>(&klo[buf][o]) = rl[i];
    }
  };
  auto kop = [&](const uint16_t* base, int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(base + l32 * ROWB + 16 * s + 8 * hh);
  };
  auto prologue = [&]() {
    load_tile(0);
    store_tile(0);
    load_tile(n_tiles > 1 ? 1 : 0);
    __syncthreads();
  };

  // ---------------- pass 1: softmax normaliser of every centroid ----------------
  float m_run = -INFINITY, s_run = 0.f;
  prologue();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    store_tile(buf ^ 1);
    load_tile(min(tile + 2, tlast));
    f32x16 big = {}, small = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kh = kop(khi[buf], s), kl = kop(klo[buf], s);
      small = mfma_bf16_32x32x16(kl, mh[s], small);
      small = mfma_bf16_32x32x16(kh, ml[s], small);
      big = mfma_bf16_32x32x16(kh, mh[s], big);
    }
    // lane: centroid l32, keys 32*tile + 8*(v/4) + 4*hh + v%4
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = 32 * tile + 8 * (v >> 2) + 4 * hh + (v & 3);
      x[v] = key < n_kbs ? big[v] + small[v] : -INFINITY;
      tmax = fmaxf(tmax, x[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax > m_run) {
      s_run *= __builtin_amdgcn_exp2f(m_run - tmax);
      m_run = tmax;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s_run += __builtin_amdgcn_exp2f(x[v] - m_run);
    __syncthreads();
  }
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
  prologue();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    store_tile(buf ^ 1);
    load_tile(min(tile + 2, tlast));
    f32x16 big = {}, small = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kh = kop(khi[buf], s), kl = kop(klo[buf], s);
      small = mfma_bf16_32x32x16(mh[s], kl, small);
      small = mfma_bf16_32x32x16(ml[s], kh, small);
      big = mfma_bf16_32x32x16(mh[s], kh, big);
    }
    // lane: key 32*tile + l32, centroid rows 32*wv + 8*(v/4) + 4*hh + v%4
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(big[v] + small[v] + a_v[v]);
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
    __syncthreads();
  }
}

template <int D, int C>
static hipError_t launch_scores_t(const Shape& s, const float* mu, const float* w,
                                  const uint16_t* kplanes, float* S, hipStream_t st) {
  constexpr int G = 128 / C;
  const int gph = (s.n_qb + G - 1) / G;
  const int n_groups = s.B * s.H * gph;
  const int64_t plane = (int64_t)s.B * s.H * s.n_kbs * s.D;
  k_scores<D, C><<<n_groups, 256, 0, st>>>(mu, w, kplanes, S, s.n_qb, s.n_kbs, gph, n_groups,
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
