// Per-query-block Lloyd k-means: the clustering half of IBCS.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques", IBCS paragraph: the queries of each 128-token block (original
// order) are grouped into clusters; each cluster keeps its centroid and the
// share of the block's queries as its weight.
//
// One work-group (4 waves) per query block.  The block's raw queries are
// staged once in LDS in their input dtype.  Thread t owns point t/2 and half
// of its dimensions in registers (the distance pass), so every iteration reads
// only the C centroids from LDS (broadcast reads).  The update pass is
// deterministic: wave 0 lists each cluster's members in ascending token order
// with ballots, then thread (dim, cluster group) sums its members in that
// order.  Init: centroid c = query floor(c*n/C); ties go to the lower
// centroid index; an empty cluster keeps its centroid; the weights come from
// the last assignment.
#include "common.h"
#include "kernels.h"

namespace abatt {

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) {
  return *p;
}

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void k_kmeans(const T* __restrict__ Q, float* __restrict__ mu_out,
                                                float* __restrict__ w_out, int N, int n_qb,
                                                int iters) {
  constexpr int QB = 128;
  constexpr int HD = D / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  T* xs = reinterpret_cast<T*>(smem);                                   // [QB][D]
  float* mus = reinterpret_cast<float*>(smem + QB * D * sizeof(T));     // [C][D]
  int* assign = reinterpret_cast<int*>(mus + C * D);                    // [QB]
  int* perm = assign + QB;                                              // [QB]
  int* cstart = perm + QB;                                              // [C]
  int* ccount = cstart + C;                                             // [C]

  const int r = blockIdx.x;
  const int qb = r % n_qb;
  const int64_t bh = r / n_qb;
  const int q0 = qb * QB;
  const int n = min(QB, N - q0);
  const int t = threadIdx.x;

  {  // stage the block's queries (n rows, contiguous) with 16-byte loads
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + (bh * N + q0) * D);
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
    const int chunks = n * D * (int)sizeof(T) / 16;
    for (int i = t; i < chunks; i += 256) dst[i] = src[i];
  }
  if (t < QB) assign[t] = -1;
  __syncthreads();
  for (int i = t; i < C * D; i += 256) {
    const int c = i / D, e = i % D;
    mus[i] = load_as_f32<T>(xs + ((c * n) / C) * D + e);
  }
  const int p = t >> 1, h = t & 1;
  const bool valid = p < n;
  float xr[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) xr[e] = valid ? load_as_f32<T>(xs + p * D + h * HD + e) : 0.f;
  __syncthreads();

  const int lane = t & 63;
  const uint32_t below_lo = lane >= 32 ? 0xffffffffu : ((1u << lane) - 1u);
  const uint32_t below_hi = lane <= 32 ? 0u : ((1u << (lane - 32)) - 1u);
  constexpr int G = 256 / D;  // cluster groups in the update pass
  const int ue = t % D, ug = t / D;

  for (int it = 0; it < iters; ++it) {
    // assignment: nearest centroid by squared distance of the differences
    float best = 0.f;
    int a = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float* m = mus + c * D + h * HD;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < HD; e += 4) {
        const f32x4 mv = *reinterpret_cast<const f32x4*>(m + e);
        const float d0 = xr[e] - mv[0], d1 = xr[e + 1] - mv[1];
        const float d2 = xr[e + 2] - mv[2], d3 = xr[e + 3] - mv[3];
        acc = fmaf(d0, d0, acc);
        acc = fmaf(d1, d1, acc);
        acc = fmaf(d2, d2, acc);
        acc = fmaf(d3, d3, acc);
      }
      const float tot = acc + __shfl_xor(acc, 1);
      if (c == 0 || tot < best) {
        best = tot;
        a = c;
      }
    }
    // an assignment equal to the previous one is a fixed point: the update
    // would reproduce the centroids and counts, and so would every later
    // iteration, so the loop ends with the same result it would reach at iters
    const bool changed = h == 0 && valid && (it == 0 || assign[p] != a);
    if (h == 0 && valid) assign[p] = a;
    if (!__syncthreads_or(changed)) break;
    // member lists in ascending token order (wave 0)
    if (t < 64) {
      const int a0 = assign[t], a1 = assign[t + 64];
      int base = 0;
      for (int c = 0; c < C; ++c) {
        const uint64_t m0 = __ballot(a0 == c), m1 = __ballot(a1 == c);
        const int c0 = __popcll(m0), c1 = __popcll(m1);
        if (a0 == c)
          perm[base + __popc((uint32_t)m0 & below_lo) + __popc((uint32_t)(m0 >> 32) & below_hi)] = t;
        if (a1 == c)
          perm[base + c0 + __popc((uint32_t)m1 & below_lo) + __popc((uint32_t)(m1 >> 32) & below_hi)] =
              t + 64;
        if (t == 0) {
          cstart[c] = base;
          ccount[c] = c0 + c1;
        }
        base += c0 + c1;
      }
    }
    __syncthreads();
    // update: mean of the members, summed in token order
    for (int c = ug; c < C; c += G) {
      const int cnt = ccount[c];
      if (cnt > 0) {
        const int st = cstart[c];
        float sum = 0.f;
        for (int i = 0; i < cnt; ++i) sum += load_as_f32<T>(xs + perm[st + i] * D + ue);
        mus[c * D + ue] = sum / (float)cnt;
      }
    }
    __syncthreads();
  }

  float* mo = mu_out + (int64_t)r * C * D;
  for (int i = t; i < C * D; i += 256) mo[i] = mus[i];
  if (t < C) w_out[(int64_t)r * C + t] = (float)ccount[t] / (float)n;
}

// bf16 queries: the same Lloyd iterations with both contractions on the
// matrix cores (v_mfma_f32_16x16x32_bf16).  Per iteration and block:
//   dots[c][p] = mu_c . x_p  as a [16 x D] centroid tile times X^T, each
//     centroid split into three bf16 planes (hi + mid + lo = its fp32 value),
//     so the products are exact and the sums fp32 as in the scalar path; the
//     queries are bf16 already;
//   sums[e][c] = sum_p x_p[e] onehot[c][p]  (exact products, fp32 sums), and
//     counts[c] from the same one-hot operand.
// Wave w owns points 32w..32w+31 in the assignment and dims D/4*w.. in the
// update; the query operands of both products are built once, in registers.
// Lane layout of the 16x16 product: A row = B column = lane % 16 (k slots by
// lane / 16), D[4*(lane/16) + v][lane % 16] in accumulator element v.  The
// update thus leaves lane (g, i) with cluster i and 4 consecutive dims, which
// it rounds to the planes with packed conversions and 8-byte writes.
template <int D, int C>
__global__ __launch_bounds__(256) void k_kmeans_mfma(const uint16_t* __restrict__ Q,
                                                     float* __restrict__ mu_out,
                                                     float* __restrict__ w_out, int N, int n_qb,
                                                     int iters) {
  constexpr int QB = 128;
  constexpr int KS = D / 32;  // k steps of the distance product
  constexpr int UT = D / 64;  // 16-dim update tiles per wave
  constexpr int XS = D + 8;   // padded row of the staged queries / planes (bf16)
  constexpr int OS = QB + 8;  // padded row of the one-hot matrix (bf16)
  static_assert(C % 4 == 0 && C <= 16, "one 16-row centroid tile");
  // the staged queries are only read while the operands are built; the
  // centroid planes reuse their space afterwards
  __shared__ __align__(16) uint16_t lds[QB * XS];
  __shared__ __align__(16) uint16_t oh[16 * OS];  // onehot[c][p] of the last assignment
  __shared__ __align__(16) float npart[4][16];    // per-wave partial |mu_c|^2
  __shared__ int wchg[2][4];                      // per-wave "assignment changed", by iteration parity
  uint16_t* xs = lds;
  uint16_t* planes = lds;  // [3][16][XS] after set-up

  const int r = blockIdx.x;
  const int qb = r % n_qb;
  const int64_t bh = r / n_qb;
  const int q0 = qb * QB;
  const int n = min(QB, N - q0);
  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63, g = l >> 4, i = l & 15;

  {  // stage the block's queries; rows past the end are zero
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + (bh * N + q0) * D);
    constexpr int CH = D / 8;
    for (int k = t; k < QB * CH; k += 256) {
      const int row = k / CH, ch = k % CH;
      const u32x4 v = row < n ? src[k] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(xs + row * XS + 8 * ch) = v;
    }
  }
  for (int k = t; k < 16 * OS / 2; k += 256) reinterpret_cast<uint32_t*>(oh)[k] = 0u;
  __syncthreads();

  // distance operand (B = X^T): point 32w + 16u + i, dims 32ks + 8g .. +7
  bf16x8 xb[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xb[u][ks] = *reinterpret_cast<const bf16x8*>(xs + (32 * w + 16 * u + i) * XS + 32 * ks + 8 * g);
  // update operand (A = X^T): dim D/4*w + 16u + i, points 32ks + 8g .. +7
  bf16x8 ub[UT][4];
#pragma unroll
  for (int u = 0; u < UT; ++u)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint16_t* col = xs + (32 * ks + 8 * g) * XS + (D / 4) * w + 16 * u + i;
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (uint32_t)col[(2 * j) * XS] | ((uint32_t)col[(2 * j + 1) * XS] << 16);
      ub[u][ks] = __builtin_bit_cast(bf16x8, v);
    }
  // centroids in registers: mreg[u][v] = mu[i][D/4*w + 16u + 4g + v]; the
  // initial centroid c is query floor(c*n/C); rows c >= C stay zero
  float mreg[UT][4];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const u32x2 x = i < C ? *reinterpret_cast<const u32x2*>(xs + ((i * n) / C) * XS + (D / 4) * w +
                                                            16 * u + 4 * g)
                          : u32x2{0u, 0u};
    mreg[u][0] = bf16_bits_to_f32(x[0] & 0xffffu);
    mreg[u][1] = bf16_bits_to_f32(x[0] >> 16);
    mreg[u][2] = bf16_bits_to_f32(x[1] & 0xffffu);
    mreg[u][3] = bf16_bits_to_f32(x[1] >> 16);
  }
  __syncthreads();

  // centroids -> bf16 planes and per-wave partial squared norms
  auto publish = [&]() {
    float sq = 0.f;
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      uint32_t hw[2], mw[2], lw[2];
#pragma unroll
      for (int v2 = 0; v2 < 2; ++v2) {
        const f32x2 m = {mreg[u][2 * v2], mreg[u][2 * v2 + 1]};
        const bf16x2 h = __builtin_convertvector(m, bf16x2);
        const f32x2 r1 = m - __builtin_convertvector(h, f32x2);
        const bf16x2 md = __builtin_convertvector(r1, bf16x2);
        const bf16x2 lo = __builtin_convertvector(r1 - __builtin_convertvector(md, f32x2), bf16x2);
        hw[v2] = __builtin_bit_cast(uint32_t, h);
        mw[v2] = __builtin_bit_cast(uint32_t, md);
        lw[v2] = __builtin_bit_cast(uint32_t, lo);
        sq = fmaf(m[0], m[0], sq);
        sq = fmaf(m[1], m[1], sq);
      }
      const int e = i * XS + (D / 4) * w + 16 * u + 4 * g;
      *reinterpret_cast<u32x2*>(planes + e) = u32x2{hw[0], hw[1]};
      *reinterpret_cast<u32x2*>(planes + 16 * XS + e) = u32x2{mw[0], mw[1]};
      *reinterpret_cast<u32x2*>(planes + 32 * XS + e) = u32x2{lw[0], lw[1]};
    }
    {
      const f32x2 r16 = pair_x16(sq);
      sq = r16[0] + r16[1];
      const f32x2 r32 = pair_x32(sq);
      sq = r32[0] + r32[1];
    }
    if (g == 0) npart[w][i] = sq;
  };
  publish();
  __syncthreads();

  int cnt = 0;
  int prev[2] = {-1, -1};  // this lane's points' assignments in the last iteration
  for (int it = 0; it < iters; ++it) {
    // assignment: nearest centroid by |mu_c|^2 - 2 x.mu_c; ties -> lower index
    bool changed = false;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(planes + pl * 16 * XS + i * XS + 32 * ks + 8 * g);
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = mfma_bf16_16x16x32(a, xb[u][ks], acc[u]);
      }
    }
    f32x4 mn = *reinterpret_cast<const f32x4*>(&npart[0][4 * g]);
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) mn += *reinterpret_cast<const f32x4*>(&npart[ww][4 * g]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float best = 0.f;
      int a = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float d = 4 * g + v < C ? fmaf(-2.f, acc[u][v], mn[v]) : __builtin_inff();
        if (v == 0 || d < best) {
          best = d;
          a = 4 * g + v;
        }
      }
      // lexicographic minimum of (distance, index) over the lane pairs l, l^16
      // (and l^32 for 16 clusters)
      auto pick = [&](const f32x2& b2, const f32x2& a2) {
        const int a0 = __float_as_int(a2[0]), a1 = __float_as_int(a2[1]);
        const bool hi = b2[1] < b2[0] || (b2[1] == b2[0] && a1 < a0);
        best = hi ? b2[1] : b2[0];
        a = hi ? a1 : a0;
      };
      pick(pair_x16(best), pair_x16(__int_as_float(a)));
      if constexpr (C > 8) pick(pair_x32(best), pair_x32(__int_as_float(a)));
      // one-hot column of point p (rows c >= C and points p >= n stay zero)
      const int p = 32 * w + 16 * u + i;
      changed |= p < n && a != prev[u];
      prev[u] = a;
      if (4 * g < C && p < n) {
#pragma unroll
        for (int v = 0; v < 4; ++v) oh[(4 * g + v) * OS + p] = a == 4 * g + v ? 0x3f80u : 0u;
      }
    }
    // an assignment equal to the previous one is a fixed point: the update
    // would reproduce the centroids and counts (and so would every later
    // iteration), so the loop ends with the result it would reach at iters.
    // One vote per wave and one barrier (which also publishes the one-hot
    // matrix); the two flag sets alternate, so a set is rewritten only after
    // the barrier that ends the next iteration.
    {
      const bool wc = __any(changed);
      if (l == 0) wchg[it & 1][w] = wc;
      __syncthreads();
      const int* f = wchg[it & 1];
      if (!(f[0] | f[1] | f[2] | f[3])) break;
    }
    // update: member sums on the matrix cores; counts from the one-hot bits
    f32x4 sum[UT];
#pragma unroll
    for (int u = 0; u < UT; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    cnt = 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(oh + i * OS + 32 * ks + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) cnt += __popc(b[j] & 0x00800080u);  // bit 7 of bf16 1.0
      const bf16x8 B = __builtin_bit_cast(bf16x8, b);
#pragma unroll
      for (int u = 0; u < UT; ++u) sum[u] = mfma_bf16_16x16x32(ub[u][ks], B, sum[u]);
    }
    cnt = sum_x32(sum_x16(cnt));  // members of cluster i
    if (cnt > 0) {
      // quotient sum / cnt: reciprocal estimate plus one residual correction
      const float fc = (float)cnt;
      const float inv = 1.f / fc;
#pragma unroll
      for (int u = 0; u < UT; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float q = sum[u][v] * inv;
          mreg[u][v] = fmaf(fmaf(-q, fc, sum[u][v]), inv, q);
        }
    }
    // every wave read this iteration's planes before the barrier above
    publish();
    __syncthreads();
  }

  if (i < C) {
    float* mo = mu_out + ((int64_t)r * C + i) * D + (D / 4) * w + 4 * g;
#pragma unroll
    for (int u = 0; u < UT; ++u)
      *reinterpret_cast<f32x4*>(mo + 16 * u) = f32x4{mreg[u][0], mreg[u][1], mreg[u][2], mreg[u][3]};
    if (w == 0 && g == 0) w_out[(int64_t)r * C + i] = (float)cnt / (float)n;
  }
}

template <typename T, int D, int C>
static hipError_t launch_kmeans_t(const Shape& s, const void* Q, float* mu, float* w,
                                  hipStream_t st) {
  const size_t lds = 128 * D * sizeof(T) + C * D * sizeof(float) + (256 + 2 * C) * sizeof(int);
  auto kern = k_kmeans<T, D, C>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  kern<<<s.R, 256, lds, st>>>((const T*)Q, mu, w, s.N, s.n_qb, s.kmeans_iters);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_kmeans_d(const Shape& s, const void* Q, float* mu, float* w,
                                  hipStream_t st) {
  if (s.n_clusters == 8) return launch_kmeans_t<T, D, 8>(s, Q, mu, w, st);
  return launch_kmeans_t<T, D, 16>(s, Q, mu, w, st);
}

template <int D, int C>
static hipError_t launch_kmeans_mfma(const Shape& s, const void* Q, float* mu, float* w,
                                     hipStream_t st) {
  k_kmeans_mfma<D, C><<<s.R, 256, 0, st>>>((const uint16_t*)Q, mu, w, s.N, s.n_qb, s.kmeans_iters);
  return hipGetLastError();
}

hipError_t launch_kmeans(const Shape& s, const void* Q, float* mu, float* w, hipStream_t st) {
  if (s.bf16) {
    if (s.n_clusters == 8)
      return s.D == 128 ? launch_kmeans_mfma<128, 8>(s, Q, mu, w, st)
                        : launch_kmeans_mfma<64, 8>(s, Q, mu, w, st);
    return s.D == 128 ? launch_kmeans_mfma<128, 16>(s, Q, mu, w, st)
                      : launch_kmeans_mfma<64, 16>(s, Q, mu, w, st);
  }
  return s.D == 128 ? launch_kmeans_d<float, 128>(s, Q, mu, w, st)
                    : launch_kmeans_d<float, 64>(s, Q, mu, w, st);
}

}  // namespace abatt
