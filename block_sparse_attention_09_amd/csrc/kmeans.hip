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
    if (h == 0 && valid) assign[p] = a;
    __syncthreads();
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

hipError_t launch_kmeans(const Shape& s, const void* Q, float* mu, float* w, hipStream_t st) {
  if (s.bf16)
    return s.D == 128 ? launch_kmeans_d<uint16_t, 128>(s, Q, mu, w, st)
                      : launch_kmeans_d<uint16_t, 64>(s, Q, mu, w, st);
  return s.D == 128 ? launch_kmeans_d<float, 128>(s, Q, mu, w, st)
                    : launch_kmeans_d<float, 64>(s, Q, mu, w, st);
}

}  // namespace abatt
