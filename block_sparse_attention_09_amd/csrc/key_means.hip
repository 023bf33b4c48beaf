// Mean key of every sparse key block (4 consecutive tokens by default).
//
// [hamidun] "AB-Attention's three techniques", IBCS paragraph: key blocks are
// scored through their averaged keys; the third technique fixes the key block
// at 4 consecutive tokens (and compares it with 128).  HBM-bound: each block's
// rows are read once (16-byte lane loads, consecutive lanes on consecutive
// bytes) and one fp32 row is written.  Blocks of kb > 4 tokens are summed in
// token order, like the 4-token form, then scaled by 1/kb (exact, kb a power
// of two).
#include "common.h"
#include "kernels.h"

namespace abatt {

// Mean of dims 8c..8c+7 of one bf16 key block whose first row is `src`.
template <int D>
__device__ __forceinline__ void block_mean8_bf16(const uint16_t* __restrict__ src, int kb,
                                                 float (&out)[8]) {
  if (kb == 4) {
    u32x4 r0 = *reinterpret_cast<const u32x4*>(src);
    u32x4 r1 = *reinterpret_cast<const u32x4*>(src + D);
    u32x4 r2 = *reinterpret_cast<const u32x4*>(src + 2 * D);
    u32x4 r3 = *reinterpret_cast<const u32x4*>(src + 3 * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = bf16_bits_to_f32(r0[e] & 0xffffu), b0 = bf16_bits_to_f32(r0[e] >> 16);
      const float a1 = bf16_bits_to_f32(r1[e] & 0xffffu), b1 = bf16_bits_to_f32(r1[e] >> 16);
      const float a2 = bf16_bits_to_f32(r2[e] & 0xffffu), b2 = bf16_bits_to_f32(r2[e] >> 16);
      const float a3 = bf16_bits_to_f32(r3[e] & 0xffffu), b3 = bf16_bits_to_f32(r3[e] >> 16);
      out[2 * e] = (((a0 + a1) + a2) + a3) * 0.25f;
      out[2 * e + 1] = (((b0 + b1) + b2) + b3) * 0.25f;
    }
  } else {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int tk = 0; tk < kb; ++tk) {
      const u32x4 rr = *reinterpret_cast<const u32x4*>(src + (int64_t)tk * D);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_bits_to_f32(rr[e] & 0xffffu);
        acc[2 * e + 1] += bf16_bits_to_f32(rr[e] >> 16);
      }
    }
    const float inv = 1.f / (float)kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = acc[e] * inv;
  }
}

// bf16 input: one thread = 8 dims of one block (4 x 16-byte loads).  Writes
// either the fp32 means or (kSplit) the means as two bf16 planes hi + lo with
// hi = bf16(mean), lo = bf16(mean - hi): the operands of the split-bf16
// scoring MFMAs, which then stage them without any conversion.
template <int D, bool kSplit>
__global__ __launch_bounds__(256) void k_key_means_bf16(const uint16_t* __restrict__ K,
                                                        float* __restrict__ kmean,
                                                        int64_t total, int N, int n_kbs,
                                                        int kb) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % CH);
    const int64_t bj = i / CH;  // bh * n_kbs + j
    const int j = (int)(bj % n_kbs);
    const int64_t bh = bj / n_kbs;
    float out[8];
    block_mean8_bf16<D>(K + (bh * N + (int64_t)kb * j) * D + 8 * c, kb, out);
    if constexpr (kSplit) {
      uint16_t* hi = reinterpret_cast<uint16_t*>(kmean);
      uint16_t* lo = hi + total * 8;
      u32x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h0 = f32_to_bf16_bits(out[2 * e]), h1 = f32_to_bf16_bits(out[2 * e + 1]);
        const uint32_t l0 = f32_to_bf16_bits(out[2 * e] - bf16_bits_to_f32(h0));
        const uint32_t l1 = f32_to_bf16_bits(out[2 * e + 1] - bf16_bits_to_f32(h1));
        h[e] = h0 | (h1 << 16);
        l[e] = l0 | (l1 << 16);
      }
      *reinterpret_cast<u32x4*>(hi + bj * D + 8 * c) = h;
      *reinterpret_cast<u32x4*>(lo + bj * D + 8 * c) = l;
    } else {
      float* dst = kmean + bj * D + 8 * c;
      *reinterpret_cast<f32x4*>(dst) = f32x4{out[0], out[1], out[2], out[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{out[4], out[5], out[6], out[7]};
    }
  }
}

// fp32 input: one thread = 4 dims of one block (same two output forms).
template <int D, bool kSplit>
__global__ __launch_bounds__(256) void k_key_means_f32(const float* __restrict__ K,
                                                       float* __restrict__ kmean,
                                                       int64_t total, int N, int n_kbs,
                                                       int kb) {
  constexpr int CH = D / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % CH);
    const int64_t bj = i / CH;
    const int j = (int)(bj % n_kbs);
    const int64_t bh = bj / n_kbs;
    const float* src = K + (bh * N + (int64_t)kb * j) * D + 4 * c;
    f32x4 o;
    if (kb == 4) {
      f32x4 r0 = *reinterpret_cast<const f32x4*>(src);
      f32x4 r1 = *reinterpret_cast<const f32x4*>(src + D);
      f32x4 r2 = *reinterpret_cast<const f32x4*>(src + 2 * D);
      f32x4 r3 = *reinterpret_cast<const f32x4*>(src + 3 * D);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (((r0[e] + r1[e]) + r2[e]) + r3[e]) * 0.25f;
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int tk = 0; tk < kb; ++tk) {
        const f32x4 rr = *reinterpret_cast<const f32x4*>(src + (int64_t)tk * D);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += rr[e];
      }
      const float inv = 1.f / (float)kb;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[e] * inv;
    }
    if constexpr (kSplit) {
      uint16_t* hi = reinterpret_cast<uint16_t*>(kmean);
      uint16_t* lo = hi + total * 4;
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16_bits(o[e]);
        l[e] = f32_to_bf16_bits(o[e] - bf16_bits_to_f32(h[e]));
      }
      *reinterpret_cast<u32x2*>(hi + bj * D + 4 * c) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *reinterpret_cast<u32x2*>(lo + bj * D + 4 * c) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    } else {
      *reinterpret_cast<f32x4*>(kmean + bj * D + 4 * c) = o;
    }
  }
}

// bf16 input, the scoring form for bf16 problems: the means of one tile of
// 32 consecutive blocks of a head (the scorer's tile) as fp16 values scaled
// by 2^-e, with e chosen so that the tile's largest magnitude lands in
// [1, 2), and 2^e in tscale[head tile] (2^-126 for a tile of zeros).  A
// power-of-two scale is exact, so every mean keeps fp16's 11 significant bits
// whatever the keys' range (no overflow; below fp16's normal range only for
// values 2^-14 below the tile's largest).  The scorer rescales whole tiles by
// powers of two on their way to LDS, which a largest value near 1 leaves
// room for in both directions.
// One work-group per (head, tile); a thread holds 8 dims of 1 (D = 64) or 2
// (D = 128) blocks, reduces the tile's largest |mean| with the others, then
// scales, rounds to nearest and stores.
template <int D>
__global__ __launch_bounds__(256) void k_key_means_f16(const uint16_t* __restrict__ K,
                                                       uint16_t* __restrict__ kh,
                                                       float* __restrict__ tscale, int N,
                                                       int n_kbs, int n_tiles, int kb) {
  constexpr int CH = D / 8;
  constexpr int NI = 32 * CH / 256;  // blocks-by-chunk items per thread
  static_assert(NI * 256 == 32 * CH, "one tile = whole items per thread");
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int tile = (int)(blockIdx.x % (unsigned)n_tiles);
  const int64_t bh = blockIdx.x / (unsigned)n_tiles;
  float out[NI][8];
  float amax = 0.f;
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int q = ii * 256 + t;
    const int key = 32 * tile + q / CH, c = q % CH;
    if (key < n_kbs) {
      block_mean8_bf16<D>(K + (bh * N + (int64_t)kb * key) * D + 8 * c, kb, out[ii]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[ii][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(out[ii][e]));
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // m = f * 2^x with f in [0.5, 1): m * 2^-(x - 1) lies in [1, 2)
  int e = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 1 : -126;
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int q = ii * 256 + t;
    const int key = 32 * tile + q / CH, c = q % CH;
    if (key < n_kbs) {
      u32x4 h;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        h[v] = pack_f16_rne(__builtin_amdgcn_ldexpf(out[ii][2 * v], -e),
                            __builtin_amdgcn_ldexpf(out[ii][2 * v + 1], -e));
      *reinterpret_cast<u32x4*>(kh + (bh * n_kbs + key) * D + 8 * c) = h;
    }
  }
  if (t == 0) tscale[blockIdx.x] = __builtin_amdgcn_ldexpf(1.f, e);
}

template <bool kSplit>
static hipError_t launch_means(const Shape& s, const void* K, float* out, hipStream_t st) {
  const int64_t blocks = (int64_t)s.B * s.H * s.n_kbs;
  const int64_t total = blocks * (s.bf16 ? s.D / 8 : s.D / 4);
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  if (s.bf16) {
    if (s.D == 128)
      k_key_means_bf16<128, kSplit><<<grid, 256, 0, st>>>((const uint16_t*)K, out, total, s.N, s.n_kbs,
                                                         s.kv_block);
    else
      k_key_means_bf16<64, kSplit><<<grid, 256, 0, st>>>((const uint16_t*)K, out, total, s.N, s.n_kbs,
                                                         s.kv_block);
  } else {
    if (s.D == 128)
      k_key_means_f32<128, kSplit><<<grid, 256, 0, st>>>((const float*)K, out, total, s.N, s.n_kbs,
                                                        s.kv_block);
    else
      k_key_means_f32<64, kSplit><<<grid, 256, 0, st>>>((const float*)K, out, total, s.N, s.n_kbs,
                                                        s.kv_block);
  }
  return hipGetLastError();
}

hipError_t launch_key_means(const Shape& s, const void* K, float* kmean, hipStream_t st) {
  return launch_means<false>(s, K, kmean, st);
}

hipError_t launch_key_means_split(const Shape& s, const void* K, uint16_t* planes, hipStream_t st) {
  return launch_means<true>(s, K, reinterpret_cast<float*>(planes), st);
}

hipError_t launch_key_means_f16(const Shape& s, const void* K, uint16_t* kh, float* tscale,
                                hipStream_t st) {
  const int n_tiles = (s.n_kbs + 31) / 32;
  const int64_t grid = (int64_t)s.B * s.H * n_tiles;
  if (s.D == 128)
    k_key_means_f16<128><<<(unsigned)grid, 256, 0, st>>>((const uint16_t*)K, kh, tscale, s.N,
                                                         s.n_kbs, n_tiles, s.kv_block);
  else
    k_key_means_f16<64><<<(unsigned)grid, 256, 0, st>>>((const uint16_t*)K, kh, tscale, s.N,
                                                        s.n_kbs, n_tiles, s.kv_block);
  return hipGetLastError();
}

}  // namespace abatt
