// Per-row SIP device code shared by the two samplers of libabatt (the
// three-kernel count / scan / fill path and the one-pass path): Philox draws,
// work-group reductions, the capped-proportional solve of pi and the row
// staging.  What each computes, with its citation, is described at the top of
// sampler.hip.
#pragma once

#include "common.h"
#include "draw_rule.h"

namespace abatt {

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round two 32x32->64
// multiplies (one v_mad_u64_u32 each), the high halves XORed into the other
// words with the key (one three-input XOR each), a Weyl key schedule, ten
// rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = (uint64_t)M0 * c[0], p1 = (uint64_t)M1 * c[2];
    // three-input XORs in one gfx950 v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
  }
}

constexpr int kSampT = 512;
constexpr int kSampWaves = kSampT / 64;
constexpr double kTwo32 = 4294967296.0;

struct Red {
  double d[kSampWaves];
  float f[kSampWaves];
  int i[kSampWaves];
};

__device__ __forceinline__ double block_sum_f64(double v, Red& red) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red.d[w] = v;
  __syncthreads();
  double s = red.d[0];
#pragma unroll
  for (int k = 1; k < kSampWaves; ++k) s += red.d[k];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float block_min_f32(float v, Red& red) {
  v = wave_min(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red.f[w] = v;
  __syncthreads();
  float s = red.f[0];
#pragma unroll
  for (int k = 1; k < kSampWaves; ++k) s = fminf(s, red.f[k]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ int block_sum_i32(int v, Red& red) {
  v = wave_sum_i32(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red.i[w] = v;
  __syncthreads();
  int s = red.i[0];
#pragma unroll
  for (int k = 1; k < kSampWaves; ++k) s += red.i[k];
  __syncthreads();
  return s;
}

struct PiSolve {
  double c;      // proportionality constant (mode 2)
  float theta;   // certain iff s >= theta (mode 2)
  int mode;      // 0: every block pi=1; 1: pi=1 on positive scores; 2: capped-proportional
};
static_assert(sizeof(PiSolve) == 16, "row solve record is 16 bytes");

__device__ __forceinline__ double pi_of(float s, const PiSolve& ps) {
  if (ps.mode == 0) return 1.0;
  if (!(s > 0.f)) return 0.0;
  if (ps.mode == 1 || s >= ps.theta) return 1.0;
  return ps.c * (double)s;
}

// First-round statistics of a row (this thread's share): positive count,
// fp64 sum of the positive scores, largest score.
struct RowStats {
  int npos = 0;
  double sum = 0.0;
  float smax = 0.f;
  // Written without a branch: a score <= 0 adds +0.0 to the sum (which
  // leaves it unchanged) and cannot raise smax above its start of 0.
  __device__ __forceinline__ void add(float v) {
    const bool pos = v > 0.f;
    npos += pos;
    sum += (double)(pos ? v : 0.f);
    smax = fmaxf(smax, v);
  }
};

__device__ inline PiSolve solve_pi(const float* s, int n, double budget, RowStats st, Red& red) {
  PiSolve ps;
  ps.c = 0.0;
  ps.theta = INFINITY;
  const double m = budget * (double)n;
  if (m >= (double)n) {
    ps.mode = 0;
    return ps;
  }
  int npos = block_sum_i32(st.npos, red);
  double part = st.sum;
  float smax = st.smax;
  if (m >= (double)npos) {
    ps.mode = 1;
    return ps;
  }
  ps.mode = 2;
  double sum = block_sum_f64(part, red);
  smax = -block_min_f32(-smax, red);
  int ncert = 0;
  float theta = INFINITY;
  for (bool first = true;; first = false) {
    if (!first) {
      part = 0.0;
      for (int j = threadIdx.x; j < n; j += kSampT) {
        const float v = s[j];
        if (v > 0.f && v < theta) part += (double)v;
      }
      sum = block_sum_f64(part, red);
    }
    if (!(sum > 0.0)) break;
    const double c = (m - (double)ncert) / sum;
    ps.c = c;
    // no uncertain score reaches 1/c: nothing more becomes certain (c*s is
    // monotonic in s, so the largest score decides; first iteration only,
    // where every positive score is uncertain)
    if (first && c * (double)smax < 1.0) break;
    float cand = INFINITY;
    for (int j = threadIdx.x; j < n; j += kSampT) {
      const float v = s[j];
      if (v > 0.f && v < theta && c * (double)v >= 1.0) cand = fminf(cand, v);
    }
    cand = block_min_f32(cand, red);
    if (cand == INFINITY) break;
    theta = cand;
    ps.theta = theta;
    int k = 0;
    for (int j = threadIdx.x; j < n; j += kSampT) k += s[j] >= theta;
    ncert = block_sum_i32(k, red);
  }
  return ps;
}

// Stage the row in LDS (or read it in place when it does not fit) and gather
// the first-round statistics on the way: 16-byte loads when the row starts
// 16-byte aligned, 4-byte loads otherwise.  Each thread issues kStageU loads
// before it uses the first, so a row costs a few memory round trips rather
// than one per load; the statistics still see the values in index order.
constexpr int kStageU = 10;

template <bool kLds>
__device__ __forceinline__ const float* stage_row(const float* g, int n, float* lds,
                                                  RowStats& st) {
  int head = 0;
  if ((reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    const int n4 = n >> 2;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    for (int q0 = threadIdx.x; q0 < n4; q0 += kStageU * kSampT) {
      f32x4 v[kStageU];
#pragma unroll
      for (int u = 0; u < kStageU; ++u) {
        const int q = q0 + u * kSampT;
        if (q < n4) v[u] = g4[q];
      }
#pragma unroll
      for (int u = 0; u < kStageU; ++u) {
        const int q = q0 + u * kSampT;
        if (q < n4) {
          if constexpr (kLds) reinterpret_cast<f32x4*>(lds)[q] = v[u];
          st.add(v[u][0]);
          st.add(v[u][1]);
          st.add(v[u][2]);
          st.add(v[u][3]);
        }
      }
    }
    head = 4 * n4;
  }
  for (int j0 = head + threadIdx.x; j0 < n; j0 += kStageU * kSampT) {
    float v[kStageU];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int j = j0 + u * kSampT;
      if (j < n) v[u] = g[j];
    }
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int j = j0 + u * kSampT;
      if (j < n) {
        if constexpr (kLds) lds[j] = v[u];
        st.add(v[u]);
      }
    }
  }
  if constexpr (kLds) {
    __syncthreads();
    return lds;
  } else {
    return g;
  }
}

// The keep decision of block j (score s, Philox word w): sip_keep(w, x)
// with x = pi_j * 2^32, which is 2^32 in a mode-0 row and for the certain
// blocks (mode 1, or s >= theta), 0 for s <= 0, and c32 * s otherwise
// (exact: c32 = c * 2^32 is pi_of's constant scaled by a power of two,
// which commutes with the product's rounding).  As w < 2^32, the cases with
// x = 2^32 keep and the case x = 0 drops without a compare; the rest
// compares.  Bitwise operators, so that no per-block branch is taken.
__device__ __forceinline__ bool keep_block(uint32_t w, float s, const PiSolve& ps, double c32) {
  const bool cert = (ps.mode == 1) | (s >= ps.theta);
  return (ps.mode == 0) | ((s > 0.f) & (cert | sip_keep(w, c32 * (double)s)));
}

// Kept-bit mask (4 bits) of blocks 4g..4g+3: one Philox call (counter g),
// word k for block 4g + k.  The four scores are read (one 16-byte read when
// the row is 16-byte aligned and the group lies inside it) before the Philox
// rounds, which then cover the read's latency.
__device__ __forceinline__ uint32_t draw_group(const float* s, int n, int g, int qb, int h, int b,
                                               uint64_t seed, const PiSolve& ps, double c32) {
  float v[4];
  if (4 * g + 3 < n && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
    const f32x4 q = reinterpret_cast<const f32x4*>(s)[g];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = q[k];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = 4 * g + k < n ? s[4 * g + k] : 0.f;
  }
  uint32_t c[4] = {(uint32_t)g, (uint32_t)qb, (uint32_t)h, (uint32_t)b};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  uint32_t mask = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    mask |= (uint32_t)((4 * g + k < n) & keep_block(c[k], v[k], ps, c32)) << k;
  return mask;
}

}  // namespace abatt
