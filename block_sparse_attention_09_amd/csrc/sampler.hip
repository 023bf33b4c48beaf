// SIP sampler: inclusion probabilities, Philox draws, CSR plan.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques", SIP paragraph: each key block is sampled with probability
// proportional to its score, the most important blocks are certain, and a
// kept block is weighted by the inverse of its probability (Horvitz-Thompson),
// applied as the logit shift log(1/pi).
//
// Per plan row (one work-group, the score row staged in LDS):
//   * pi: m = budget * n expected blocks; repeat c = (m - #certain) /
//     sum(uncertain positive scores) and make every uncertain block with
//     c*s >= 1 certain, until none is added (the first round's count, sum
//     and maximum are gathered while the row is staged).  The certain set is always a top
//     set of the scores, so it is held as a threshold theta (certain iff
//     s >= theta).  float64 throughout; sums are fixed-order tree reductions,
//     so every run gives the same bits.
//   * draws: block j uses words 2(j%2), 2(j%2)+1 of Philox4x32-10 with
//     counter (j/2, qb, h, b) and key (seed low, seed high) as one 53-bit
//     uniform (32 bits from the first word, the top 21 of the second); kept
//     iff it is < pi_j * 2^53 (exact compare).
// k_sip_count solves pi, draws, and records the row's kept-block bitmask, its
// count and its solve (mode, c, theta); k_scan turns counts into row_ptr (and
// flags a plan that exceeds its capacity); k_sip_fill walks the bitmask and
// writes ascending block ids with logw = -ln(pi) (float64 log, rounded to
// fp32; 0 where pi = 1), re-deriving pi of each kept block from its score and
// the recorded solve.  Forced (text) blocks follow the sampled ones with
// logw 0.
#include "common.h"
#include "kernels.h"

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
  __device__ __forceinline__ void add(float v) {
    if (v > 0.f) {
      ++npos;
      sum += (double)v;
      smax = fmaxf(smax, v);
    }
  }
};

__device__ PiSolve solve_pi(const float* s, int n, double budget, RowStats st, Red& red) {
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
// 16-byte aligned, 4-byte loads otherwise.
template <bool kLds>
__device__ __forceinline__ const float* stage_row(const float* g, int n, float* lds,
                                                  RowStats& st) {
  int head = 0;
  if ((reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    const int n4 = n >> 2;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    for (int q = threadIdx.x; q < n4; q += kSampT) {
      const f32x4 v = g4[q];
      if constexpr (kLds) reinterpret_cast<f32x4*>(lds)[q] = v;
      st.add(v[0]);
      st.add(v[1]);
      st.add(v[2]);
      st.add(v[3]);
    }
    head = 4 * n4;
  }
  for (int j = head + threadIdx.x; j < n; j += kSampT) {
    const float v = g[j];
    if constexpr (kLds) lds[j] = v;
    st.add(v);
  }
  if constexpr (kLds) {
    __syncthreads();
    return lds;
  } else {
    return g;
  }
}

// pi_j * 2^32, exactly: pi_of scaled by a power of two (c32 = c * 2^32, and
// a power-of-two factor commutes with the product's rounding).
__device__ __forceinline__ double pi_x32(float s, const PiSolve& ps, double c32) {
  if (ps.mode == 0) return kTwo32;
  if (!(s > 0.f)) return 0.0;
  if (ps.mode == 1 || s >= ps.theta) return kTwo32;
  return c32 * (double)s;
}

// Kept-bit mask (4 bits) of blocks 4g..4g+3: two Philox calls (counters 2g
// and 2g+1), each giving two 53-bit uniforms u = w0 * 2^21 + (w1 >> 11)
// (words 0,1 and 2,3); kept iff u < pi * 2^53.  With x = pi * 2^32 and
// f = floor(min(x, 2^32 - 1)), w0 < f implies u < (w0 + 1) * 2^21 <= pi * 2^53
// and w0 > f implies u >= (f + 1) * 2^21 > pi * 2^53 (for pi < 1; pi = 1
// gives f = 2^32 - 1 and no w0 above it), so only w0 == f (probability 2^-32)
// needs the 53-bit compare.
__device__ __forceinline__ uint32_t draw_group(const float* s, int n, int g, int qb, int h, int b,
                                               uint64_t seed, const PiSolve& ps, double c32) {
  uint32_t mask = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t c[4] = {(uint32_t)(2 * g + i), (uint32_t)qb, (uint32_t)h, (uint32_t)b};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 4 * g + 2 * i + k;
      if (j < n) {
        const double x = pi_x32(s[j], ps, c32);
        const uint32_t w0 = c[2 * k];
        const uint32_t f = x < 4294967295.0 ? (uint32_t)x : 0xffffffffu;
        bool keep = w0 < f;
        if (w0 == f) {
          const double u = (double)(((uint64_t)w0 << 21) | (c[2 * k + 1] >> 11));
          keep = u < x * 2097152.0;
        }
        if (keep) mask |= 1u << (2 * i + k);
      }
    }
  }
  return mask;
}

template <bool kLds>
__global__ __launch_bounds__(kSampT) void k_sip_count(const float* __restrict__ S, int n,
                                                     int n_forced, int n_qb, int H,
                                                     double budget, uint64_t seed,
                                                     int32_t* __restrict__ counts,
                                                     uint32_t* __restrict__ masks,
                                                     PiSolve* __restrict__ solves) {
  extern __shared__ __align__(16) float srow[];
  __shared__ Red red;
  const int r = blockIdx.x;
  const int qb = r % n_qb, bh = r / n_qb, h = bh % H, b = bh / H;
  RowStats st;
  const float* s = stage_row<kLds>(S + (int64_t)r * n, n, srow, st);
  const PiSolve ps = solve_pi(s, n, budget, st, red);
  const double c32 = ps.c * kTwo32;
  const int groups = (n + 3) / 4;
  const int words = (n + 31) / 32;
  uint32_t* mrow = masks + (int64_t)r * words;
  const int t = threadIdx.x;
  int cnt = 0;
  for (int base = 0; base < 8 * words; base += kSampT) {
    const int g = base + t;
    const uint32_t nib = g < groups ? draw_group(s, n, g, qb, h, b, seed, ps, c32) : 0u;
    cnt += __popc(nib);
    // eight consecutive groups (threads) make one 32-bit mask word
    uint32_t wv = nib << (4 * (t & 7));
    wv |= __shfl_xor(wv, 1);
    wv |= __shfl_xor(wv, 2);
    wv |= __shfl_xor(wv, 4);
    if ((t & 7) == 0 && g / 8 < words) mrow[g / 8] = wv;
  }
  cnt = block_sum_i32(cnt, red);
  if (t == 0) {
    counts[r] = cnt + n_forced;
    solves[r] = ps;
  }
}

// Exclusive scan of the row counts -> row_ptr (single work-group).
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ counts, int R,
                                               int32_t* __restrict__ row_ptr, int64_t capacity,
                                               int32_t* __restrict__ status) {
  __shared__ int64_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (R + 1023) / 1024;
  const int lo = min(t * per, R), hi = min(lo + per, R);
  int64_t local = 0;
  for (int i = lo; i < hi; ++i) local += counts[i];
  // inclusive scan within the wave
  int64_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int64_t before = 0, total = 0;
  for (int k = 0; k < 16; ++k) {
    if (k < w) before += wsum[k];
    total += wsum[k];
  }
  int64_t run = before + incl - local;
  const int64_t cap32 = 0x7fffffff;
  for (int i = lo; i < hi; ++i) {
    row_ptr[i] = (int32_t)(run < cap32 ? run : cap32);
    run += counts[i];
  }
  if (t == 0) {
    row_ptr[R] = (int32_t)(total < cap32 ? total : cap32);
    *status = (total > capacity || total > cap32) ? 1 : 0;
  }
}

__global__ __launch_bounds__(kSampT) void k_sip_fill(const float* __restrict__ S, int n,
                                                    int n_forced,
                                                    const uint32_t* __restrict__ masks,
                                                    const PiSolve* __restrict__ solves,
                                                    const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ status,
                                                    int32_t* __restrict__ col_idx,
                                                    float* __restrict__ logw) {
  __shared__ int wtot[kSampWaves];
  // kept blocks of one pass over kSampT mask words, as offsets from the
  // pass's first block (< 32 * kSampT = 16384, so 16 bits suffice)
  __shared__ uint16_t list[32 * kSampT];
  if (*status != 0) return;  // plan exceeded its capacity: nothing is written
  const int r = blockIdx.x;
  const int words = (n + 31) / 32;
  const uint32_t* mrow = masks + (int64_t)r * words;
  const float* srow = S + (int64_t)r * n;
  const PiSolve ps = solves[r];
  const int64_t start = row_ptr[r];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int run = 0;
  for (int base = 0; base < words; base += kSampT) {
    const int wi = base + t;
    const uint32_t m = wi < words ? mrow[wi] : 0u;
    const int k = __popc(m);
    int incl = k;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < kSampWaves; ++q) {
      if (q < w) before += wtot[q];
      tot += wtot[q];
    }
    // compact this word's kept blocks (ascending) into the list
    int pos = before + incl - k;
    uint32_t mm = m;
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      list[pos++] = (uint16_t)(32 * t + bit);
    }
    __syncthreads();
    // every thread takes kept blocks i, i + kSampT, ...: coalesced writes
    const int64_t out = start + run;
    for (int i = t; i < tot; i += kSampT) {
      const int j = 32 * base + list[i];
      const double pi = pi_of(srow[j], ps);
      col_idx[out + i] = j;
      logw[out + i] = pi == 1.0 ? 0.0f : (float)(-log(pi));
    }
    run += tot;
    __syncthreads();
  }
  for (int i = t; i < n_forced; i += kSampT) {
    col_idx[start + run + i] = n + i;
    logw[start + run + i] = 0.0f;
  }
}

constexpr size_t kSampLdsMax = 150 * 1024;

template <bool kLds>
static hipError_t launch_sampler_t(const Shape& s, const float* S, double budget, uint64_t seed,
                                   void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                                   int64_t capacity, int32_t* status, hipStream_t st) {
  const size_t lds = kLds ? (size_t)s.n_kbs * sizeof(float) : 0;
  const int n_forced = s.n_kb - s.n_kbs;
  SamplerWs l = sampler_ws_layout(s);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + l.counts);
  uint32_t* masks = reinterpret_cast<uint32_t*>(base + l.masks);
  PiSolve* solves = reinterpret_cast<PiSolve*>(base + l.solves);
  if (kLds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_sip_count<kLds>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k_sip_count<kLds><<<s.R, kSampT, lds, st>>>(S, s.n_kbs, n_forced, s.n_qb, s.H, budget, seed,
                                              counts, masks, solves);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_scan<<<1, 1024, 0, st>>>(counts, s.R, row_ptr, capacity, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_sip_fill<<<s.R, kSampT, 0, st>>>(S, s.n_kbs, n_forced, masks, solves, row_ptr, status,
                                     col_idx, logw);
  return hipGetLastError();
}

SamplerWs sampler_ws_layout(const Shape& s) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SamplerWs l;
  l.counts = 0;
  l.masks = up((size_t)s.R * sizeof(int32_t));
  l.solves = l.masks + up((size_t)s.R * ((s.n_kbs + 31) / 32) * sizeof(uint32_t));
  l.total = l.solves + up((size_t)s.R * sizeof(PiSolve));
  return l;
}

hipError_t launch_sampler(const Shape& s, const float* S, double budget, uint64_t seed,
                          void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                          int64_t capacity, int32_t* status, hipStream_t st) {
  if ((size_t)s.n_kbs * sizeof(float) <= kSampLdsMax)
    return launch_sampler_t<true>(s, S, budget, seed, ws, row_ptr, col_idx, logw, capacity,
                                  status, st);
  return launch_sampler_t<false>(s, S, budget, seed, ws, row_ptr, col_idx, logw, capacity,
                                 status, st);
}

}  // namespace abatt
