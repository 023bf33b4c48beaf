// SIP sampler: inclusion probabilities, Philox draws, CSR plan.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques", SIP paragraph: the draw probability pi of a key block scales
// with its score and is capped at 1 (top-scored blocks always drawn); a drawn
// block carries the Horvitz-Thompson weight 1/pi, applied as the logit shift
// log(1/pi).
//
// Per plan row (one work-group; the count kernel reads the score row in
// place, the one-pass kernel stages it in LDS when it fits):
//   * pi: m = budget * n expected blocks; repeat c = (m - #certain) /
//     sum(uncertain positive scores) and make every uncertain block with
//     c*s >= 1 certain, until none is added (the first round's count, sum
//     and maximum are gathered in the row's first read).  The certain set
//     is always a top set of the scores, so it is held as a threshold theta
//     (certain iff s >= theta).  float64 throughout; sums are fixed-order
//     tree reductions, so every run gives the same bits.
//   * draws: block j uses word j%4 of Philox4x32-10 with counter
//     (j/4, qb, h, b) and key (seed low, seed high) as a 32-bit uniform
//     integer w; kept iff w < pi_j * 2^32 (exact compare), so it enters with
//     probability ceil(pi_j * 2^32) / 2^32, within 2^-32 of pi_j.
// k_sip_count solves pi, draws, and records the row's kept-block bitmask, its
// count and its solve (mode, c, theta); k_scan turns counts into row_ptr (and
// flags a plan that exceeds its capacity); k_sip_fill walks the bitmask and
// writes ascending block ids with logw = -ln(pi) (float64 log, rounded to
// fp32; 0 where pi = 1), re-deriving pi of each kept block from its score and
// the recorded solve.  Forced (text) blocks follow the sampled ones with
// logw 0.
#include "common.h"
#include "kernels.h"
#include "sip_rows.h"

namespace abatt {

// The row is read in place: its first pass gathers the statistics, the
// solve (when it iterates) and the draws read it again from L2.
__global__ __launch_bounds__(kSampT) void k_sip_count(const float* __restrict__ S, int n,
                                                     int n_forced, int n_qb, int H,
                                                     double budget, uint64_t seed,
                                                     int32_t* __restrict__ counts,
                                                     uint32_t* __restrict__ masks,
                                                     PiSolve* __restrict__ solves) {
  __shared__ Red red;
  const int r = blockIdx.x;
  const int qb = r % n_qb, bh = r / n_qb, h = bh % H, b = bh / H;
  RowStats st;
  const float* s = stage_row<false>(S + (int64_t)r * n, n, nullptr, st);
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

constexpr int kFillU = 4;

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
    // every thread takes kept blocks i, i + kSampT, ...: coalesced writes;
    // the scores of kFillU of them are requested before the first is used
    const int64_t out = start + run;
    for (int i0 = t; i0 < tot; i0 += kFillU * kSampT) {
      int jj[kFillU];
      float sv[kFillU];
#pragma unroll
      for (int u = 0; u < kFillU; ++u) {
        const int i = i0 + u * kSampT;
        jj[u] = i < tot ? 32 * base + list[i] : 0;
        if (i < tot) sv[u] = srow[jj[u]];
      }
#pragma unroll
      for (int u = 0; u < kFillU; ++u) {
        const int i = i0 + u * kSampT;
        if (i < tot) {
          const double pi = pi_of(sv[u], ps);
          col_idx[out + i] = jj[u];
          logw[out + i] = pi == 1.0 ? 0.0f : (float)(-log(pi));
        }
      }
    }
    run += tot;
    __syncthreads();
  }
  for (int i = t; i < n_forced; i += kSampT) {
    col_idx[start + run + i] = n + i;
    logw[start + run + i] = 0.0f;
  }
}

// The count kernel reads its row in place rather than staging it in LDS:
// without the 75.6 KB of LDS per row, four work-groups share a CU instead of
// two, and the draws read each group's four scores in one 16-byte load ahead
// of the Philox rounds.  (At 18 900 blocks: 0.619 ms in place, 0.709 ms
// staged.)
hipError_t launch_sampler(const Shape& s, const float* S, double budget, uint64_t seed,
                          void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                          int64_t capacity, int32_t* status, hipStream_t st) {
  const int n_forced = s.n_kb - s.n_kbs;
  SamplerWs l = sampler_ws_layout(s);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + l.counts);
  uint32_t* masks = reinterpret_cast<uint32_t*>(base + l.masks);
  PiSolve* solves = reinterpret_cast<PiSolve*>(base + l.solves);
  k_sip_count<<<s.R, kSampT, 0, st>>>(S, s.n_kbs, n_forced, s.n_qb, s.H, budget, seed, counts,
                                      masks, solves);
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


}  // namespace abatt
