// SIP sampler in one pass: the fused form of the sampler, for comparison
// with the three-kernel path of sampler.hip.  It computes the same plan, bit
// for bit (same pi, same draws, same rows), from the same per-row code
// (sip_rows.h); see sampler.hip for what that computes and where the pages
// say so.
//
// One pass over the rows (k_sip_plan): a work-group solves pi for its row,
// draws, keeps the row's kept-block bitmask in LDS, takes its offset in the
// plan from the counts of the rows before it (decoupled look-back over
// per-row records, the single-pass scan of Merrill and Garland, "Single-pass
// Parallel Prefix Scan with Decoupled Look-back", 2016; rows handed out in
// ticket order), and writes row_ptr and
// the ascending block ids with logw = -ln(pi) (float64 log, rounded to fp32;
// 0 where pi = 1) right away, while its scores are still in the caches, so
// the score matrix comes from memory once and no scan or fill launch
// follows.  Forced (text) blocks follow
// the sampled ones with logw 0.  k_sip_init clears the tickets, the records
// and the plan status first.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "sip_rows.h"

namespace abatt {

// Look-back record of a plan row, one 64-bit word: the state in the high half
// (0 = nothing published yet, 1 = the row's own count, 2 = the inclusive
// prefix through the row), the value in the low half.
constexpr uint64_t kFlagAgg = 1ull << 32;
constexpr uint64_t kFlagIncl = 2ull << 32;
constexpr uint32_t kSat32 = 0xffffffffu;
// bound on the look-back spin (each round sleeps ~128 cycles): rows only ever
// wait for rows that started before them, so it is never reached; if it were,
// the plan is marked invalid (status 2) instead of hanging
constexpr int kSpinMax = 1 << 22;

// Clears the row tickets, the look-back records and the plan status (a
// kernel, not a memset, so that the sequence can be captured in a graph).
__global__ __launch_bounds__(256) void k_sip_init(uint32_t* __restrict__ ticket,
                                                  uint64_t* __restrict__ flags, int R,
                                                  int32_t* __restrict__ status) {
  const int stride = gridDim.x * 256;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < R; i += stride) flags[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *ticket = 0;
    *status = 0;
  }
}

// A record carries its whole payload (state and count) in one 64-bit word, so
// relaxed device-coherent accesses suffice: no other data is published with
// it, and acquire/release would write back or invalidate the whole L2 of the
// XCD on every access.
__device__ __forceinline__ uint64_t load_flag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_flag(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of the row counts before row r (wave 0; every lane returns
// it): decoupled look-back over the records of rows r-1, r-2, ..., 64 at a
// time, lane i reading row r-1-i.  Rows before r hold tickets taken before r's,
// so they are running or done and publish their counts.  Returns false if the
// spin bound was hit.
__device__ __forceinline__ bool look_back(const uint64_t* flags, int r, uint64_t& prefix) {
  const int lane = threadIdx.x & 63;
  prefix = 0;
  int base = r - 1;
  int spins = 0;
  while (base >= 0) {
    const int j = base - lane;
    const uint64_t f = j >= 0 ? load_flag(flags + j) : kFlagIncl;
    const uint32_t state = (uint32_t)(f >> 32);
    const uint64_t incl = __ballot(state == 2);
    const uint64_t none = __ballot(state == 0);
    // lanes up to and including the closest inclusive record are needed
    const int stop = incl ? __ffsll((unsigned long long)incl) - 1 : 63;
    const uint64_t needed = stop == 63 ? ~0ull : ((2ull << stop) - 1);
    if (none & needed) {
      if (++spins > kSpinMax) return false;
      __builtin_amdgcn_s_sleep(2);
      continue;
    }
    uint64_t v = lane <= stop ? (f & 0xffffffffull) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    prefix += v;
    if (incl) return true;
    base -= 64;
  }
  return true;
}

// One plan row per work-group, rows taken in ticket order: read the row's
// scores in place (statistics, solve, draws: the count kernel's code), keep
// the kept-block bitmask in LDS, find the row's offset in the plan by
// look-back, then write row_ptr and the row's ids and log-weights (ascending,
// forced blocks last).  A row whose entries do not fit in the capacity writes
// nothing; the last row writes row_ptr[R] (the total needed) and the
// overflow status.
__global__ __launch_bounds__(kSampT) void k_sip_plan(
    const float* __restrict__ S, int n, int n_forced, int n_qb, int H, int R, double budget,
    uint64_t seed, uint32_t* __restrict__ ticket, uint64_t* __restrict__ flags,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx, float* __restrict__ logw,
    int64_t capacity, int32_t* __restrict__ status) {
  extern __shared__ __align__(16) uint32_t mask[];  // the row's kept-block bitmask
  __shared__ Red red;
  __shared__ int s_row;
  __shared__ uint64_t s_prefix;
  __shared__ int s_ok;
  __shared__ int wtot[kSampWaves];
  // kept blocks of one pass over kSampT mask words, as offsets from the
  // pass's first block (< 32 * kSampT = 16384, so 16 bits suffice)
  __shared__ uint16_t list[32 * kSampT];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) s_row = (int)atomicAdd(ticket, 1u);
  __syncthreads();
  const int r = s_row;
  const int qb = r % n_qb, bh = r / n_qb, h = bh % H, b = bh / H;
  const int words = (n + 31) / 32;
  RowStats st;
  const float* s = stage_row<false>(S + (int64_t)r * n, n, nullptr, st);
  const PiSolve ps = solve_pi(s, n, budget, st, red);
  const double c32 = ps.c * kTwo32;
  const int groups = (n + 3) / 4;
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
    if ((t & 7) == 0 && g / 8 < words) mask[g / 8] = wv;
  }
  cnt = block_sum_i32(cnt, red) + n_forced;   // also orders the mask stores before the reads below

  if (w == 0) {
    const uint64_t own = (uint64_t)(uint32_t)cnt;
    if (t == 0) store_flag(flags + r, (r == 0 ? kFlagIncl : kFlagAgg) | own);
    uint64_t prefix = 0;
    const bool ok = r == 0 || look_back(flags, r, prefix);
    if (prefix > kSat32) prefix = kSat32;
    if (t == 0) {
      const uint64_t incl = prefix + own > kSat32 ? kSat32 : prefix + own;
      store_flag(flags + r, kFlagIncl | incl);
      s_prefix = prefix;
      s_ok = ok;
    }
  }
  __syncthreads();
  const uint64_t prefix = s_prefix;
  const int64_t cap32 = 0x7fffffff;
  if (t == 0) {
    if (!s_ok) atomicMax(status, 2);
    row_ptr[r] = (int32_t)((int64_t)prefix < cap32 ? (int64_t)prefix : cap32);
    if (r == R - 1) {
      const int64_t total = (int64_t)prefix + cnt;
      row_ptr[R] = (int32_t)(total < cap32 ? total : cap32);
      if (total > capacity || total > cap32) atomicMax(status, 1);
    }
  }
  if (!s_ok || (int64_t)prefix + cnt > capacity || (int64_t)prefix + cnt > cap32) return;

  // ids and log-weights of the kept blocks, kSampT mask words at a time: the
  // exclusive prefix of the words' kept counts places each thread's word in
  // an LDS list (ascending), then every thread takes entries i, i + kSampT,
  // ... of the list, so consecutive entries go to consecutive slots; the
  // scores of kFillU of them are requested before the first is used
  constexpr int kFillU = 4;
  const int64_t start = (int64_t)prefix;
  int run = 0;
  for (int base = 0; base < words; base += kSampT) {
    const int wi = base + t;
    const uint32_t m = wi < words ? mask[wi] : 0u;
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
    int pos = before + incl - k;
    uint32_t mm = m;
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      list[pos++] = (uint16_t)(32 * t + bit);
    }
    __syncthreads();
    const int64_t out = start + run;
    for (int i0 = t; i0 < tot; i0 += kFillU * kSampT) {
      int jj[kFillU];
      float sv[kFillU];
#pragma unroll
      for (int u = 0; u < kFillU; ++u) {
        const int i = i0 + u * kSampT;
        jj[u] = i < tot ? 32 * base + list[i] : 0;
        if (i < tot) sv[u] = s[jj[u]];
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

OnePassWs onepass_ws_layout(const Shape& s) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  OnePassWs l;
  l.ticket = 0;
  l.flags = 256;
  l.total = l.flags + up((size_t)s.R * sizeof(uint64_t));
  return l;
}

hipError_t launch_sampler_onepass(const Shape& s, const float* S, double budget, uint64_t seed,
                                  void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                                  int64_t capacity, int32_t* status, hipStream_t st) {
  // dynamic LDS: the mask words (2.4 KB at 18 900 blocks); with the 32 KB
  // list, four work-groups share a CU
  const size_t lds = (size_t)(s.n_kbs + 31) / 32 * sizeof(uint32_t);
  const int n_forced = s.n_kb - s.n_kbs;
  const OnePassWs l = onepass_ws_layout(s);
  char* base = static_cast<char*>(ws);
  uint32_t* ticket = reinterpret_cast<uint32_t*>(base + l.ticket);
  uint64_t* flags = reinterpret_cast<uint64_t*>(base + l.flags);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_sip_plan),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int init_blocks = (int)std::min<int64_t>(((int64_t)s.R + 255) / 256, 1024);
  k_sip_init<<<init_blocks, 256, 0, st>>>(ticket, flags, s.R, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_sip_plan<<<s.R, kSampT, lds, st>>>(S, s.n_kbs, n_forced, s.n_qb, s.H, s.R, budget, seed,
                                       ticket, flags, row_ptr, col_idx, logw, capacity, status);
  return hipGetLastError();
}

}  // namespace abatt
