// Gathered-KV flash attention with the Horvitz-Thompson logit shift, and the
// dense path built from the same tile core.
//
// [hamidun] = news.hamidun.com, "AB-Attention speeds up video generation by up
// to 2.23x and skips 92% of attention", section "AB-Attention's three
// techniques": SIP keeps ordinary softmax attention and adds log(1/pi) to the
// logits of a kept block; the third technique gathers the kept 4-token K/V
// blocks by index into full compute tiles without permuting tokens
// ([zerohour] = zerohour.day, "AB-Attention approximates dense video attention
// at high sparsity", key facts, says the same of the kernel).
//
// bf16 kernel (gfx950), one work-group of 4 waves per plan row (128 queries):
//   * wave w owns queries 32w..32w+31; its Q slice stays in registers as the
//     B operand of S^T = K Q^T (bf16 MFMA 32x32x16, fp32 accumulation), so a
//     lane ends up holding 32 logits of ONE query (lane%32) and the row max
//     needs a single exchange between the two half-waves;
//   * keys arrive in chunks of 32 = 8 groups of 4 consecutive keys of the
//     row's key sequence (one kept 4-token block per group; longer blocks
//     span several groups; dense rows take every group in order), small
//     enough that three work-groups fit on a CU.  A group of a head is
//     4*D*2 contiguous bytes, so one wave-wide 16-byte load moves a whole
//     group (D=128).  The block ids
//     of a chunk are fetched once per wave and broadcast with readlane.  K
//     goes straight to LDS by direct buffer loads into a tile with an XOR
//     slot swizzle; V is loaded into registers and converted to
//     fp16 while it is staged (exact for bf16 values in fp16's normal range),
//     then stored row-major.  K and V of a group come from one row
//     computation, and at D=128 the group's row base is wave-uniform and
//     rides in the loads' scalar offset, so the gather costs few vector
//     instructions (about 4 per MFMA, exponentials included: at that ratio
//     they co-issue with the MFMAs of the other waves on the SIMD; what holds
//     the matrix cores back is the dependency chain QK^T -> softmax -> PV
//     inside each wave, which more waves per SIMD cover better).  The PV operand is read with the gfx950 LDS
//     transpose read, so PV runs as O^T = V^T P^T on fp16 MFMA with the
//     probabilities straight from the softmax registers: the key order inside
//     an MFMA k-step is chosen to match what each lane already holds;
//   * two LDS stages: K and V of chunk c+1 arrive while chunk c is computed,
//     one barrier per chunk;
//   * online softmax in the exp2 domain against a reference that trails the
//     running max: probabilities are formed against it first, and only when
//     a half-chunk's fp16 sum passes 2^15 (a value may leave fp16's range)
//     does the wave take the chunk's exact max, move the reference (when the
//     max passes it by more than 8, log2 units), rescale the accumulators
//     and form them again.  Most chunks take no max at all;
//   * work-groups run in plan-row order, so all XCDs share one head at a time
//     and its K/V stays resident in the Infinity Cache; a layer whose whole
//     K/V fits that cache gives each XCD a contiguous range of rows instead.
// fp32 kernel: plain fp32 arithmetic (one thread per query), used for fp32
// problems.
#include "common.h"
#include "kernels.h"

namespace abatt {

constexpr float kRescaleLog2 = 8.0f;

typedef short v4i16 __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose read: within each 16-lane group, lane r supplies the
// address of 4 consecutive 16-bit elements; lane i receives element i%4 of the
// lanes 4k + i/4 (k = 0..3).  With lane r pointing at row k0 + r/4, columns
// c0 + 4*(r%4) of a row-major tile, lane i gets column c0 + i of rows
// k0..k0+3 -- the K-contiguous operand layout of a 32x32x16 MFMA.
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}

// V tile swizzle: 16-byte chunk c of row r is stored at chunk c ^ vswz(r), so
// the four rows a transpose read touches fall on different banks.
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return (4 * (row & 3)) & (D / 8 - 1);
}

// s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (no wait),
// lgkmcnt 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Work-group barrier for stages filled by direct-to-LDS loads, which the
// compiler does not track: wait for all of this wave's vector memory
// operations and LDS accesses, then s_barrier; the empty asm statements keep
// the compiler from moving memory operations across it.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from byte soff + voff of a buffer straight into LDS, lane
// l's bytes at lds_addr + 16 l (the range check covers voff, not the
// wave-uniform soff).  Written as inline asm so that the compiler does not
// track it: its own wait insertion would otherwise make every later LDS read
// wait for it.  The caller waits (dma_barrier) before the stage is read.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                                  uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(soff), "s"(lds_addr)
               : "memory", "m0");
}

// Buffer resource for a head's K or V (bounds-checked: loads past the end
// return zero, which the dense path relies on for its last partial block).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes,
                                           0x00020000);
}

// kV16: V arrives already converted to fp16 and moves to LDS by direct loads
// like K.  Rows run in 32-key chunks, which keeps a work-group within 33 KB of
// LDS and about 160 VGPRs, so three work-groups share a CU (three waves per
// SIMD: measured 1.5-4% faster than two with 64-key chunks on gathered rows,
// 6% on dense ones).
template <int D, bool kGather, bool kV16>
__global__ __launch_bounds__(256, 3) void k_attend_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const float* __restrict__ logw, int64_t capacity,
    const int32_t* __restrict__ status, uint16_t* __restrict__ O, float* __restrict__ lse, int N,
    int n_qb, int n_kb, int R, float scale_log2, int lkb, int xcd_contig) {
  constexpr int KS = D / 16;          // QK^T k-steps
  constexpr int DT = D / 32;          // PV output tiles
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CK = 32;                 // keys per chunk
  constexpr int NG = CK / 4;             // 4-key groups per chunk
  constexpr int TT = CK / 32;            // 32-key tiles per chunk
  constexpr int WG = NG / 4;             // groups each wave moves per chunk
  constexpr int BPS = 64 / (4 * CPR);    // 4-key groups covered by one wave-wide load (1 or 2)
  constexpr int SLOTS = WG / BPS;        // 16-byte loads per lane per chunk, for K and for V
  constexpr int GROUP_BYTES = 4 * D * 2;  // one group of 4 keys
  static_assert(SLOTS * BPS == WG && SLOTS >= 1, "a wave moves whole loads of each chunk");
  // K tile: row-major, 16-byte slot s of row r stored at s ^ (r % CPR)
  // (conflict-free operand reads without padding; the direct loads place each
  // lane's 16 bytes at a fixed LDS position, so the swizzle is chosen through
  // the source address)
  __shared__ __align__(16) uint16_t Ks[2][CK * D];
  __shared__ __align__(16) uint16_t Vs[2][CK * D];
  __shared__ float lwb[2][NG];

  // Row order.  The dispatcher deals consecutive work-groups to the 8 XCDs in
  // turn.  Large layers take rows in plan order, so all XCDs work on the same
  // head at once and that head's K/V (38.7 MB at 75600 tokens) stays in the
  // 256 MB Infinity Cache (giving each XCD its own contiguous rows there
  // spreads the XCDs over 8 heads and measured 4% slower).  When the layer's
  // whole K/V fits the Infinity Cache (xcd_contig), each XCD takes a
  // contiguous range of rows instead, so its L2 serves fewer heads at a time
  // (2% faster at 12 heads of 32760 tokens).
  const int r = xcd_contig ? xcd_remap(blockIdx.x, R) : (int)blockIdx.x;
  const int qb = r % n_qb;
  const int64_t bh = r / n_qb;
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);

  int64_t start = 0;
  int nblk;
  if constexpr (kGather) {
    const int64_t a = row_ptr[r], b = row_ptr[r + 1];
    const bool bad = (status != nullptr && *status != 0) || a < 0 || b < a || b > capacity;
    start = a;
    nblk = bad ? 0 : (int)(b - a);
  } else {
    nblk = (N + 3) / 4;
  }
  // keys of the row: nblk blocks of 2^lkb tokens (dense rows: 4-token groups)
  const int nchunk = (int)((((int64_t)nblk << lkb) + CK - 1) / CK);
  const int kbmask = (1 << lkb) - 1;

  const __amdgpu_buffer_rsrc_t krs = head_rsrc(K + bh * N * D, N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(V + bh * N * D, N * D * 2);

  const int qrow = qb * 128 + 32 * wv + l32;
  bf16x8 qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < N)
      qreg[s] = *reinterpret_cast<const bf16x8*>(Q + (bh * N + qrow) * D + 16 * s + 8 * hh);
    else
      qreg[s] = bf16x8{};
  }

  // A chunk is CK consecutive keys of the row's key sequence, NG groups of 4;
  // group g of chunk c starts at key CK*c + 4g, in block (CK*c + 4g) >> lkb at
  // token (CK*c + 4g) & kbmask of the block.  Lane j holds the block id and
  // shift of group j & 15 (repeated for blocks longer than 4), branch-free.
  auto group_block = [&](int c, int g) { return (CK * c + 4 * g) >> lkb; };
  auto group_token = [&](int c, int g) { return (CK * c + 4 * g) & kbmask; };
  // The row's ids and shifts are read through bounds-checked buffers: entries
  // past the row read zero, and valid_id rejects them by position.
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(col_idx + start), (short)0, nblk * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(logw + start), (short)0, nblk * 4, 0x00020000);
  auto fetch_ids = [&](int c, int& id, float& lw) {
    const int idx = group_block(c, lane & (NG - 1)) * 4;
    id = (int)__builtin_amdgcn_raw_buffer_load_b32(crs, idx, 0, 0);
    lw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lrs, idx, 0, 0));
  };
  // validity is applied when the ids are first used (keeps the loads in flight)
  auto valid_id = [&](int c, int raw) -> bool {
    return group_block(c, lane & (NG - 1)) < nblk && raw >= 0 && raw < n_kb;
  };

  // lane -> (group within a load, key within the group, 16-byte chunk); one
  // wave-wide 16-byte load covers BPS groups of 4 rows
  const int sub = lane / (4 * CPR);
  const int key = (lane % (4 * CPR)) / CPR;
  const int dc = lane % CPR;
  constexpr int ROW_BYTES = D * 2;
  // the lane's part of a group's offset: its row in the group and its 16-byte
  // chunk, plain for V, slot-swizzled for the K tile (group g holds tile rows
  // 4g..4g+3)
  const int vlane = key * ROW_BYTES + (dc << 4);
  auto klane = [&](int g) { return key * ROW_BYTES + ((dc ^ ((4 * g + key) % CPR)) << 4); };
  // fp16 V by direct loads: the lane's source chunk carries the V tile's swizzle
  // (chunk c of tile row r at c ^ vswz(r)), and group g's 4 rows land at row 4g
  auto vlane_t = [&](int g) { return key * ROW_BYTES + ((dc ^ vswz<D>(4 * g + key)) << 4); };
  auto vlds = [&](int stage, int g) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(
        &Vs[stage][g * (GROUP_BYTES / 2)]);
  };

  // K goes straight to LDS by direct loads; V too when it arrives as fp16,
  // otherwise through registers (converted to fp16 on its way to LDS).
  u32x4 vpre[kV16 ? 1 : SLOTS];
  int id_next = 0;                   // raw ids of the next chunk to start (gathered rows)
  float lw_next = 0.f;

  // K and V of chunk c into stage `stage`, from one row computation per group.
  // Gathered rows: the ids `idv` are validated, so every row lies inside the
  // head; when a load covers one group (D = 128) the group's row base is
  // wave-uniform and goes in the scalar offset.  Dense rows: group g of chunk
  // c is keys CK*c + 4g .. +3; rows past N (a partial last group, or whole
  // groups of the last chunk) are clamped to row N-1, and their logits are
  // masked.
  auto issue_kv = [&](int c, int idv, int stage) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int b0 = WG * wv + BPS * j;
      const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)(
          &Ks[stage][b0 * (GROUP_BYTES / 2)]);
      if constexpr (kGather && BPS == 1) {
        const int soff = __builtin_amdgcn_readfirstlane(
            ((__builtin_amdgcn_readlane(idv, b0) << lkb) + group_token(c, b0)) * ROW_BYTES);
        buffer_load_lds16(krs, klane(b0), soff, lds);
        if constexpr (kV16)
          buffer_load_lds16(vrs, vlane_t(b0), soff, vlds(stage, b0));
        else
          vpre[j] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vlane, soff, 0));
      } else {
        int rowoff;
        if constexpr (kGather) {
          const int r0 = (__builtin_amdgcn_readlane(idv, b0) << lkb) + group_token(c, b0);
          const int r1 = (__builtin_amdgcn_readlane(idv, b0 + 1) << lkb) + group_token(c, b0 + 1);
          rowoff = (sub ? r1 : r0) * ROW_BYTES;
        } else {
          // this lane's key row, clamped; key * ROW_BYTES is part of klane/vlane
          const int row = CK * c + 4 * (b0 + sub) + key;
          rowoff = ((row < N ? row : N - 1) - key) * ROW_BYTES;
        }
        buffer_load_lds16(krs, rowoff + klane(b0 + sub), 0, lds);
        if constexpr (kV16)
          buffer_load_lds16(vrs, rowoff + vlane_t(b0 + sub), 0, vlds(stage, b0));
        else
          vpre[j] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, rowoff + vlane, 0, 0));
      }
    }
  };
  // Chunk c into stage `stage`; gathered rows first validate the ids of the
  // chunk (in id_next) once and record its shifts.
  auto start_chunk = [&](int c, int stage) {
    if constexpr (kGather) {
      const bool ok = valid_id(c, id_next);
      if (t < NG) lwb[stage][t] = ok ? lw_next * kLog2e : -INFINITY;
      issue_kv(c, ok ? id_next : 0, stage);
    } else {
      issue_kv(c, 0, stage);
    }
  };
  // V of a chunk from registers into stage buf, converted to fp16 (exact for
  // bf16 values in fp16's normal range; as it is with fp16 V).
  auto store_regs = [&](int buf) {
    uint16_t* vst = Vs[buf];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int row = 4 * (WG * wv + i * BPS + sub) + key;
      u32x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hv[e] = pack_f16_rtz(__uint_as_float(vpre[i][e] << 16),
                             __uint_as_float(vpre[i][e] & 0xffff0000u));
      *reinterpret_cast<u32x4*>(&vst[row * D + 8 * (dc ^ vswz<D>(row))]) = hv;
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
  float m_used = -INFINITY;
  float lsum = 0.f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // Pipeline: chunk c is computed from LDS stage c%2; the other stage is free
  // during iteration c.  At the top of iteration c, K of chunk c+1 goes to the
  // free stage by direct loads and V of chunk c+1 to it as well (fp16 V) or to
  // registers, converted into the free stage after the chunk's PV.  Gathered
  // rows validate the ids of chunk c+1 (fetched during iteration c-1) first
  // and request those of chunk c+2.  The barrier that ends iteration c waits
  // for all of it, so every load has a whole iteration to land.  Chunk
  // indices are clamped to the last chunk so the prefetch code runs
  // unconditionally; the cost is a few redundant loads at the end.
  const int clast = nchunk > 0 ? nchunk - 1 : 0;
  if (nchunk > 0) {
    if constexpr (kGather) fetch_ids(0, id_next, lw_next);
    start_chunk(0, 0);
    if constexpr (kGather) fetch_ids(min(1, clast), id_next, lw_next);
    if constexpr (!kV16) store_regs(0);
  }
  dma_barrier();

  // transpose-read geometry (per lane, fixed)
  const int tr_r = lane & 15;
  const int tr_g = (lane >> 4) & 1;

  auto step = [&](int c, int buf) {
    const uint16_t* kst = Ks[buf];
    const uint16_t* vst = Vs[buf];
    start_chunk(min(c + 1, clast), buf ^ 1);                                // K, V of chunk c+1
    if constexpr (kGather) fetch_ids(min(c + 2, clast), id_next, lw_next);  // ids of chunk c+2

    // S^T tile: lane holds query l32, keys 32*tt + 8*g + 4*hh + (0..3) = group 8tt+2g+hh
    f32x16 sacc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) sacc[tt] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int krow = 32 * tt + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &kst[krow * D + (((2 * s + hh) ^ (krow % CPR)) << 3)]);
        sacc[tt] = mfma_bf16_32x32x16(a, qreg[s], sacc[tt]);
      }
    }
    // keep four K operand reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < TT * KS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if constexpr (!kGather) {
      if (c == nchunk - 1) {  // keys past N in the last dense chunk
        const int base = CK * c;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (base + 32 * tt + 8 * (v >> 2) + 4 * hh + (v & 3) >= N) sacc[tt][v] = -INFINITY;
      }
    }
    float lwg[4 * TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int g = 0; g < 4; ++g) lwg[4 * tt + g] = kGather ? lwb[buf][8 * tt + 2 * g + hh] : 0.f;
    uint32_t pk[8 * TT];
    // fp16 probabilities of half gp of tile tt (this lane's groups 2gp and
    // 2gp+1) against the reference mr; returns their sum (the row sum takes
    // the same fp16 values as the numerator)
    auto probs = [&](int tt, int gp, float mr) -> float {
      float cs = 0.f;
#pragma unroll
      for (int g = 2 * gp; g < 2 * gp + 2; ++g) {
        const float sh = lwg[4 * tt + g] - mr;
        float p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          p[q] = __builtin_amdgcn_exp2f(fmaf(sacc[tt][4 * g + q], scale_log2, sh));
        pk[8 * tt + 2 * g] = pack_f16_rne(p[0], p[1]);
        pk[8 * tt + 2 * g + 1] = pack_f16_rne(p[2], p[3]);
        cs = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[8 * tt + 2 * g]), ones, cs, false);
        cs = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[8 * tt + 2 * g + 1]), ones, cs, false);
      }
      return cs;
    };
    // exact shifted maximum of the chunk; the reference moves to it when it
    // passes the reference by more than kRescaleLog2, and the accumulators
    // follow
    auto rescale = [&]() {
      float mloc = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        // an opaque copy keeps this maximum on the rare path (the compiler
        // would otherwise hoist part of it above the branch)
        f32x16 sx = sacc[tt];
        asm volatile("" : "+v"(sx));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float gm = fmaxf(fmaxf(sx[4 * g], sx[4 * g + 1]), fmaxf(sx[4 * g + 2], sx[4 * g + 3]));
          mloc = fmaxf(mloc, fmaf(gm, scale_log2, lwg[4 * tt + g]));
        }
      }
      const f32x2 mp = pair_x32(mloc);
      const float mrow = fmaxf(mp[0], mp[1]);
      const bool need = mrow > m_used + kRescaleLog2;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_used - mrow) : 1.f;
      if (need) m_used = mrow;
      lsum *= alpha;
#pragma unroll
      for (int u = 0; u < DT; ++u) oacc[u] *= alpha;
    };
    // O^T += V^T P^T, one half-tile at a time.  k-step (tt, gp) covers keys
    // 32tt+16gp .. +15 in the order lane-half hh holds them: 4hh+{0..3}, then
    // 8+4hh+{0..3}.  Each half's probabilities are formed against the current
    // reference first; if their sum passes 2^15 on any lane (so that a value
    // may leave fp16's range; also inf or NaN while the reference is still
    // -inf), the wave takes the exact maximum, moves the reference and forms
    // them again.  Otherwise every value is at most 2^15, and the half goes
    // straight to its MFMAs.
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float cs = probs(tt, gp, m_used);
        if (__builtin_expect(__any(__float_as_uint(cs) > 0x47000000u), 0)) {
          rescale();
          cs = probs(tt, gp, m_used == -INFINITY ? 0.f : m_used);
        }
        lsum += cs;
        const int pb = 8 * tt + 4 * gp;
        const f16x8 pop =
            __builtin_bit_cast(f16x8, u32x4{pk[pb], pk[pb + 1], pk[pb + 2], pk[pb + 3]});
        const int rowa = 32 * tt + 16 * gp + 4 * hh + (tr_r >> 2);
        const int rowb = rowa + 8;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
          const int d0 = 32 * u + 16 * tr_g + 4 * (tr_r & 3);
          const v4i16 va = lds_read_tr16(&vst[rowa * D + 8 * ((d0 >> 3) ^ vswz<D>(rowa)) + (d0 & 7)]);
          const v4i16 vb = lds_read_tr16(&vst[rowb * D + 8 * ((d0 >> 3) ^ vswz<D>(rowb)) + (d0 & 7)]);
          const f16x8 vop = __builtin_bit_cast(
              f16x8, u32x4{__builtin_bit_cast(u32x2, va)[0], __builtin_bit_cast(u32x2, va)[1],
                           __builtin_bit_cast(u32x2, vb)[0], __builtin_bit_cast(u32x2, vb)[1]});
          oacc[u] = mfma_f16_32x32x16(vop, pop, oacc[u]);
        }
      }
    }
    if constexpr (!kV16) store_regs(buf ^ 1);   // V of chunk c+1 -> free stage
    dma_barrier();
  };
  // unrolled by two so that stage addresses are constants (measured faster,
  // gathered and dense rows alike)
  for (int c = 0; c < nchunk; c += 2) {
    step(c, 0);
    if (c + 1 < nchunk) step(c + 1, 1);
  }

  // epilogue: O^T lane layout = query l32, dims 32u + 8g + 4hh + (0..3)
  const f32x2 lp = pair_x32(lsum);
  const float ltot = lp[0] + lp[1];
  if (qrow < N) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* orow = O + (bh * N + qrow) * D;
#pragma unroll
    for (int u = 0; u < DT; ++u) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t b0 = f32_to_bf16_bits(oacc[u][4 * g] * inv);
        const uint32_t b1 = f32_to_bf16_bits(oacc[u][4 * g + 1] * inv);
        const uint32_t b2 = f32_to_bf16_bits(oacc[u][4 * g + 2] * inv);
        const uint32_t b3 = f32_to_bf16_bits(oacc[u][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * u + 8 * g + 4 * hh) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
      }
    }
    if (hh == 0 && lse != nullptr)
      lse[bh * N + qrow] = ltot > 0.f ? (m_used + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per query, 32-key chunks staged in LDS.
// ---------------------------------------------------------------------------
template <int D, bool kGather>
__global__ __launch_bounds__(128) void k_attend_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const float* __restrict__ logw, int64_t capacity, const int32_t* __restrict__ status,
    float* __restrict__ O, float* __restrict__ lse, int N, int n_qb, int n_kb, int R,
    float scale_log2, int lkb) {
  constexpr int CK = 32;  // keys per chunk
  __shared__ __align__(16) float Kf[CK * D];
  __shared__ __align__(16) float Vf[CK * D];
  __shared__ float lwk[CK];

  const int r = xcd_remap(blockIdx.x, R);
  const int qb = r % n_qb;
  const int64_t bh = r / n_qb;
  const int t = threadIdx.x;
  const int qrow = qb * 128 + t;

  int64_t start = 0;
  int nblk;
  if constexpr (kGather) {
    const int64_t a = row_ptr[r], b = row_ptr[r + 1];
    const bool bad = (status != nullptr && *status != 0) || a < 0 || b < a || b > capacity;
    start = a;
    nblk = bad ? 0 : (int)(b - a);
  } else {
    nblk = (N + 3) / 4;
  }
  // key kap of the row's key sequence: block kap >> lkb, token kap & kbmask
  const int nchunk = (int)((((int64_t)nblk << lkb) + CK - 1) / CK);
  const int kbmask = (1 << lkb) - 1;
  const float* Kh = K + bh * N * D;
  const float* Vh = V + bh * N * D;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = qrow < N ? Q[(bh * N + qrow) * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int c = 0; c < nchunk; ++c) {
    __syncthreads();
    for (int i = t; i < CK * D / 4; i += 128) {
      const int key = (4 * i) / D, e = (4 * i) % D;
      const int kap = c * CK + key;
      const int idx = kap >> lkb;
      int id = 0;
      float lw = -INFINITY;
      if constexpr (kGather) {
        if (idx < nblk) {
          const int cid = col_idx[start + idx];
          if (cid >= 0 && cid < n_kb) {
            id = cid;
            lw = logw[start + idx] * kLog2e;
          }
        }
      } else {
        id = idx;
        lw = kap < N ? 0.f : -INFINITY;
      }
      int64_t tok = ((int64_t)id << lkb) + (kap & kbmask);
      if (tok >= N) tok = N - 1;
      *reinterpret_cast<f32x4*>(&Kf[key * D + e]) = *reinterpret_cast<const f32x4*>(Kh + tok * D + e);
      *reinterpret_cast<f32x4*>(&Vf[key * D + e]) = *reinterpret_cast<const f32x4*>(Vh + tok * D + e);
      if (e == 0) lwk[key] = lw;
    }
    __syncthreads();
    float z[CK];
    float cm = -INFINITY;
#pragma unroll
    for (int k = 0; k < CK; ++k) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&Kf[k * D + e]);
        dot = fmaf(q[e], kv[0], dot);
        dot = fmaf(q[e + 1], kv[1], dot);
        dot = fmaf(q[e + 2], kv[2], dot);
        dot = fmaf(q[e + 3], kv[3], dot);
      }
      z[k] = fmaf(dot, scale_log2, lwk[k]);
      cm = fmaxf(cm, z[k]);
    }
    const float mn = fmaxf(m, cm);
    if (mn == -INFINITY) continue;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int k = 0; k < CK; ++k) {
      const float p = __builtin_amdgcn_exp2f(z[k] - m);
      l += p;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&Vf[k * D + e]);
        o[e] = fmaf(p, vv[0], o[e]);
        o[e + 1] = fmaf(p, vv[1], o[e + 1]);
        o[e + 2] = fmaf(p, vv[2], o[e + 2]);
        o[e + 3] = fmaf(p, vv[3], o[e + 3]);
      }
    }
  }
  if (qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = O + (bh * N + qrow) * D;
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<f32x4*>(orow + e) = f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    if (lse != nullptr) lse[bh * N + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// bf16 V to fp16 once per call, for the fp16-V form of the gathered kernel:
// the conversion that kernel otherwise applies while staging V (round toward
// zero, exact in fp16's normal range), 16 bytes per thread per step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_v_to_f16(const u32x4* __restrict__ V,
                                                  u32x4* __restrict__ V16, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 x = V[i];
    u32x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = pack_f16_rtz(__uint_as_float(x[e] << 16), __uint_as_float(x[e] & 0xffff0000u));
    V16[i] = h;
  }
}

hipError_t launch_v_to_f16(const Shape& s, const void* V, void* V16, hipStream_t st) {
  const int64_t n16 = (int64_t)s.B * s.H * s.N * s.D / 8;   // D is a multiple of 8
  const int64_t blocks = (n16 + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  k_v_to_f16<<<grid, 256, 0, st>>>((const u32x4*)V, (u32x4*)V16, n16);
  return hipGetLastError();
}

template <int D, bool kGather, bool kV16>
static void launch_attend_t(const Shape& s, const void* Q, const void* K, const void* V,
                            const int32_t* row_ptr, const int32_t* col_idx, const float* logw,
                            int64_t capacity, const int32_t* status, void* O, float* lse,
                            hipStream_t st) {
  const float sl2 = s.scale * kLog2e;
  // gathered rows use the problem's key-block size; dense rows run in groups of 4
  int lkb = 2;
  if (kGather)
    while ((1 << lkb) < s.kv_block) ++lkb;
  if (s.bf16) {
    // K and V (2 bytes an element each) of the whole layer within 224 MB: the
    // rows of each XCD are taken as one contiguous range
    const int xcd_contig = (size_t)s.B * s.H * s.N * s.D * 4 <= ((size_t)224 << 20) ? 1 : 0;
    k_attend_bf16<D, kGather, kV16><<<s.R, 256, 0, st>>>(
        (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, row_ptr, col_idx, logw,
        capacity, status, (uint16_t*)O, lse, s.N, s.n_qb, s.n_kb, s.R, sl2, lkb, xcd_contig);
  } else {
    k_attend_f32<D, kGather><<<s.R, 128, 0, st>>>(
        (const float*)Q, (const float*)K, (const float*)V, row_ptr, col_idx, logw, capacity,
        status, (float*)O, lse, s.N, s.n_qb, s.n_kb, s.R, sl2, lkb);
  }
}

hipError_t launch_attend(const Shape& s, const void* Q, const void* K, const void* V,
                         const int32_t* row_ptr, const int32_t* col_idx, const float* logw,
                         int64_t capacity, const int32_t* status, void* O, float* lse,
                         bool gather, bool v16, hipStream_t st) {
#define ABATT_ATTEND(Dv)                                                                     \
  if (v16 && gather)                                                                         \
    launch_attend_t<Dv, true, true>(s, Q, K, V, row_ptr, col_idx, logw, capacity, status, O, \
                                    lse, st);                                                \
  else if (v16)                                                                              \
    launch_attend_t<Dv, false, true>(s, Q, K, V, row_ptr, col_idx, logw, capacity, status,   \
                                     O, lse, st);                                            \
  else if (gather)                                                                           \
    launch_attend_t<Dv, true, false>(s, Q, K, V, row_ptr, col_idx, logw, capacity, status,   \
                                     O, lse, st);                                            \
  else                                                                                       \
    launch_attend_t<Dv, false, false>(s, Q, K, V, row_ptr, col_idx, logw, capacity, status,  \
                                      O, lse, st);
  if (s.D == 128) {
    ABATT_ATTEND(128)
  } else {
    ABATT_ATTEND(64)
  }
#undef ABATT_ATTEND
  return hipGetLastError();
}

}  // namespace abatt
