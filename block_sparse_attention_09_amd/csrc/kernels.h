// Host-side launchers of the gfx950 kernels (internal to libabatt).
// Each returns the hipError_t of its launch(es); shapes are checked by the
// caller (abatt.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abatt {

struct Shape {
  int B, H, N, D;
  int q_block, kv_block, n_clusters, kmeans_iters;
  int n_qb;      // ceil(N / q_block)
  int n_kbs;     // sparse (scored) key blocks
  int n_kb;      // all key blocks incl. forced
  int R;         // B*H*n_qb plan rows
  float scale;
  bool bf16;     // dtype of Q/K/V/O
};

// key_means.hip: fp32 means [B,H,n_kbs,D]; for the scorer either the same
// means as two bf16 planes (hi then lo, each [B,H,n_kbs,D]; fp32 problems) or
// (bf16 problems) one fp16 plane [B,H,n_kbs,D] scaled per 32-block tile, with
// the tiles' scales [B,H,ceil(n_kbs/32)] in tscale
hipError_t launch_key_means(const Shape& s, const void* K, float* kmean, hipStream_t st);
hipError_t launch_key_means_split(const Shape& s, const void* K, uint16_t* planes, hipStream_t st);
hipError_t launch_key_means_f16(const Shape& s, const void* K, uint16_t* kh, float* tscale,
                                hipStream_t st);

// kmeans.hip: centroids [R, C, D] fp32 and weights [R, C] fp32
hipError_t launch_kmeans(const Shape& s, const void* Q, float* mu, float* w, hipStream_t st);

// score.hip: S [R, n_kbs] fp32 from centroids, weights and the key means in
// their scoring form (split planes, tscale null; or the scaled fp16 plane).
// Layers with few work-groups split each group's key tiles over two
// launches; `partial` (scores_partial_bytes, 0 when unsplit) holds the
// splits' partial normalisers between them.
size_t scores_partial_bytes(const Shape& s);
hipError_t launch_scores(const Shape& s, const float* mu, const float* w, const uint16_t* kplanes,
                         const float* tscale, float* S, void* partial, hipStream_t st);

// sampler.hip: counts -> row_ptr -> col_idx/logw.  The sampler's scratch
// (row counts, kept-block bitmasks, per-row solves) lives in `ws`.
struct SamplerWs {
  size_t counts, masks, solves, total;
};
SamplerWs sampler_ws_layout(const Shape& s);
hipError_t launch_sampler(const Shape& s, const float* S, double budget, uint64_t seed,
                          void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                          int64_t capacity, int32_t* status, hipStream_t st);

// sampler_onepass.hip: the same plan in one pass (decoupled look-back over
// per-row records); its scratch (a ticket and one record per row) in `ws`.
// Status 2 marks a plan whose look-back hit its spin bound.
struct OnePassWs {
  size_t ticket, flags, total;
};
OnePassWs onepass_ws_layout(const Shape& s);
hipError_t launch_sampler_onepass(const Shape& s, const float* S, double budget, uint64_t seed,
                                  void* ws, int32_t* row_ptr, int32_t* col_idx, float* logw,
                                  int64_t capacity, int32_t* status, hipStream_t st);

// attend.hip: gathered (plan != null) or dense attention; v16: V given as
// fp16 (bf16 problems)
hipError_t launch_attend(const Shape& s, const void* Q, const void* K, const void* V,
                         const int32_t* row_ptr, const int32_t* col_idx, const float* logw,
                         int64_t capacity, const int32_t* status, void* O, float* lse,
                         bool gather, bool v16, hipStream_t st);
// attend.hip: V [B,H,N,D] bf16 -> fp16 (round toward zero)
hipError_t launch_v_to_f16(const Shape& s, const void* V, void* V16, hipStream_t st);

// scratch.hip: device address of the library's static scratch array
// (ABATT_SCRATCH_BYTES) on the current device, looked up on first use
hipError_t scratch_ptr(void** out);

}  // namespace abatt
