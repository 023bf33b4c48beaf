// C ABI of libabatt: argument checks, workspace layout, kernel launches.
// Every check runs on the host before any HIP call, so invalid arguments come
// back as a status code with nothing enqueued (and without a GPU present).
#include "abatt.h"

#include <cmath>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

using abatt::Shape;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device tensors and workspaces are read and written 16 bytes at a time: a
// pointer that is NULL or not 16-byte aligned is rejected.
static bool bad(const void* x) { return x == nullptr || (reinterpret_cast<uintptr_t>(x) & 15) != 0; }

// Validates *p; fills *s.  Returns ABATT_OK, ABATT_EINVAL or ABATT_EUNSUPPORTED.
abatt_status make_shape(const abatt_problem_t* p, Shape* s) {
  if (p == nullptr) return ABATT_EINVAL;
  if (p->B <= 0 || p->H <= 0 || p->N <= 0 || p->D <= 0) return ABATT_EINVAL;
  if (p->q_block <= 0 || p->kv_block <= 0 || p->n_clusters <= 0 || p->kmeans_iters <= 0)
    return ABATT_EINVAL;
  if (p->n_forced_tail < 0 || p->n_forced_tail >= p->N) return ABATT_EINVAL;
  if (p->n_forced_tail % p->kv_block != 0) return ABATT_EINVAL;
  if ((p->N - p->n_forced_tail) % p->kv_block != 0) return ABATT_EINVAL;
  if (!(p->scale > 0.0f) || !std::isfinite(p->scale)) return ABATT_EINVAL;
  if (p->dtype != ABATT_F32 && p->dtype != ABATT_BF16) return ABATT_EINVAL;
  if (p->n_clusters > p->q_block) return ABATT_EINVAL;
  // what the kernels implement
  if (p->D != 64 && p->D != 128) return ABATT_EUNSUPPORTED;
  if (p->q_block != 128) return ABATT_EUNSUPPORTED;
  // key blocks: a power of two from 4 to 128 tokens
  if (p->kv_block < 4 || p->kv_block > 128 || (p->kv_block & (p->kv_block - 1)) != 0)
    return ABATT_EUNSUPPORTED;
  if (p->n_clusters != 8 && p->n_clusters != 16) return ABATT_EUNSUPPORTED;
  const int64_t n_qb = (p->N + p->q_block - 1) / p->q_block;
  const int64_t R = (int64_t)p->B * p->H * n_qb;
  if (R > INT32_MAX / 2) return ABATT_EUNSUPPORTED;
  // one head of K or V is addressed through a 32-bit buffer range
  if ((int64_t)p->N * p->D * 4 > INT32_MAX) return ABATT_EUNSUPPORTED;
  s->B = p->B;
  s->H = p->H;
  s->N = p->N;
  s->D = p->D;
  s->q_block = p->q_block;
  s->kv_block = p->kv_block;
  s->n_clusters = p->n_clusters;
  s->kmeans_iters = p->kmeans_iters;
  s->n_qb = (int)n_qb;
  s->n_kbs = (p->N - p->n_forced_tail) / p->kv_block;
  s->n_kb = s->n_kbs + p->n_forced_tail / p->kv_block;
  s->R = (int)R;
  s->scale = p->scale;
  s->bf16 = p->dtype == ABATT_BF16;
  return ABATT_OK;
}

// Dense attention accepts any N (keys past N are masked) and ignores the
// key-block size and the forced tail (it runs over every key in groups of 4);
// the other checks are the same as for the plan problem.
abatt_status make_dense_shape(const abatt_problem_t* p, Shape* s) {
  if (p == nullptr) return ABATT_EINVAL;
  abatt_problem_t q = *p;
  q.n_forced_tail = 0;
  q.kv_block = 4;
  const int N = q.N;
  if (N > 0 && N % 4 != 0) q.N = N + (4 - N % 4);  // only for the block checks
  abatt_status st = make_shape(&q, s);
  if (st != ABATT_OK) return st;
  s->N = N;
  s->n_qb = (N + s->q_block - 1) / s->q_block;
  s->R = s->B * s->H * s->n_qb;
  return ABATT_OK;
}

struct PlanWs {
  size_t kmean, mu, w, S, partial, sampler, total;
};

// the sampler's scratch, for either sampler
size_t sampler_region(const Shape& s) {
  const size_t a = abatt::sampler_ws_layout(s).total, b = abatt::onepass_ws_layout(s).total;
  return a > b ? a : b;
}

PlanWs plan_ws_layout(const Shape& s) {
  PlanWs l;
  size_t off = 0;
  l.kmean = off;
  off = align_up(off + (size_t)s.B * s.H * s.n_kbs * s.D * sizeof(float));
  l.mu = off;
  off = align_up(off + (size_t)s.R * s.n_clusters * s.D * sizeof(float));
  l.w = off;
  off = align_up(off + (size_t)s.R * s.n_clusters * sizeof(float));
  l.S = off;
  off = align_up(off + (size_t)s.R * s.n_kbs * sizeof(float));
  l.partial = off;
  off = align_up(off + abatt::scores_partial_bytes(s));
  l.sampler = off;
  off = align_up(off + sampler_region(s));
  l.total = off;
  return l;
}

size_t sampler_ws_bytes(const Shape& s) { return align_up(sampler_region(s)); }

abatt_status hip_status(hipError_t e) { return e == hipSuccess ? ABATT_OK : ABATT_EHIP; }

// A second stream per device, owned by the library (default priority), and
// the two events that fork it from a caller's stream and join it back.
struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
Side g_side[kMaxDevices];

// The current device's side stream, created on first use; nullptr when it is
// not to be used: `stream` is under capture (a stream that joins a capture
// stays part of it until the capture ends, so eager calls from other threads
// would be captured too; captured plans run on `stream` alone), the device
// index is out of range, creation failed, or the stream does not exist yet
// and may not be created (`may_create` false).  Called with g_side_mu held.
Side* side_stream(hipStream_t stream, bool may_create) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();  // the launches that follow report their own errors
    return nullptr;
  }
  if (cs != hipStreamCaptureStatusNone) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  Side& sd = g_side[dev];
  if (sd.s != nullptr) return &sd;
  if (!may_create) return nullptr;
  Side n;
  if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) == hipSuccess &&
      hipEventCreateWithFlags(&n.join, hipEventDisableTiming) == hipSuccess) {
    sd = n;
    return &sd;
  }
  if (n.join != nullptr) (void)hipEventDestroy(n.join);
  if (n.fork != nullptr) (void)hipEventDestroy(n.fork);
  if (n.s != nullptr) (void)hipStreamDestroy(n.s);
  return nullptr;
}

// Key means in their scoring form, centroids and weights, scores.  The
// key-mean region holds two bf16 planes (fp32 problems) or one fp16 plane
// followed by the per-tile scales (bf16 problems), which fits in the same
// space.
//
// The key means (K only, bound by HBM) and k-means (Q only, bound by the
// latency of its Lloyd iterations) do not depend on each other, so they run
// side by side: the key means on the side stream, forked from `stream` by an
// event, k-means on `stream`, which waits for the side stream's join event
// before the scorer.  The call thus stays ordered on `stream`.  Without a
// side stream (and always under graph capture) both run on `stream`, one
// after the other, with the same results.
hipError_t run_scores(const Shape& s, const PlanWs& l, char* ws, const void* Q, const void* K,
                      float* mu, float* w, float* S, hipStream_t stream, bool may_create = true) {
  uint16_t* kplanes = reinterpret_cast<uint16_t*>(ws + l.kmean);
  float* tscale = s.bf16 ? reinterpret_cast<float*>(kplanes + (size_t)s.B * s.H * s.n_kbs * s.D)
                         : nullptr;
  auto key_means = [&](hipStream_t st) {
    return s.bf16 ? abatt::launch_key_means_f16(s, K, kplanes, tscale, st)
                  : abatt::launch_key_means_split(s, K, kplanes, st);
  };
  hipError_t e;
  {
    // one fork / join at a time: the events are shared by every call on the device
    std::lock_guard<std::mutex> lock(g_side_mu);
    Side* sd = side_stream(stream, may_create);
    if (sd == nullptr) {
      e = key_means(stream);
      if (e == hipSuccess) e = abatt::launch_kmeans(s, Q, mu, w, stream);
    } else {
      e = hipEventRecord(sd->fork, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
      if (e == hipSuccess) {
        // joined whatever the launches return: `stream` always waits for
        // the side stream's work before it goes on
        const hipError_t ek = key_means(sd->s);
        const hipError_t er = hipEventRecord(sd->join, sd->s);
        const hipError_t em = abatt::launch_kmeans(s, Q, mu, w, stream);
        const hipError_t ej = er == hipSuccess ? hipStreamWaitEvent(stream, sd->join, 0) : er;
        e = ek != hipSuccess ? ek : (em != hipSuccess ? em : ej);
      }
    }
  }
  if (e == hipSuccess) e = abatt::launch_scores(s, mu, w, kplanes, tscale, S, ws + l.partial, stream);
  return e;
}

// The whole plan (selector, then sampler) on the workspace `ws` laid out as l;
// onepass selects the one-pass sampler (the same plan).
hipError_t run_plan(const Shape& s, const PlanWs& l, char* ws, const void* Q, const void* K,
                    double budget, uint64_t seed, const abatt_plan_t* plan, hipStream_t stream,
                    bool onepass = false, bool may_create = true) {
  float* mu = reinterpret_cast<float*>(ws + l.mu);
  float* w = reinterpret_cast<float*>(ws + l.w);
  float* S = reinterpret_cast<float*>(ws + l.S);
  hipError_t e = run_scores(s, l, ws, Q, K, mu, w, S, stream, may_create);
  if (e == hipSuccess)
    e = (onepass ? abatt::launch_sampler_onepass : abatt::launch_sampler)(
        s, S, budget, seed, ws + l.sampler, plan->row_ptr, plan->col_idx, plan->logw,
        plan->capacity, plan->status, stream);
  return e;
}

bool budget_ok(double budget) { return budget > 0.0 && budget <= 1.0 && std::isfinite(budget); }

abatt_status check_plan(const Shape& s, const abatt_plan_t* plan, bool need_status) {
  if (plan == nullptr || plan->row_ptr == nullptr || plan->col_idx == nullptr ||
      plan->logw == nullptr)
    return ABATT_EINVAL;
  if (need_status && plan->status == nullptr) return ABATT_EINVAL;
  if (plan->capacity < 0) return ABATT_EINVAL;
  return ABATT_OK;
}

}  // namespace

extern "C" {

int64_t abatt_plan_rows(const abatt_problem_t* p) {
  Shape s;
  return make_shape(p, &s) == ABATT_OK ? (int64_t)s.R : -1;
}

int64_t abatt_plan_max_nnz(const abatt_problem_t* p) {
  Shape s;
  if (make_shape(p, &s) != ABATT_OK) return -1;
  return (int64_t)s.R * s.n_kb;
}

int64_t abatt_plan_nnz_bound(const abatt_problem_t* p, double budget) {
  Shape s;
  if (make_shape(p, &s) != ABATT_OK || !budget_ok(budget)) return -1;
  const double m = budget * (double)s.n_kbs;
  double per = std::ceil(m + 10.0 * std::sqrt(m) + 16.0);
  if (per > (double)s.n_kbs) per = (double)s.n_kbs;
  return (int64_t)s.R * ((int64_t)per + (s.n_kb - s.n_kbs));
}

size_t abatt_plan_workspace_bytes(const abatt_problem_t* p) {
  Shape s;
  if (make_shape(p, &s) != ABATT_OK) return 0;
  return plan_ws_layout(s).total;
}

size_t abatt_sampler_workspace_bytes(const abatt_problem_t* p) {
  Shape s;
  if (make_shape(p, &s) != ABATT_OK) return 0;
  return sampler_ws_bytes(s);
}

abatt_status abatt_key_means(const abatt_problem_t* p, const void* K, float* kmean,
                             hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(K) || bad(kmean)) return ABATT_EINVAL;
  return hip_status(abatt::launch_key_means(s, K, kmean, stream));
}

abatt_status abatt_scores(const abatt_problem_t* p, const void* Q, const void* K, float* S,
                          float* centroids, float* weights, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || S == nullptr || bad(workspace)) return ABATT_EINVAL;
  const PlanWs l = plan_ws_layout(s);
  if (workspace_bytes < l.total) return ABATT_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* mu = centroids ? centroids : reinterpret_cast<float*>(ws + l.mu);
  float* w = weights ? weights : reinterpret_cast<float*>(ws + l.w);
  return hip_status(run_scores(s, l, ws, Q, K, mu, w, S, stream));
}

abatt_status abatt_plan_from_scores(const abatt_problem_t* p, const float* S, double budget,
                                    uint64_t seed, void* workspace, size_t workspace_bytes,
                                    abatt_plan_t* plan, hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (S == nullptr || bad(workspace) || !budget_ok(budget)) return ABATT_EINVAL;
  st = check_plan(s, plan, true);
  if (st != ABATT_OK) return st;
  if (workspace_bytes < sampler_ws_bytes(s)) return ABATT_EWORKSPACE;
  if (plan->capacity < (int64_t)s.R * (s.n_kb - s.n_kbs)) return ABATT_ECAPACITY;
  return hip_status(abatt::launch_sampler(s, S, budget, seed, workspace, plan->row_ptr,
                                          plan->col_idx, plan->logw, plan->capacity,
                                          plan->status, stream));
}

abatt_status abatt_plan(const abatt_problem_t* p, const void* Q, const void* K, double budget,
                        uint64_t seed, void* workspace, size_t workspace_bytes,
                        abatt_plan_t* plan, hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || bad(workspace) || !budget_ok(budget))
    return ABATT_EINVAL;
  st = check_plan(s, plan, true);
  if (st != ABATT_OK) return st;
  const PlanWs l = plan_ws_layout(s);
  if (workspace_bytes < l.total) return ABATT_EWORKSPACE;
  if (plan->capacity < (int64_t)s.R * (s.n_kb - s.n_kbs)) return ABATT_ECAPACITY;
  return hip_status(run_plan(s, l, static_cast<char*>(workspace), Q, K, budget, seed, plan,
                             stream));
}

abatt_status abatt_plan_onepass(const abatt_problem_t* p, const void* Q, const void* K,
                                double budget, uint64_t seed, void* workspace,
                                size_t workspace_bytes, abatt_plan_t* plan, hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || bad(workspace) || !budget_ok(budget))
    return ABATT_EINVAL;
  st = check_plan(s, plan, true);
  if (st != ABATT_OK) return st;
  const PlanWs l = plan_ws_layout(s);
  if (workspace_bytes < l.total) return ABATT_EWORKSPACE;
  if (plan->capacity < (int64_t)s.R * (s.n_kb - s.n_kbs)) return ABATT_ECAPACITY;
  return hip_status(run_plan(s, l, static_cast<char*>(workspace), Q, K, budget, seed, plan,
                             stream, true));
}

abatt_status abatt_plan_noalloc(const abatt_problem_t* p, const void* Q, const void* K,
                                double budget, uint64_t seed, abatt_plan_t* plan,
                                hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || !budget_ok(budget)) return ABATT_EINVAL;
  st = check_plan(s, plan, true);
  if (st != ABATT_OK) return st;
  const PlanWs l = plan_ws_layout(s);
  if (l.total > (size_t)ABATT_SCRATCH_BYTES) return ABATT_ESCRATCH;
  if (plan->capacity < (int64_t)s.R * (s.n_kb - s.n_kbs)) return ABATT_ECAPACITY;
  void* ws = nullptr;
  hipError_t e = abatt::scratch_ptr(&ws);
  if (e != hipSuccess) return ABATT_EHIP;
  // creates no side stream (it uses one an earlier call made)
  return hip_status(run_plan(s, l, static_cast<char*>(ws), Q, K, budget, seed, plan, stream,
                             false, false));
}

abatt_status abatt_attend(const abatt_problem_t* p, const void* Q, const void* K, const void* V,
                          const abatt_plan_t* plan, void* O, float* lse, hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || bad(V) || bad(O)) return ABATT_EINVAL;
  st = check_plan(s, plan, false);
  if (st != ABATT_OK) return st;
  return hip_status(abatt::launch_attend(s, Q, K, V, plan->row_ptr, plan->col_idx, plan->logw,
                                         plan->capacity, plan->status, O, lse, true, false,
                                         stream));
}

abatt_status abatt_v_to_f16(const abatt_problem_t* p, const void* V, void* V16,
                            hipStream_t stream) {
  // an elementwise conversion: any N (as for dense attention) is fine
  Shape s;
  abatt_status st = make_dense_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (!s.bf16) return ABATT_EUNSUPPORTED;
  if (bad(V) || bad(V16) || V == V16) return ABATT_EINVAL;
  return hip_status(abatt::launch_v_to_f16(s, V, V16, stream));
}

abatt_status abatt_attend_v16(const abatt_problem_t* p, const void* Q, const void* K,
                              const void* V16, const abatt_plan_t* plan, void* O, float* lse,
                              hipStream_t stream) {
  Shape s;
  abatt_status st = make_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (!s.bf16) return ABATT_EUNSUPPORTED;
  if (bad(Q) || bad(K) || bad(V16) || bad(O)) return ABATT_EINVAL;
  st = check_plan(s, plan, false);
  if (st != ABATT_OK) return st;
  return hip_status(abatt::launch_attend(s, Q, K, V16, plan->row_ptr, plan->col_idx,
                                         plan->logw, plan->capacity, plan->status, O, lse, true,
                                         true, stream));
}

abatt_status abatt_dense(const abatt_problem_t* p, const void* Q, const void* K, const void* V,
                         void* O, float* lse, hipStream_t stream) {
  Shape s;
  abatt_status st = make_dense_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (bad(Q) || bad(K) || bad(V) || bad(O)) return ABATT_EINVAL;
  return hip_status(abatt::launch_attend(s, Q, K, V, nullptr, nullptr, nullptr, 0, nullptr, O,
                                         lse, false, false, stream));
}

abatt_status abatt_dense_v16(const abatt_problem_t* p, const void* Q, const void* K,
                             const void* V16, void* O, float* lse, hipStream_t stream) {
  Shape s;
  abatt_status st = make_dense_shape(p, &s);
  if (st != ABATT_OK) return st;
  if (!s.bf16) return ABATT_EUNSUPPORTED;
  if (bad(Q) || bad(K) || bad(V16) || bad(O)) return ABATT_EINVAL;
  return hip_status(abatt::launch_attend(s, Q, K, V16, nullptr, nullptr, nullptr, 0, nullptr, O,
                                         lse, false, true, stream));
}

const char* abatt_status_str(abatt_status s) {
  switch (s) {
    case ABATT_OK: return "ok";
    case ABATT_EINVAL: return "invalid argument";
    case ABATT_EUNSUPPORTED: return "unsupported problem (D, block sizes or cluster count)";
    case ABATT_EWORKSPACE: return "workspace too small";
    case ABATT_ECAPACITY: return "plan capacity too small";
    case ABATT_EHIP: return "HIP launch failed";
    case ABATT_ESCRATCH: return "plan workspace exceeds the library's static scratch (ABATT_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* abatt_version(void) { return "abatt 0.1 (gfx950)"; }

}  // extern "C"
