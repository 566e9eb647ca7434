// libkvpop C ABI: host-side validation, workspace sizing and dispatch.
// Nothing here allocates device memory or synchronises; every entry point
// validates all arguments before its first launch.
#include <math.h>

#include <atomic>

#include "kvpop.h"
#include "kvpop_internal.h"

#define KVPOP_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using kvpop::Dims;

constexpr int kMaxSeq = 262144;
constexpr long long kMaxBudget = 1LL << 30;

bool dtype_ok(int32_t d) { return d == KVPOP_BF16 || d == KVPOP_F32; }

// Shape checks shared by every call; `call` selects the per-call rules.
kvpop_status make_dims(int32_t call, const kvpop_problem* pr, Dims* d) {
  if (!pr) return KVPOP_ERR_ARG;
  if (pr->batch < 1 || pr->n_q_heads < 1 || pr->n_kv_heads < 1) return KVPOP_ERR_ARG;
  if (pr->n_q_heads % pr->n_kv_heads != 0) return KVPOP_ERR_ARG;
  if (pr->sink < 0 || pr->window < 0 || pr->topk < 0) return KVPOP_ERR_ARG;
  const long long budget = (long long)pr->sink + pr->window + pr->topk;
  if (budget > kMaxBudget) return KVPOP_ERR_ARG;
  if (!dtype_ok(pr->qkv_dtype) || !dtype_ok(pr->out_dtype)) return KVPOP_ERR_ARG;
  if (!(pr->softmax_scale == pr->softmax_scale) || isinf(pr->softmax_scale)) return KVPOP_ERR_ARG;
  // sizes whose products the launch geometry and the index arithmetic hold:
  // (sequence, KV head) pairs on a grid's y/z axis, query heads x sequences
  // in a 30-bit grid, and at most 2^40 elements per prefill tensor
  if ((long long)pr->batch * pr->n_kv_heads > 65535) return KVPOP_ERR_UNSUPPORTED;
  if ((long long)pr->batch * pr->n_q_heads > (1LL << 20)) return KVPOP_ERR_UNSUPPORTED;
  if (call != KVPOP_CALL_DECODE &&
      (long long)pr->batch * pr->n_q_heads * (long long)pr->seq_len * pr->head_dim > (1LL << 40))
    return KVPOP_ERR_UNSUPPORTED;
  const int G = pr->n_q_heads / pr->n_kv_heads;
  if (call != KVPOP_CALL_THRESHOLDS && call != KVPOP_CALL_TARGET_SCORE &&
      call != KVPOP_CALL_BOUNDARY_LABELS) {
    if (pr->head_dim != 64 && pr->head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
    if (G > 32) return KVPOP_ERR_UNSUPPORTED;
  }
  if (call == KVPOP_CALL_DECODE) {
    if (pr->window < 1 || budget < 1) return KVPOP_ERR_ARG;
  } else {
    if (call == KVPOP_CALL_CACHE_FROM_PREFILL && pr->window < 1) return KVPOP_ERR_ARG;
    if (pr->seq_len < 1) return KVPOP_ERR_ARG;
    if (pr->seq_len > kMaxSeq) return KVPOP_ERR_UNSUPPORTED;
    if ((call == KVPOP_CALL_MASKED_FWD || call == KVPOP_CALL_MASKED_BWD) && pr->window < 1)
      return KVPOP_ERR_ARG;
    if (call == KVPOP_CALL_MASKED_BWD && pr->qkv_dtype != KVPOP_BF16)
      return KVPOP_ERR_UNSUPPORTED;
  }
  d->b = pr->batch;
  d->Hq = pr->n_q_heads;
  d->Hkv = pr->n_kv_heads;
  d->G = G;
  d->S = call == KVPOP_CALL_DECODE ? 0 : pr->seq_len;
  d->D = pr->head_dim;
  d->s = pr->sink;
  d->w = pr->window;
  d->k = pr->topk;
  d->scale = pr->softmax_scale > 0.0f ? pr->softmax_scale : 1.0f / sqrtf((float)pr->head_dim);
  d->f32_in = pr->qkv_dtype == KVPOP_F32;
  d->f32_out = pr->out_dtype == KVPOP_F32;
  return KVPOP_OK;
}

size_t ws_bytes(int32_t call, const Dims& d) {
  switch (call) {
    case KVPOP_CALL_THRESHOLDS: return kvpop::thresholds_ws_bytes(d);
    case KVPOP_CALL_MASKED_FWD: return kvpop::fwd_ws_bytes(d);
    case KVPOP_CALL_FUTURE_TARGET: return kvpop::target_ws_bytes(d);
    case KVPOP_CALL_DECODE: return kvpop::decode_ws_bytes(d);
    case KVPOP_CALL_MASKED_BWD: return kvpop::bwd_ws_bytes(d);
    default: return 0;
  }
}

kvpop_status check_ws(int32_t call, const Dims& d, const void* ws, size_t ws_len) {
  const size_t need = ws_bytes(call, d);
  if (need == 0) return KVPOP_OK;
  if (!ws || ws_len < need) return KVPOP_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return KVPOP_ERR_ARG;   // regions are carved 256-aligned
  return KVPOP_OK;
}

kvpop_status finish(hipError_t e) { return e == hipSuccess ? KVPOP_OK : KVPOP_ERR_HIP; }

}  // namespace

KVPOP_EXPORT size_t kvpop_workspace_size(int32_t call, const kvpop_problem* pr) {
  Dims d;
  if (call < KVPOP_CALL_THRESHOLDS || call > KVPOP_CALL_MASKED_BWD) return 0;
  if (make_dims(call, pr, &d) != KVPOP_OK) return 0;
  return ws_bytes(call, d);
}

KVPOP_EXPORT kvpop_status kvpop_thresholds(const kvpop_problem* pr, const float* prio,
                                           int32_t* rank, int32_t* tau, void* ws,
                                           size_t ws_bytes_, hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_THRESHOLDS, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!prio || !rank || !tau) return KVPOP_ERR_ARG;
  st = check_ws(KVPOP_CALL_THRESHOLDS, d, ws, ws_bytes_);
  if (st != KVPOP_OK) return st;
  return finish(kvpop::launch_thresholds(d, prio, rank, tau, ws, stream));
}

KVPOP_EXPORT kvpop_status kvpop_masked_attn_fwd(const kvpop_problem* pr, const void* q,
                                                const void* k, const void* v,
                                                const int32_t* rank, const int32_t* tau, void* o,
                                                float* lse, void* ws, size_t ws_bytes_,
                                                hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_MASKED_FWD, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !v || !rank || !tau || !o || !lse) return KVPOP_ERR_ARG;
  st = check_ws(KVPOP_CALL_MASKED_FWD, d, ws, ws_bytes_);
  if (st != KVPOP_OK) return st;
  return finish(kvpop::launch_masked_fwd(d, q, k, v, rank, tau, o, lse, ws, stream));
}

KVPOP_EXPORT kvpop_status kvpop_future_target(const kvpop_problem* pr, const void* q,
                                              const void* k, const float* lse, float* target,
                                              void* ws, size_t ws_bytes_, hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_FUTURE_TARGET, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !lse || !target) return KVPOP_ERR_ARG;
  st = check_ws(KVPOP_CALL_FUTURE_TARGET, d, ws, ws_bytes_);
  if (st != KVPOP_OK) return st;
  return finish(kvpop::launch_future_target(d, q, k, lse, target, ws, stream));
}

KVPOP_EXPORT kvpop_status kvpop_decode_step(const kvpop_problem* pr, const kvpop_cache* cache,
                                            const int32_t* pos, const void* q, const void* k_new,
                                            const void* v_new, const float* prio_leaving,
                                            void* o, float* lse, void* ws, size_t ws_bytes_,
                                            hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_DECODE, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!cache || !cache->k || !cache->v || !cache->slot_pos || !cache->slot_prio || !cache->ring)
    return KVPOP_ERR_ARG;
  if ((uintptr_t)cache->state % 16 != 0) return KVPOP_ERR_ARG;   // read as 16-byte records
  if (!pos || !q || !k_new || !v_new || !prio_leaving || !o) return KVPOP_ERR_ARG;
  st = check_ws(KVPOP_CALL_DECODE, d, ws, ws_bytes_);
  if (st != KVPOP_OK) return st;
  kvpop::CacheArgs c{cache->k, cache->v, cache->slot_pos, cache->slot_prio, cache->ring,
                     cache->state};
  return finish(kvpop::launch_decode(d, c, pos, q, k_new, v_new, prio_leaving, o, lse, ws, stream));
}

KVPOP_EXPORT kvpop_status kvpop_decode_step_noalloc(const kvpop_problem* pr,
                                                    const kvpop_cache* cache, const int32_t* pos,
                                                    const void* q, const void* k_new,
                                                    const void* v_new, const float* prio_leaving,
                                                    void* o, float* lse, hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_DECODE, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!cache || !cache->k || !cache->v || !cache->slot_pos || !cache->slot_prio || !cache->ring)
    return KVPOP_ERR_ARG;
  if ((uintptr_t)cache->state % 16 != 0) return KVPOP_ERR_ARG;   // read as 16-byte records
  if (!pos || !q || !k_new || !v_new || !prio_leaving || !o) return KVPOP_ERR_ARG;
  const size_t need = ws_bytes(KVPOP_CALL_DECODE, d);
  if (need > kvpop::decode_noalloc_scratch_bytes()) return KVPOP_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && kvpop::decode_noalloc_scratch(stream, &ws) != hipSuccess) return KVPOP_ERR_HIP;
  kvpop::CacheArgs c{cache->k, cache->v, cache->slot_pos, cache->slot_prio, cache->ring,
                     cache->state};
  return finish(kvpop::launch_decode(d, c, pos, q, k_new, v_new, prio_leaving, o, lse, ws, stream));
}

KVPOP_EXPORT kvpop_status kvpop_cache_from_prefill(const kvpop_problem* pr,
                                                   const kvpop_cache* cache, const void* k,
                                                   const void* v, const float* prio,
                                                   const int32_t* rank, const int32_t* tau,
                                                   hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_CACHE_FROM_PREFILL, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!cache || !cache->k || !cache->v || !cache->slot_pos || !cache->slot_prio || !cache->ring)
    return KVPOP_ERR_ARG;
  if ((uintptr_t)cache->state % 16 != 0) return KVPOP_ERR_ARG;   // read as 16-byte records
  if (!k || !v || !prio || !rank || !tau) return KVPOP_ERR_ARG;
  kvpop::CacheArgs c{cache->k, cache->v, cache->slot_pos, cache->slot_prio, cache->ring,
                     cache->state};
  return finish(kvpop::launch_cache_from_prefill(d, c, k, v, prio, rank, tau, stream));
}

KVPOP_EXPORT kvpop_status kvpop_target_score(const kvpop_problem* pr, const float* target,
                                             float eps, float* score, hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_TARGET_SCORE, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!target || !score) return KVPOP_ERR_ARG;
  if (!(eps >= 0.0f) || isinf(eps)) return KVPOP_ERR_ARG;
  return finish(kvpop::launch_target_score(d, target, eps, score, stream));
}

KVPOP_EXPORT kvpop_status kvpop_masked_attn_bwd(const kvpop_problem* pr, const void* q,
                                                const void* k, const void* v, const void* o,
                                                const float* lse, const int32_t* rank,
                                                const int32_t* tau, const void* dout, float* dq,
                                                float* dk, float* dv, void* ws, size_t ws_bytes_,
                                                hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_MASKED_BWD, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !v || !o || !lse || !rank || !tau || !dout || !dq || !dk || !dv)
    return KVPOP_ERR_ARG;
  st = check_ws(KVPOP_CALL_MASKED_BWD, d, ws, ws_bytes_);
  if (st != KVPOP_OK) return st;
  return finish(kvpop::launch_masked_bwd(d, q, k, v, o, lse, rank, tau, dout, dq, dk, dv, ws,
                                         stream));
}

KVPOP_EXPORT kvpop_status kvpop_boundary_labels(const kvpop_problem* pr, const float* score,
                                                const float* log_gamma, int32_t decay_step,
                                                int32_t* t_bnd, int32_t* y, hipStream_t stream) {
  Dims d;
  kvpop_status st = make_dims(KVPOP_CALL_BOUNDARY_LABELS, pr, &d);
  if (st != KVPOP_OK) return st;
  if (!score || !log_gamma || !t_bnd || !y) return KVPOP_ERR_ARG;
  if (decay_step < 1) return KVPOP_ERR_ARG;
  if (d.S > kvpop::labels_max_seq()) return KVPOP_ERR_UNSUPPORTED;
  return finish(kvpop::launch_boundary_labels(d, score, log_gamma, decay_step, t_bnd, y, stream));
}

KVPOP_EXPORT const char* kvpop_status_string(int32_t st) {
  switch (st) {
    case KVPOP_OK: return "ok";
    case KVPOP_ERR_ARG: return "invalid argument";
    case KVPOP_ERR_UNSUPPORTED: return "unsupported problem";
    case KVPOP_ERR_WORKSPACE: return "workspace too small";
    case KVPOP_ERR_HIP: return "HIP launch failed";
    case KVPOP_ERR_SCRATCH: return "problem exceeds the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

KVPOP_EXPORT int32_t kvpop_abi_version(void) { return KVPOP_ABI_VERSION; }

namespace kvpop {
namespace {
std::atomic<int> g_reverse_launch{0};
}  // namespace
int launch_order_reversed() { return g_reverse_launch.load(std::memory_order_relaxed); }
}  // namespace kvpop

KVPOP_EXPORT void kvpop_debug_reverse_launch_order(int32_t on) {
  kvpop::g_reverse_launch.store(on != 0 ? 1 : 0, std::memory_order_relaxed);
}
