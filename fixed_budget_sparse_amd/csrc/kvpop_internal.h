// Internal definitions shared by the libkvpop HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvpop {

// ---------------------------------------------------------------- problem
struct Dims {
  int b, Hq, Hkv, G, S, D;
  int s, w, k;
  float scale;        // softmax scale (resolved: > 0)
  bool f32_in;        // q/k/v (and decode cache) in float32, else bfloat16
  bool f32_out;       // attention output in float32, else bfloat16
  int nseg() const { return b * Hkv; }
  long long budget() const { return (long long)s + w + k; }
};

// Workspace carving: every region is 256-byte aligned.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes, tilings and launchers of each call (defined in the .hip files).
size_t thresholds_ws_bytes(const Dims& d);
hipError_t launch_thresholds(const Dims& d, const float* prio, int* rank, int* tau,
                             void* ws, hipStream_t st);

int launch_order_reversed();               // testing aid: last tile first when nonzero
int fwd_rows_per_head(const Dims& d);          // query rows per head in one tile
size_t fwd_ws_bytes(const Dims& d);
hipError_t launch_masked_fwd(const Dims& d, const void* q, const void* k, const void* v,
                             const int* rank, const int* tau, void* o, float* lse,
                             void* ws, hipStream_t st);

// The forward's per-tile key plan (tiles of m query rows per head; listed
// long-range keys of each tile's first row in rank order), built into the
// first fwd_ws_bytes(d) bytes of `ws`; the backward reuses it.
struct FwdPlan {
  const int2* list;   // [nseg, ntiles, cap] (token, q_end(token))
  const int* count;   // [nseg, ntiles]
  const int* qend;    // [nseg, S]: the last row that keeps each token
  int m, ntiles, cap;
};
FwdPlan launch_fwd_plan(const Dims& d, const int* rank, const int* tau, void* ws,
                        hipStream_t st);

size_t bwd_ws_bytes(const Dims& d);
hipError_t launch_masked_bwd(const Dims& d, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const int* rank, const int* tau,
                             const void* dout, float* dq, float* dk, float* dv, void* ws,
                             hipStream_t st);

size_t target_ws_bytes(const Dims& d);
hipError_t launch_future_target(const Dims& d, const void* q, const void* k, const float* lse,
                                float* target, void* ws, hipStream_t st);

struct CacheArgs {
  void* k;
  void* v;
  int* slot_pos;
  float* slot_prio;
  int* ring;
  int* state;   // may be null
};
int decode_splits(const Dims& d);
size_t decode_ws_bytes(const Dims& d);
hipError_t launch_decode(const Dims& d, const CacheArgs& c, const int* pos, const void* q,
                         const void* k_new, const void* v_new, const float* prio_leaving,
                         void* o, float* lse, void* ws, hipStream_t st);
// The fixed device scratch of the no-allocation decode entry point: its size,
// and its device address on the device of stream `st` (which must be the
// current device; hipErrorInvalidDevice otherwise).
size_t decode_noalloc_scratch_bytes();
hipError_t decode_noalloc_scratch(hipStream_t st, void** out);

hipError_t launch_cache_from_prefill(const Dims& d, const CacheArgs& c, const void* k,
                                     const void* v, const float* prio, const int* rank,
                                     const int* tau, hipStream_t st);
hipError_t launch_target_score(const Dims& d, const float* target, float eps, float* score,
                               hipStream_t st);

int labels_max_seq();
hipError_t launch_boundary_labels(const Dims& d, const float* score, const float* log_gamma,
                                  int decay_step, int32_t* t_bnd, int32_t* y, hipStream_t st);

}  // namespace kvpop
