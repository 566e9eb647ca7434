/* kvpop.h — C ABI of libkvpop: the data-parallel hot path of KVpop's
 * fixed-budget sparse KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title):
 *   [Notes]  "KVpop -- Key-Value Cache Compression with Predictive Online Pruning
 *            精读笔记" (reading notes on arXiv 2607.05061), the page with the
 *            method's formulas.
 *   [Sum-zh] "技术摘要：KVpop — 基于预测性在线剪枝的键值（KV）缓存压缩".
 * Every KV head keeps B = s + w + k entries ([Notes] §2.1): s sink tokens, the
 * w most recent tokens (a protected window) and the k best older tokens under a
 * static per-token priority.  The sparse mask of [Notes] §2.3 is
 *   M[q,t] = (t < s) or (q - t < w) or (s <= t <= q - w and rank(t) <= tau_q)
 * taken together with causality (t <= q), where rank(t) is the place of t in
 * the priority order and tau_q the rank of the k-th best eligible token.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers, allocated and owned by the caller.  The
 *     library allocates and frees nothing and keeps no state between calls.
 *   - Every call only enqueues kernels on `stream` and returns; nothing
 *     synchronises.  Arguments are validated on the host first: on any error
 *     nothing is launched and a non-zero status is returned.  A failed launch
 *     returns KVPOP_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Tensors are contiguous, row-major, in the shapes given below.
 *   - `ws` is caller-owned scratch of at least kvpop_workspace_size(call, pr)
 *     bytes (NULL allowed when that size is 0); its contents on entry are
 *     ignored and on exit undefined.  Calls that share a workspace or outputs
 *     must not overlap in time.
 *   - Priority order: higher priority first, ties to the lower token index;
 *     -0 equals +0 and NaN counts as -inf.
 *   - Query head h reads KV head h / (Hq / Hkv).  Priorities, ranks, cutoffs
 *     and decode caches are per KV head.
 *   - Logs are natural logs.
 */
#ifndef KVPOP_H
#define KVPOP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVPOP_ABI_VERSION 6

typedef enum {
  KVPOP_OK = 0,
  KVPOP_ERR_ARG = 1,          /* invalid argument (shape, NULL pointer, budget) */
  KVPOP_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement  */
  KVPOP_ERR_WORKSPACE = 3,    /* ws_bytes smaller than kvpop_workspace_size()   */
  KVPOP_ERR_HIP = 4,          /* a kernel launch failed                          */
  KVPOP_ERR_SCRATCH = 5       /* kvpop_decode_step_noalloc: the problem needs more
                                 than KVPOP_NOALLOC_SCRATCH_BYTES of scratch    */
} kvpop_status;

/* Size of the fixed device scratch of kvpop_decode_step_noalloc (per GPU). */
#define KVPOP_NOALLOC_SCRATCH_BYTES (8u << 20)

typedef enum { KVPOP_BF16 = 0, KVPOP_F32 = 1 } kvpop_dtype;

typedef enum {
  KVPOP_CALL_THRESHOLDS = 0,
  KVPOP_CALL_MASKED_FWD = 1,
  KVPOP_CALL_FUTURE_TARGET = 2,
  KVPOP_CALL_DECODE = 3,
  KVPOP_CALL_CACHE_FROM_PREFILL = 4,
  KVPOP_CALL_TARGET_SCORE = 5,
  KVPOP_CALL_BOUNDARY_LABELS = 6,
  KVPOP_CALL_MASKED_BWD = 7
} kvpop_call;

/* Problem description shared by all calls.
 *   batch       sequences (>= 1)
 *   n_q_heads   Hq; n_kv_heads Hkv; Hq % Hkv == 0 and 1 <= Hq/Hkv <= 32;
 *               batch * Hkv <= 65535, batch * Hq <= 2^20 and, for prefill
 *               calls, batch * Hq * S * D <= 2^40 (KVPOP_ERR_UNSUPPORTED above)
 *   seq_len     S (prefill calls; 1 <= S <= 262144); ignored by decode
 *   head_dim    D in {64, 128}
 *   sink, window, topk   s >= 0, w >= 0, k >= 0 with s + w + k <= 2^30;
 *               w >= 1 for the forward and decode calls
 *   softmax_scale  logit scale; <= 0 selects 1/sqrt(D)
 *   qkv_dtype   KVPOP_BF16 or KVPOP_F32 (dtype of q, k, v and the decode cache)
 *   out_dtype   dtype of the attention output o (KVPOP_BF16 or KVPOP_F32) */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t sink;
  int32_t window;
  int32_t topk;
  float softmax_scale;
  int32_t qkv_dtype;
  int32_t out_dtype;
} kvpop_problem;

/* Fixed-size decode cache of capacity Bc = s + w + k slots per (sequence, KV
 * head) ([Notes] §2.3: inference keeps only the compact cache; [Sum-zh] §4.3:
 * the fixed per-head budget keeps memory constant).  All arrays are caller
 * owned, persist between decode calls and may be copied to checkpoint.
 *   k, v       [batch, Hkv, Bc, D] in qkv_dtype
 *   slot_pos   [batch, Hkv, Bc] int32: token position held by each slot
 *   slot_prio  [batch, Hkv, Bc] float: priority of the long-range token held
 *   ring       [batch, Hkv, w]  int32: slot of window position p mod w
 *   state      [batch, Hkv, KVPOP_CACHE_STATE_WORDS] int32, or NULL: a record
 *              derived from the arrays above that spares the next step a scan
 *              of every slot: the step p + 1 it is for, then the priority
 *              (float bits), position and slot of the worst held long-range
 *              token after step p (slot -1: none), then spare words.  Each
 *              decode step writes it for the next step; a step uses it only
 *              when its first word equals the step's p, and otherwise scans
 *              the slots (as every step does with NULL).  Zero-filled is
 *              valid; kvpop_cache_from_prefill marks it stale.  Save and
 *              restore it together with the other arrays.  16-byte aligned
 *              (KVPOP_ERR_ARG otherwise).
 * Slots 0 .. min(p, Bc)-1 are the held tokens before step p; slot order is
 * unspecified. */
#define KVPOP_CACHE_STATE_WORDS 8
typedef struct {
  void* k;
  void* v;
  int32_t* slot_pos;
  float* slot_prio;
  int32_t* ring;
  int32_t* state;
} kvpop_cache;

/* Bytes of scratch the call needs for problem `pr` (0 for an invalid problem). */
size_t kvpop_workspace_size(int32_t call, const kvpop_problem* pr);

/* Per-token ranks and per-query top-k cutoffs ([Notes] §2.3: rank(t) by the
 * static priority, tau_q = rank of the k-th best token of E(q); [Notes] §2.2:
 * E(q) = {t | s <= t <= q - w}; [Sum-zh] §2.4: a running threshold over static
 * priorities replaces per-row sorting).
 *   prio  [batch, Hkv, S] float (values for t < s are read but never matter)
 *   rank  [batch, Hkv, S] int32 out: a permutation of 0..S-1 per (b, h)
 *   tau   [batch, Hkv, S] int32 out: for |E(q)| >= k >= 1 the k-th smallest
 *         rank over E(q); INT32_MAX when |E(q)| < k; -1 when k == 0.
 * Exact: results are unique integers. */
kvpop_status kvpop_thresholds(const kvpop_problem* pr, const float* prio,
                              int32_t* rank, int32_t* tau,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Causal GQA attention restricted to the sparse mask M above, generated in the
 * kernel from (rank, tau) with no S x S mask stored ([Notes] §2.3, Figure 1;
 * [Sum-zh] §2.2: the sparse operator also returns the log-sum-exp).
 *   q    [batch, Hq, S, D]  qkv_dtype
 *   k, v [batch, Hkv, S, D] qkv_dtype
 *   rank, tau  as produced by kvpop_thresholds for the same (s, w, k)
 *   o    [batch, Hq, S, D]  out_dtype: softmax over the kept keys of each row
 *   lse  [batch, Hq, S] float: ln sum_{kept t} exp(scale <q_q, k_t>)
 * Float results; accumulation in float32.  With k >= S this is dense causal
 * attention, whose lse is the teacher LSE kvpop_future_target takes. */
kvpop_status kvpop_masked_attn_fwd(const kvpop_problem* pr, const void* q,
                                   const void* k, const void* v,
                                   const int32_t* rank, const int32_t* tau,
                                   void* o, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Training-only transposed pass ([Notes] §2.2 future mass m_t, §2.3 Eq. (8)
 * and Figure 2): keys act as queries and queries as keys, the original
 * query's LSE is subtracted and only d >= t + w is summed, so no S x S
 * probability map is formed.
 *   q    [batch, Hq, S, D], k [batch, Hkv, S, D]  qkv_dtype
 *   lse  [batch, Hq, S] float: the dense causal (teacher) LSE of each query
 *   target [batch, Hq, S] float out:
 *          ln sum_{d = t+w}^{S-1} exp(scale <q_d, k_t> - lse_d), -inf when t + w > S - 1
 * This is the first term of Eq. (8) per query head (no -ln N_t, no average
 * over the query group).  w >= 0.  Any finite lse is accepted: the teacher's
 * dense causal LSE (every exponent <= 0, the fast path: the sum runs without
 * a running maximum) or an approximation such as the sparse operator's LSE
 * ([Sum-zh] §2.2, [Notes] §2.3), which can lie below a dropped key's logit;
 * a tile whose max-free sums leave float32's safe range [2^-100, 2^100] is
 * recomputed in the same launch with a running maximum per row, so the
 * result never overflows to +inf and never underflows to -inf for a
 * non-empty range.  A non-finite lse gives unspecified values. */
kvpop_status kvpop_future_target(const kvpop_problem* pr, const void* q,
                                 const void* k, const float* lse, float* target,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* One decode step for every sequence ([Notes] §2.2 newcomer t_new = q - w,
 * §2.4 the token leaving the window is scored then; [Sum-zh] §2.1 budget).
 * At position p of sequence b, for each KV head:
 *   1. token p enters the window;
 *   2. token u = p - w, if u >= s, leaves the window: it is kept when fewer
 *      than k long-range tokens are held, otherwise it replaces the worst held
 *      long-range token (lowest priority, ties: highest position) iff its
 *      priority is strictly larger, else it is dropped; the freed slot takes
 *      token p;
 *   3. the G query heads attend over the min(p+1, Bc) held tokens.
 *   cache      as above (updated in place)
 *   pos        [batch] int32 device: p of each sequence; p == 0 starts a new
 *              sequence (the cache contents are ignored); p < 0 skips the
 *              sequence (cache untouched, o = 0, lse = -inf).  Steps of one
 *              sequence must come in order p = 0, 1, 2, ...
 *   q          [batch, Hq, D]  qkv_dtype
 *   k_new, v_new [batch, Hkv, D] qkv_dtype: K/V of token p
 *   prio_leaving [batch, Hkv] float: priority of token p - w (read iff p - w >= s)
 *   o          [batch, Hq, D] out_dtype;  lse [batch, Hq] float or NULL
 * Cache membership is exact and equals the kept set of forward row p for the
 * same priorities. */
kvpop_status kvpop_decode_step(const kvpop_problem* pr, const kvpop_cache* cache,
                               const int32_t* pos, const void* q,
                               const void* k_new, const void* v_new,
                               const float* prio_leaving, void* o, float* lse,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* kvpop_decode_step without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code being captured into a
 * HIP graph, tight per-token serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels, results and cache update as kvpop_decode_step
 * (bit for bit).  The split-K partials that kvpop_decode_step keeps in `ws`
 * live instead in a fixed array of KVPOP_NOALLOC_SCRATCH_BYTES (8 MiB) in
 * device memory, one per GPU, held from the library's first call on that GPU
 * until the process ends; a problem needing more (kvpop_workspace_size of
 * KVPOP_CALL_DECODE above that size: only 32-head query groups with at
 * most about 32 (sequence, KV head) pairs) returns KVPOP_ERR_SCRATCH and launches nothing.  Nothing in
 * the array has to start at any value (every word a step reads is written
 * earlier in the same step), but every call on one GPU shares it: calls that
 * overlap in time on one GPU (two streams, two threads) race and must be
 * ordered by the caller.  When the problem uses scratch (several splits),
 * `stream` must belong to the current device (KVPOP_ERR_HIP otherwise), and
 * the first such call on a device looks the array's address up once (no
 * allocation). */
kvpop_status kvpop_decode_step_noalloc(const kvpop_problem* pr, const kvpop_cache* cache,
                                       const int32_t* pos, const void* q, const void* k_new,
                                       const void* v_new, const float* prio_leaving, void* o,
                                       float* lse, hipStream_t stream);

/* Prefill -> decode handoff ([Notes] §2.3: inference keeps only the compact
 * cache; after a prompt it holds the kept set of the prompt's last row under
 * the mask above).  For each (sequence, KV head), with p = S - 1 (S =
 * seq_len, the prompt length):
 *   cache  out: slots 0 .. min(S, Bc)-1 hold the sinks (t < s), the
 *          long-range tokens of E(p) with rank(t) <= tau_p, and the window
 *          (p - t < w); a long-range slot's slot_prio is the token's priority
 *          (NaN as -inf, -0 as +0), other slots get 0; ring[t mod w] is the
 *          slot of each window token; slots min(S, Bc) .. Bc-1 get slot_pos
 *          -1.  The K/V rows are copied into their slots.  This is the state
 *          kvpop_decode_step reaches after steps 0 .. p with the same
 *          priorities (up to slot order), so decoding continues at p = S.
 *   k, v   [batch, Hkv, S, D] qkv_dtype: the prompt's keys and values
 *   prio   [batch, Hkv, S] float; rank, tau from kvpop_thresholds for the same
 *          (s, w, k)
 * Requires w >= 1 and D in {64, 128}; uses no workspace. */
kvpop_status kvpop_cache_from_prefill(const kvpop_problem* pr, const kvpop_cache* cache,
                                      const void* k, const void* v, const float* prio,
                                      const int32_t* rank, const int32_t* tau,
                                      hipStream_t stream);

/* Target score of each (KV head, token) ([Notes] §2.2: the future mass
 * m_t = (1/N_t) sum_{d=t+w}^{S-1} A_{d,t} of query group g, aggregated as
 * r_{h,t} = log(eps + (1/G) sum_g m_t^{(h,g)})).  N_t = S - t - w, the number
 * of future queries.
 *   target [batch, Hq, S] float: kvpop_future_target's output,
 *          ln sum_{d >= t+w} A_{d,t} per query head
 *   eps    >= 0, finite
 *   score  [batch, Hkv, S] float out: log(eps + (1/G) sum_g exp(target_g - ln N_t));
 *          where t + w > S - 1 (N_t = 0) the mean is 0 and score = log(eps)
 *          (-inf for eps = 0).  The mean is taken relative to the group's
 *          largest exponent, so targets above ln N_t (a sparse LSE) do not
 *          overflow.
 * Uses no workspace. */
kvpop_status kvpop_target_score(const kvpop_problem* pr, const float* target, float eps,
                                float* score, hipStream_t stream);

/* Teacher boundary labels ([Notes] §2.2: the decayed target score
 * r(q, t) = r_t + floor((q - t)/n) log(gamma_h), the teacher's top-k over
 * E(q) = {t | s <= t <= q - w}, the boundary token t_bnd and the label y of
 * the newcomer t_new = q - w).  For each (sequence, KV head, query q):
 *   the decayed score is computed in float32 as one rounded product and one
 *   rounded sum (NaN counts as -inf, -0 as +0); the teacher keeps the first
 *   min(k, |E(q)|) tokens of E(q) in the order (decayed score descending,
 *   index ascending);
 *   t_bnd  [batch, Hkv, S] int32 out: the last kept token in that order (it may
 *          be t_new itself)
 *   y      [batch, Hkv, S] int32 out: +1 if t_new is kept, -1 if it is not
 *   rows with q - w < s (no newcomer) get t_bnd = -1, y = 0; with k = 0
 *   nothing is kept and rows with a newcomer get t_bnd = -1, y = -1.
 *   score      [batch, Hkv, S] float: the target score r_t (kvpop_target_score)
 *   log_gamma  [Hkv] float (device): log(gamma_h), expected finite (the pages
 *              take gamma_h in (0, 1), i.e. a negative value)
 *   decay_step n >= 1
 * Requires S <= 32768 (KVPOP_ERR_UNSUPPORTED above); head_dim and the dtypes
 * are ignored.  Uses no workspace. */
kvpop_status kvpop_boundary_labels(const kvpop_problem* pr, const float* score,
                                   const float* log_gamma, int32_t decay_step, int32_t* t_bnd,
                                   int32_t* y, hipStream_t stream);

/* Backward of kvpop_masked_attn_fwd: the gradients that training the sparse
 * student needs ([Notes] §2.3: attention over the kept set M[q,t]; §2.1:
 * distillation against the dense teacher).  With P the kept-set
 * probabilities rebuilt from the forward's LSE and dO the gradient of O:
 *   D_i = <dO_i, O_i>,  dS_it = P_it (<dO_i, v_t> - D_i),
 *   dq_i = scale sum_t dS_it k_t,  dk_t = scale sum_i dS_it q_i,
 *   dv_t = sum_i P_it dO_i,
 * dk and dv summed over the query heads that share the KV head; the LSE
 * output is taken as not differentiated.
 *   q, dout [batch, Hq, S, D] bf16; k, v [batch, Hkv, S, D] bf16
 *   o      [batch, Hq, S, D] out_dtype: the forward's output
 *   lse    [batch, Hq, S] float: the forward's LSE
 *   rank, tau  the same arrays the forward took
 *   dq     [batch, Hq, S, D] float out; dk, dv [batch, Hkv, S, D] float out
 *          (every element written)
 * Requires qkv_dtype = KVPOP_BF16 (KVPOP_ERR_UNSUPPORTED otherwise),
 * D in {64, 128}, w >= 1; P and dS are rounded to bf16 as MFMA operands,
 * sums in float32.  Workspace: kvpop_workspace_size(KVPOP_CALL_MASKED_BWD). */
kvpop_status kvpop_masked_attn_bwd(const kvpop_problem* pr, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse,
                                   const int32_t* rank, const int32_t* tau, const void* dout,
                                   float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* A short description of status `st` (a kvpop_status value; any other value
 * gives "unknown status").  The returned string is static. */
const char* kvpop_status_string(int32_t st);
int32_t kvpop_abi_version(void);

/* Testing aid, for callers that check determinism: with on != 0, the
 * masked forward, the future target and the masked backward launch their
 * workgroups in reverse order (the last tile first) until called again with
 * 0.  Each workgroup's result depends only on its own tile, so every output
 * is unchanged bit for bit; only timing and cache locality change.  The
 * setting is process-wide and read when a call launches. */
void kvpop_debug_reverse_launch_order(int32_t on);

#ifdef __cplusplus
}
#endif
#endif /* KVPOP_H */
