// kvpop_cache_from_prefill: the decode cache as it stands after a prompt.
//
// Inference keeps only the compact cache (KVpop reading notes §2.3); after a
// prompt of S tokens the cache must hold the kept set of the last prompt row
// p = S - 1 under the forward's mask (§2.3: sinks t < s, the protected window
// q - t < w, and the long-range tokens of E(p) = [s, p - w] with
// rank(t) <= tau_p), which is exactly the set decode reaches after steps
// 0 .. p with the same static priorities.  One workgroup per (sequence, KV
// head):
//   1. the long-range survivors of row p are counted, prefix-summed over the
//      four waves and placed with wave ballots, in token order;
//   2. slots 0 .. n-1 (n = min(S, s + w + k)) receive the sinks, the
//      long-range tokens and the window, in that order; a long-range slot
//      keeps the token's priority (NaN as -inf, -0 as +0, as the decode step
//      compares them), ring[t mod w] = slot of each window token, and slots
//      n .. Bc-1 are marked empty (position -1);
//   3. after a barrier the K and V rows are copied into their slots, 16
//      bytes per lane.
// Decode then continues at p = S; while S < Bc the next tokens take slots
// S, S+1, ... as in a decode that started at 0.
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // rank loads in flight per lane

struct HandoffArgs {
  void* ck;
  void* cv;
  int* slot_pos;
  float* slot_prio;
  int* ring;
  const void* k;
  const void* v;
  const float* prio;
  const int* rank;
  const int* tau;
  int Hkv, S, s, w, topk, Bc, row_bytes;
};

__global__ __launch_bounds__(kThreads) void cache_from_prefill_kernel(HandoffArgs a) {
  __shared__ int s_cnt[kThreads / 64];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int S = a.S, s = a.s, w = a.w, Bc = a.Bc;
  const int p = S - 1;
  const int* rk = a.rank + seg * S;
  const float* pr = a.prio + seg * S;
  const int tau_p = a.tau[seg * S + p];
  int* spos = a.slot_pos + seg * Bc;
  float* sprio = a.slot_prio + seg * Bc;
  int* ring = a.ring + seg * w;

  const int n_sink = min(s, S);
  const int e_lo = s, e_hi = p - w;                    // E(p)
  const int n_e = max(0, e_hi - e_lo + 1);
  const int win_lo = max(s, p - w + 1);
  const int n_win = max(0, p - win_lo + 1);

  // ---- 1. long-range survivors: each wave owns a contiguous token range
  const int per_wave = (n_e + 3) / 4;
  const int t_lo = e_lo + wave * per_wave, t_hi = min(e_hi + 1, t_lo + per_wave);
  // branch-free test; the load index is clamped into the range (loops below
  // only run while base < t_hi, so t_hi - 1 is a valid token)
  auto kept = [&](int t) { return (t < t_hi) & (rk[min(t, t_hi - 1)] <= tau_p); };
  int cnt = 0;
  for (int base = t_lo; base < t_hi; base += 64 * kUnroll) {
    bool kp[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) kp[u] = kept(base + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) cnt += __builtin_popcountll(wave_ballot(kp[u]));
  }
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  int slot = n_sink;                                   // long-range slots follow the sinks
  for (int wv = 0; wv < wave; ++wv) slot += s_cnt[wv];
  int n_long = 0;
  for (int wv = 0; wv < kThreads / 64; ++wv) n_long += s_cnt[wv];
  for (int base = t_lo; base < t_hi; base += 64 * kUnroll) {
    bool kp[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) kp[u] = kept(base + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t m = wave_ballot(kp[u]);
      if (kp[u]) {
        const int j = slot + lanes_below(m);
        const int t = base + 64 * u + lane;
        spos[j] = t;
        sprio[j] = canonical_priority(pr[t]);
      }
      slot += __builtin_popcountll(m);
    }
  }

  // ---- 2. sinks, window, ring, empty slots
  const int n = n_sink + n_long + n_win;               // = min(S, Bc)
  for (int j = tid; j < n_sink; j += kThreads) {
    spos[j] = j;
    sprio[j] = 0.0f;
    if (j > p - w) ring[j % w] = j;                    // a sink inside the last w positions
  }
  for (int i = tid; i < n_win; i += kThreads) {
    const int j = n_sink + n_long + i, t = win_lo + i;
    spos[j] = t;
    sprio[j] = 0.0f;
    ring[t % w] = j;
  }
  for (int j = n + tid; j < Bc; j += kThreads) {
    spos[j] = -1;
    sprio[j] = 0.0f;
  }
  __syncthreads();   // slot positions written above are read back below

  // ---- 3. K/V rows into their slots
  const int pieces = a.row_bytes / 16;
  const unsigned char* kg = (const unsigned char*)a.k + seg * (size_t)S * a.row_bytes;
  const unsigned char* vg = (const unsigned char*)a.v + seg * (size_t)S * a.row_bytes;
  unsigned char* kc = (unsigned char*)a.ck + seg * (size_t)Bc * a.row_bytes;
  unsigned char* vc = (unsigned char*)a.cv + seg * (size_t)Bc * a.row_bytes;
  for (long long i = tid; i < (long long)n * pieces; i += kThreads) {
    const int j = (int)(i / pieces), pc = (int)(i % pieces);
    const int t = spos[j];
    const size_t src = (size_t)t * a.row_bytes + (size_t)pc * 16;
    const size_t dst = (size_t)j * a.row_bytes + (size_t)pc * 16;
    *(uint4*)(kc + dst) = *(const uint4*)(kg + src);
    *(uint4*)(vc + dst) = *(const uint4*)(vg + src);
  }
}

}  // namespace

hipError_t launch_cache_from_prefill(const Dims& d, const CacheArgs& c, const void* k,
                                     const void* v, const float* prio, const int* rank,
                                     const int* tau, hipStream_t st) {
  HandoffArgs a;
  a.ck = c.k; a.cv = c.v; a.slot_pos = c.slot_pos; a.slot_prio = c.slot_prio; a.ring = c.ring;
  a.k = k; a.v = v; a.prio = prio; a.rank = rank; a.tau = tau;
  a.Hkv = d.Hkv; a.S = d.S; a.s = d.s; a.w = d.w; a.topk = d.k;
  a.Bc = (int)d.budget();
  a.row_bytes = d.D * (d.f32_in ? 4 : 2);
  hipLaunchKernelGGL(cache_from_prefill_kernel, dim3(d.Hkv, d.b), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvpop
