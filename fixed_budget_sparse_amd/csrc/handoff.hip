// kvpop_cache_from_prefill: the decode cache as it stands after a prompt.
//
// Inference keeps only the compact cache (KVpop reading notes §2.3); after a
// prompt of S tokens the cache must hold the kept set of the last prompt row
// p = S - 1 under the forward's mask (§2.3: sinks t < s, the protected window
// q - t < w, and the long-range tokens of E(p) = [s, p - w] with
// rank(t) <= tau_p), which is exactly the set decode reaches after steps
// 0 .. p with the same static priorities.
//
// Slots 0 .. n-1 (n = min(S, s + w + k)) receive the sinks, the long-range
// tokens in token order and the window, in that order; slots n .. Bc-1 are
// marked empty (position -1).  A long-range slot keeps the token's priority
// (NaN as -inf, -0 as +0, as the decode step compares them) and
// ring[t mod w] = slot of each token of the last w positions.
//
// Grid (Hkv, batch, ceil(Bc / kSlots)): one workgroup per (sequence, KV head,
// block of kSlots slots), so the row copies spread over the whole chip.  Each
// workgroup counts the long-range survivors of its (sequence, head) (per-wave
// counts over contiguous token ranges, prefix-summed over the waves), places
// with wave ballots only those that land in its slot block, writes that
// block's slot metadata and ring entries and keeps the block's token
// positions in LDS; after a barrier it copies its K and V rows, 16 bytes per
// lane.  Decode then continues at p = S; while S < Bc the next tokens take
// slots S, S+1, ... as in a decode that started at 0.  The pair's record of
// the next step's worst long-range token is marked stale (step 0), so the
// first step scans the slots.
#include "kvpop.h"
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;    // rank loads in flight per lane
constexpr int kSlots = 512;   // cache slots per workgroup
constexpr int kCopyUnroll = 4;
constexpr int kStateWords = KVPOP_CACHE_STATE_WORDS;   // first word: the step it is for

struct HandoffArgs {
  void* ck;
  void* cv;
  int* slot_pos;
  float* slot_prio;
  int* ring;
  int* state;
  const void* k;
  const void* v;
  const float* prio;
  const int* rank;
  const int* tau;
  int Hkv, S, s, w, topk, Bc, row_bytes;
};

__global__ __launch_bounds__(kThreads) void cache_from_prefill_kernel(HandoffArgs a) {
  __shared__ int s_cnt[kWaves];
  __shared__ int s_pos[kSlots];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int S = a.S, s = a.s, w = a.w, Bc = a.Bc;
  const int j0 = blockIdx.z * kSlots, j1 = min(j0 + kSlots, Bc);   // this block's slots
  const int p = S - 1;
  const int* rk = a.rank + seg * S;
  const float* pr = a.prio + seg * S;
  const int tau_p = a.tau[seg * S + p];
  int* spos = a.slot_pos + seg * Bc;
  float* sprio = a.slot_prio + seg * Bc;
  int* ring = a.ring + seg * w;
  if (a.state && blockIdx.z == 0 && tid == 0) a.state[seg * kStateWords] = 0;

  const int n_sink = min(s, S);
  const int e_lo = s, e_hi = p - w;                    // E(p)
  const int n_e = max(0, e_hi - e_lo + 1);
  const int win_lo = max(s, p - w + 1);
  const int n_win = max(0, p - win_lo + 1);

  // ---- 1. long-range survivors: each wave owns a contiguous token range
  const int per_wave = (n_e + kWaves - 1) / kWaves;
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
  for (int wv = 0; wv < kWaves; ++wv) n_long += s_cnt[wv];
  // place only where this wave's slots [slot, slot + cnt) meet [j0, j1)
  if (slot < j1 && slot + cnt > j0) {
    for (int base = t_lo; base < t_hi && slot < j1; base += 64 * kUnroll) {
      bool kp[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) kp[u] = kept(base + 64 * u + lane);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint64_t m = wave_ballot(kp[u]);
        const int j = slot + lanes_below(m);
        if (kp[u] && j >= j0 && j < j1) {
          const int t = base + 64 * u + lane;
          s_pos[j - j0] = t;
          spos[j] = t;
          sprio[j] = canonical_priority(pr[t]);
        }
        slot += __builtin_popcountll(m);
      }
    }
  }

  // ---- 2. sinks, window, ring and empty slots of this block
  const int n = n_sink + n_long + n_win;               // = min(S, Bc)
  const int w_lo = n_sink + n_long;                    // first window slot
  for (int j = j0 + tid; j < j1; j += kThreads) {
    int t = -1;
    if (j < n_sink) {
      t = j;
    } else if (j >= w_lo && j < n) {
      t = win_lo + (j - w_lo);
    } else if (j < n) {
      continue;                                        // long-range: placed above
    }
    s_pos[j - j0] = t;
    spos[j] = t;
    sprio[j] = 0.0f;
    if (t >= 0 && t > p - w) ring[t % w] = j;          // a token of the last w positions
  }
  __syncthreads();   // s_pos complete

  // ---- 3. K/V rows of this block's occupied slots
  const int pieces = a.row_bytes / 16;
  const int nj = max(0, min(j1, n) - j0);
  const long long total = (long long)nj * pieces;
  const unsigned char* kg = (const unsigned char*)a.k + seg * (size_t)S * a.row_bytes;
  const unsigned char* vg = (const unsigned char*)a.v + seg * (size_t)S * a.row_bytes;
  unsigned char* kc = (unsigned char*)a.ck + (seg * (size_t)Bc + j0) * a.row_bytes;
  unsigned char* vc = (unsigned char*)a.cv + (seg * (size_t)Bc + j0) * a.row_bytes;
  for (long long base = tid; base < total; base += (long long)kThreads * kCopyUnroll) {
    uint4 kr[kCopyUnroll], vr[kCopyUnroll];
    size_t dst[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const long long i = min(base + (long long)kThreads * u, total - 1);   // clamped: in range
      const int jj = (int)(i / pieces), pc = (int)(i % pieces);
      const size_t src = (size_t)s_pos[jj] * a.row_bytes + (size_t)pc * 16;
      dst[u] = (size_t)jj * a.row_bytes + (size_t)pc * 16;
      kr[u] = *(const uint4*)(kg + src);
      vr[u] = *(const uint4*)(vg + src);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      if (base + (long long)kThreads * u < total) {
        *(uint4*)(kc + dst[u]) = kr[u];
        *(uint4*)(vc + dst[u]) = vr[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_from_prefill(const Dims& d, const CacheArgs& c, const void* k,
                                     const void* v, const float* prio, const int* rank,
                                     const int* tau, hipStream_t st) {
  HandoffArgs a;
  a.ck = c.k; a.cv = c.v; a.slot_pos = c.slot_pos; a.slot_prio = c.slot_prio; a.ring = c.ring;
  a.state = c.state;
  a.k = k; a.v = v; a.prio = prio; a.rank = rank; a.tau = tau;
  a.Hkv = d.Hkv; a.S = d.S; a.s = d.s; a.w = d.w; a.topk = d.k;
  a.Bc = (int)d.budget();
  a.row_bytes = d.D * (d.f32_in ? 4 : 2);
  const unsigned parts = (unsigned)((a.Bc + kSlots - 1) / kSlots);
  hipLaunchKernelGGL(cache_from_prefill_kernel, dim3(d.Hkv, d.b, parts), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvpop
