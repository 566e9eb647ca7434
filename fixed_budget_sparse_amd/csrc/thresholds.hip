// kvpop_thresholds: per-token ranks and per-query top-k cutoffs.
//
// rank(t) is the place of token t in the static priority order and tau_q the
// rank of the k-th best token of E(q) = {t | s <= t <= q - w} (KVpop reading
// notes, §2.2 and §2.3; the running threshold over static priorities of the
// gist.science summary §2.4).  Both are exact integers.
//
// Rank: a stable least-significant-digit radix sort (4 passes of 8 bits) of
// order-preserving 32-bit priority keys with the token index as payload.
// Stability keeps equal priorities in index order, which is the tie rule.
// Within a tile each wave ranks equal digits with ballots (no atomics), so
// the sort is deterministic.
//
// Cutoffs: the sequential Fenwick-tree scan is replaced by independent chunks
// of queries.  A workgroup builds an S-bit LDS bitmap of the ranks of E(q0) for
// its first query q0, selects the k-th set bit with a block prefix count, then
// steps through the chunk: each step adds the rank of the newcomer q - w; while
// fewer than k tokens are eligible the cutoff is open (INT32_MAX); when the
// k-th arrives the cutoff is the highest set bit; afterwards a newcomer ranked
// below the cutoff moves it to the next lower set bit (inserting one element
// below the k-th order statistic moves it to its predecessor), found with a
// wavefront ballot over 64 bitmap words at a time.
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;                          // keys per lane
constexpr int kSortTile = kSortThreads * kSortItems;    // keys per workgroup
constexpr int kRadix = 256;

int sort_tiles(int S) { return (S + kSortTile - 1) / kSortTile; }

int tau_chunk(int S) { return S <= 32768 ? 256 : 512; }

// ---------------------------------------------------------------- sort
template <bool kFirst>
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(
    const float* __restrict__ prio, const uint32_t* __restrict__ keys, int S, int ntiles,
    int shift, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kRadix];
  const int tile = blockIdx.x, seg = blockIdx.y;
  for (int i = threadIdx.x; i < kRadix; i += kSortThreads) h[i] = 0;
  __syncthreads();
  const size_t base = (size_t)seg * S;
  const int t0 = tile * kSortTile;
  for (int i = threadIdx.x; i < kSortTile; i += kSortThreads) {
    const int idx = t0 + i;
    if (idx < S) {
      const uint32_t key = kFirst ? priority_sort_key(prio[base + idx]) : keys[base + idx];
      atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  for (int dg = threadIdx.x; dg < kRadix; dg += kSortThreads)
    hist[((size_t)seg * kRadix + dg) * ntiles + tile] = h[dg];
}

// Exclusive prefix of one segment's histogram in (digit, tile) order.
__global__ __launch_bounds__(kRadix) void radix_scan_kernel(uint32_t* __restrict__ hist,
                                                            int ntiles) {
  __shared__ uint32_t tot[kRadix];
  const int seg = blockIdx.x, dg = threadIdx.x;
  uint32_t* row = hist + ((size_t)seg * kRadix + dg) * ntiles;
  uint32_t sum = 0;
  for (int t = 0; t < ntiles; ++t) sum += row[t];
  tot[dg] = sum;
  __syncthreads();
  for (int off = 1; off < kRadix; off <<= 1) {
    const uint32_t add = dg >= off ? tot[dg - off] : 0u;
    __syncthreads();
    tot[dg] += add;
    __syncthreads();
  }
  uint32_t run = tot[dg] - sum;
  for (int t = 0; t < ntiles; ++t) {
    const uint32_t c = row[t];
    row[t] = run;
    run += c;
  }
}

// Mask of the lanes holding the same 8-bit digit (valid lanes only).
__device__ __forceinline__ uint64_t same_digit_lanes(uint32_t dig, bool valid) {
  uint64_t m = wave_ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool set = (dig >> bit) & 1u;
    const uint64_t bb = wave_ballot(set);
    m &= set ? bb : ~bb;
  }
  return m;
}

template <bool kFirst>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const float* __restrict__ prio, const uint32_t* __restrict__ keys_in,
    const int* __restrict__ vals_in, uint32_t* __restrict__ keys_out, int* __restrict__ vals_out,
    const uint32_t* __restrict__ hist, int S, int ntiles, int shift) {
  __shared__ uint32_t offs[4][kRadix];   // per-wave running write offset of each digit
  const int tile = blockIdx.x, seg = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kRadix; i += kSortThreads) (&offs[0][0])[i] = 0;
  __syncthreads();
  const size_t base = (size_t)seg * S;
  // wave `wave` owns keys [wbase, wbase + 1024) of the tile, in index order
  const int wbase = tile * kSortTile + wave * (kSortTile / 4);
  uint32_t key[kSortItems];
  int val[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = wbase + i * 64 + lane;
    if (idx < S) {
      key[i] = kFirst ? priority_sort_key(prio[base + idx]) : keys_in[base + idx];
      val[i] = kFirst ? idx : vals_in[base + idx];
    } else {
      key[i] = 0xffffffffu;
      val[i] = -1;
    }
  }
  // pass 1: count each digit per wave
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const bool valid = wbase + i * 64 + lane < S;
    const uint32_t dig = (key[i] >> shift) & 255u;
    const uint64_t peers = same_digit_lanes(dig, valid);
    if (valid && lane == __builtin_ctzll(peers)) offs[wave][dig] += (uint32_t)__builtin_popcountll(peers);
  }
  __syncthreads();
  for (int dg = threadIdx.x; dg < kRadix; dg += kSortThreads) {
    uint32_t run = hist[((size_t)seg * kRadix + dg) * ntiles + tile];
    for (int wv = 0; wv < 4; ++wv) {
      const uint32_t c = offs[wv][dg];
      offs[wv][dg] = run;
      run += c;
    }
  }
  __syncthreads();
  // pass 2: place every key; lanes of one digit read the running offset, then
  // the lowest of them advances it (LDS operations of a wave execute in order)
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const bool valid = wbase + i * 64 + lane < S;
    const uint32_t dig = (key[i] >> shift) & 255u;
    const uint64_t peers = same_digit_lanes(dig, valid);
    uint32_t start = 0;
    if (valid) {
      start = offs[wave][dig];
      const uint32_t pos = start + (uint32_t)lanes_below(peers);
      keys_out[base + pos] = key[i];
      vals_out[base + pos] = val[i];
    }
    wave_lds_fence();
    if (valid && lane == __builtin_ctzll(peers))
      offs[wave][dig] = start + (uint32_t)__builtin_popcountll(peers);
    wave_lds_fence();
  }
}

__global__ __launch_bounds__(256) void rank_from_order_kernel(const int* __restrict__ order,
                                                              int* __restrict__ rank, int S,
                                                              long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long seg = i / S;
  const int place = (int)(i - seg * S);
  const int t = order[i];
  if ((unsigned)t < (unsigned)S) rank[seg * S + t] = place;
}

// ---------------------------------------------------------------- cutoffs
// Highest set bit of the bitmap with index < x (-1 if none).  Called by all 64
// lanes of one wave with the same x.
__device__ int highest_bit_below(const uint32_t* bm, int x, int lane) {
  const int wi = x >> 5, b = x & 31;
  if (b) {
    const uint32_t wd = bm[wi] & ((1u << b) - 1u);
    if (wd) return (wi << 5) + 31 - __builtin_clz(wd);
  }
  for (int hi = wi - 1; hi >= 0; hi -= 64) {
    const int j = hi - lane;                 // lane 0 looks at the highest word
    const uint32_t v = j >= 0 ? bm[j] : 0u;
    const uint64_t m = wave_ballot(v != 0u);
    if (m) {
      const int L = __builtin_ctzll(m);
      const uint32_t vv = (uint32_t)__shfl((int)v, L);
      return ((hi - L) << 5) + 31 - __builtin_clz(vv);
    }
  }
  return -1;
}

__global__ __launch_bounds__(256) void tau_kernel(const int* __restrict__ rank,
                                                  int* __restrict__ tau, int S, int s, int w,
                                                  int k, int chunk) {
  extern __shared__ uint32_t smem[];
  __shared__ int cnt[256];
  __shared__ int s_tau0;
  const int nwords = (S + 31) >> 5;
  uint32_t* bitmap = smem;
  int* newr = (int*)(smem + nwords);        // rank of the newcomer of each chunk row
  int* taus = newr + chunk;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int seg = blockIdx.y;
  const int q0 = blockIdx.x * chunk;
  const int nq = min(chunk, S - q0);
  const int* rk = rank + (size_t)seg * S;
  int* out = tau + (size_t)seg * S + q0;
  if (k == 0) {
    for (int i = tid; i < nq; i += 256) out[i] = -1;
    return;
  }
  if (tid == 0) s_tau0 = kInt32Max;   // stays open unless the k-th bit is found
  for (int i = tid; i < nwords; i += 256) bitmap[i] = 0u;
  for (int i = tid; i < nq; i += 256) {
    const int t = q0 + i - w;
    const int r = t >= s ? rk[t] : -1;
    newr[i] = (unsigned)r < (unsigned)S ? r : -1;
  }
  __syncthreads();
  const int e_hi = q0 - w;                  // E(q0) = [s, e_hi]
  const int n0 = max(0, e_hi - s + 1);
  for (int t = s + tid; t <= e_hi; t += 256) {
    const int r = rk[t];
    if ((unsigned)r < (unsigned)S) atomicOr(&bitmap[r >> 5], 1u << (r & 31));
  }
  __syncthreads();
  if (n0 >= k) {
    // k-th smallest set bit: per-thread word range, block prefix of counts
    const int wpt = (nwords + 255) / 256;
    const int w0 = tid * wpt, w1 = min(nwords, w0 + wpt);
    int c = 0;
    for (int i = w0; i < w1; ++i) c += __builtin_popcount(bitmap[i]);
    cnt[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = tid >= off ? cnt[tid - off] : 0;
      __syncthreads();
      cnt[tid] += add;
      __syncthreads();
    }
    const int excl = cnt[tid] - c;
    if (excl < k && excl + c >= k) {
      int need = k - excl;
      for (int i = w0; i < w1; ++i) {
        uint32_t wd = bitmap[i];
        const int pc = __builtin_popcount(wd);
        if (need <= pc) {
          for (int j = 1; j < need; ++j) wd &= wd - 1u;
          s_tau0 = (i << 5) + __builtin_ctz(wd);
          break;
        }
        need -= pc;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    int tc = s_tau0;
    int n = n0;
    if (lane == 0) taus[0] = n < k ? kInt32Max : tc;
    for (int i = 1; i < nq; ++i) {
      const int r = newr[i];
      if (r >= 0) {
        if (lane == 0) bitmap[r >> 5] |= 1u << (r & 31);
        wave_lds_fence();
        ++n;
        if (n == k)
          tc = highest_bit_below(bitmap, S, lane);
        else if (n > k && r < tc)
          tc = highest_bit_below(bitmap, tc, lane);
      }
      if (lane == 0) taus[i] = n < k ? kInt32Max : tc;
    }
  }
  __syncthreads();
  for (int i = tid; i < nq; i += 256) out[i] = taus[i];
}

}  // namespace

size_t thresholds_ws_bytes(const Dims& d) {
  const size_t n = (size_t)d.nseg() * d.S;
  size_t bytes = 4 * align256(n * 4);                                     // keys/vals x2
  bytes += align256((size_t)d.nseg() * kRadix * sort_tiles(d.S) * 4);     // histograms
  return bytes;
}

hipError_t launch_thresholds(const Dims& d, const float* prio, int* rank, int* tau, void* ws,
                             hipStream_t st) {
  const int S = d.S, nseg = d.nseg(), ntiles = sort_tiles(S);
  const size_t n = (size_t)nseg * S;
  char* p = (char*)ws;
  uint32_t* keysA = (uint32_t*)p; p += align256(n * 4);
  uint32_t* keysB = (uint32_t*)p; p += align256(n * 4);
  int* valsA = (int*)p; p += align256(n * 4);
  int* valsB = (int*)p; p += align256(n * 4);
  uint32_t* hist = (uint32_t*)p;

  const dim3 g(ntiles, nseg);
  uint32_t* kin = nullptr;
  int* vin = nullptr;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    uint32_t* kout = (pass & 1) ? keysB : keysA;
    int* vout = (pass & 1) ? valsB : valsA;
    if (pass == 0) {
      hipLaunchKernelGGL(radix_hist_kernel<true>, g, dim3(kSortThreads), 0, st, prio, nullptr, S,
                         ntiles, shift, hist);
    } else {
      hipLaunchKernelGGL(radix_hist_kernel<false>, g, dim3(kSortThreads), 0, st, nullptr, kin, S,
                         ntiles, shift, hist);
    }
    hipLaunchKernelGGL(radix_scan_kernel, dim3(nseg), dim3(kRadix), 0, st, hist, ntiles);
    if (pass == 0) {
      hipLaunchKernelGGL(radix_scatter_kernel<true>, g, dim3(kSortThreads), 0, st, prio, nullptr,
                         nullptr, kout, vout, hist, S, ntiles, shift);
    } else {
      hipLaunchKernelGGL(radix_scatter_kernel<false>, g, dim3(kSortThreads), 0, st, nullptr, kin,
                         vin, kout, vout, hist, S, ntiles, shift);
    }
    kin = kout;
    vin = vout;
  }
  const long long total = (long long)n;
  hipLaunchKernelGGL(rank_from_order_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, vin, rank, S, total);
  const int chunk = tau_chunk(S);
  const int nchunks = (S + chunk - 1) / chunk;
  const size_t lds = (size_t)((S + 31) >> 5) * 4 + (size_t)chunk * 8;
  hipLaunchKernelGGL(tau_kernel, dim3(nchunks, nseg), dim3(256), lds, st, rank, tau, S, d.s, d.w,
                     d.k, chunk);
  return hipGetLastError();
}

}  // namespace kvpop
