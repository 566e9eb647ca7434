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
// its first query q0 (ballots over the rank order), selects the k-th set bit
// with a block prefix count, and then either computes every later query of
// the chunk in parallel from a small candidate set (when k tokens are already
// eligible at q0; see tau_kernel) or, in the early chunks, steps through it:
// each step adds the rank of the newcomer q - w; while fewer than k tokens are
// eligible the cutoff is open (INT32_MAX); when the k-th arrives the cutoff is
// the highest set bit; afterwards a newcomer ranked below the cutoff moves it
// to the next lower set bit (inserting one element below the k-th order
// statistic moves it to its predecessor), found with a wavefront ballot over
// 64 bitmap words at a time.
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;                          // keys per lane
constexpr int kSortTile = kSortThreads * kSortItems;    // keys per workgroup
constexpr int kRadix = 256;

int sort_tiles(int S) { return (S + kSortTile - 1) / kSortTile; }

int tau_chunk(int S) { return S <= 16384 ? 64 : S <= 65536 ? 128 : 256; }

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

// One pass of the stable scatter.  Every workgroup derives its own write
// offsets from the segment's per-tile digit counts (exclusive prefix over
// digits of the totals, plus the counts of the earlier tiles); the last pass
// writes rank[token] = place and order[place] = token instead of keys.
template <bool kFirst, bool kLast>
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const float* __restrict__ prio, const uint32_t* __restrict__ keys_in,
    const int* __restrict__ vals_in, uint32_t* __restrict__ keys_out, int* __restrict__ vals_out,
    int* __restrict__ rank_out, const uint32_t* __restrict__ hist, int S, int ntiles, int shift) {
  static_assert(kSortThreads == kRadix, "one thread per digit");
  __shared__ uint32_t offs[4][kRadix];   // per-wave running write offset of each digit
  __shared__ uint32_t dsum[kRadix];
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
  {
    // this tile's first write position of each digit
    const int dg = threadIdx.x;
    const uint32_t* row = hist + ((size_t)seg * kRadix + dg) * ntiles;
    uint32_t tot = 0, before = 0;
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t c = row[t];
      before += t < tile ? c : 0u;
      tot += c;
    }
    dsum[dg] = tot;
    __syncthreads();
    for (int off = 1; off < kRadix; off <<= 1) {
      const uint32_t add = dg >= off ? dsum[dg - off] : 0u;
      __syncthreads();
      dsum[dg] += add;
      __syncthreads();
    }
    uint32_t run = dsum[dg] - tot + before;
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
      if constexpr (kLast) {
        rank_out[base + val[i]] = (int)pos;
        vals_out[base + pos] = val[i];
      } else {
        keys_out[base + pos] = key[i];
        vals_out[base + pos] = val[i];
      }
    }
    wave_lds_fence();
    if (valid && lane == __builtin_ctzll(peers))
      offs[wave][dig] = start + (uint32_t)__builtin_popcountll(peers);
    wave_lds_fence();
  }
}


// The whole sort of one sequence's priorities in one workgroup when they fit
// in LDS (S <= 16384: 4-byte keys and 2-byte token indices): the same four
// stable 8-bit passes, with the keys kept in registers and exchanged through
// LDS between passes instead of through HBM, so the rank costs one launch.
// 16 waves; wave `wave` owns places [wave * 64 * ipl, +64 * ipl) of the
// current order, item i of a lane at place wbase + 64 i + lane.
constexpr int kLdsSortThreads = 1024;
constexpr int kLdsSortWaves = kLdsSortThreads / 64;
constexpr int kLdsSortItems = 16;
constexpr int kLdsSortMaxS = kLdsSortThreads * kLdsSortItems;

size_t lds_sort_bytes(int S) {
  return (size_t)kLdsSortWaves * kRadix * 4 + 16 + (size_t)S * 4 + align256((size_t)S * 2);
}

__global__ __launch_bounds__(kLdsSortThreads) void lds_rank_kernel(const float* __restrict__ prio,
                                                                   int S, int* __restrict__ rank,
                                                                   int* __restrict__ order) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  uint32_t* offs = reinterpret_cast<uint32_t*>(dyn);          // [waves][256]
  int* wtot = reinterpret_cast<int*>(offs + kLdsSortWaves * kRadix);   // [4]
  uint32_t* skey = reinterpret_cast<uint32_t*>(wtot + 4);     // [S]
  uint16_t* sval = reinterpret_cast<uint16_t*>(skey + S);     // [S]
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const size_t base = (size_t)blockIdx.x * S;
  const int ipl = (S + kLdsSortThreads - 1) / kLdsSortThreads;   // items per lane
  const int wbase = wave * 64 * ipl;
  uint32_t key[kLdsSortItems], pos[kLdsSortItems];
  int val[kLdsSortItems];
#pragma unroll
  for (int i = 0; i < kLdsSortItems; ++i) {
    const int idx = wbase + 64 * i + lane;
    const bool valid = i < ipl && idx < S;
    key[i] = valid ? priority_sort_key(prio[base + idx]) : 0xffffffffu;
    val[i] = idx;
    pos[i] = 0;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    for (int j = tid; j < kLdsSortWaves * kRadix; j += kLdsSortThreads) offs[j] = 0;
    __syncthreads();
    // count each digit per wave; every key keeps its place among the wave's
    // keys of its digit (the running count read before the lowest lane of its
    // digit advances it; LDS operations of a wave execute in order)
#pragma unroll
    for (int i = 0; i < kLdsSortItems; ++i) {
      if (i < ipl) {
        const bool valid = wbase + 64 * i + lane < S;
        const uint32_t dig = (key[i] >> shift) & 255u;
        const uint64_t peers = same_digit_lanes(dig, valid);
        uint32_t run = 0;
        if (valid) {
          run = offs[wave * kRadix + dig];
          pos[i] = run + (uint32_t)lanes_below(peers);
        }
        wave_lds_fence();
        if (valid && lane == __builtin_ctzll(peers))
          offs[wave * kRadix + dig] = run + (uint32_t)__builtin_popcountll(peers);
        wave_lds_fence();
      }
    }
    __syncthreads();
    // first place of each (wave, digit): digits in order, waves in order
    int tot = 0, incl = 0;
    if (tid < kRadix) {
      for (int wv = 0; wv < kLdsSortWaves; ++wv) tot += (int)offs[wv * kRadix + tid];
      incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      if (lane == 63) wtot[wave] = incl;
    }
    __syncthreads();
    if (tid < kRadix) {
      uint32_t run = (uint32_t)(incl - tot);
      for (int wv = 0; wv < wave; ++wv) run += (uint32_t)wtot[wv];
      for (int wv = 0; wv < kLdsSortWaves; ++wv) {
        const uint32_t c = offs[wv * kRadix + tid];
        offs[wv * kRadix + tid] = run;
        run += c;
      }
    }
    __syncthreads();
    // place every key: its (wave, digit) start plus its place among them
#pragma unroll
    for (int i = 0; i < kLdsSortItems; ++i) {
      if (i < ipl && wbase + 64 * i + lane < S)
        pos[i] += offs[wave * kRadix + ((key[i] >> shift) & 255u)];
    }
    if (pass < 3) {
      // every wave finished reading the previous order before the last barrier
#pragma unroll
      for (int i = 0; i < kLdsSortItems; ++i) {
        if (i < ipl && wbase + 64 * i + lane < S) {
          skey[pos[i]] = key[i];
          sval[pos[i]] = (uint16_t)val[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kLdsSortItems; ++i) {
        const int idx = wbase + 64 * i + lane;
        if (i < ipl && idx < S) {
          key[i] = skey[idx];
          val[i] = (int)sval[idx];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLdsSortItems; ++i) {
        if (i < ipl && wbase + 64 * i + lane < S) {
          rank[base + val[i]] = (int)pos[i];
          order[base + pos[i]] = val[i];
        }
      }
    }
  }
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

// Block-wide inclusive prefix sum of v (one value per thread, 256 threads).
__device__ int block_scan_incl(int v, int* sc) {
  const int tid = threadIdx.x;
  sc[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += add;
    __syncthreads();
  }
  const int r = sc[tid];
  __syncthreads();
  return r;
}

// One workgroup per chunk of queries [q0, q0 + nq) of one segment.
//   E(q0) bitmap: bit r set iff the token of rank r (order[r]) lies in
//   [s, q0 - w]; built with wave ballots over the rank order (no atomics).
//   tau0 = k-th smallest set bit (a block prefix of word popcounts).
// If |E(q0)| >= k every later query of the chunk is computed in parallel:
// a newcomer u = q - w matters only if its rank is below tau0 (otherwise the
// k smallest do not change); with J such newcomers in the chunk, T = the
// min(J+1, k) largest of the k smallest ranks of E(q0) and N = the J
// newcomers, tau_q is the (j_q + 1)-th largest of the candidates present at q
// (T always, a newcomer from its arrival on), j_q = newcomers arrived by q.
// (Each such arrival moves the k-th order statistic down by one place among
// the present candidates, and it never falls below T's smallest.)
// Otherwise (early chunks, fewer than k eligible at q0) one wave steps
// through the chunk: while fewer than k tokens are eligible the cutoff is
// open; when the k-th arrives it is the highest set bit; afterwards a
// newcomer ranked below the cutoff moves it to the next lower set bit.
__global__ __launch_bounds__(256) void tau_kernel(const int* __restrict__ rank,
                                                  const int* __restrict__ order,
                                                  int* __restrict__ tau, int S, int s, int w,
                                                  int k, int chunk) {
  extern __shared__ uint32_t smem[];
  __shared__ int sc[256];
  __shared__ int s_tau0, s_J, s_nT;
  const int nwords = (S + 31) >> 5;
  uint32_t* bitmap = smem;
  int* newr = (int*)(smem + nwords);        // rank of the newcomer at each chunk position
  int* taus = newr + chunk;
  int* jpre = taus + chunk;                 // newcomers below tau0 arrived by each position
  int* Tv = jpre + chunk;                   // T ascending (<= chunk + 1 entries)
  int* Nv = Tv + chunk + 1;                 // N ranks (arrival order)
  int* Na = Nv + chunk;                     // N arrival positions
  int* Cv = Na + chunk;                     // candidates, descending rank (<= 2 chunk + 1)
  int* Ca = Cv + 2 * chunk + 1;             // their arrival positions (0 for T)
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int seg = blockIdx.y;
  const int q0 = blockIdx.x * chunk;
  const int nq = min(chunk, S - q0);
  const int* rk = rank + (size_t)seg * S;
  const int* ord = order + (size_t)seg * S;
  int* out = tau + (size_t)seg * S + q0;
  if (k == 0) {
    for (int i = tid; i < nq; i += 256) out[i] = -1;
    return;
  }
  if (tid == 0) s_tau0 = kInt32Max;   // stays open unless the k-th bit is found
  for (int i = tid; i < nq; i += 256) {
    const int t = q0 + i - w;
    const int r = t >= s ? rk[t] : -1;
    newr[i] = (unsigned)r < (unsigned)S ? r : -1;
  }
  const int e_hi = q0 - w;                  // E(q0) = [s, e_hi]
  const int n0 = max(0, e_hi - s + 1);
  constexpr int kU = 8;   // rank-order loads in flight per lane
  for (int base = wave * 64 * kU; base < S; base += 256 * kU) {
    int tv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r = base + 64 * u + lane;
      tv[u] = r < S ? ord[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int r0 = base + 64 * u;
      const uint64_t m = wave_ballot(tv[u] >= s && tv[u] <= e_hi);
      if (lane == 0 && r0 < S) {
        bitmap[r0 >> 5] = (uint32_t)m;
        if ((r0 >> 5) + 1 < nwords) bitmap[(r0 >> 5) + 1] = (uint32_t)(m >> 32);
      }
    }
  }
  __syncthreads();
  // per-thread word range and its popcount prefix (reused for T below)
  const int wpt = (nwords + 255) / 256;
  const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
  int c = 0;
  for (int i = w0; i < w1; ++i) c += __builtin_popcount(bitmap[i]);
  const int excl = block_scan_incl(c, sc) - c;
  if (n0 >= k && excl < k && excl + c >= k) {
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
  __syncthreads();
  const int tau0 = s_tau0;

  if (n0 >= k) {
    // ---- parallel path
    const int ppt = (nq + 255) / 256;           // positions per thread (contiguous)
    const int p0 = min(nq, tid * ppt), p1 = min(nq, p0 + ppt);
    int mine = 0;
    for (int i = p0; i < p1; ++i) mine += (i > 0) & (newr[i] >= 0) & (newr[i] < tau0);
    const int incl = block_scan_incl(mine, sc);
    int run = incl - mine;
    for (int i = p0; i < p1; ++i) {
      const bool mt = (i > 0) & (newr[i] >= 0) & (newr[i] < tau0);
      if (mt) {
        Nv[run] = newr[i];
        Na[run] = i;
      }
      run += mt;
      jpre[i] = run;
    }
    if (tid == 255) {
      s_J = incl;
      s_nT = min(incl + 1, k);
    }
    __syncthreads();
    const int J = s_J, nT = s_nT;
    // T: set bits with global index in [k - nT, k - 1], ascending
    if (excl < k && excl + c > k - nT) {
      int g = excl;
      for (int i = w0; i < w1 && g < k; ++i) {
        uint32_t wd = bitmap[i];
        while (wd && g < k) {
          const int b = __builtin_ctz(wd);
          wd &= wd - 1u;
          if (g >= k - nT) Tv[g - (k - nT)] = (i << 5) + b;
          ++g;
        }
      }
    }
    __syncthreads();
    // candidate positions in descending rank order (ranks are distinct)
    for (int a = tid; a < nT + J; a += 256) {
      int v, arr;
      if (a < nT) {
        v = Tv[a];
        arr = 0;
      } else {
        v = Nv[a - nT];
        arr = Na[a - nT];
      }
      int above = 0;
      for (int b = 0; b < J; ++b) above += Nv[b] > v;
      if (a < nT) {
        above += nT - 1 - a;
      } else {
        for (int b = 0; b < nT; ++b) above += Tv[b] > v;
      }
      Cv[above] = v;
      Ca[above] = arr;
    }
    __syncthreads();
    // each wave steps through the candidates in lockstep (broadcast reads
    // whose addresses do not depend on the data), 8 at a time, until every
    // lane has found its (j + 1)-th present candidate
    const int nC = nT + J;
    for (int ib = wave * 64; ib < nq; ib += 256) {
      const int i = ib + lane;
      const int need = i < nq ? jpre[i] + 1 : 0;
      int cnt = 0, t = tau0;
      bool done = i >= nq;
      for (int a0 = 0; a0 < nC; a0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int a = a0 + u;
          const bool pres = a < nC && Ca[a] <= i;
          cnt += pres;
          if (!done && pres && cnt == need) {
            t = Cv[a];
            done = true;
          }
        }
        if (wave_ballot(!done) == 0) break;
      }
      if (i < nq) taus[i] = t;
    }
  } else if (wave == 0) {
    // ---- sequential path (fewer than k eligible at q0)
    int tc = tau0;
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
  const bool in_lds = S <= kLdsSortMaxS;
  if (in_lds) {
    const size_t lds = lds_sort_bytes(S);
    // more than 64 KiB of dynamic LDS must be allowed explicitly (160 KiB per CU)
    (void)hipFuncSetAttribute((const void*)lds_rank_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(lds_rank_kernel, dim3(nseg), dim3(kLdsSortThreads), lds, st, prio, S, rank,
                       valsA);
    vin = valsA;
  }
  for (int pass = 0; pass < 4 && !in_lds; ++pass) {
    const int shift = 8 * pass;
    uint32_t* kout = (pass & 1) ? keysB : keysA;
    int* vout = (pass & 1) ? valsB : valsA;
    if (pass == 0) {
      hipLaunchKernelGGL(radix_hist_kernel<true>, g, dim3(kSortThreads), 0, st, prio, nullptr, S,
                         ntiles, shift, hist);
      hipLaunchKernelGGL((radix_scatter_kernel<true, false>), g, dim3(kSortThreads), 0, st, prio,
                         nullptr, nullptr, kout, vout, nullptr, hist, S, ntiles, shift);
    } else {
      hipLaunchKernelGGL(radix_hist_kernel<false>, g, dim3(kSortThreads), 0, st, nullptr, kin, S,
                         ntiles, shift, hist);
      if (pass < 3)
        hipLaunchKernelGGL((radix_scatter_kernel<false, false>), g, dim3(kSortThreads), 0, st,
                           nullptr, kin, vin, kout, vout, nullptr, hist, S, ntiles, shift);
      else   // last pass: rank and the rank order (the token at each place)
        hipLaunchKernelGGL((radix_scatter_kernel<false, true>), g, dim3(kSortThreads), 0, st,
                           nullptr, kin, vin, nullptr, vout, rank, hist, S, ntiles, shift);
    }
    kin = kout;
    vin = vout;
  }
  const int chunk = tau_chunk(S);
  const int nchunks = (S + chunk - 1) / chunk;
  // bitmap + newr, taus, jpre, T, N (rank, arrival), candidates (rank, arrival)
  const size_t lds = (size_t)((S + 31) >> 5) * 4 + (size_t)(10 * chunk + 3) * 4;
  hipLaunchKernelGGL(tau_kernel, dim3(nchunks, nseg), dim3(256), lds, st, rank, vin, tau, S,
                     d.s, d.w, d.k, chunk);
  return hipGetLastError();
}

}  // namespace kvpop
