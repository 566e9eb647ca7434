// kvpop_masked_attn_fwd: causal GQA attention under the fixed-budget sparse
// mask (KVpop reading notes §2.3: M[q,t] = 1[t<s] or 1[q-t<w] or
// (1[t in E(q)] and 1[rank(t) <= tau_q]); Figure 1: softmax over the retained
// set; gist.science summary §2.2: the operator returns the log-sum-exp).
//
// Design (gfx950):
//  * A workgroup owns one query tile of one KV head: m = 256 / G query rows of
//    each of the G query heads that share the KV head, stacked into 256 MFMA
//    rows (8 waves x 32).  The G heads share priorities, hence the mask and
//    the key list, so one gathered key set feeds all of them.
//  * The tile's candidate keys are the sinks, the long-range keys of its first
//    row q0 ({t in E(q0) : rank(t) <= tau_q0}, exactly k keys, listed in rank
//    order by a small pre-pass) and the contiguous band [q0-w+1, q_hi].  Since
//    tau is non-increasing in q once k tokens are eligible and an evicted
//    token never returns, this covers every kept key of every row.  Kept keys
//    are scattered over the whole prefix, so instead of skipping key blocks
//    the kernel gathers the candidates into dense 64-key chunks in LDS.
//  * Per chunk: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (each lane then owns
//    one query row), the A8 mask only on chunks that are not kept by every
//    row, as the interval test t <= q <= q_end(t) (q_end from a small
//    pre-pass: tau never increases with q, so the rows that keep a token are
//    one interval), online softmax in the exp2
//    domain, and O^T = V^T P^T, so P feeds the second MFMA straight from
//    registers and O stays row-per-lane.  V is gathered like K (16 lanes per
//    256-byte row, coalesced) and kept row-major in LDS with its 16-byte
//    pieces XOR-swizzled by row; the V^T operand is read with gfx950's
//    transposing LDS load (ds_read_b64_tr_b16), which hands each lane four
//    consecutive keys of one dim, so no lane shuffles or pairs rows itself.
//  * float32 inputs use v_mfma_f32_32x32x2_f32 with the same lane layouts.
#include <type_traits>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 512;       // 8 waves
constexpr int kRowsPerTile = 256;   // stacked query rows per workgroup (8 waves x 32)
constexpr int kChunk = 64;          // keys per chunk
constexpr int kDesc = 8;            // key-descriptor slots (bf16: chunks c .. c+4 live)

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* rank;
  const int* tau;
  const int2* list;    // [nseg, ntiles, cap] (token, q_end) of listed long-range keys
  const int* count;    // [nseg, ntiles]
  const int* qend;     // [nseg, S] last row that keeps each token
  void* o;
  float* lse;
  int S, Hq, Hkv, G, m, ntiles, s, w, cap;
  int reverse;         // launch order reversed (testing aid)
  float scale_log2;    // softmax scale * log2(e)
};

// Per token t of each (sequence, KV head): order[rank[t]] = t, and q_end(t),
// the last row that keeps t.  tau never increases with q, so the rows that
// keep t are the interval [t, q_end(t)]: S - 1 for a sink or a token whose
// window reaches the end, t + w - 1 when the token is not kept once it
// leaves the window, else the last q >= t + w with tau_q >= rank(t), found
// by bisection.  Row q then keeps t iff t <= q <= q_end(t).
__global__ __launch_bounds__(256) void key_end_kernel(const int* __restrict__ rank,
                                                      const int* __restrict__ tau,
                                                      int* __restrict__ order,
                                                      int* __restrict__ qend, int S, int s, int w,
                                                      long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long seg = i / S;
  const int t = (int)(i - seg * S);
  const int* tq = tau + seg * S;
  const int r = rank[i];
  if ((unsigned)r < (unsigned)S) order[seg * S + r] = t;
  int e;
  if (t < s || t + w > S - 1) {
    e = S - 1;
  } else {
    int lo = t + w, hi = S - 1;
    if (tq[lo] < r) {
      e = t + w - 1;
    } else {
      while (lo < hi) {                 // invariant: tq[lo] >= r
        const int mid = lo + (hi - lo + 1) / 2;
        if (tq[mid] >= r) lo = mid;
        else hi = mid - 1;
      }
      e = lo;
    }
  }
  qend[i] = e;
}

// Lists, in rank order, the long-range keys of each tile's first row q0 when
// its cutoff is finite: tokens t in [s, q0 - w] with rank(t) <= tau_q0.  The
// places 0 .. tau_q0 of the rank order (up to the whole sequence for the
// first tiles, where few tokens are eligible) are split into one contiguous
// run per wave: a counting pass (eight loads in flight per lane, a ballot per
// 64 places), one barrier for the prefix over the waves, then a placing pass
// over the same run.  Entries are (token, q_end(token)).
constexpr int kListThreads = 512;
__global__ __launch_bounds__(kListThreads) void tile_list_kernel(
    const int* __restrict__ order, const int* __restrict__ tau, const int* __restrict__ qend,
    int S, int s, int w, int m, int ntiles, int cap, int2* __restrict__ list,
    int* __restrict__ count) {
  constexpr int kU = 8;
  constexpr int kWaves = kListThreads / 64;
  __shared__ int wsum[kWaves];
  const int tile = blockIdx.x, seg = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int q0 = tile * m;
  const int e_hi = q0 - w;
  const int tq0 = tau[(size_t)seg * S + q0];
  int* cnt_out = count + (size_t)seg * ntiles + tile;
  if (e_hi < s || tq0 < 0 || tq0 == kInt32Max || cap == 0) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  const int n_places = min(tq0, S - 1) + 1;
  const int* ord = order + (size_t)seg * S;
  const int* qe = qend + (size_t)seg * S;
  int2* out = list + ((size_t)seg * ntiles + tile) * cap;
  // this wave's run of places, a multiple of 64 long
  const int per = ((n_places + kWaves * 64 - 1) / (kWaves * 64)) * 64;
  const int r0 = wave * per, r1 = min(r0 + per, n_places);
  auto eligible = [&](int t) { return t >= s && t <= e_hi; };
  int wcount = 0;
  for (int b0 = r0; b0 < r1; b0 += 64 * kU) {
    int t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = b0 + 64 * u + lane;
      t[u] = i < r1 ? ord[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) wcount += __builtin_popcountll(wave_ballot(eligible(t[u])));
  }
  if (lane == 0) wsum[wave] = wcount;
  __syncthreads();
  int pos = 0, total = 0;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    const int c = wsum[j];
    pos += j < wave ? c : 0;
    total += c;
  }
  for (int b0 = r0; b0 < r1; b0 += 64 * kU) {
    int t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = b0 + 64 * u + lane;
      t[u] = i < r1 ? ord[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool keep = eligible(t[u]);
      const uint64_t bal = wave_ballot(keep);
      const int at = pos + lanes_below(bal);
      if (keep && at < cap) out[at] = make_int2(t[u], qe[t[u]]);
      pos += __builtin_popcountll(bal);
    }
  }
  if (tid == 0) *cnt_out = min(total, cap);
}

// LDS geometry
template <int D, bool kF32>
struct FwdLds {
  // bf16: K and V row-major [64][D], 16-byte pieces XOR-swizzled by row
  // f32:  K row-major [64][D+1]; V row-major [64][D+4]
  static constexpr int KS = kF32 ? D + 1 : D;
  static constexpr int VS = kF32 ? D + 4 : D;
  static constexpr int kBytes = kF32 ? kChunk * KS * 4 : kChunk * KS * 2;
  static constexpr int vBytes = kF32 ? kChunk * VS * 4 : kChunk * VS * 2;
};

typedef short short4v __attribute__((ext_vector_type(4)));

// One key of a chunk as fetched by the descriptor reads: its token (-2: token
// and q_end come from the tile's list entry l), and q_end(t) otherwise.
struct KeyDesc {
  int t, r;
  int2 l;
};

// Byte offset of 16-byte piece `piece` of key row `key` in a bf16 K chunk.
// The QK operand read has the 16 lanes served together read one piece of 16
// consecutive rows; XORing the piece index with key mod 16 (D = 128) or
// (key / 2) mod 8 (D = 64, where two rows share a 64-bank line) spreads them
// over all 64 banks.
template <int D>
__device__ __forceinline__ int k_piece_offset(int key, int piece) {
  const int sw = D == 128 ? (key & 15) : ((key >> 1) & 7);
  return key * (D * 2) + ((piece ^ sw) << 4);
}

// Byte offset of 16-byte piece `piece` of key row `key` in a bf16 V chunk.
// The piece index is XORed with a function of the row that stays inside the
// row (D = 128: 16 pieces, XOR 4 (key mod 4); D = 64: 8 pieces, XOR
// 4 ((key / 2) mod 2)), so that the transposed reads below, where a half wave
// reads 32- or 64-byte runs of four consecutive rows, touch 64 distinct banks.
template <int D>
__device__ __forceinline__ int v_piece_offset(int key, int piece) {
  const int sw = D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
  return key * (D * 2) + ((piece ^ sw) << 4);
}

// Per-lane byte offsets, one per 32-dim output block db, of the transposed
// V^T operand reads.  ds_read_b64_tr_b16 gives lane i of a 16-lane group
// element (i mod 4) of the 64-bit words read by lanes 4e + i/4 (e = 0..3) of
// the group (checked on the device).  Lane j of the group reading row
// key0 + j/4, dims d0 + 4(j mod 4) .. +3 therefore receives
// V[key0 + e][d0 + i] for e = 0..3: four consecutive keys of one dim.  For
// lane (li, hh) of the wave: key0 = 16 ks + 8 a + 4 hh, d0 = 32 db + 16 (li/16),
// so the pair of reads (a = 0, 1) is the MFMA operand element 4a + r =
// V[16 ks + 8 a + 4 hh + r][32 db + li], the key order of the P operand.
template <int D>
__device__ __forceinline__ void v_tr_offsets(int lane, int (&off)[D / 32]) {
  const int hh = lane >> 5, li = lane & 31;
  const int half = li >> 4, j = li & 15, jq = j >> 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int dim = 32 * db + 16 * half + 4 * (j & 3);
    off[db] = v_piece_offset<D>(4 * hh + jq, dim >> 3) + (dim & 7) * 2;
  }
}

// V^T operand (output block db, k-step ks) from a bf16 V chunk at `vb`.
template <int D>
__device__ __forceinline__ bf16x8 v_tr_operand(const unsigned char* vb, const int (&off)[D / 32],
                                               int db, int ks) {
  typedef __attribute__((address_space(3))) short4v lds_s4;
  const unsigned char* p = vb + off[db] + 16 * ks * (D * 2);
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + 8 * (D * 2)));
  typedef short short8v __attribute__((ext_vector_type(8)));
  const short8v v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int D, bool kF32In, bool kF32Out>
__global__ __launch_bounds__(kThreads, 1) void masked_fwd_kernel(FwdArgs a) {
  using L = FwdLds<D, kF32In>;
  // K and V buffers as separate arrays (bf16: three of each, float32: two):
  // the bf16 pipeline names each by a compile-time index, so the compiler can
  // tell that the direct loads into one buffer never alias the reads of
  // another and need not wait for them before every LDS read.  The compiler
  // lays arrays of one size out in name order, so the V buffers come first:
  // the three V buffers and K buffer 0 then lie where the 16-bit immediate
  // offset of an LDS read reaches them from one set of per-lane offsets; K
  // buffers 1 and 2 (D = 128: above 64 KB) are read through a second base
  // 64 KB higher.  (Any other layout stays correct, with a few more adds.)
  constexpr int kThirdK = kF32In ? 16 : L::kBytes;
  constexpr int kThirdV = kF32In ? 16 : L::vBytes;
  __shared__ __attribute__((aligned(16))) unsigned char ldsa_v0[L::vBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ldsa_v1[L::vBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ldsa_v2[kThirdV];
  __shared__ __attribute__((aligned(16))) unsigned char ldsb_k0[L::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ldsb_k1[L::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ldsb_k2[kThirdK];
  // buffer i: a run-time int (float32 path, 0 or 1) or a std::integral_constant
  auto kbuf = [&](auto i) -> unsigned char* {
    if constexpr (std::is_integral<decltype(i)>::value) return i ? ldsb_k1 : ldsb_k0;
    else if constexpr (decltype(i)::value == 0) return ldsb_k0;
    else if constexpr (decltype(i)::value == 1) return ldsb_k1;
    else return ldsb_k2;
  };
  auto vbuf = [&](auto i) -> unsigned char* {
    if constexpr (std::is_integral<decltype(i)>::value) return i ? ldsa_v1 : ldsa_v0;
    else if constexpr (decltype(i)::value == 0) return ldsa_v0;
    else if constexpr (decltype(i)::value == 1) return ldsa_v1;
    else return ldsa_v2;
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  __shared__ __attribute__((aligned(16))) int kd_t[kDesc][kChunk];
  __shared__ __attribute__((aligned(16))) int kd_r[kDesc][kChunk];
  __shared__ int s_flag[kDesc];
  __shared__ int s_redo;   // some row needs the exact (running-maximum) mode

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int hh = lane >> 5, li = lane & 31;
  if (tid == 0) s_redo = 0;   // read only after the barriers that follow
  const int Lb = xcd_logical_block(launch_block(a.reverse), (int)gridDim.x);
  const int tile = Lb % a.ntiles;
  const int h = (Lb / a.ntiles) % a.Hkv;
  const int b = Lb / (a.ntiles * a.Hkv);
  const int S = a.S, s = a.s, w = a.w, m = a.m, G = a.G;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int* qend = a.qend + seg * S;
  const int* tau = a.tau + seg * S;
  const int q0 = tile * m;
  const int q_hi = min(q0 + m - 1, S - 1);

  // this lane's query row
  const int rr = wave * 32 + li;
  const int g = rr / m;
  const int q = q0 + (rr - g * m);
  const bool row_ok = g < G && q < S;
  const int hq = h * G + (g < G ? g : 0);


  // key segments of the tile: sinks | long-range | band
  const int n_sink = min(s, q_hi + 1);
  const int e_hi = q0 - w;
  const int tq0 = tau[q0];
  int n_long = 0;
  bool listed = false;
  if (e_hi >= s && tq0 >= 0) {
    if (tq0 == kInt32Max) {
      n_long = e_hi - s + 1;
    } else {
      listed = true;
      n_long = a.count[seg * a.ntiles + tile];
    }
  }
  const int band_lo = max(s, q0 - w + 1);
  const int n_band = max(0, q_hi - band_lo + 1);
  const int nk = n_sink + n_long + n_band;
  const int2* lst = a.list + (seg * a.ntiles + tile) * (size_t)a.cap;

  // query operand (B of S^T = K Q^T): lane holds row li, dims [16ks + 8hh, +8)
  constexpr int NKS = kF32In ? D / 2 : D / 16;
  typedef typename std::conditional<kF32In, float, bf16x8>::type QOp;
  QOp qop[NKS];
  {
    const size_t qrow = (((size_t)b * a.Hq + hq) * S + (row_ok ? q : 0)) * D;
    if constexpr (kF32In) {
      const float* qp = (const float*)a.q + qrow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qop[ks] = row_ok ? qp[2 * ks + hh] : 0.0f;
    } else {
      const uint16_t* qp = (const uint16_t*)a.q + qrow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row_ok) u = *(const uint4*)(qp + 16 * ks + 8 * hh);
        qop[ks] = as_bf16x8(u);
      }
    }
  }

  // the query loads stay in flight while the prologue fetches descriptors
  // and the first chunks; complete_q marks them complete before the chunk
  // loop (loads still in flight at the loop entry made the compiler wait for
  // every newer load, the whole next-chunk gather, before the first MFMA of
  // each chunk)
  auto complete_q = [&] {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qop[ks]));
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  const size_t kvbase = seg * (size_t)S * D;

  // ---- key descriptors of the chunk starting at c0, built by wave 0 in two
  // halves: desc_load issues the (branch-free, clamped) global reads into
  // registers, desc_store, one compute phase later, publishes the token and
  // its span q_end(t) - t to LDS with the chunk's mask class: 0 when every
  // key is kept by every row of the tile (t <= q0 and q_end(t) >= q_hi), so no
  // mask runs, else 2: row q keeps key t iff t <= q <= q_end(t), the A8 mask
  // as one unsigned compare (tau never increases with q, so the rows that
  // keep a key are one interval); padding keys (token -1, span 0) fail it.
  auto desc_fetch = [&](int c0, KeyDesc& d) {
    if (wave == 0) {
      const int j = c0 + lane;
      const bool in_sink = j < n_sink;
      const bool in_long = !in_sink && j < n_sink + n_long;
      const bool in_band = !in_sink && !in_long && j < nk;
      const int t = in_sink ? j
                    : in_long ? s + (j - n_sink)
                    : in_band ? band_lo + (j - n_sink - n_long) : -1;
      if (listed) d.l = lst[min(max(j - n_sink, 0), max(n_long - 1, 0))];
      d.r = qend[min(max(t, 0), S - 1)];
      d.t = (in_long && listed) ? -2 : t;    // -2: token and q_end from the list
    }
  };
  auto desc_put = [&](int db, const KeyDesc& d) {
    if (wave == 0) {
      int t = d.t == -2 ? d.l.x : d.t;
      const int e = d.t == -2 ? d.l.y : d.r;
      if (t >= S) t = -1;
      kd_t[db][lane] = t;
      kd_r[db][lane] = t >= 0 ? e - t : 0;
      const bool always = (t >= 0) & (t <= q0) & (e >= q_hi);
      const uint64_t not_always = wave_ballot(!always);
      if (lane == 0) s_flag[db] = not_always == 0 ? 0 : 2;
    }
  };
  KeyDesc pd{-1, 0, make_int2(-1, 0)};   // the chunk in flight in the loop
  auto desc_load = [&](int c0) { desc_fetch(c0, pd); };
  auto desc_store = [&](int db) { desc_put(db, pd); };

  // ---- gathers of K and V rows.  bf16: direct loads from global memory into
  // LDS (global_load_lds_dwordx4), no registers and no LDS store
  // instructions: K of chunk c+3 and V of chunk c+1 are issued at the start
  // of iteration c into the buffers the previous iteration finished reading,
  // and awaited before the closing barrier of iteration c+1, so each load has
  // two iterations to arrive (waiting on the loads of the same iteration made
  // every chunk pay a full cache round trip).  Each instruction
  // fills 1 KB of LDS (lane L writes bytes 16L .. 16L+15 of its block, checked
  // on the device), i.e. 1024 / (2 D) rows; lane L fetches the global piece
  // that the row's swizzle places at its slot.  float32: registers -> LDS,
  // K two chunks ahead, V one chunk ahead.
  constexpr int PPR = kF32In ? D / 4 : D / 8;            // 16-byte pieces per row
  constexpr int KP = kChunk * PPR / kThreads;            // f32 pieces per thread
  static_assert(kChunk * PPR % kThreads == 0, "pieces per thread");
  constexpr int RPI = 512 / D;                           // rows per 1 KB direct load
  constexpr int NDMA = kChunk / RPI / (kThreads / 64);   // direct loads per wave per chunk
  static_assert(kF32In || NDMA * RPI * (kThreads / 64) == kChunk, "direct-load tiling");
  // native 4-wide vectors: HIP's uint4 arrays captured by the lambdas below
  // were placed in scratch memory
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v kst[kF32In ? KP : 1];
  u32x4v vst4[kF32In ? KP : 1];
  // per-lane offsets of the transposed V^T operand reads and of the swizzled
  // K operand reads (bf16: row li, piece 2 ks + hh)
  int vtr_off[D / 32];
  // K: the offset of piece 2 ks + hh of row li is k_piece_offset(li, hh) XOR
  // 32 ks (the swizzle XORs the piece index, and 2 ks only sets piece bits
  // that the row offset does not use), so one per-lane base serves every
  // k-step; k_hi is the same base plus 64 KB for the buffers above 64 KB
  int k_lo = 0, k_hi = 0;
  if constexpr (!kF32In) {
    v_tr_offsets<D>(lane, vtr_off);
    k_lo = k_piece_offset<D>(li, hh);
    k_hi = k_lo + 65536;
  }
  // K operand of k-step ks, 32-key block blk, from K buffer kb; `base` is
  // k_lo or k_hi as rebound by k_base (opaque to the compiler, so that the
  // eight XORs stay in the loop instead of occupying eight registers)
  constexpr bool kHiK = !kF32In && 3 * L::vBytes + 2 * L::kBytes > 65536;
  auto k_base = [&](auto kb) {
    int x = (kHiK && decltype(kb)::value >= 1) ? k_hi : k_lo;
    asm volatile("" : "+v"(x));
    return x;
  };
  auto k_operand = [&](auto kb, int base, int ks, int blk) {
    constexpr int bias = (kHiK && decltype(kb)::value >= 1) ? 65536 : 0;
    const unsigned char* p = kbuf(kb) + blk * 32 * (D * 2) + ((base ^ (32 * ks)) - bias);
    return as_bf16x8(*(const uint4*)p);
  };
  // Padding slots (token -1) load row 0 instead: every such key is masked
  // (its probability is exactly 0), so only finiteness matters, and the loads
  // stay unconditional (no exec-masked branches, all addresses issued at once).
  typedef __attribute__((address_space(3))) void lds_void;
  auto dma_rows = [&](const void* src, unsigned char* dst, int db, bool is_k) {
    const unsigned char* g = (const unsigned char*)src + kvbase * 2;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r0 = (wave * NDMA + i) * RPI;      // first row of this 1 KB block
      const int row = r0 + lane / PPR, slot = lane % PPR;
      const int t = min(max(kd_t[db][row], 0), S - 1);   // padding (-1) reads row 0
      const int sw = is_k ? k_piece_offset<D>(row, slot) : v_piece_offset<D>(row, slot);
      const int piece = (sw >> 4) & (PPR - 1);     // the logical piece stored at this slot
      __builtin_amdgcn_global_load_lds((const void*)(g + ((size_t)t * PPR + piece) * 16),
                                       (lds_void*)(dst + r0 * (D * 2)), 16, 0, 0);
    }
  };
  auto dma_k = [&](int db, auto kb) { dma_rows(a.k, kbuf(kb), db, true); };
  auto dma_v = [&](int db, auto vb) { dma_rows(a.v, vbuf(vb), db, false); };
  auto dma_wait = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)
  // vmcnt(2 NDMA): every load but the direct loads of the current iteration
  auto dma_wait_prev = [] { __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NDMA)); };
  static_assert(kF32In || 2 * NDMA < 16, "vmcnt field");
  auto load_k = [&](int db) {
    const unsigned char* kg = (const unsigned char*)a.k + kvbase * 4;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int p = tid + i * kThreads;
      const int t = max(kd_t[db][p / PPR], 0);
      kst[i] = *(const u32x4v*)(kg + ((size_t)t * PPR + p % PPR) * 16);
    }
  };
  auto load_v = [&](int db) {
    const unsigned char* vg = (const unsigned char*)a.v + kvbase * 4;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int p = tid + i * kThreads;
      const int t = max(kd_t[db][p / PPR], 0);
      vst4[i] = *(const u32x4v*)(vg + ((size_t)t * PPR + p % PPR) * 16);
    }
  };
  auto store_k = [&](auto kb) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int p = tid + i * kThreads;
      float* kd = (float*)kbuf(kb) + (p / PPR) * L::KS + (p % PPR) * 4;
      kd[0] = __uint_as_float(kst[i].x);
      kd[1] = __uint_as_float(kst[i].y);
      kd[2] = __uint_as_float(kst[i].z);
      kd[3] = __uint_as_float(kst[i].w);
    }
  };
  auto store_v = [&](auto vb) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int p = tid + i * kThreads;
      float* vl = (float*)vbuf(vb);
      *(u32x4v*)(vl + (p / PPR) * L::VS + (p % PPR) * 4) = vst4[i];
    }
  };

  // ---- S^T = K Q^T for one chunk (32 keys x 32 rows per block, 2 blocks)
  auto qk = [&](auto kb, f32x16 (&acc)[2]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      acc[blk] = f32x16{};
      if constexpr (!kF32In) {
        const int base = k_base(kb);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          acc[blk] = mfma32x32x16(k_operand(kb, base, ks, blk), qop[ks], acc[blk]);
      } else {
        const float* kl = (const float*)kbuf(kb) + (32 * blk + li) * L::KS + hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc[blk] = mfma32x32x2(kl[2 * ks], qop[ks], acc[blk]);
      }
    }
  };

  // ---- the A8 mask of one chunk (in place on the scores), only on chunks
  // that some row of the tile does not keep wholly
  auto apply_mask = [&](f32x16 (&sc)[2], int db) {
    const int mclass = __builtin_amdgcn_readfirstlane(s_flag[db]);   // uniform
    if (mclass != 0) {
      // branch-free: one unsigned compare and a select per score (a
      // short-circuit form of an older mask was compiled into divergent
      // branches that lost a store)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int jj = 32 * blk + 8 * (e >> 2) + 4 * hh + (e & 3);
          const bool keep = (unsigned)(q - kd_t[db][jj]) <= (unsigned)kd_r[db][jj];
          sc[blk][e] = keep ? sc[blk][e] : kNegInf;
        }
    }
  };
  // ---- online-softmax bookkeeping of one chunk; returns the exponent bias
  // -m_run * c.  A lazily moved reference max (m_run, raw units) moves only
  // when some row's max grows by more than 2^8 in the exp2 domain, so the O
  // rescale is skipped on most chunks; probabilities stay <= 2^8
  auto update_max = [&](f32x16 (&sc)[2], auto&& before_rescale) -> float {
    float mc = sc[0][0];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mc = fmaxf(mc, sc[blk][e]);
    mc = halves_max(mc);
    const float c = a.scale_log2;
    if (wave_ballot(mc * c > m_run * c + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mc);
      const float alpha = m_new == kNegInf ? 1.0f : exp2_fast((m_run - m_new) * c);
      before_rescale();   // pending PV work joins O before it is rescaled
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) oacc[d2] *= alpha;
    }
    return m_run == kNegInf ? 0.0f : -m_run * c;
  };
  auto softmax_pre = [&](f32x16 (&sc)[2], int db, auto&& before_rescale) -> float {
    apply_mask(sc, db);
    return update_max(sc, before_rescale);
  };
  // ---- probabilities: exp2, row sum, bf16 pack (straight-line)
  typedef typename std::conditional<kF32In, f32x16, bf16x8>::type POp;
  constexpr int NP = kF32In ? 2 : 4;
  auto softmax_exp = [&](f32x16 (&sc)[2], float mb, POp (&pk)[NP]) {
    const float c = a.scale_log2;
    float ps = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[blk][e] = exp2_fast(fmaf(sc[blk][e], c, mb));
        ps += sc[blk][e];
      }
    l_run += ps;
    if constexpr (!kF32In) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& src = sc[ks >> 1];
        const int o8 = 8 * (ks & 1);
        uint4 u;
        u.x = pack_bf16x2(src[o8 + 0], src[o8 + 1]);
        u.y = pack_bf16x2(src[o8 + 2], src[o8 + 3]);
        u.z = pack_bf16x2(src[o8 + 4], src[o8 + 5]);
        u.w = pack_bf16x2(src[o8 + 6], src[o8 + 7]);
        pk[ks] = as_bf16x8(u);
      }
    } else {
      pk[0] = sc[0];
      pk[1] = sc[1];
    }
  };

  // ---- O^T += V^T P^T
  auto pv = [&](auto vb, const POp (&pk)[NP]) {
    if constexpr (!kF32In) {
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          oacc[d2] = mfma32x32x16(v_tr_operand<D>(vbuf(vb), vtr_off, d2, ks), pk[ks], oacc[d2]);
    } else {
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) {
        const float* vl = (const float*)vbuf(vb) + 32 * d2 + li;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 32 * blk + 8 * (e >> 2) + 4 * hh + (e & 3);
            oacc[d2] = mfma32x32x2(vl[key * L::VS], pk[blk][e], oacc[d2]);
          }
      }
    }
  };

  // ---- bf16: one fused region per chunk, in explicit issue order (a wave
  // issues in order, so the overlap of the matrix and vector units is
  // written out; a scheduling fence after each slot keeps the compiler from
  // regrouping).  Slot i issues QK MFMA i of chunk c+1 (the two 32-key
  // blocks alternate: independent accumulators), PV MFMA i of chunk c-1 (the
  // output blocks rotate), and the exps of chunk c (32 / slots per slot);
  // exps are summed and packed to bf16 one slot later, so nothing waits on an
  // exp just issued; P(c-1) operand p is last read in the slot where P(c)
  // operand p is still being built.  LDS operand reads run two slots ahead.
  constexpr int NQM = 2 * NKS;          // QK MFMAs per chunk (= slots)
  constexpr int NB = D / 32;            // output blocks of O^T
  constexpr int NPV = NB * 4;           // PV MFMAs per chunk
  constexpr int EPM = 32 / NQM;         // exps per slot
  static_assert(kF32In || (NQM == NPV && NQM >= 4 && 32 % NQM == 0), "slot schedule");
  auto region = [&](auto kb, f32x16 (&nx)[2], f32x16 (&sc)[2], float mb, POp (&pk)[NP], auto vb,
                    float& ps) {
    if constexpr (!kF32In) {
      const int kbase = k_base(kb);
      auto rk = [&](int i) {   // QK operand i: block i & 1, k-step i >> 1
        return k_operand(kb, kbase, i >> 1, i & 1);
      };
      auto rv = [&](int j) {   // PV operand j: output block j % NB, k-step j / NB
        return v_tr_operand<D>(vbuf(vb), vtr_off, j % NB, j / NB);
      };
      auto pack = [&](int pidx) {
        const f32x16& src = sc[pidx >> 1];
        const int o8 = 8 * (pidx & 1);
        uint4 u;
        u.x = pack_bf16x2(src[o8 + 0], src[o8 + 1]);
        u.y = pack_bf16x2(src[o8 + 2], src[o8 + 3]);
        u.z = pack_bf16x2(src[o8 + 4], src[o8 + 5]);
        u.w = pack_bf16x2(src[o8 + 6], src[o8 + 7]);
        pk[pidx] = as_bf16x8(u);
      };
      const float c = a.scale_log2;
      bf16x8 kn = rk(0), vn = rv(0);   // operands one slot ahead
      nx[0] = f32x16{};
      nx[1] = f32x16{};
      ps = 0.0f;
#pragma unroll
      for (int i = 0; i <= NQM; ++i) {
        if (i < NQM) {
          const bf16x8 ak = kn, av = vn;
          if (i + 1 < NQM) {
            kn = rk(i + 1);
            vn = rv(i + 1);
          }
          nx[i & 1] = mfma32x32x16(ak, qop[i >> 1], nx[i & 1]);
          oacc[i % NB] = mfma32x32x16(av, pk[i / NB], oacc[i % NB]);
#pragma unroll
          for (int u = 0; u < EPM; ++u) {
            const int e = EPM * i + u;
            sc[e >> 4][e & 15] = exp2_fast(fmaf(sc[e >> 4][e & 15], c, mb));
          }
        }
        if (i > 0) {
          // row sums in float32 (summing the bf16-rounded values instead
          // moves a row dominated by one key by up to 2^-9 relative)
#pragma unroll
          for (int u = 0; u < EPM; ++u) {
            const int e = EPM * (i - 1) + u;
            ps += sc[e >> 4][e & 15];
          }
          if ((EPM * i) % 8 == 0) {   // elements 8p .. 8p+7 done
            const int pidx = EPM * i / 8 - 1;
            pack(pidx);
            // used here: P(c) is consumed only in the next iteration, and the
            // exps would otherwise be sunk past the region to the loop's end
            asm volatile("" ::"v"(pk[pidx]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      asm volatile("" ::"v"(ps));
    }
  };

  const int nchunk = (nk + kChunk - 1) / kChunk;
  // descriptors of chunks 0 .. n-1 (tokens -1 past the end): every read
  // issued before the first store, so the prologue waits once
  auto publish_first_descriptors = [&](auto n) {
    constexpr int N = decltype(n)::value;
    KeyDesc d0[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      d0[j] = KeyDesc{-1, 0, make_int2(-1, 0)};
      desc_fetch(j * kChunk, d0[j]);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) desc_put(j, d0[j]);
    __syncthreads();
  };
  f32x16 sA[2], sB[2];
  // P operands: in the bf16 region P(c-1) operand p is last read by a PV
  // MFMA one slot before P(c) operand p is packed into the same registers
  POp pk[NP];
  float l_tot;
  if constexpr (!kF32In) {
    // ---- bf16 software pipeline.  Entering iteration c >= 1: the scores of
    // chunk c and P of chunk c-1 are in registers; K(c+1) and V(c-1) are in
    // LDS, K(c+2) and V(c) are arriving; descriptors of c .. c+3 are
    // published.  Per iteration: the descriptor reads of chunk c+4 and the
    // direct loads of K(c+3) and V(c+1) are issued (into the buffers read
    // last in iteration c-1); mask of chunk c; the fused region (QK c+1, exps
    // c, PV c-1); descriptors of chunk c+4 are stored; the loads issued one
    // iteration earlier are awaited; barrier.  Past the last chunk the loads
    // and QK run on descriptors of tokens -1 (row 0) and their results are
    // unused, which keeps the region free of branches (the direct loads still
    // in flight when the workgroup ends are awaited by its end of program).  Buffers rotate over
    // three and score / P registers over two, so the loop is unrolled by six
    // and every buffer index is a compile-time constant.
    //
    // Two modes.  Fixed reference (first run): each row's maximum over the
    // first chunk is its reference for the whole tile, so later chunks need
    // no maximum and O is never rescaled; a probability of up to 2^64 (a
    // later score up to 64 binary orders above the reference) is harmless in
    // float32 (sums of thousands of such terms stay far below 2^128, and the
    // relative precision of every term is unchanged).  A row whose final sum
    // leaves [2^-64, 2^64] (a larger score, a row with nothing kept in the
    // first chunk, NaN) makes the workgroup rerun the tile in the exact mode:
    // the running maximum, moved lazily by more than 2^8, with rescales.
    auto run = [&](auto exact) {
      constexpr bool kExact = decltype(exact)::value;
      publish_first_descriptors(std::integral_constant<int, 4>{});
      dma_k(0, C0{});
      dma_k(1, C1{});
      dma_k(2, C2{});
      dma_v(0, C0{});
      {   // V buffer 2 starts at zero: iteration 0 runs its PV slots on it
        uint4* vz = (uint4*)vbuf(C2{});
        for (int i = tid; i < (int)(L::vBytes / 16); i += kThreads) vz[i] = make_uint4(0, 0, 0, 0);
      }
      dma_wait();
      complete_q();
      __syncthreads();
      qk(C0{}, sA);
      float mb0;
      {   // iteration 0: no PV yet
        desc_load(4 * kChunk);
        __builtin_amdgcn_sched_barrier(0);   // descriptor reads before the direct loads
        dma_v(1, C1{});
        mb0 = softmax_pre(sA, 0, [] {});
#pragma unroll
        for (int p = 0; p < NP; ++p) pk[p] = POp{};
        // K(3) goes over K(0): every wave's qk(0) must have read it (later
        // iterations overwrite a buffer read before the last barrier)
        __syncthreads();
        dma_k(3, C0{});
        float ps;
        region(C1{}, sB, sA, mb0, pk, C2{}, ps);
        l_run += ps;
        desc_store(4);
        dma_wait_prev();
        __syncthreads();
      }
      // iteration c with R = c mod 3 (compile-time): direct loads into K
      // buffer R and V buffer (R+1) mod 3, reads of K buffer (R+1) mod 3 and
      // V buffer (R+2) mod 3; scores of chunks c and c+1 alternate between
      // sA and sB with the parity of c
      auto step = [&](int c, auto rr, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        constexpr int R = decltype(rr)::value;
        using Kw = std::integral_constant<int, R>;
        using Vw = std::integral_constant<int, (R + 1) % 3>;
        using Kr = std::integral_constant<int, (R + 1) % 3>;
        using Vr = std::integral_constant<int, (R + 2) % 3>;
        desc_load((c + 4) * kChunk);
        __builtin_amdgcn_sched_barrier(0);
        dma_k((c + 3) % kDesc, Kw{});
        dma_v((c + 1) % kDesc, Vw{});
        float mb = mb0;
        if constexpr (kExact) {
          // a rescale first completes PV(c-1) and zeroes P(c-1), so the
          // region's PV MFMAs then add exactly 0
          mb = softmax_pre(cur, c % kDesc, [&] {
            pv(Vr{}, pk);
#pragma unroll
            for (int p = 0; p < NP; ++p) pk[p] = POp{};
          });
        } else {
          apply_mask(cur, c % kDesc);
        }
        float ps;
        region(Kr{}, nxt, cur, mb, pk, Vr{}, ps);
        l_run += ps;
        desc_store((c + 4) % kDesc);
        dma_wait_prev();
        __syncthreads();
      };
      for (int c = 1; c < nchunk; c += 6) {
        step(c, C1{}, sB, sA);
        if (c + 1 >= nchunk) break;
        step(c + 1, C2{}, sA, sB);
        if (c + 2 >= nchunk) break;
        step(c + 2, C0{}, sB, sA);
        if (c + 3 >= nchunk) break;
        step(c + 3, C1{}, sA, sB);
        if (c + 4 >= nchunk) break;
        step(c + 4, C2{}, sB, sA);
        if (c + 5 >= nchunk) break;
        step(c + 5, C0{}, sA, sB);
      }
      // PV of the last chunk: its V is in buffer (nchunk - 1) mod 3
      switch ((nchunk - 1) % 3) {
        case 0: pv(C0{}, pk); break;
        case 1: pv(C1{}, pk); break;
        default: pv(C2{}, pk); break;
      }
      l_tot = halves_sum(l_run);
    };
    run(std::false_type{});
    const bool bad = row_ok && !(l_tot >= 0x1p-64f && l_tot <= 0x1p64f);
    if (wave_ballot(bad) != 0 && lane == 0) s_redo = 1;
    __syncthreads();
    if (s_redo) {
      m_run = kNegInf;
      l_run = 0.0f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
      run(std::true_type{});
    }
  } else {
    // ---- float32 inputs: K one chunk ahead, V staged with it, steps in order
    publish_first_descriptors(std::integral_constant<int, 3>{});
    complete_q();
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      load_k((c + 1) % kDesc);
      load_v((c + 1) % kDesc);
      desc_load((c + 3) * kChunk);
      qk(c & 1, sA);
      const float mb = softmax_pre(sA, c % kDesc, [] {});
      softmax_exp(sA, mb, pk);
      pv(c & 1, pk);
      store_k((c + 1) & 1);
      store_v((c + 1) & 1);
      desc_store((c + 3) % kDesc);
      __syncthreads();
    }
    l_tot = halves_sum(l_run);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  if (row_ok) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const size_t orow = (((size_t)b * a.Hq + hq) * S + q) * D;
#pragma unroll
    for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * d2 + 8 * j + 4 * hh;
        const float o0 = oacc[d2][4 * j] * inv, o1 = oacc[d2][4 * j + 1] * inv;
        const float o2 = oacc[d2][4 * j + 2] * inv, o3 = oacc[d2][4 * j + 3] * inv;
        if constexpr (kF32Out) {
          *(float4*)((float*)a.o + orow + d) = make_float4(o0, o1, o2, o3);
        } else {
          *(uint2*)((uint16_t*)a.o + orow + d) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
      }
    if (hh == 0)
      a.lse[((size_t)b * a.Hq + hq) * S + q] =
          l_tot > 0.0f ? (m_run * a.scale_log2 + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, bool kF32In, bool kF32Out>
void launch_fwd_kernel(const FwdArgs& a, int n_wg, hipStream_t st) {
  hipLaunchKernelGGL((masked_fwd_kernel<D, kF32In, kF32Out>), dim3((unsigned)n_wg), dim3(kThreads),
                     0, st, a);
}

}  // namespace

int fwd_rows_per_head(const Dims& d) { return kRowsPerTile / d.G; }

static int fwd_ntiles(const Dims& d) {
  const int m = fwd_rows_per_head(d);
  return (d.S + m - 1) / m;
}

static int fwd_list_cap(const Dims& d) { return d.k < d.S ? d.k : d.S; }

size_t fwd_ws_bytes(const Dims& d) {
  const size_t nseg = d.nseg(), nt = fwd_ntiles(d);
  size_t bytes = align256(nseg * d.S * 4);                              // order
  bytes += align256(nseg * d.S * 4);                                    // q_end
  bytes += align256(nseg * nt * 4);                                     // counts
  bytes += align256(nseg * nt * (size_t)fwd_list_cap(d) * 8);           // lists
  return bytes;
}

FwdPlan launch_fwd_plan(const Dims& d, const int* rank, const int* tau, void* ws,
                        hipStream_t st) {
  const int nseg = d.nseg(), nt = fwd_ntiles(d), m = fwd_rows_per_head(d);
  const int cap = fwd_list_cap(d);
  char* p = (char*)ws;
  int* order = (int*)p; p += align256((size_t)nseg * d.S * 4);
  int* qend = (int*)p; p += align256((size_t)nseg * d.S * 4);
  int* count = (int*)p; p += align256((size_t)nseg * nt * 4);
  int2* list = (int2*)p;

  const long long total = (long long)nseg * d.S;
  const unsigned nblk = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(key_end_kernel, dim3(nblk), dim3(256), 0, st, rank, tau, order, qend, d.S,
                     d.s, d.w, total);
  hipLaunchKernelGGL(tile_list_kernel, dim3(nt, nseg), dim3(kListThreads), 0, st, order, tau,
                     qend, d.S, d.s, d.w, m, nt, cap, list, count);
  FwdPlan pl;
  pl.list = list; pl.count = count; pl.qend = qend; pl.m = m; pl.ntiles = nt; pl.cap = cap;
  return pl;
}

hipError_t launch_masked_fwd(const Dims& d, const void* q, const void* k, const void* v,
                             const int* rank, const int* tau, void* o, float* lse, void* ws,
                             hipStream_t st) {
  const FwdPlan pl = launch_fwd_plan(d, rank, tau, ws, st);
  const int2* list = pl.list;
  const int* count = pl.count;
  const int m = pl.m, nt = pl.ntiles, cap = pl.cap;

  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.rank = rank; a.tau = tau; a.list = list; a.count = count;
  a.qend = pl.qend;
  a.o = o; a.lse = lse;
  a.S = d.S; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.m = m; a.ntiles = nt;
  a.s = d.s; a.w = d.w; a.cap = cap;
  a.reverse = launch_order_reversed();
  a.scale_log2 = d.scale * 1.4426950408889634f;
  const int n_wg = nt * d.Hkv * d.b;   // one workgroup per tile
  if (d.D == 128) {
    if (d.f32_in) {
      if (d.f32_out) launch_fwd_kernel<128, true, true>(a, n_wg, st);
      else launch_fwd_kernel<128, true, false>(a, n_wg, st);
    } else {
      if (d.f32_out) launch_fwd_kernel<128, false, true>(a, n_wg, st);
      else launch_fwd_kernel<128, false, false>(a, n_wg, st);
    }
  } else {
    if (d.f32_in) {
      if (d.f32_out) launch_fwd_kernel<64, true, true>(a, n_wg, st);
      else launch_fwd_kernel<64, true, false>(a, n_wg, st);
    } else {
      if (d.f32_out) launch_fwd_kernel<64, false, true>(a, n_wg, st);
      else launch_fwd_kernel<64, false, false>(a, n_wg, st);
    }
  }
  return hipGetLastError();
}

}  // namespace kvpop
