// kvpop_masked_attn_bwd: gradients of the fixed-budget sparse attention.
//
// The student's forward attends over the kept set of KVpop reading notes §2.3
// (M[q,t] = 1[t<s] or 1[q-t<w] or (1[t in E(q)] and 1[rank(t) <= tau_q]),
// causal); training the sparse student (§2.1: distillation against the dense
// teacher) needs its backward.  With P the renormalised probabilities over the
// kept keys (rebuilt from the forward's LSE), for an upstream gradient dO:
//   dP_it = <dO_i, v_t>,  D_i = <dO_i, O_i> (= sum_t P_it dP_it),
//   dS_it = P_it (dP_it - D_i),
//   dQ_i = scale sum_t dS_it k_t,  dK_t = scale sum_i dS_it q_i,
//   dV_t = sum_i P_it dO_i,
// with dK, dV summed over the query heads that share the KV head.
//
// Design (gfx950):
//  * bwd_dot_kernel: D_i from dO and the forward's O, and the row's LSE in
//    the exp2 domain.
//  * dQ, query-major (bwd_dq_kernel): the forward's tiles (m rows of each of
//    the G query heads stacked into 256 rows, 8 waves of 32) and its key plan
//    (sinks, the listed long-range keys of the tile's first row, the band);
//    per 64-key chunk the K and V rows are direct-loaded into one of two
//    swizzled LDS stages (the next chunk's loads in flight during the math),
//    then per wave S^T = K Q^T and dP^T = V dO^T on MFMA, dS in registers,
//    and dQ^T += K^T dS^T on MFMA with K^T read transposed from the same
//    stage and dS as the B operand.
//  * dK, dV, key-major (bwd_dkdv_kernel): key t is kept by the contiguous rows
//    [t, q_end(t)] (tau never increases with q), so a tile of keys needs the
//    rows [min t, max q_end], and the mask of a (row, key) pair is the
//    interval test t <= q <= q_end(t).  The forward plan finds q_end(t);
//    bwd_key_order_kernel orders the keys into 128-key tiles (short-lived
//    keys by token, long-lived ones by q_end band and token band), and
//    bwd_tile_plan_kernel lists each tile's 32-row chunks as one work item,
//    or two split at the fixed row S / 2 when it spans more than half the
//    sequence (the second half's sums added by bwd_dkdv_merge_kernel in a
//    fixed order).  Per workgroup (4 waves of 32 keys, K and V operands in
//    registers) the (query head, chunk) items stream through six LDS stages
//    by direct loads, three items ahead: S = Q K^T and dP = dO V^T of the
//    next item, dV^T += dO^T P and dK^T += Q^T dS of the previous one (Q^T
//    and dO^T read transposed from the same stage) and the P / dS math of
//    the current one are interleaved MFMA by MFMA.
//  * bf16 inputs, float32 accumulation, P and dS rounded to bf16 as MFMA
//    operands; dQ, dK, dV are written in float32.
#include <mutex>
#include <type_traits>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kQThreads = 512;      // dQ: 8 waves x 32 stacked rows
constexpr int kQChunk = 64;         // dQ: keys per chunk
constexpr int kKGroups = 4;         // dK/dV: 32-key groups per tile, one wave pair each
constexpr int kKTile = 32 * kKGroups;
constexpr int kKThreads = 128 * kKGroups;
constexpr int kRChunk = 32;         // dK/dV: query rows per chunk

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- D_i
// D_i = sum_d dO[i, d] O[i, d] per row, and the row's LSE times log2 e
template <int D, bool kF32Out>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const uint16_t* __restrict__ dout,
                                                      const void* __restrict__ o,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ dvec,
                                                      float* __restrict__ lse2, long long rows) {
  constexpr int LPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPW = 64 / LPR;       // rows per wave
  const long long wv = ((long long)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int lane = lane_id();
  const long long row = wv * RPW + lane / LPR;
  const int part = lane % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const uint4 u = *(const uint4*)(dout + row * D + part * 8);
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
    float ov[8];
    if constexpr (kF32Out) {
      const float4 a = *(const float4*)((const float*)o + row * D + part * 8);
      const float4 b = *(const float4*)((const float*)o + row * D + part * 8 + 4);
      ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
      ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
    } else {
      const uint4 x = *(const uint4*)((const uint16_t*)o + row * D + part * 8);
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ov[2 * i] = bf16_bits_to_f32(xw[i] & 0xffffu);
        ov[2 * i + 1] = bf16_bits_to_f32(xw[i] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_bits_to_f32(uw[i] & 0xffffu) * ov[2 * i];
      acc += bf16_bits_to_f32(uw[i] >> 16) * ov[2 * i + 1];
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && row < rows) {
    dvec[row] = acc;
    lse2[row] = lse[row] * kLog2e;   // the LSE in the exp2 domain, for both kernels
  }
}

// Buckets of the dK/dV key order for sequence length S: keys living at most
// w + 64 rows by t / 64 (a tile of them visits about w + 64 rows); the
// others by (q_end band, t band) with S / 8-row q_end bands and S / 64-token
// t bands, so the keys of a tile end and start near each other and the rows
// it streams ([min t, max q_end]) are mostly rows its keys keep.  (On the
// 16k layer this keeps about two thirds of the streamed (key, row) pairs,
// against one half when long-lived keys are ordered by q_end alone.)
struct KeyBuckets {
  int nb1, qb, tb, ntb, nb;
  __host__ __device__ explicit KeyBuckets(int S) {
    nb1 = (S + 63) / 64;
    qb = ((S + 7) / 8 + 63) / 64 * 64;
    tb = ((S + 63) / 64 + 63) / 64 * 64;
    ntb = (S + tb - 1) / tb;
    nb = nb1 + ((S + qb - 1) / qb) * ntb;
  }
};

// Exclusive prefix sums of cnt[0 .. n) into off[0 .. n) by all 1024 threads
// of the workgroup (n <= 8192): with rev, in descending index order (off[i]
// = the sum of cnt[j] for j > i).  Integer sums: the same offsets as a serial
// pass.  cnt and off must not overlap; wtot holds 16 wave totals.
__device__ void block_excl_scan_1024(const int* cnt, int* off, int n, int* wtot, bool rev) {
  constexpr int kPer = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[kPer];
  int local = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid * kPer + u;
    v[u] = i < n ? cnt[rev ? n - 1 - i : i] : 0;
    local += v[u];
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int j = 0; j < wave; ++j) run += wtot[j];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid * kPer + u;
    if (i < n) off[rev ? n - 1 - i : i] = run;
    run += v[u];
  }
  __syncthreads();
}

// Key order of the dK/dV tiles, one workgroup per (sequence, KV head): a
// counting sort over the KeyBuckets (order inside a bucket is free: a key's
// sums do not depend on its tile).
__global__ __launch_bounds__(1024) void bwd_key_order_kernel(const int* __restrict__ qend,
                                                             int* __restrict__ korder, int S,
                                                             int w) {
  extern __shared__ int bk[];       // nb counters, then nb offsets
  __shared__ int wtot[16];
  const int seg = blockIdx.x, tid = threadIdx.x;
  const KeyBuckets kb(S);
  const int nb = kb.nb;
  const int* qe = qend + (size_t)seg * S;
  int* out = korder + (size_t)seg * S;
  for (int i = tid; i < nb; i += 1024) bk[i] = 0;
  __syncthreads();
  auto bucket = [&](int t) {
    const int e = qe[t];
    return (e - t + 1 <= w + 64) ? t / 64 : kb.nb1 + (e / kb.qb) * kb.ntb + t / kb.tb;
  };
  for (int t = tid; t < S; t += 1024) atomicAdd(&bk[bucket(t)], 1);
  __syncthreads();
  block_excl_scan_1024(bk, bk + nb, nb, wtot, false);   // nb <= S / 64 + 512
  for (int t = tid; t < S; t += 1024) out[atomicAdd(&bk[nb + bucket(t)], 1)] = t;
}

// ---------------------------------------------------------------- dQ
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* dvec;
  const float* lse2;   // LSE log2 e per row
  const int* rank;
  const int* tau;
  const int* qend;
  const int* korder;
  const int4* tplan;   // [nseg, 2 ktiles] dK/dV work items (tile, part, first chunk, end chunk)
  const int* tsplit;   // [nseg, ktiles] 1 if the tile's rows are split over two items
  float* part1;        // [nseg, ktiles, kKTile, 2, D] second-half sums of split tiles
  const int2* list;
  const int* count;
  float* dq;
  float* dk;
  float* dv;
  int S, Hq, Hkv, G, m, ntiles, ktiles, s, w, cap;
  int reverse;         // launch order reversed (testing aid)
  float scale, scale_log2;
};

// LDS layout of the dQ kernel's K and V chunks: row-major 64-key chunks of
// 16-byte pieces, piece p of row r in slot p XOR dq_swz(r).  Row reads (the A
// operands of S^T = K Q^T and dP^T = V dO^T: 16 lanes read one piece of 16
// aligned rows) need dq_swz to take 16 distinct slot values over those rows;
// the transposed reads of K (the A operand K^T of dQ^T += K^T dS^T: a wave
// reads 64 bytes of each of 8 aligned rows, 16 lanes 32 bytes of 4 rows)
// need every 16-byte slot of the bank line hit exactly twice.  D = 128 (one
// row per 256-byte bank line): the two bit pairs of r mod 16 swapped;
// D = 64 (two rows per line, the row's parity picking the half): a
// permutation of (r / 2) mod 8 whose top bit is r / 2 mod 2.
template <int D>
__device__ __forceinline__ int dq_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offsets, per lane, of the transposed K^T operand reads (output block
// db, half a of the k-step's 8 keys): lane (li, hh) reads row
// 16 ks + 8 a + 4 hh + jq, dims 32 db + 16 (li / 16) + 4 (j mod 4) .. + 3 with
// j = li mod 16, jq = j / 4; ds_read_b64_tr_b16 then hands lane i of each
// 16-lane group element (i mod 4) of the words read by lanes 4e + i/4, so
// the pair a = 0, 1 is the MFMA operand element 4 a + r = K[16 ks + 8 a +
// 4 hh + r][32 db + li].  The row's swizzle depends on a but not on ks, so
// ks enters as an immediate.
template <int D>
__device__ __forceinline__ void dq_tr_offsets(int lane, int (&off)[D / 32][2]) {
  const int hh = lane >> 5, li = lane & 31;
  const int half = li >> 4, j = li & 15, jq = j >> 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a8 = 0; a8 < 2; ++a8) {
      const int row = 8 * a8 + 4 * hh + jq;          // ks = 0
      const int dim = 32 * db + 16 * half + 4 * (j & 3);
      off[db][a8] = row * (D * 2) + (((dim >> 3) ^ dq_swz<D>(row)) << 4) + (dim & 7) * 2;
    }
}

// dQ, query-major on the forward's tiles and key plan (8 waves, 256 stacked
// rows): per 64-key chunk, S^T = K Q^T and dP^T = V dO^T on MFMA (each lane
// owns one row), P = exp(S scale - LSE) on kept keys, dS = P (dP - D) packed
// to bf16, and dQ^T += K^T dS^T with the K^T operand read transposed from
// the same LDS chunk.  K and V arrive by direct loads into two LDS stages:
// the gathers of chunk c+2 are issued after the barrier that ends chunk c
// into the buffers chunk c used, and awaited before the barrier that ends
// chunk c+1; the key descriptors (token, q_end - t) of chunk c+2 are read by
// wave 0 during chunk c and stored before that barrier.
template <int D>
__global__ __launch_bounds__(kQThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NKS = D / 16;
  constexpr int PPR = D / 8;                 // 16-byte pieces per row
  constexpr int RB = D * 2;                  // bytes per row
  constexpr int CB = kQChunk * RB;           // bytes per chunk buffer
  constexpr int RPI = 1024 / RB;             // rows per 1 KB direct load
  constexpr int NDMA = kQChunk / RPI / (kQThreads / 64);   // direct loads per wave per chunk
  static_assert(NDMA * RPI * (kQThreads / 64) == kQChunk, "direct-load tiling");
  constexpr int kSlots = 4;                  // descriptor slots (chunks c .. c+2 live)
  // K buffers first (their transposed reads reach furthest past their base);
  // equal-sized arrays are laid out in name order
  __shared__ __attribute__((aligned(16))) unsigned char dqa_k0[CB];
  __shared__ __attribute__((aligned(16))) unsigned char dqa_k1[CB];
  __shared__ __attribute__((aligned(16))) unsigned char dqb_v0[CB];
  __shared__ __attribute__((aligned(16))) unsigned char dqb_v1[CB];
  __shared__ __attribute__((aligned(16))) int kd_t[kSlots][kQChunk];
  __shared__ __attribute__((aligned(16))) int kd_span[kSlots][kQChunk];   // q_end(t) - t
  __shared__ int kd_flag[kSlots];   // 0: every row of the tile keeps every key of the chunk
  auto kbuf = [&](auto i) -> unsigned char* {
    if constexpr (decltype(i)::value == 0) return dqa_k0;
    else return dqa_k1;
  };
  auto vbuf = [&](auto i) -> unsigned char* {
    if constexpr (decltype(i)::value == 0) return dqb_v0;
    else return dqb_v1;
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;

  const int lane = lane_id(), wave = wave_id();
  const int hh = lane >> 5, li = lane & 31;
  const int bid = launch_block(a.reverse);
  const int tile = bid % a.ntiles;
  const int h = (bid / a.ntiles) % a.Hkv;
  const int b = bid / (a.ntiles * a.Hkv);
  const int S = a.S, s = a.s, w = a.w, m = a.m, G = a.G;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int* qend = a.qend + seg * S;
  const int* tau = a.tau + seg * S;
  const int q0 = tile * m;
  const int q_hi = min(q0 + m - 1, S - 1);

  const int rr = wave * 32 + li;
  const int g = rr / m;
  const int q = q0 + (rr - g * m);
  const bool row_ok = g < G && q < S;
  const int hq = h * G + (g < G ? g : 0);
  const size_t qrow = ((size_t)b * a.Hq + hq) * S + (row_ok ? q : 0);
  const float lse2 = row_ok ? a.lse2[qrow] : 0.0f;
  const float drow = row_ok ? a.dvec[qrow] : 0.0f;

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
  const int nchunk = (nk + kQChunk - 1) / kQChunk;
  const int2* lst = a.list + (seg * a.ntiles + tile) * (size_t)a.cap;

  // B operands: Q^T and dO^T of this lane's row, dims [16 ks + 8 hh, +8)
  // (unconditional loads of a valid row, zeroed for padding rows; completed
  // before the chunk loop so that it does not wait on them)
  bf16x8 qop[NKS], dop[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4v u = *(const u32x4v*)(a.q + qrow * D + 16 * ks + 8 * hh);
    u32x4v x = *(const u32x4v*)(a.dout + qrow * D + 16 * ks + 8 * hh);
    if (!row_ok) u = x = u32x4v{0, 0, 0, 0};
    qop[ks] = __builtin_bit_cast(bf16x8, u);
    dop[ks] = __builtin_bit_cast(bf16x8, x);
  }
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) dqacc[d2] = f32x16{};

  // ---- key descriptors of the chunk starting at c0: wave 0 reads them
  // (branch-free, clamped) into registers, and stores token and span
  // q_end(t) - t (token -1, span 0 for padding) one phase later, with the
  // chunk's mask flag: 0 when every key is kept by every row of the tile
  // (t <= q0 and q_end(t) >= q_hi), so no mask runs
  struct Desc {
    int t, r;
    int2 l;
  };
  auto desc_fetch = [&](int c0, Desc& d) {
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
  auto desc_put = [&](int slot, const Desc& d) {
    if (wave == 0) {
      int t = d.t == -2 ? d.l.x : d.t;
      const int e = d.t == -2 ? d.l.y : d.r;
      if (t >= S) t = -1;
      kd_t[slot][lane] = t;
      kd_span[slot][lane] = t >= 0 ? e - t : 0;
      const bool always = (t >= 0) & (t <= q0) & (e >= q_hi);
      const uint64_t not_always = wave_ballot(!always);
      if (lane == 0) kd_flag[slot] = not_always == 0 ? 0 : 2;
    }
  };

  // ---- gathers: each 1 KB direct load fills RPI rows; lane L fetches the
  // global piece that the row's swizzle places at its slot (padding keys
  // read row 0: they are masked, so only finiteness matters)
  typedef __attribute__((address_space(3))) void lds_void;
  const size_t kvbase = seg * (size_t)S * D;
  auto dma_rows = [&](const uint16_t* src, unsigned char* dst, int slot) {
    const unsigned char* gsrc = (const unsigned char*)(src + kvbase);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r0 = (wave * NDMA + i) * RPI;
      const int row = r0 + lane / PPR, sl = lane % PPR;
      const int t = min(max(kd_t[slot][row], 0), S - 1);
      const int piece = sl ^ dq_swz<D>(row);
      __builtin_amdgcn_global_load_lds((const void*)(gsrc + ((size_t)t * PPR + piece) * 16),
                                       (lds_void*)(dst + r0 * RB), 16, 0, 0);
    }
  };
  auto dma_chunk = [&](int c, auto bi) {
    dma_rows(a.k, kbuf(bi), c % kSlots);
    dma_rows(a.v, vbuf(bi), c % kSlots);
  };

  // per-lane LDS offsets: row reads (row li, piece 2 ks + hh: base XOR 32 ks)
  // and the transposed K^T reads
  int tro[D / 32][2];
  dq_tr_offsets<D>(lane, tro);
  const int row_base = li * RB + ((hh ^ dq_swz<D>(li)) << 4);

  // ---- one chunk from the buffers bi: S, dP, dS, dQ
  auto chunk = [&](int c, auto bi) {
    const unsigned char* kl = kbuf(bi);
    const unsigned char* vl = vbuf(bi);
    int rb = row_base;
    asm volatile("" : "+v"(rb));   // keeps the eight XORs below in the loop
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = f32x16{};
      pacc[blk] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int off = 32 * blk * RB + (rb ^ (32 * ks));
        sacc[blk] = mfma32x32x16(as_bf16x8(*(const uint4*)(kl + off)), qop[ks], sacc[blk]);
        pacc[blk] = mfma32x32x16(as_bf16x8(*(const uint4*)(vl + off)), dop[ks], pacc[blk]);
      }
    }
    // dS = P (dP - D_i), P = exp(S scale - LSE_i) on kept keys: the exp of
    // every score, then, only on chunks with a key that some row of the
    // tile does not keep (a wave-uniform branch), a select (a masked score's
    // exp may overflow; it is never used; key data in 4-wide reads).  Rows
    // past the tile need no mask: their Q and dO operands are zero and their
    // LSE and D are 0, so their dS is exactly 0.
    const int slot = c % kSlots;
    float pr[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) pr[blk][e] = exp2_fast(fmaf(sacc[blk][e], a.scale_log2, -lse2));
    if (__builtin_amdgcn_readfirstlane(kd_flag[slot]) != 0) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j0 = 32 * blk + 8 * jj + 4 * hh;
          const int4 t4 = *(const int4*)(&kd_t[slot][j0]);
          const int4 r4 = *(const int4*)(&kd_span[slot][j0]);
          const int tv[4] = {t4.x, t4.y, t4.z, t4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * jj + r;
            const bool kp = row_ok & ((unsigned)(q - tv[r]) <= (unsigned)rv[r]);
            pr[blk][e] = kp ? pr[blk][e] : 0.0f;
          }
        }
    }
    float dsv[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) dsv[blk][e] = pr[blk][e] * (pacc[blk][e] - drow);
    bf16x8 pk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pk[ks] = pack_bf16x8(&dsv[ks >> 1][8 * (ks & 1)]);
    // dQ^T += K^T dS^T
    typedef __attribute__((address_space(3))) short4v lds_s4;
#pragma unroll
    for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(kl + tro[d2][0] + 16 * ks * RB));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(kl + tro[d2][1] + 16 * ks * RB));
        const short8v v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dqacc[d2] = mfma32x32x16(__builtin_bit_cast(bf16x8, v8), pk[ks], dqacc[d2]);
      }
  };

  // ---- prologue: descriptors of chunks 0 and 1 (every read issued before
  // the first store), their gathers, the query loads completed
  {
    Desc d0{-1, 0, make_int2(-1, 0)}, d1{-1, 0, make_int2(-1, 0)};
    desc_fetch(0, d0);
    desc_fetch(kQChunk, d1);
    desc_put(0, d0);
    desc_put(1, d1);
    __syncthreads();
    dma_chunk(0, C0{});
    dma_chunk(1, C1{});
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qop[ks]), "+v"(dop[ks]));
    __syncthreads();
  }
  // ---- chunk c reads buffers c mod 2; after the barrier that ends it, the
  // gathers of chunk c+2 go into those buffers (compile-time buffer indices:
  // unrolled by two)
  Desc pd{-1, 0, make_int2(-1, 0)};
  auto step = [&](int c, auto bi) {
    desc_fetch((c + 2) * kQChunk, pd);
    chunk(c, bi);
    desc_put((c + 2) % kSlots, pd);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the gathers of chunk c+1
    __syncthreads();
    if (c + 2 < nchunk) dma_chunk(c + 2, bi);
  };
  for (int c = 0; c < nchunk; c += 2) {
    step(c, C0{});
    if (c + 1 < nchunk) step(c + 1, C1{});
  }

  if (row_ok) {
    float* out = a.dq + qrow * D;
#pragma unroll
    for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * d2 + 8 * j + 4 * hh;
        *(float4*)(out + d) = make_float4(dqacc[d2][4 * j] * a.scale, dqacc[d2][4 * j + 1] * a.scale,
                                          dqacc[d2][4 * j + 2] * a.scale,
                                          dqacc[d2][4 * j + 3] * a.scale);
      }
  }
}

// ---------------------------------------------------------------- dK, dV plan
// Work items of the dK/dV kernel, one workgroup per (sequence, KV head): each
// 128-key tile of the key order needs the 32-row chunks [min t, max q_end];
// a tile whose chunks cross the fixed split row R = S/2 (rounded down to a
// chunk) becomes two items, the chunks below R and the chunks from R on, so
// no single workgroup streams more than half the sequence (the sinks' tile
// and the tiles of early tokens kept to the end otherwise set the kernel's
// length alone).  The split row is the same for every tile, so every key
// whose rows cross R is summed as (rows below R) + (rows from R), and any
// other key gets an exact zero from its tile's other half, whatever tile the
// key order put it in (the order inside a bucket is not fixed): dk and dv do
// not depend on the order.  The items are listed longest first (a counting
// sort on the chunk count), so each XCD starts its longest items first;
// empty item slots (the second slot of an unsplit tile) come last and exit
// at once.
__device__ __forceinline__ int split_chunk(int S) { return (S / 2) / kRChunk; }
// bins of the longest-first sort: one per chunk count up to 4095 (32 KB of
// LDS for counters and offsets), longer items share the last bin
__host__ __device__ inline int plan_bins(int S) { return min(S / kRChunk + 2, 4096); }

__global__ __launch_bounds__(1024) void bwd_tile_plan_kernel(const int* __restrict__ korder,
                                                             const int* __restrict__ qend, int S,
                                                             int ktiles, int4* __restrict__ tmp,
                                                             int4* __restrict__ plan,
                                                             int* __restrict__ tsplit) {
  extern __shared__ int hist[];     // nbins counters, then nbins offsets
  __shared__ int wtot[16];
  const int seg = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int nbins = plan_bins(S);     // chunk counts, the longest in one bin
  const int n_ent = 2 * ktiles;
  const int* ko = korder + (size_t)seg * S;
  const int* qe = qend + (size_t)seg * S;
  int4* tm = tmp + (size_t)seg * n_ent;
  int4* pl = plan + (size_t)seg * n_ent;
  for (int i = tid; i < 2 * nbins; i += 1024) hist[i] = 0;
  __syncthreads();
  // one wave per tile: 64 lanes x 2 keys, then a wave reduction
  for (int tile = wave; tile < ktiles; tile += 1024 / 64) {
    int lo = kInt32Max, hi = -1;
#pragma unroll
    for (int r = 0; r < kKTile / 64; ++r) {
      const int slot = tile * kKTile + 64 * r + lane;
      if (slot < S) {
        const int t = ko[slot];
        lo = min(lo, t);
        hi = max(hi, qe[t]);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off));
      hi = max(hi, __shfl_xor(hi, off));
    }
    if (lane == 0) {
      const int c0 = lo <= hi ? lo / kRChunk : 0;
      const int n = lo <= hi ? hi / kRChunk - c0 + 1 : 0;
      int4 e0, e1;
      const int cs = split_chunk(S);
      if (c0 < cs && cs < c0 + n) {
        e0 = make_int4(tile, 0, c0, cs);
        e1 = make_int4(tile, 1, cs, c0 + n);
      } else {
        e0 = make_int4(tile, 0, c0, c0 + n);
        e1 = make_int4(tile, -1, 0, 0);
      }
      tsplit[(size_t)seg * ktiles + tile] = e1.y >= 0 ? 1 : 0;
      tm[2 * tile] = e0;
      tm[2 * tile + 1] = e1;
      atomicAdd(&hist[min(e0.w - e0.z, nbins - 1)], 1);
      atomicAdd(&hist[min(e1.w - e1.z, nbins - 1)], 1);
    }
  }
  __syncthreads();
  block_excl_scan_1024(hist, hist + nbins, nbins, wtot, true);   // offsets, longest first
  for (int i = tid; i < n_ent; i += 1024) {
    const int4 e = tm[i];
    pl[atomicAdd(&hist[nbins + min(e.w - e.z, nbins - 1)], 1)] = e;
  }
}

// dK, dV of split tiles: the first half's sums (written to dk, dv) plus the
// second half's, one float32 add per element.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_merge_kernel(BwdArgs a) {
  const int tile = blockIdx.x % a.ktiles, sg = blockIdx.x / a.ktiles;
  if (!a.tsplit[(size_t)sg * a.ktiles + tile]) return;
  const int S = a.S;
  const size_t kvbase = (size_t)sg * S * D;
  const float* src = a.part1 + ((size_t)sg * a.ktiles + tile) * kKTile * 2 * D;
  constexpr int PPK = 2 * D / 4;          // float4 pieces per key (dK then dV)
  constexpr int KPI = 256 / PPK;          // keys per pass of the workgroup
  constexpr int NIT = kKTile / KPI;       // passes
  constexpr int kU = 8;                   // passes in flight: their key, part and row reads issued together
  static_assert(NIT % kU == 0, "merge passes");
  const int pc = threadIdx.x % PPK, j0 = threadIdx.x / PPK;
  const size_t col = 4 * (pc % (D / 4));
  float* base = pc < D / 4 ? a.dk : a.dv;
  for (int i0 = 0; i0 < NIT; i0 += kU) {
    int t[kU];
    float4 x[kU], y[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + KPI * (i0 + u);
      const int slot = tile * kKTile + j;
      t[u] = slot < S ? a.korder[(size_t)sg * S + slot] : -1;
      x[u] = *(const float4*)(src + (size_t)j * 2 * D + 4 * pc);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      y[u] = t[u] >= 0 ? *(const float4*)(base + kvbase + (size_t)t[u] * D + col)
                       : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (t[u] < 0) continue;
      y[u].x += x[u].x; y[u].y += x[u].y; y[u].z += x[u].z; y[u].w += x[u].w;
      *(float4*)(base + kvbase + (size_t)t[u] * D + col) = y[u];
    }
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(kKThreads) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NKS = D / 16;
  constexpr int NB = D / 32;                         // 32-dim output blocks
  constexpr int PPR = D / 8;                         // 16-byte pieces per row
  constexpr int RB = D * 2;                          // bytes per row
  constexpr int CB = kRChunk * RB;                   // bytes of one tensor's chunk
  constexpr int RPI = 1024 / RB;                     // rows per 1 KB direct load
  constexpr int NW = kKThreads / 64;                 // waves
  constexpr int NBLK = kRChunk / RPI;                // 1 KB blocks per tensor and item
  constexpr int LPW = 2 * NBLK / NW;                 // row loads per wave and item
  constexpr int NLD = LPW + 1;                       // direct loads per wave and item
  static_assert(LPW >= 1 && LPW * NW == 2 * NBLK, "direct-load tiling");
  static_assert(kRChunk == 32, "row values: 64 floats per item");
  // Six stages of one item each: the rows' LSE log2 e and D (64 floats),
  // then the Q rows, then the dO rows (row-major, swizzled like the dQ
  // kernel's K: read as rows for S and dP and transposed for dK and dV).
  // Stage offsets are multiples of 256 bytes, so adding one to a lane's
  // in-stage offset commutes with the XORs of the swizzle (bits 4..7).
  // Then the exchange of P from the S waves to the dP waves: per step
  // parity, per key group, 16 floats per lane in the MFMA result layout.
  constexpr int NST = 6;
  constexpr int RV = 2 * kRChunk * 4;                // bytes of row values
  constexpr int SB = RV + 2 * CB;                    // bytes per stage
  static_assert(SB % 256 == 0, "stage alignment");
  constexpr int XB = kKGroups * 16 * 64 * 4;         // bytes of one exchange buffer
  __shared__ __attribute__((aligned(256))) unsigned char kvst[NST * SB + 2 * XB];
  unsigned char* const xbuf = kvst + NST * SB;

  const int lane = lane_id(), wave = wave_id();
  const int hh = lane >> 5, li = lane & 31;
  // Two roles per key group, one wave each (waves g and g + 4 share a SIMD):
  // role 0 computes S, P and dV, role 1 dP, dS and dK.  The roles split the
  // work of a group without repeating any of it, and each holds half the
  // operands and accumulators, so two waves fit on every SIMD and the MFMA
  // stream of one overlaps the exp and select math of the other.
  const int grp = wave & 3, role = wave >> 2;
  // the items of one (sequence, KV head) go to one XCD, longest first, so
  // the workgroups sharing an L2 read overlapping rows
  const int Lb = xcd_logical_block(launch_block(a.reverse), (int)gridDim.x);
  const int n_ent = 2 * a.ktiles;
  const int sg = Lb / n_ent;
  const int4 item = a.tplan[(size_t)sg * n_ent + Lb % n_ent];
  if (item.y < 0) return;            // the empty slot of an unsplit tile (uniform)
  const int tile = item.x, part = item.y;
  const int h = sg % a.Hkv, b = sg / a.Hkv;
  const int S = a.S, G = a.G;
  const size_t seg = (size_t)b * a.Hkv + h;

  // this lane's key
  const int slot = tile * kKTile + 32 * grp + li;
  const int t = slot < S ? a.korder[seg * S + slot] : -1;
  const int qe = t >= 0 ? a.qend[seg * S + t] : -1;
  // The rows that keep key t are exactly [t, q_end(t)]: tau never increases
  // with q, so once a key leaves the kept set it never returns (sinks and
  // keys whose window reaches the end have q_end = S - 1).  A row q keeps it
  // iff 0 <= q - t <= q_end(t) - t: one unsigned compare, the same decision as
  // the mask test from rank and tau.  Rows past S - 1 exceed q_end; a padding
  // slot takes t = S + 32, above every row a chunk holds (q - t wraps to a
  // large unsigned value), with span 0.
  const unsigned span = t >= 0 ? (unsigned)(qe - t) : 0u;
  const int t_m = t >= 0 ? t : S + kRChunk;
  const size_t kvbase = seg * (size_t)S * D;

  // B operand of the role's S or dP product: K^T (role 0) or V^T (role 1)
  // of this lane's key, dims [16 ks + 8 hh, +8) (loaded unconditionally from
  // a clamped row, then zeroed for padding, and completed here: loads still
  // pending at the loop would make the compiler wait for the loop's own
  // prefetch before the first MFMA of every chunk)
  bf16x8 bop[NKS];
  {
    const uint16_t* src = (role ? a.v : a.k) + kvbase + (size_t)(t >= 0 ? t : 0) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4v u = *(const u32x4v*)(src + 16 * ks + 8 * hh);
      if (t < 0) u = u32x4v{0, 0, 0, 0};
      bop[ks] = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(bop[ks]));
  }
  // work items: (query head, 32-row chunk) pairs over the item's chunks,
  // aligned to 32 rows (the plan's [min t, max q_end] of the tile, or one
  // part of it)
  const int c_first = item.z;
  const int n_chunk = item.w - item.z;
  const int n_items = G * n_chunk;

  // items in order: query head gg, then chunk ci; the (gg, ci) of an item are
  // stepped rather than divided out of its index
  struct ItemPos {
    int gg, ci;
  };
  auto next_pos = [&](ItemPos p) {
    return p.ci + 1 < n_chunk ? ItemPos{p.gg, p.ci + 1} : ItemPos{p.gg + 1, 0};
  };
  // positions past the last item (query head G and beyond) load the last
  // head's rows instead; those items are masked or never used
  auto clamp_pos = [&](ItemPos p) { return ItemPos{min(p.gg, G - 1), p.ci}; };
  // ---- staging of one item into the stage at byte offset so, all by
  // direct loads (lane L of a load writes 16 L, or 4 L, bytes past the
  // load's LDS base): the Q and dO rows (1 KB blocks spread over the waves),
  // lane L fetching the global piece its swizzled slot holds, and the rows'
  // LSE log2 e (lanes 0..31) and D (lanes 32..63), loaded by every wave (the
  // same bytes; no branch).  Rows past the end read row S - 1 and are
  // masked.  Each wave issues NLD loads.
  auto dma_item = [&](ItemPos ip, int so) {
    const size_t hrow = ((size_t)b * a.Hq + h * G + ip.gg) * S;
    const int c0 = (c_first + ip.ci) * kRChunk;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int L = wave * LPW + i;
      const int tensor = L / NBLK, r0 = (L % NBLK) * RPI;   // tensor: wave-uniform
      const int row = r0 + lane / PPR, sl = lane % PPR;
      const int qq = min(c0 + row, S - 1);
      const uint32_t off = (uint32_t)qq * RB + ((sl ^ dq_swz<D>(row)) << 4);
      const unsigned char* base = (const unsigned char*)(tensor ? a.dout : a.q) + hrow * RB;
      dma_lds_x4_so(base, off, kvst + so + RV + tensor * CB + r0 * RB);
    }
    const int qq = min(c0 + li, S - 1);
    dma_lds_x1((hh ? a.dvec : a.lse2) + hrow + qq, kvst + so);
  };

  // per-lane in-stage LDS offsets: row reads (row li, piece 2 ks + hh: base
  // XOR 32 ks) and the transposed reads
  int tro[NB][2];
  dq_tr_offsets<D>(lane, tro);
  const int row_base = li * RB + ((hh ^ dq_swz<D>(li)) << 4);
  typedef __attribute__((address_space(3))) short4v lds_s4;

  // ---- the pipeline.  Item i lives in stage i mod 6; every wave loads
  // its share of item it+3 in iteration it, waits for its loads of item
  // it+2 at the end and meets the others at a barrier.  Iteration it:
  //   role 0: S of item it+1; dV^T += dO^T P of item it-1 (P packed in the
  //           previous iteration); P of item it from its S (computed in the
  //           previous iteration): exp, then the interval select, written to
  //           the exchange buffer and packed.
  //   role 1: dP of item it; dK^T += Q^T dS of item it-2 (dS packed in the
  //           previous iteration); dS of item it-1 = P (from the exchange
  //           buffer, written by role 0 in the previous iteration) times
  //           (dP - D), packed.
  // Each role's MFMAs read their operands kPf MFMAs ahead, with the math
  // between them.  The count is padded to even with masked items and runs
  // two iterations past the last so that role 1 finishes; stages and
  // exchange buffers that those and the first iterations read before any
  // item reaches them are zeroed (zero P or dS times stale data could be
  // NaN).
  constexpr int kPf = 4;                             // operand reads ahead of their MFMA
  const int n_pad = (n_items + 1) & ~1;
  const int n_loop = n_pad > 0 ? n_pad + 2 : 0;
  auto stage_of = [&](int i) { return (i % NST) * SB; };
  auto mask_c0 = [&](int i, ItemPos p) {   // first row of item i, or far away when padding
    return i < n_items ? (c_first + p.ci) * kRChunk : -(1 << 30);
  };
  // operand ks of the S (role 0, Q rows) or dP (role 1, dO rows) product of
  // the item whose row-read base (row_base plus its stage offset) is rb
  auto row_operand = [&](int rb, int ks) {
    const unsigned char* p = kvst + (rb ^ (32 * ks)) + (role ? CB : 0);
    return as_bf16x8(*(const uint4*)p);
  };

  ItemPos cur{0, 0}, nx1{0, 0}, nx2{0, 0}, nx3{0, 0};   // items it .. it+3
  if (n_items > 0) {
    dma_item(cur, stage_of(0));
    nx1 = next_pos(cur);
    dma_item(clamp_pos(nx1), stage_of(1));
    nx2 = next_pos(nx1);
    dma_item(clamp_pos(nx2), stage_of(2));
    nx3 = next_pos(nx2);
    // stages 4 and 5 (read as items -2 and -1) and both exchange buffers
    uint4* z = (uint4*)(kvst + stage_of(4));
    for (int i = threadIdx.x; i < (2 * SB + 2 * XB) / 16; i += kKThreads) {
      uint4* zp = i < 2 * SB / 16 ? z + i : (uint4*)xbuf + (i - 2 * SB / 16);
      *zp = make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | NLD);   // items 0 and 1 landed
    lds_barrier();
  }

  f32x16 acc[NB];                    // dV (role 0) or dK (role 1)
#pragma unroll
  for (int d2 = 0; d2 < NB; ++d2) acc[d2] = f32x16{};

  // one role's loop; X: S (role 0) or dP (role 1) of items with even / odd
  // index, pk: packed P (role 0) or dS (role 1) likewise
  auto run = [&](auto role_c) {
    constexpr int R = decltype(role_c)::value;
    f32x16 XA = f32x16{}, XB_ = f32x16{};
    bf16x8 pkA[2] = {}, pkB[2] = {};
    if constexpr (R == 0) {
      if (n_items > 0) {   // S of item 0
        const int rb = row_base + stage_of(0) + RV;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) XA = mfma32x32x16(row_operand(rb, ks), bop[ks], XA);
      }
    }
    // iteration it: Xp / Xn: X of the item this role reads / writes in it
    // (role 0: S of it / it+1; role 1: dP of it-1 / it), pk_use: packed P or
    // dS consumed (role 0: item it-1; role 1: it-2), pk_new: produced
    // (role 0: item it; role 1: it-1)
    auto step = [&](int it, f32x16& Xp, f32x16& Xn, const bf16x8 (&pk_use)[2],
                    bf16x8 (&pk_new)[2]) {
      constexpr int NMF = NKS + 2 * NB;              // MFMAs of the role per iteration
      constexpr int EPS = (16 + NMF - 1) / NMF;      // scores per MFMA slot
      const int c0 = mask_c0(it, cur);
      dma_item(clamp_pos(nx3), stage_of(it + 3));
      __builtin_amdgcn_sched_barrier(0);
      // row reads: S of it+1 (role 0) or dP of it (role 1)
      int rb = row_base + stage_of(R == 0 ? it + 1 : it) + RV;
      asm volatile("" : "+v"(rb));
      // transposed reads: dO^T of item it-1 (role 0) or Q^T of item it-2
      // (role 1); opaque per-lane bases, constant parts in the offset field
      int trb[NB][2];
#pragma unroll
      for (int d2 = 0; d2 < NB; ++d2)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          trb[d2][x] = tro[d2][x] + stage_of(it + NST - (R == 0 ? 1 : 2)) + RV + (R == 0 ? CB : 0);
          asm volatile("" : "+v"(trb[d2][x]));
        }
      auto tr_operand = [&](int m) {   // block m / 2, k-step m mod 2
        const int d2 = m >> 1, ks = m & 1;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(kvst + trb[d2][0] + 16 * ks * RB));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(kvst + trb[d2][1] + 16 * ks * RB));
        const short8v v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v8);
      };
      auto operand = [&](int q) { return q < NKS ? row_operand(rb, q) : tr_operand(q - NKS); };
      // the math's inputs: role 0 the LSE of item it; role 1 D of item it-1
      // and P of item it-1 from the exchange buffer
      const float* rvals = (const float*)(kvst + stage_of(R == 0 ? it : it + NST - 1));
      float4* xb = (float4*)(xbuf + ((R == 0 ? it : it + 1) & 1) * XB) + grp * 4 * 64 + lane;
      f32x4 rv4[4];
      float4 px[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rv4[j] = *(const f32x4*)(rvals + (R == 0 ? 0 : kRChunk) + 8 * j + 4 * hh);
        if constexpr (R == 1) px[j] = xb[64 * j];
      }
      bf16x8 op[NMF];
#pragma unroll
      for (int q = 0; q < kPf; ++q) op[q] = operand(q);
      __builtin_amdgcn_sched_barrier(0);
      Xn = f32x16{};
      float pv[16];
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        if (q + kPf < NMF) op[q + kPf] = operand(q + kPf);
        if (q < NKS) {
          Xn = mfma32x32x16(op[q], bop[q], Xn);
        } else {
          const int m = q - NKS;
          acc[m >> 1] = mfma32x32x16(op[q], pk_use[m & 1], acc[m >> 1]);
        }
#pragma unroll
        for (int e = q * EPS; e < (q + 1) * EPS && e < 16; ++e) {
          const int j = e >> 2, r = e & 3;
          if constexpr (R == 0) {
            // P: the exp of every score, then a select (a masked score's
            // exp may overflow; it is never used)
            const bool kp = (unsigned)(c0 + 8 * j + 4 * hh + r - t_m) <= span;
            const float ex = exp2_fast(fmaf(Xp[e], a.scale_log2, -rv4[j][r]));
            pv[e] = kp ? ex : 0.0f;
          } else {
            const float p = r == 0 ? px[j].x : r == 1 ? px[j].y : r == 2 ? px[j].z : px[j].w;
            pv[e] = p * (Xp[e] - rv4[j][r]);   // dS
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (R == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xb[64 * j] = make_float4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pk_new[ks] = pack_bf16x8(&pv[8 * ks]);
      // the packed values complete in this iteration (left alone, the
      // compiler moves that math next to its use in the next one)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) asm volatile("" ::"v"(pk_new[ks]));
      __builtin_amdgcn_s_waitcnt(0x0F70 | NLD);   // item it+2 landed
      cur = nx1;
      nx1 = nx2;
      nx2 = nx3;
      nx3 = next_pos(nx3);
      lds_barrier();
    };
    for (int it = 0; it < n_loop; it += 2) {
      if constexpr (R == 0) {
        step(it, XA, XB_, pkB, pkA);         // S of it (even) / it+1; P of it-1 / it
        step(it + 1, XB_, XA, pkA, pkB);
      } else {
        step(it, XB_, XA, pkA, pkB);         // dP of it-1 (odd) / it; dS of it-2 / it-1
        step(it + 1, XA, XB_, pkB, pkA);
      }
    }
  };
  if (role == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
  if (n_items > 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // the loads past the end

  if (t >= 0) {
    // the first (or only) part writes dk (role 1) or dv (role 0); the second
    // part of a split tile writes its sums beside them for the merge
    float* p1 = a.part1 + (((size_t)sg * a.ktiles + tile) * kKTile + 32 * grp + li) * 2 * D;
    float* out = part ? p1 + (role ? 0 : D) : (role ? a.dk : a.dv) + kvbase + (size_t)t * D;
    const float sc = role ? a.scale : 1.0f;
#pragma unroll
    for (int d2 = 0; d2 < NB; ++d2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * d2 + 8 * j + 4 * hh;
        *(float4*)(out + d) = make_float4(acc[d2][4 * j] * sc, acc[d2][4 * j + 1] * sc,
                                          acc[d2][4 * j + 2] * sc, acc[d2][4 * j + 3] * sc);
      }
  }
}

template <int D>
void launch_dot_dq(const Dims& d, BwdArgs a, const void* o, hipStream_t st, hipEvent_t dot_done) {
  const long long rows = (long long)d.b * d.Hq * d.S;
  constexpr int RPB = 4 * (64 / (D / 8));     // rows per 256-thread block
  const unsigned nblk = (unsigned)((rows + RPB - 1) / RPB);
  if (d.f32_out)
    hipLaunchKernelGGL((bwd_dot_kernel<D, true>), dim3(nblk), dim3(256), 0, st, a.dout, o, a.lse,
                       (float*)a.dvec, (float*)a.lse2, rows);
  else
    hipLaunchKernelGGL((bwd_dot_kernel<D, false>), dim3(nblk), dim3(256), 0, st, a.dout, o, a.lse,
                       (float*)a.dvec, (float*)a.lse2, rows);
  if (dot_done) (void)hipEventRecord(dot_done, st);   // a failure shows in hipGetLastError
  const long long nq = (long long)a.ntiles * d.Hkv * d.b;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)nq), dim3(kQThreads), 0, st, a);
}

template <int D>
void launch_dkdv(const Dims& d, BwdArgs a, hipStream_t st) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)(2 * a.ktiles * d.nseg())),
                     dim3(kKThreads), 0, st, a);
  hipLaunchKernelGGL((bwd_dkdv_merge_kernel<D>), dim3((unsigned)(a.ktiles * d.nseg())), dim3(256), 0,
                     st, a);
}

// A second stream per device for the key-major half of the backward (key
// order, tile plan, dK/dV, merge), which needs only q_end and D_i: it runs
// beside the dot product and dQ, forked from the caller's stream after the
// forward plan and joined back before the call returns, through events.
// Created on the first backward on a device (default priority); a device
// where that fails runs everything on the caller's stream (so does a first
// call made while the caller's stream is being captured).  The lock makes
// concurrent callers enqueue one at a time (each wait refers to the event's
// record made just before it, so the events can be reused at once).
constexpr int kMaxBwdDevices = 64;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, dot_done = nullptr, join = nullptr;
  int state = 0;   // 0: not tried, 1: ready, -1: unavailable
};
SideStream g_side[kMaxBwdDevices];
std::mutex g_side_mu;

SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxBwdDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.state == 0) {
    // no creation while the caller's stream is being captured into a graph
    // (it would end the capture); such a call runs on the caller's stream
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
      (void)hipGetLastError();
      return nullptr;
    }
    bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ss.dot_done, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
    ss.state = ok ? 1 : -1;
    if (!ok) (void)hipGetLastError();   // leave no error behind for the launches
  }
  return ss.state == 1 ? &ss : nullptr;
}

}  // namespace

static int bwd_ktiles(const Dims& d) { return (d.S + kKTile - 1) / kKTile; }

size_t bwd_ws_bytes(const Dims& d) {
  const size_t rows = (size_t)d.b * d.Hq * d.S, keys = (size_t)d.nseg() * d.S;
  const size_t nt = (size_t)d.nseg() * bwd_ktiles(d);
  return fwd_ws_bytes(d) + 2 * align256(rows * 4) + align256(keys * 4) +
         2 * align256(nt * 2 * 16) +                  // item plan and its unsorted copy
         align256(nt * 4) +                           // split flags
         align256(nt * kKTile * 2 * (size_t)d.D * 4);  // second-half sums of split tiles
}

hipError_t launch_masked_bwd(const Dims& d, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const int* rank, const int* tau,
                             const void* dout, float* dq, float* dk, float* dv, void* ws,
                             hipStream_t st) {
  const FwdPlan pl = launch_fwd_plan(d, rank, tau, ws, st);
  char* p = (char*)ws + fwd_ws_bytes(d);
  const size_t rows = (size_t)d.b * d.Hq * d.S, keys = (size_t)d.nseg() * d.S;
  float* dvec = (float*)p; p += align256(rows * 4);
  float* lse2 = (float*)p; p += align256(rows * 4);
  int* korder = (int*)p; p += align256(keys * 4);
  const int ktiles = bwd_ktiles(d);
  const size_t nt = (size_t)d.nseg() * ktiles;
  int4* tplan = (int4*)p; p += align256(nt * 2 * 16);
  int4* tplan_tmp = (int4*)p; p += align256(nt * 2 * 16);
  int* tsplit = (int*)p; p += align256(nt * 4);
  float* part1 = (float*)p;
  const int* qend = pl.qend;   // q_end(t), computed by the forward plan

  BwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout; a.lse = lse; a.dvec = dvec; a.lse2 = lse2;
  a.rank = rank; a.tau = tau;
  a.qend = qend; a.korder = korder; a.list = pl.list; a.count = pl.count;
  a.tplan = tplan; a.tsplit = tsplit; a.part1 = part1;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.S = d.S; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.m = pl.m; a.ntiles = pl.ntiles;
  a.ktiles = ktiles;
  a.s = d.s; a.w = d.w; a.cap = pl.cap;
  a.reverse = launch_order_reversed();
  a.scale = d.scale;
  a.scale_log2 = d.scale * 1.4426950408889634f;

  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream* ss = side_stream(st);
  hipStream_t ks = st;   // stream of the key-major half
  if (ss) {
    hipError_t e = hipEventRecord(ss->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return e;
    ks = ss->s;
  }
  const int nb = KeyBuckets(d.S).nb;
  hipLaunchKernelGGL(bwd_key_order_kernel, dim3(d.nseg()), dim3(1024), (size_t)nb * 2 * 4, ks, qend,
                     korder, d.S, d.w);
  const int nbins = plan_bins(d.S);
  hipLaunchKernelGGL(bwd_tile_plan_kernel, dim3(d.nseg()), dim3(1024), (size_t)nbins * 2 * 4, ks,
                     korder, qend, d.S, ktiles, tplan_tmp, tplan, tsplit);
  if (d.D == 128) launch_dot_dq<128>(d, a, o, st, ss ? ss->dot_done : nullptr);
  else launch_dot_dq<64>(d, a, o, st, ss ? ss->dot_done : nullptr);
  if (ss) {
    const hipError_t e = hipStreamWaitEvent(ks, ss->dot_done, 0);
    if (e != hipSuccess) return e;
  }
  if (d.D == 128) launch_dkdv<128>(d, a, ks);
  else launch_dkdv<64>(d, a, ks);
  if (ss) {
    hipError_t e = hipEventRecord(ss->join, ks);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->join, 0);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace kvpop
