// kvpop_future_target: the training-only transposed-attention pass.
//
// KVpop reading notes §2.2 define the future attention mass of key t as the
// sum over future queries d >= t + w of the dense causal probabilities
// A[d,t]; §2.3 Eq. (8) rewrites its log as
//   log sum_{d=t+w}^{S-1} exp(l(d,t) - LSE_d) - log N_t,
// and Figure 2 computes the first term with an attention pass whose queries
// are the keys and whose keys are the queries, with the original query's LSE
// subtracted and d >= t + w masked.  This kernel returns that first term per
// query head (the aggregation over the query group, epsilon and N_t are left
// to the caller).
//
// Design (gfx950):
//  * A workgroup owns 256 key rows t of one query head: each of its 4 waves
//    keeps two 32-row blocks of K as MFMA B operands in registers, so every
//    Q operand read from LDS feeds two v_mfma_f32_32x32x16_bf16.
//  * The future queries d stream through LDS in 64-row chunks shared by the 4
//    waves, double-buffered: the global loads of chunk c+1 are issued before
//    the math of chunk c and stored to the other buffer after it, so one
//    barrier per chunk suffices and the load latency hides behind the MFMAs.
//    Their LSE biases take three slots, since the exps of a chunk's last
//    column block run in the next iteration.
//  * X^T = Q K^T leaves every lane owning one row t; each score becomes
//    exp2(x * scale log2 e - LSE_d log2 e) and is summed directly: with the
//    dense LSE every exponent is <= 0, so no running maximum is needed.
//  * Any other LSE (the sparse operator's, which can lie below a dropped
//    key's logit) may push a term past float32's range.  Such a sum cannot
//    overflow unnoticed: a row whose max-free total leaves [2^-100, 2^100]
//    makes its workgroup recompute the tile with a running maximum per row
//    (rescaling its sum whenever the maximum grows), which is exact for any
//    finite LSE.  With the dense LSE every total lies in that range (it is a
//    sum of at most S probabilities, each <= 1, of which the largest is not
//    tiny unless the target is below -69), so the dense path pays one flag
//    and one barrier.
//  * Chunks wholly below a wave's first row + w are skipped; the d >= t + w
//    test (a select) runs only on chunks that straddle the band.
//  * Blocks are renumbered so that each XCD (its own L2) works through whole
//    heads: consecutive logical blocks are consecutive key tiles of one head,
//    which read the same Q stream.
#include <type_traits>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kRB = 2;                           // 32-row MFMA blocks per wave
constexpr int kWaveRows = 32 * kRB;
constexpr int kRowsPerTile = 4 * kWaveRows;
constexpr int kChunk = 64;

struct TgtArgs {
  const void* q;
  const void* k;
  const float* lse;
  float* target;
  int S, Hq, Hkv, G, w, ntiles;
  int reverse;         // launch order reversed (testing aid)
  float scale_log2;
};

template <int D, bool kF32>
struct TgtGeom {
  static constexpr int esz = kF32 ? 4 : 2;
  static constexpr int QS = kF32 ? D + 1 : D + 8;           // LDS row stride (elements)
  static constexpr int bufBytes = ((kChunk * QS * esz + 15) / 16) * 16;
  static constexpr int PPR = D * esz / 16;                   // 16-byte pieces per Q row
  static constexpr int NPIECE = kChunk * PPR / kThreads;     // pieces per thread per chunk
  static constexpr int NKS = kF32 ? D / 2 : D / 16;          // MFMA k-steps
};

// The exact pass for an arbitrary (finite) LSE: the tile's future queries
// stream through LDS one 64-row chunk at a time; each lane keeps, for each of
// its rows, a running maximum m of the exponents (log2 units) and the sum of
// exp2(e - m), rescaled whenever m grows; the two lanes of a row merge theirs
// at the end.  Slow next to the max-free pipeline, and only run for tiles
// whose max-free sums left float32's range.  Writes the tile's targets.
template <int D, bool kF32In, typename KOp>
__device__ __forceinline__ void rescaled_pass(
    const TgtArgs& a, const KOp (&kop)[kRB][TgtGeom<D, kF32In>::NKS],
    unsigned char (&q_lds)[2][TgtGeom<D, kF32In>::bufBytes], float (&nlse)[3][kChunk], int rbase,
    int t0, int b, int hq) {
  using Gm = TgtGeom<D, kF32In>;
  const int tid = threadIdx.x, lane = lane_id();
  const int hh = lane >> 5, li = lane & 31;
  const int S = a.S, w = a.w;
  const int d_start = t0 + w;
  const unsigned char* qg = (const unsigned char*)a.q + ((size_t)b * a.Hq + hq) * S * D * Gm::esz;
  const float* lse = a.lse + ((size_t)b * a.Hq + hq) * S;
  float m[kRB], l[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.0f;
  }
  for (int d0 = d_start; d0 < S; d0 += kChunk) {
    __syncthreads();   // every wave is done with the previous chunk
    for (int p = tid; p < kChunk * Gm::PPR; p += kThreads) {
      const int row = p / Gm::PPR, piece = p % Gm::PPR;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (d0 + row < S) u = *(const uint4*)(qg + ((size_t)(d0 + row) * D) * Gm::esz + piece * 16);
      if constexpr (kF32In) {
        float* dst = (float*)q_lds[0] + row * Gm::QS + piece * 4;
        dst[0] = __uint_as_float(u.x);
        dst[1] = __uint_as_float(u.y);
        dst[2] = __uint_as_float(u.z);
        dst[3] = __uint_as_float(u.w);
      } else {
        *(uint4*)((uint16_t*)q_lds[0] + row * Gm::QS + piece * 8) = u;
      }
    }
    if (tid < kChunk) nlse[0][tid] = d0 + tid < S ? -lse[d0 + tid] * kLog2e : kNegInf;
    __syncthreads();
    if (d0 + kChunk - 1 < rbase + w) continue;   // every row of this wave starts later
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x16 acc[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) acc[rb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < Gm::NKS; ++ks) {
        if constexpr (kF32In) {
          const float av = ((const float*)q_lds[0])[(32 * cb + li) * Gm::QS + hh + 2 * ks];
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb] = mfma32x32x2(av, kop[rb][ks], acc[rb]);
        } else {
          const bf16x8 av = as_bf16x8(
              *(const uint4*)((const uint16_t*)q_lds[0] + (32 * cb + li) * Gm::QS + 8 * hh + 16 * ks));
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) acc[rb] = mfma32x32x16(av, kop[rb][ks], acc[rb]);
        }
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int t = rbase + 32 * rb + li;
        // exponent of element i in log2 units, -inf outside d >= t + w, d < S
        // (evaluated twice, for the block maximum and for the sum, rather
        // than held: this pass is rare and registers are not)
        auto expo = [&](int i) {
          const int dl = 32 * cb + 8 * (i >> 2) + 4 * hh + (i & 3);
          const int d = d0 + dl;
          const float x = fmaf(acc[rb][i], a.scale_log2, nlse[0][dl]);
          return (d >= t + w && d < S) ? x : kNegInf;
        };
        float bm = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) bm = fmaxf(bm, expo(i));
        if (bm == kNegInf) continue;   // nothing of this block in the row's range
        if (bm > m[rb]) {
          l[rb] *= exp2_fast(m[rb] - bm);   // m = -inf: l is 0 and stays 0
          m[rb] = bm;
        }
        float acc_l = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_l += exp2_fast(expo(i) - m[rb]);
        l[rb] += acc_l;
      }
    }
  }
  float* out = a.target + ((size_t)b * a.Hq + hq) * S;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float mm = halves_max(m[rb]);
    const float part = mm == kNegInf ? 0.0f : l[rb] * exp2_fast(m[rb] - mm);
    const float ll = halves_sum(part);
    const int t = rbase + 32 * rb + li;
    if (hh == 0 && t < S) out[t] = ll > 0.0f ? (mm + log2f(ll)) * kLn2 : kNegInf;
  }
}

template <int D, bool kF32In>
__global__ __launch_bounds__(kThreads, 2) void future_target_kernel(TgtArgs a) {
  using Gm = TgtGeom<D, kF32In>;
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[2][Gm::bufBytes];
  // -LSE_d * log2(e) of a chunk's queries, in three slots: a wave still
  // reading the previous chunk's biases (the exps of its last block run in
  // the next iteration) must not see them overwritten by the store of the
  // chunk after next, which other waves may reach first
  __shared__ __attribute__((aligned(16))) float nlse[3][kChunk];
  __shared__ int redo;   // some row of the tile needs the running-maximum pass

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int hh = lane >> 5, li = lane & 31;
  const int L = xcd_logical_block(launch_block(a.reverse), (int)gridDim.x);
  const int tile = L % a.ntiles;
  const int hq = (L / a.ntiles) % a.Hq;
  const int b = L / (a.ntiles * a.Hq);
  const int S = a.S, w = a.w;
  const int h = hq / a.G;
  const int t0 = tile * kRowsPerTile;
  const int rbase = t0 + wave * kWaveRows;        // this wave's first key row
  float* out = a.target + ((size_t)b * a.Hq + hq) * S;

  const int d_start = t0 + w;                      // first query any row of the tile needs
  if (d_start > S - 1) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int t = rbase + 32 * rb + li;
      if (hh == 0 && t < S) out[t] = kNegInf;
    }
    return;
  }

  // key operands (B of X^T = Q K^T): rows rbase + 32 rb + li, dims [16ks + 8hh, +8)
  typedef typename std::conditional<kF32In, float, bf16x8>::type KOp;
  KOp kop[kRB][Gm::NKS];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int t = rbase + 32 * rb + li;
    const bool ok = t < S;
    const size_t krow = (((size_t)b * a.Hkv + h) * S + (ok ? t : 0)) * D;
    if constexpr (kF32In) {
      const float* kp = (const float*)a.k + krow;
#pragma unroll
      for (int ks = 0; ks < Gm::NKS; ++ks) kop[rb][ks] = ok ? kp[2 * ks + hh] : 0.0f;
    } else {
      const uint16_t* kp = (const uint16_t*)a.k + krow;
#pragma unroll
      for (int ks = 0; ks < Gm::NKS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (ok) u = *(const uint4*)(kp + 16 * ks + 8 * hh);
        kop[rb][ks] = as_bf16x8(u);
      }
    }
  }

  // complete the key loads here: loads still in flight at the loop entry make
  // the compiler wait for every newer load before the loop's first MFMA
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < Gm::NKS; ++ks) asm volatile("" : "+v"(kop[rb][ks]));

  const unsigned char* qg = (const unsigned char*)a.q + ((size_t)b * a.Hq + hq) * S * D * Gm::esz;
  const float* lse = a.lse + ((size_t)b * a.Hq + hq) * S;

  // staging of one chunk: global -> registers, registers -> LDS buffer
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v stage[Gm::NPIECE];
  float stage_lse = 0.0f;
  auto load_chunk = [&](int d0) {
    // a buffer descriptor over rows d0 .. S-1: each lane's offset is the same
    // for every chunk and rows past the end read as zeros (their -LSE is
    // -inf, so they add 0), with no per-chunk address arithmetic
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qg + (size_t)d0 * D * Gm::esz), (short)0, (S - d0) * D * Gm::esz, 0x00020000);
#pragma unroll
    for (int i = 0; i < Gm::NPIECE; ++i) {
      const int p = tid + i * kThreads;
      const int row = p / Gm::PPR, piece = p % Gm::PPR;
      stage[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * D * Gm::esz + piece * 16, 0, 0);
    }
    // the raw value only: arithmetic on it here would wait for all the loads
    // above; it is scaled when stored
    if (tid < kChunk) stage_lse = lse[min(d0 + tid, S - 1)];
  };
  auto store_chunk = [&](int buf, int nsl, int d0) {
#pragma unroll
    for (int i = 0; i < Gm::NPIECE; ++i) {
      const int p = tid + i * kThreads;
      const int row = p / Gm::PPR, piece = p % Gm::PPR;
      if constexpr (kF32In) {
        float* dst = (float*)q_lds[buf] + row * Gm::QS + piece * 4;
        dst[0] = __uint_as_float(stage[i][0]);
        dst[1] = __uint_as_float(stage[i][1]);
        dst[2] = __uint_as_float(stage[i][2]);
        dst[3] = __uint_as_float(stage[i][3]);
      } else {
        *(u32x4v*)((uint16_t*)q_lds[buf] + row * Gm::QS + piece * 8) = stage[i];
      }
    }
    if (tid < kChunk) nlse[nsl][tid] = d0 + tid < S ? -stage_lse * kLog2e : kNegInf;
  };

  // four partial sums per row block (by column mod 4), so consecutive adds
  // of a group do not wait on each other
  float sum[kRB][4];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[rb][r] = 0.0f;
  const int nchunks = (S - d_start + kChunk - 1) / kChunk;
  if (tid == 0) redo = 0;
  load_chunk(d_start);
  store_chunk(0, 0, d_start);
  __syncthreads();

  // One 32-column block of MFMAs: acc[rb] = Q_block K_rb^T.
  auto mfma_block = [&](f32x16 (&acc)[kRB], int buf, int cb) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) acc[rb] = f32x16{};
    if constexpr (!kF32In) {
      const uint16_t* ql = (const uint16_t*)q_lds[buf] + (32 * cb + li) * Gm::QS + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < Gm::NKS; ++ks) {
        const bf16x8 av = as_bf16x8(*(const uint4*)(ql + 16 * ks));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[rb] = mfma32x32x16(av, kop[rb][ks], acc[rb]);
      }
    } else {
      const float* ql = (const float*)q_lds[buf] + (32 * cb + li) * Gm::QS + hh;
#pragma unroll
      for (int ks = 0; ks < Gm::NKS; ++ks) {
        const float av = ql[2 * ks];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[rb] = mfma32x32x2(av, kop[rb][ks], acc[rb]);
      }
    }
  };
  // exp2 and row sums of one block: the lane holds columns
  // d = d0 + 32cb + 8j + 4hh + r of rows rbase + 32rb + li
  auto exp_block = [&](const f32x16 (&acc)[kRB], int slot, int cb, int d0, auto masked) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dl = 32 * cb + 8 * j + 4 * hh;
      const f32x4 bias = *(const f32x4*)(&nlse[slot][dl]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          float p = exp2_fast(fmaf(acc[rb][4 * j + r], a.scale_log2, bias[r]));
          if constexpr (decltype(masked)::value) {   // selects, no branches
            const int d = d0 + dl + r;
            p = ((d >= rbase + 32 * rb + li + w) & (d < S)) ? p : 0.0f;
          }
          sum[rb][r] += p;
        }
    }
  };
  // The MFMAs of one block interleaved with the exp work of another
  // (independent) block, in a fixed order so the matrix and vector units run
  // together: the first operand reads and the block's biases first, then 8
  // groups of two MFMAs and four scores (fma, exp2, add) each, pinned with
  // scheduling barriers.
  auto fused = [&](auto doM, auto doE, auto maskE, f32x16 (&accM)[kRB], int mbuf, int mcb,
                   const f32x16 (&accE)[kRB], int eslot, int ecb, int d0E) {
    constexpr bool kM = decltype(doM)::value, kE = decltype(doE)::value;
    constexpr bool kMask = decltype(maskE)::value;
    constexpr int NK = Gm::NKS;              // 8 (D = 128, bf16)
    constexpr int kPer = 32 / NK;            // scores per group: 4, all with one bias vector
    const uint16_t* ql = (const uint16_t*)q_lds[mbuf] + (32 * mcb + li) * Gm::QS + 8 * hh;
    const float* nb = &nlse[eslot][32 * ecb + 4 * hh];
    // operands two k-steps ahead; the block's biases (four vectors per lane:
    // its columns 8j + 4hh + r, shared by both row blocks) are read once, at
    // the start, instead of once per group
    bf16x8 a0{}, a1{};
    f32x4 bb[4] = {};
    if constexpr (kE) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = *(const f32x4*)(nb + 8 * j);
    }
    if constexpr (kM) {
      a0 = as_bf16x8(*(const uint4*)(ql));
      a1 = as_bf16x8(*(const uint4*)(ql + 16));
      accM[0] = accM[1] = f32x16{};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const f32x4 b0 = bb[ks & 3];
      bf16x8 a2 = a1;
      if constexpr (kM)
        if (ks + 2 < NK) a2 = as_bf16x8(*(const uint4*)(ql + 16 * (ks + 2)));
      if constexpr (kM) {
        accM[0] = mfma32x32x16(a0, kop[0][ks], accM[0]);
        accM[1] = mfma32x32x16(a0, kop[1][ks], accM[1]);
      }
      if constexpr (kE) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int idx = kPer * ks + i, rb = idx >> 4, e = idx & 15;
          float p = exp2_fast(fmaf(accE[rb][e], a.scale_log2, b0[e & 3]));
          if constexpr (kMask) {   // a select, no branch
            const int d = d0E + 32 * ecb + 8 * (e >> 2) + 4 * hh + (e & 3);
            p = ((d >= rbase + 32 * rb + li + w) & (d < S)) ? p : 0.0f;
          }
          sum[rb][e & 3] += p;
        }
      }
      a0 = a1;
      a1 = a2;
      // within the group: one MFMA, half the scores' VALU work, the other
      // MFMA, the rest (each MFMA then has VALU work of this wave to overlap;
      // two MFMAs back to back measured 2-4 % slower)
      if constexpr (kM && kE) {
        constexpr int kV = kMask ? 12 : 6;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // Software pipeline over chunks: while the MFMAs of column block 0 of chunk
  // c run, the exps of block 1 of chunk c-1 are computed; while the MFMAs of
  // block 1 of chunk c run, the exps of block 0 of chunk c are computed.
  f32x16 accA[kRB], accB[kRB];
  bool pend = false, pend_mask = false;   // block 1 of the previous chunk awaits its exps
  int pend_d0 = 0, pend_nsl = 0;
  int nsl = 0;                            // bias slot of chunk c (c mod 3)
  for (int c = 0; c < nchunks; ++c) {
    const int d0 = d_start + c * kChunk;
    const int buf = c & 1;
    const bool has_next = c + 1 < nchunks;
    if (has_next) load_chunk(d0 + kChunk);
    // this wave's rows need d >= t + w: chunks wholly below are skipped; the
    // d >= t + w test is compiled only into the straddling-chunk variant
    const bool active = d0 + kChunk - 1 >= rbase + w;
    const bool msk = d0 < rbase + kWaveRows - 1 + w || d0 + kChunk - 1 > S - 1;
    if constexpr (!kF32In && kRB == 2 && D == 128) {
      // block 0 of chunk c (MFMA) with block 1 of chunk c-1 (exp), then
      // block 1 of chunk c (MFMA) with block 0 of chunk c (exp)
      if (active && pend) {
        if (pend_mask) fused(T_{}, T_{}, T_{}, accA, buf, 0, accB, pend_nsl, 1, pend_d0);
        else fused(T_{}, T_{}, F_{}, accA, buf, 0, accB, pend_nsl, 1, pend_d0);
      } else if (active) {
        fused(T_{}, F_{}, F_{}, accA, buf, 0, accB, pend_nsl, 1, pend_d0);
      } else if (pend) {
        if (pend_mask) fused(F_{}, T_{}, T_{}, accA, buf, 0, accB, pend_nsl, 1, pend_d0);
        else fused(F_{}, T_{}, F_{}, accA, buf, 0, accB, pend_nsl, 1, pend_d0);
      }
      if (active) {
        if (msk) fused(T_{}, T_{}, T_{}, accB, buf, 1, accA, nsl, 0, d0);
        else fused(T_{}, T_{}, F_{}, accB, buf, 1, accA, nsl, 0, d0);
      }
    } else {
      if (active) mfma_block(accA, buf, 0);
      if (pend) {
        if (pend_mask) exp_block(accB, pend_nsl, 1, pend_d0, std::true_type{});
        else exp_block(accB, pend_nsl, 1, pend_d0, std::false_type{});
      }
      if (active) {
        mfma_block(accB, buf, 1);
        if (msk) exp_block(accA, nsl, 0, d0, std::true_type{});
        else exp_block(accA, nsl, 0, d0, std::false_type{});
      }
    }
    pend = active;
    pend_mask = msk;
    pend_d0 = d0;
    pend_nsl = nsl;
    nsl = nsl == 2 ? 0 : nsl + 1;
    if (has_next) store_chunk(buf ^ 1, nsl, d0 + kChunk);
    __syncthreads();
  }
  if (pend) {
    if constexpr (!kF32In && kRB == 2 && D == 128) {
      if (pend_mask) fused(F_{}, T_{}, T_{}, accA, 0, 0, accB, pend_nsl, 1, pend_d0);
      else fused(F_{}, T_{}, F_{}, accA, 0, 0, accB, pend_nsl, 1, pend_d0);
    } else {
      if (pend_mask) exp_block(accB, pend_nsl, 1, pend_d0, std::true_type{});
      else exp_block(accB, pend_nsl, 1, pend_d0, std::false_type{});
    }
  }

  // A row whose range d >= t + w is not empty has a total in [2^-100, 2^100]
  // unless its exponents left the range the max-free sum covers; then the
  // whole workgroup (barriers) recomputes the tile with a running maximum.
  float tot[kRB];
  bool bad = false;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float part = (sum[rb][0] + sum[rb][1]) + (sum[rb][2] + sum[rb][3]);
    tot[rb] = halves_sum(part);
    const int t = rbase + 32 * rb + li;
    const bool nonempty = t + w <= S - 1;
    bad |= nonempty && !(tot[rb] >= 0x1p-100f && tot[rb] <= 0x1p100f);
  }
  if (bad) redo = 1;   // every writer stores the same value
  __syncthreads();
  if (redo) {
    rescaled_pass<D, kF32In>(a, kop, q_lds, nlse, rbase, t0, b, hq);
    return;
  }
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int t = rbase + 32 * rb + li;
    if (hh == 0 && t < S) out[t] = tot[rb] > 0.0f ? log2f(tot[rb]) * kLn2 : kNegInf;
  }
}

template <int D, bool kF32In>
void launch_tgt(TgtArgs a, int b, hipStream_t st) {
  a.ntiles = (a.S + kRowsPerTile - 1) / kRowsPerTile;
  const long long n = (long long)a.ntiles * a.Hq * b;
  hipLaunchKernelGGL((future_target_kernel<D, kF32In>), dim3((unsigned)n), dim3(kThreads), 0, st,
                     a);
}

}  // namespace

size_t target_ws_bytes(const Dims&) { return 0; }

hipError_t launch_future_target(const Dims& d, const void* q, const void* k, const float* lse,
                                float* target, void*, hipStream_t st) {
  TgtArgs a;
  a.q = q; a.k = k; a.lse = lse; a.target = target;
  a.S = d.S; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.w = d.w; a.ntiles = 0;
  a.reverse = launch_order_reversed();
  a.scale_log2 = d.scale * 1.4426950408889634f;
  if (d.D == 128) {
    if (d.f32_in) launch_tgt<128, true>(a, d.b, st);
    else launch_tgt<128, false>(a, d.b, st);
  } else {
    if (d.f32_in) launch_tgt<64, true>(a, d.b, st);
    else launch_tgt<64, false>(a, d.b, st);
  }
  return hipGetLastError();
}

// Target score ([Notes] §2.2): r_{h,t} = log(eps + (1/G) sum_g m_t^{(h,g)}) with
// m_t = exp(target_g[t]) / N_t, N_t = S - t - w future queries (the mean is 0
// where there are none).  One thread per (b, h, t).  The exponents
// x_g = target_g[t] - ln N_t are <= 0 for the dense LSE (a probability sum
// over N_t queries is at most N_t) but not for a sparse one, so the mean is
// taken relative to the group's largest exponent m:
//   mean = e^m A,  A = (1/G) sum_g e^(x_g - m) in [1/G, 1],
//   score = log(eps + e^m A)            for m <= 0 (e^m cannot overflow),
//         = m + log(eps e^-m + A)       for m > 0  (e^-m cannot overflow).
namespace {
__global__ __launch_bounds__(256) void target_score_kernel(const float* __restrict__ target,
                                                           float* __restrict__ score, int Hq,
                                                           int Hkv, int S, int w, float eps,
                                                           long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int G = Hq / Hkv;
  const long long bh = i / S;
  const int t = (int)(i - bh * S);
  const int b = (int)(bh / Hkv), h = (int)(bh % Hkv);
  const int nt = S - t - w;
  const float* tg = target + ((size_t)b * Hq + (size_t)h * G) * S + t;
  float r = logf(eps);                        // no future query: the mean is 0
  if (nt > 0) {
    const float lnn = logf((float)nt);
    float m = kNegInf;
    for (int g = 0; g < G; ++g) m = fmaxf(m, tg[(size_t)g * S] - lnn);
    if (m != kNegInf) {
      float acc = 0.0f;
      for (int g = 0; g < G; ++g) acc += expf(tg[(size_t)g * S] - lnn - m);
      const float A = acc / (float)G;
      if (m > 0.0f) r = m + logf(eps * expf(-m) + A);
      else if (eps > 0.0f) r = logf(eps + expf(m) * A);
      else r = m + logf(A);
    }
  }
  score[i] = r;
}
}  // namespace

hipError_t launch_target_score(const Dims& d, const float* target, float eps, float* score,
                               hipStream_t st) {
  const long long total = (long long)d.b * d.Hkv * d.S;
  hipLaunchKernelGGL(target_score_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     target, score, d.Hq, d.Hkv, d.S, d.w, eps, total);
  return hipGetLastError();
}

}  // namespace kvpop
