// kvpop_decode_step: one decode step over the compact fixed-size cache.
//
// KVpop reading notes §2.3: inference keeps only the compact cache; §2.2 and
// §2.4: at query q the token u = q - w leaves the protected window and is
// scored then (the delayed readout), competing for the k long-range slots;
// gist.science summary §2.1: B = s + w + k entries per KV head.
//
// One kernel per step (two with split-K), on the caller's stream:
//  1. attend, one workgroup per (sequence, KV head, split): first the step's
//     decision — the slot token p takes (slot p while the cache fills;
//     afterwards the slot of u when u is dropped, or of the worst held
//     long-range token when u replaces it).  The worst token comes from the
//     pair's record in the cache's state array, written by the previous step
//     for this one; without a current record (no state array, a new handoff,
//     a record marked stale) every slot's metadata is scanned, with wave
//     shuffle and LDS reductions.  Every split computes the same decision,
//     and each also scans its own slots, as the update leaves them, for the
//     next step's worst token (one split: it writes the record; several:
//     their candidates go to the combine, which writes it).
//     Then every wave streams 32-slot blocks of K and V from HBM with
//     coalesced loads, the new token's row read from k_new / v_new in place
//     of its slot, prefetching the next block into registers while the
//     current one is in its private LDS region (V transposed), and runs
//     S^T = K Q^T and O^T = V^T P^T on MFMA with the G query heads of the KV
//     head as the MFMA rows, keeping an online softmax.  The 4 waves merge in
//     LDS; with one split the workgroup writes o and lse and the metadata
//     update, otherwise a partial (max, sum, unnormalised O), split 0 records
//     the decision.  The split owning the new token's slot writes its K/V row
//     there at the end (no other workgroup reads that slot in this step).
//  2. combine (only with several splits, after every split has read the
//     metadata): applies the recorded metadata update, writes the next
//     step's record and merges the partials into o and lse.
// A device-scope fence per workgroup (to let the last one merge) would write
// back and invalidate the L2 of its XCD on this multi-XCD part, so the merge
// across workgroups is a separate kernel.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "kvpop.h"
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBlk = 32;          // slots per wave iteration
constexpr int kTargetBlocks = 512;   // 2 resident workgroups per CU

struct DecArgs {
  void* ck;
  void* cv;
  int* slot_pos;
  float* slot_prio;
  int* ring;
  const int* pos;
  const void* q;
  const void* k_new;
  const void* v_new;
  const float* prio_leaving;
  void* o;
  float* lse;
  float* part;          // [b, Hq, nsplit, D + 2]: max (log2 units), sum, unnormalised O
  int* dec;             // [b, Hkv, 4] the step's decision, applied by the combine (splits > 1)
  int* cand;            // [b, Hkv, nsplit, 4] each split's worst candidate for the next step
  int* state;           // [b, Hkv, 8] the next step's worst long-range token per pair, or null
  int Hq, Hkv, G, s, w, k, Bc, spl, nsplit;
  float scale_log2;
};

// (priority, position, slot) of the worst long-range candidate seen so far:
// lowest priority, ties to the highest position; slot < 0 means none.
struct Worst {
  float p;
  int pos, slot;
};

__device__ __forceinline__ bool worse_than(const Worst& a, const Worst& b) {
  return a.slot >= 0 && (b.slot < 0 || a.p < b.p || (a.p == b.p && a.pos > b.pos));
}

constexpr int kDecideThreads = 256;
constexpr int kDecideUnroll = 8;   // slot loads in flight per thread
constexpr int kStateWords = KVPOP_CACHE_STATE_WORDS;   // per-pair record of the next step
constexpr int kRescanEarly = 2;    // next-step candidate slots per thread loaded before the math

__device__ __forceinline__ void wave_reduce_worst(Worst& best) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    Worst o;
    o.p = __shfl_xor(best.p, off);
    o.pos = __shfl_xor(best.pos, off);
    o.slot = __shfl_xor(best.slot, off);
    if (worse_than(o, best)) best = o;
  }
}

// The leave decision of step p for one (sequence, KV head), from the slot
// metadata as it stands before the step: the slot token p takes (slot p while
// the cache fills; afterwards the slot of u = p - w when u is dropped, or of
// the worst held long-range token when u replaces it) and the priority u
// keeps.  Every workgroup of the pair computes it (all its threads take part;
// the slot scan issues all its loads before comparing, then a wave and a
// workgroup reduction).  ns < 0: no step (p < 0) or an inconsistent cache.
struct Decision {
  int ns, u_slot;
  float pu;
  bool keep_u;
};

__device__ Decision decide_step(const DecArgs& a, size_t seg, int p, Worst* s_worst) {
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int s = a.s, w = a.w, k = a.k, Bc = a.Bc;
  const int* spos = a.slot_pos + seg * Bc;
  const float* sprio = a.slot_prio + seg * Bc;
  const int* ring = a.ring + seg * w;
  Decision dc{-1, -1, 0.0f, false};
  if (p < 0) return dc;
  const int u = p - w;
  if (p < Bc) {
    // filling: token p takes slot p; u (if eligible) joins the long-range set
    dc.ns = p;
    if (p > 0 && u >= s) {
      dc.u_slot = ring[p % w];
      dc.pu = canonical_priority(a.prio_leaving[seg]);
      dc.keep_u = true;
    }
  } else {
    // full: u = p - w >= s + k; it is kept iff it beats the worst long-range token
    dc.u_slot = ring[p % w];
    dc.pu = canonical_priority(a.prio_leaving[seg]);
    // the worst held long-range token: from the pair's record when the
    // previous step wrote it for this step, else from a scan of every slot
    Worst best{__builtin_huge_valf(), -1, -1};
    bool have = false;
    if (k > 0 && a.state) {
      const int4 r = *(const int4*)(a.state + seg * kStateWords);
      if (__builtin_amdgcn_readfirstlane(r.x) == p) {
        best = Worst{__int_as_float(r.y), r.z, r.w};
        have = true;
      }
    }
    if (k == 0) {
      dc.ns = dc.u_slot;
    } else if (have) {
      dc.keep_u = best.slot >= 0 && dc.pu > best.p;
      dc.ns = dc.keep_u ? best.slot : dc.u_slot;
    } else {
      for (int j0 = tid; j0 < Bc; j0 += kDecideThreads * kDecideUnroll) {
        int sp[kDecideUnroll];
        float pr[kDecideUnroll];
#pragma unroll
        for (int i = 0; i < kDecideUnroll; ++i) {
          const int j = j0 + i * kDecideThreads;
          sp[i] = j < Bc ? spos[j] : -1;
          pr[i] = j < Bc ? sprio[j] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kDecideUnroll; ++i) {
          const Worst c{pr[i], sp[i], j0 + i * kDecideThreads};
          if (sp[i] >= s && sp[i] < u && worse_than(c, best)) best = c;
        }
      }
      wave_reduce_worst(best);
      if (lane == 0) s_worst[wave] = best;
      __syncthreads();
      best = s_worst[0];
#pragma unroll
      for (int i = 1; i < kDecideThreads / 64; ++i)
        if (worse_than(s_worst[i], best)) best = s_worst[i];
      dc.keep_u = best.slot >= 0 && dc.pu > best.p;
      dc.ns = dc.keep_u ? best.slot : dc.u_slot;
    }
  }
  if ((unsigned)dc.ns >= (unsigned)Bc) dc.ns = -1;   // inconsistent cache state: no update
  return dc;
}

// The metadata update of a decision (one thread).
__device__ __forceinline__ void apply_decision(const DecArgs& a, size_t seg, int p,
                                               const Decision& dc) {
  const int Bc = a.Bc, w = a.w;
  if (dc.ns < 0) return;
  float* sprio = a.slot_prio + seg * Bc;
  if (dc.keep_u && (unsigned)dc.u_slot < (unsigned)Bc) sprio[dc.u_slot] = dc.pu;
  a.ring[seg * w + p % w] = dc.ns;
  a.slot_pos[seg * Bc + dc.ns] = p;
  sprio[dc.ns] = 0.0f;
}

// Folds slot j into the next step's worst long-range candidate `best`, with
// the metadata (sp, pr) as read before step p's update dc: after the update
// slot dc.ns holds token p (not a candidate), slot dc.u_slot holds u = p - w
// with priority dc.pu when u is kept; a candidate of step p + 1 has
// s <= position <= p - w.
__device__ __forceinline__ void fold_candidate(Worst& best, int j, int sp, float pr,
                                               const Decision& dc, int s, int u) {
  if (j == dc.ns) return;
  if (dc.keep_u && j == dc.u_slot) pr = dc.pu;
  const Worst c{pr, sp, j};
  if (sp >= s && sp <= u && worse_than(c, best)) best = c;
}

template <int D, bool kF32>
struct DecLds {
  // bf16: K [32][D+8]; V^T [D][32+8] (permuted columns)
  // f32:  K [32][D+1]; V [32][D+4]
  static constexpr int KS = kF32 ? D + 1 : D + 8;
  static constexpr int VS = kF32 ? D + 4 : kBlk + 8;
  static constexpr int kBytes = kF32 ? kBlk * KS * 4 : kBlk * KS * 2;
  static constexpr int vBytes = kF32 ? kBlk * VS * 4 : D * VS * 2;
  static constexpr int waveBytes = ((kBytes + vBytes + 15) / 16) * 16;
  // K: 16-byte pieces per lane; bf16 V: (slot pair, 8-dim octet) tasks per
  // lane, each two 16-byte row loads
  static constexpr int KPL = kBlk * (D * (kF32 ? 4 : 2) / 16) / 64;
  static constexpr int VTL = (kBlk / 2) * (D / 8) / 64;
};

// Two workgroups per CU, except for float32 caches at D = 128, whose staging
// registers allow one.
template <int D, bool kF32, bool kF32Out>
__global__ __launch_bounds__(kThreads, (kF32 && D == 128) ? 1 : 2) void decode_attend_kernel(DecArgs a) {
  using L = DecLds<D, kF32>;
  static_assert(kWaves * L::waveBytes >= kWaves * 32 * (D + 2) * 4, "merge area");
  __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * L::waveBytes];
  __shared__ Worst s_worst[kWaves];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int hh = lane >> 5, li = lane & 31;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Bc = a.Bc, G = a.G;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int p = a.pos[b];
  const int n_valid = p < 0 ? 0 : min(p + 1, Bc);
  const int j_lo = split * a.spl;
  const int j_hi = min(j_lo + a.spl, n_valid);
  unsigned char* my = lds + wave * L::waveBytes;

  // query operand: row li is query head h*G + li (rows >= G are zero)
  const bool row_ok = li < G;
  const int hq = h * G + (row_ok ? li : 0);
  constexpr int NKS = kF32 ? D / 2 : D / 16;
  typedef typename std::conditional<kF32, float, bf16x8>::type QOp;
  QOp qop[NKS];
  {
    const size_t qrow = ((size_t)b * a.Hq + hq) * D;
    if constexpr (kF32) {
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

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const size_t cbase = seg * (size_t)Bc * D;

  // ---- staging of one 32-slot block: HBM -> registers -> this wave's LDS.
  // The slot the step's new token takes (ns_sub) is read from k_new / v_new
  // in place of its old content.
  int ns_sub = -1;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  uint4 kst[L::KPL];
  u32x4v vpair[kF32 ? 1 : 2 * L::VTL];
  uint4 vst4[kF32 ? L::KPL : 1];
  // (slots at or past `lim` read as zeros)
  auto load_blk = [&](int blk, int lim) {
    if constexpr (!kF32) {
      const uint16_t* kg = (const uint16_t*)a.ck + cbase;
      const uint16_t* vg = (const uint16_t*)a.cv + cbase;
      const uint16_t* kn = (const uint16_t*)a.k_new + seg * D;
      const uint16_t* vn = (const uint16_t*)a.v_new + seg * D;
      auto krow = [&](int slot) { return slot == ns_sub ? kn : kg + (size_t)slot * D; };
      auto vrow = [&](int slot) { return slot == ns_sub ? vn : vg + (size_t)slot * D; };
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        const int slot = blk + pi / PPR;
        kst[i] = slot < lim ? *(const uint4*)(krow(slot) + (pi % PPR) * 8)
                             : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < L::VTL; ++i) {
        const int task = lane + 64 * i;
        const int pr = task & 15, oc = task >> 4;      // pairs fastest: distinct LDS banks
        const int s0 = blk + 2 * pr;
        const u32x4v z = {0u, 0u, 0u, 0u};
        vpair[2 * i] = s0 < lim ? *(const u32x4v*)(vrow(s0) + 8 * oc) : z;
        vpair[2 * i + 1] = s0 + 1 < lim ? *(const u32x4v*)(vrow(s0 + 1) + 8 * oc) : z;
      }
    } else {
      const float* kg = (const float*)a.ck + cbase;
      const float* vg = (const float*)a.cv + cbase;
      const float* kn = (const float*)a.k_new + seg * D;
      const float* vn = (const float*)a.v_new + seg * D;
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        const int slot = blk + pi / PPR;
        const int piece = (pi % PPR) * 4;
        const float* kr = slot == ns_sub ? kn : kg + (size_t)slot * D;
        const float* vr = slot == ns_sub ? vn : vg + (size_t)slot * D;
        kst[i] = slot < lim ? *(const uint4*)(kr + piece) : make_uint4(0, 0, 0, 0);
        vst4[i] = slot < lim ? *(const uint4*)(vr + piece) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_blk = [&]() {
    if constexpr (!kF32) {
      uint16_t* kl = (uint16_t*)my;
      uint16_t* vl = (uint16_t*)(my + L::kBytes);
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        *(uint4*)(kl + (pi / PPR) * L::KS + (pi % PPR) * 8) = kst[i];
      }
      // V^T: column c = 16*ks + 8*hh + 4*a + r of LDS row d holds slot
      // 16*ks + 8*a + 4*hh + r of the block (the P operand layout); a slot
      // pair lands in two adjacent columns, so each dim is one 32-bit word
#pragma unroll
      for (int i = 0; i < L::VTL; ++i) {
        const int task = lane + 64 * i;
        const int pr = task & 15, oc = task >> 4;
        const int j0 = 2 * pr;
        const int c0 = 16 * (j0 >> 4) + 8 * ((j0 >> 2) & 1) + 4 * ((j0 >> 3) & 1) + (j0 & 3);
        const u32x4v x0 = vpair[2 * i], x1 = vpair[2 * i + 1];
        uint16_t* col = vl + (8 * oc) * L::VS + c0;
#pragma unroll
        for (int dp = 0; dp < 4; ++dp) {
          *(uint32_t*)(col + (2 * dp) * L::VS) = (x0[dp] & 0xffffu) | (x1[dp] << 16);
          *(uint32_t*)(col + (2 * dp + 1) * L::VS) = (x0[dp] >> 16) | (x1[dp] & 0xffff0000u);
        }
      }
    } else {
      float* kl = (float*)my;
      float* vl = (float*)(my + L::kBytes);
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        const int row = pi / PPR, piece = pi % PPR;
        float* kd = kl + row * L::KS + piece * 4;
        kd[0] = __uint_as_float(kst[i].x);
        kd[1] = __uint_as_float(kst[i].y);
        kd[2] = __uint_as_float(kst[i].z);
        kd[3] = __uint_as_float(kst[i].w);
        *(uint4*)(vl + row * L::VS + piece * 4) = vst4[i];
      }
    }
  };

  // the first block's loads are issued before the step's position arrives,
  // bounded by the split's end in the cache (every such slot exists; those
  // past the held ones are zeroed below), and before the step's decision
  // (the new token's slot is patched afterwards); the new token's K/V row is
  // written to its slot at the end by the split that owns the slot (no other
  // workgroup reads that slot in this step)
  int blk = j_lo + wave * kBlk;
  const int j_cap = min(j_lo + a.spl, Bc);
  if (blk < j_cap) load_blk(blk, j_cap);
  const Decision dc = decide_step(a, seg, p, s_worst);
  const int ns = dc.ns;
  // The next step's record: this split's share of the scan for the worst
  // long-range token after this step's update.  The metadata is read before
  // anything updates it (with one split the update is applied at the end of
  // this workgroup; with several, by the combine kernel); the first
  // kRescanEarly slots per thread are loaded now, behind the K/V stream.
  const bool track = a.state != nullptr && p >= 0;
  const int* spos = a.slot_pos + seg * Bc;
  const float* sprio = a.slot_prio + seg * Bc;
  int r_sp[kRescanEarly];
  float r_pr[kRescanEarly];
#pragma unroll
  for (int i = 0; i < kRescanEarly; ++i) {
    const int j = j_lo + tid + i * kThreads;
    const bool ok = track && j < j_hi;
    r_sp[i] = ok ? spos[j] : -1;
    r_pr[i] = ok ? sprio[j] : 0.0f;
  }
  if (tid == 0 && a.nsplit > 1 && split == 0) {
    int* rec = a.dec + seg * 4;
    rec[0] = ns;
    rec[1] = dc.u_slot;
    rec[2] = dc.keep_u ? 1 : 0;
    rec[3] = __float_as_int(dc.pu);
  }
  ns_sub = ns;
  if (blk < j_hi && blk + kBlk > j_hi) {
    // the first block straddles the held slots' end (a filling cache): rows
    // past it become zeros, as for every later block
    if constexpr (!kF32) {
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i)
        if (blk + (lane + 64 * i) / PPR >= j_hi) kst[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < L::VTL; ++i) {
        const int s0 = blk + 2 * ((lane + 64 * i) & 15);
        const u32x4v z = {0u, 0u, 0u, 0u};
        if (s0 >= j_hi) vpair[2 * i] = z;
        if (s0 + 1 >= j_hi) vpair[2 * i + 1] = z;
      }
    } else {
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i)
        if (blk + (lane + 64 * i) / PPR >= j_hi) {
          kst[i] = make_uint4(0, 0, 0, 0);
          vst4[i] = make_uint4(0, 0, 0, 0);
        }
    }
  }
  if (blk < j_hi && ns >= blk && ns < blk + kBlk) {
    // patch the new token's row into the first block (unconditional loads of
    // the one new row, then selects)
    const int r = ns - blk;
    if constexpr (!kF32) {
      const uint16_t* kn = (const uint16_t*)a.k_new + seg * D;
      const uint16_t* vn = (const uint16_t*)a.v_new + seg * D;
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        const uint4 nk = *(const uint4*)(kn + (pi % PPR) * 8);
        if (pi / PPR == r) kst[i] = nk;
      }
#pragma unroll
      for (int i = 0; i < L::VTL; ++i) {
        const int task = lane + 64 * i;
        const int pr = task & 15, oc = task >> 4;
        const u32x4v nv = *(const u32x4v*)(vn + 8 * oc);
        if (2 * pr == r) vpair[2 * i] = nv;
        if (2 * pr + 1 == r) vpair[2 * i + 1] = nv;
      }
    } else {
      const float* kn = (const float*)a.k_new + seg * D;
      const float* vn = (const float*)a.v_new + seg * D;
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < L::KPL; ++i) {
        const int pi = lane + 64 * i;
        const uint4 nk = *(const uint4*)(kn + (pi % PPR) * 4);
        const uint4 nv = *(const uint4*)(vn + (pi % PPR) * 4);
        if (pi / PPR == r) {
          kst[i] = nk;
          vst4[i] = nv;
        }
      }
    }
  }
  for (; blk < j_hi; blk += kWaves * kBlk) {
    store_blk();
    wave_lds_fence();
    if (blk + kWaves * kBlk < j_hi) load_blk(blk + kWaves * kBlk, j_hi);   // in flight during the math

    // ---- S^T = K Q^T (32 slots x 32 rows)
    f32x16 sacc = f32x16{};
    if constexpr (!kF32) {
      const uint16_t* kl = (const uint16_t*)my + li * L::KS + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        sacc = mfma32x32x16(as_bf16x8(*(const uint4*)(kl + 16 * ks)), qop[ks], sacc);
    } else {
      const float* kl = (const float*)my + li * L::KS + hh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sacc = mfma32x32x2(kl[2 * ks], qop[ks], sacc);
    }
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int slot = blk + 8 * (e >> 2) + 4 * hh + (e & 3);
      x[e] = slot < j_hi ? sacc[e] * a.scale_log2 : kNegInf;
    }
    float mc = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mc = fmaxf(mc, x[e]);
    mc = halves_max(mc);
    const float m_new = fmaxf(m_run, mc);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[e] = exp2_fast(x[e] - m_use);
      ps += x[e];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T
    if constexpr (!kF32) {
      const bf16x8 pk0 = pack_bf16x8(&x[0]), pk1 = pack_bf16x8(&x[8]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vl = (const uint16_t*)(my + L::kBytes) + (32 * db + li) * L::VS + 8 * hh;
        oacc[db] = mfma32x32x16(as_bf16x8(*(const uint4*)(vl)), pk0, oacc[db]);
        oacc[db] = mfma32x32x16(as_bf16x8(*(const uint4*)(vl + 16)), pk1, oacc[db]);
      }
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float* vl = (const float*)(my + L::kBytes) + 32 * db + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = 8 * (e >> 2) + 4 * hh + (e & 3);
          oacc[db] = mfma32x32x2(vl[key * L::VS], x[e], oacc[db]);
        }
      }
    }
    wave_lds_fence();
  }

  // ---- merge the 4 waves in LDS: mg[wave][row][0] = max, [1] = sum, [2..] = O
  const float l_tot = halves_sum(l_run);
  __syncthreads();                               // staging areas are free now
  float* mg = (float*)lds;
  constexpr int RS = D + 2;
  if (row_ok) {
    float* r = mg + (wave * 32 + li) * RS;
    if (hh == 0) {
      r[0] = m_run;
      r[1] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) r[2 + 32 * db + 8 * j + 4 * hh + rr] = oacc[db][4 * j + rr];
  }
  __syncthreads();

  const int nsplit = a.nsplit;
  auto write_out = [&](int g, int d, float M, float Ls, float Od) {
    const size_t oi = ((size_t)b * a.Hq + h * G + g) * D + d;
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    if constexpr (kF32Out) ((float*)a.o)[oi] = Od * inv;
    else ((__bf16*)a.o)[oi] = (__bf16)(Od * inv);
    if (d == 0 && a.lse)
      a.lse[(size_t)b * a.Hq + h * G + g] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : kNegInf;
  };
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, mg[(wv * 32 + g) * RS]);
    float Ls = 0.0f, Od = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        const float* r = mg + (wv * 32 + g) * RS;
        const float wt = exp2_fast(r[0] - M);
        Ls += r[1] * wt;
        Od += r[2 + d] * wt;
      }
    }
    if (nsplit == 1) {
      write_out(g, d, M, Ls, Od);
    } else {
      float* pp = a.part + (((size_t)b * a.Hq + h * G + g) * nsplit + split) * RS;
      if (d == 0) {
        pp[0] = M;
        pp[1] = Ls;
      }
      pp[2 + d] = Od;
    }
  }
  // this split's candidate for the next step's record (the slots loaded
  // early, then the rest of its range, kDecideUnroll loads in flight)
  if (track) {
    Worst best{__builtin_huge_valf(), -1, -1};
    const int u = p - a.w;
#pragma unroll
    for (int i = 0; i < kRescanEarly; ++i)
      fold_candidate(best, j_lo + tid + i * kThreads, r_sp[i], r_pr[i], dc, a.s, u);
    for (int j0 = j_lo + tid + kRescanEarly * kThreads; j0 < j_hi;
         j0 += kThreads * kDecideUnroll) {
      int sp[kDecideUnroll];
      float pr[kDecideUnroll];
#pragma unroll
      for (int i = 0; i < kDecideUnroll; ++i) {
        const int j = j0 + i * kThreads;
        sp[i] = j < j_hi ? spos[j] : -1;
        pr[i] = j < j_hi ? sprio[j] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kDecideUnroll; ++i)
        fold_candidate(best, j0 + i * kThreads, sp[i], pr[i], dc, a.s, u);
    }
    wave_reduce_worst(best);
    if (lane == 0) s_worst[wave] = best;
    __syncthreads();
    if (tid == 0) {
      best = s_worst[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i)
        if (worse_than(s_worst[i], best)) best = s_worst[i];
      const int4 rec = make_int4(p + 1, __float_as_int(best.p), best.pos, best.slot);
      if (nsplit == 1) *(int4*)(a.state + seg * kStateWords) = rec;
      else *(int4*)(a.cand + (seg * nsplit + split) * 4) = rec;
    }
  }
  // with one split the metadata update is this workgroup's (every read of
  // the metadata above is complete)
  if (tid == 0 && nsplit == 1) apply_decision(a, seg, p, dc);
  // the new token's K/V row into its slot, by the split that owns the slot
  if (ns >= j_lo && ns < j_hi) {
    constexpr int kWords = D * (kF32 ? 4 : 2) / 4;
    const uint32_t* knw = (const uint32_t*)a.k_new + seg * kWords;
    const uint32_t* vnw = (const uint32_t*)a.v_new + seg * kWords;
    uint32_t* kc = (uint32_t*)a.ck + (seg * Bc + ns) * kWords;
    uint32_t* vc = (uint32_t*)a.cv + (seg * Bc + ns) * kWords;
    for (int i = tid; i < kWords; i += kThreads) {
      kc[i] = knw[i];
      vc[i] = vnw[i];
    }
  }
}

// The metadata side of the combine for one (sequence, KV head): the step's
// update (recorded by split 0; every split has read the metadata by now) and
// the next step's record, the worst of the splits' candidates (wave 0, one
// candidate per lane).
__device__ __forceinline__ void combine_metadata(const DecArgs& a, int b, int h, int d) {
  const size_t seg = (size_t)b * a.Hkv + h;
  const int p = a.pos[b];
  if (a.state && p >= 0 && d < 64) {
    Worst best{__builtin_huge_valf(), -1, -1};
    for (int j = d; j < a.nsplit; j += 64) {
      const int4 c = *(const int4*)(a.cand + (seg * a.nsplit + j) * 4);
      const Worst cw{__int_as_float(c.y), c.z, c.w};
      if (worse_than(cw, best)) best = cw;
    }
    wave_reduce_worst(best);
    if (d == 0)
      *(int4*)(a.state + seg * kStateWords) =
          make_int4(p + 1, __float_as_int(best.p), best.pos, best.slot);
  }
  if (d == 0) {
    const int* rec = a.dec + seg * 4;
    const Decision dc{rec[0], rec[1], __int_as_float(rec[3]), rec[2] != 0};
    apply_decision(a, seg, p, dc);
  }
}

// Merges the per-split partials into o and lse: one workgroup per
// (sequence, query head), one thread per output dim, every partial of the
// row read at once (the split maxima, sums and this dim's unnormalised O);
// the workgroup of the first query head of each KV head also applies the
// step's metadata update (recorded by split 0: every split has read the
// metadata by now) and writes the next step's record, the worst of the
// splits' candidates (wave 0, one candidate per lane).  Every load of the
// workgroup is issued before its first store, so the metadata costs no
// round trip of its own.
template <int D, bool kF32Out, int kMaxSplit>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  static_assert(kMaxSplit <= 64, "one split candidate per lane of wave 0");
  constexpr int RS = D + 2;
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = a.G, nsplit = a.nsplit;
  const size_t row = (size_t)b * a.Hq + hq;
  const float* pp = a.part + row * nsplit * RS;
  float m[kMaxSplit], l[kMaxSplit], od[kMaxSplit];
#pragma unroll
  for (int j = 0; j < kMaxSplit; ++j) {
    const bool ok = j < nsplit;
    m[j] = ok ? pp[j * RS] : kNegInf;
    l[j] = ok ? pp[j * RS + 1] : 0.0f;
    od[j] = ok ? pp[j * RS + 2 + d] : 0.0f;
  }
  const bool meta = hq % G == 0;
  const size_t seg = (size_t)b * a.Hkv + hq / G;
  int p = -1;
  int4 rec = make_int4(-1, -1, 0, 0), cnd = make_int4(0, 0, -1, -1);
  if (meta) {
    p = a.pos[b];
    rec = *(const int4*)(a.dec + seg * 4);
    if (a.state && d < nsplit) cnd = *(const int4*)(a.cand + (seg * nsplit + d) * 4);
  }
  float M = kNegInf;
#pragma unroll
  for (int j = 0; j < kMaxSplit; ++j) M = fmaxf(M, m[j]);
  float Ls = 0.0f, Od = 0.0f;
  if (M != kNegInf) {
#pragma unroll
    for (int j = 0; j < kMaxSplit; ++j) {
      const float wt = m[j] == kNegInf ? 0.0f : exp2_fast(m[j] - M);
      Ls += l[j] * wt;
      Od += od[j] * wt;
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  if constexpr (kF32Out) ((float*)a.o)[row * D + d] = Od * inv;
  else ((__bf16*)a.o)[row * D + d] = (__bf16)(Od * inv);
  if (d == 0 && a.lse) a.lse[row] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : kNegInf;
  if (!meta) return;
  if (a.state && p >= 0 && d < 64) {
    Worst best{__builtin_huge_valf(), -1, -1};
    const Worst cw{__int_as_float(cnd.y), cnd.z, cnd.w};
    if (d < nsplit && worse_than(cw, best)) best = cw;
    wave_reduce_worst(best);
    if (d == 0)
      *(int4*)(a.state + seg * kStateWords) =
          make_int4(p + 1, __float_as_int(best.p), best.pos, best.slot);
  }
  if (d == 0) apply_decision(a, seg, p, Decision{rec.x, rec.y, __int_as_float(rec.w), rec.z != 0});
}

// The same merge for any number of splits (more than the unrolled variants
// hold): the partials of a row are read in a loop.
template <int D, bool kF32Out>
__global__ __launch_bounds__(D) void decode_combine_any_kernel(DecArgs a) {
  constexpr int RS = D + 2;
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = a.G, nsplit = a.nsplit;
  if (hq % G == 0) combine_metadata(a, b, hq / G, d);
  const size_t row = (size_t)b * a.Hq + hq;
  const float* pp = a.part + row * nsplit * RS;
  float M = kNegInf;
  for (int j = 0; j < nsplit; ++j) M = fmaxf(M, pp[j * RS]);
  float Ls = 0.0f, Od = 0.0f;
  if (M != kNegInf) {
    for (int j = 0; j < nsplit; ++j) {
      const float mj = pp[j * RS];
      const float wt = mj == kNegInf ? 0.0f : exp2_fast(mj - M);
      Ls += pp[j * RS + 1] * wt;
      Od += pp[j * RS + 2 + d] * wt;
    }
  }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  if constexpr (kF32Out) ((float*)a.o)[row * D + d] = Od * inv;
  else ((__bf16*)a.o)[row * D + d] = (__bf16)(Od * inv);
  if (d == 0 && a.lse) a.lse[row] = Ls > 0.0f ? (M + log2f(Ls)) * kLn2 : kNegInf;
}

template <int D, bool kF32, bool kF32Out>
void launch_dec(const DecArgs& a, int b, hipStream_t st) {
  hipLaunchKernelGGL((decode_attend_kernel<D, kF32, kF32Out>), dim3(a.nsplit, a.Hkv, b),
                     dim3(kThreads), 0, st, a);
  if (a.nsplit > 1) {
    const dim3 grid(a.Hq, b);
    if (a.nsplit <= 8)
      hipLaunchKernelGGL((decode_combine_kernel<D, kF32Out, 8>), grid, dim3(D), 0, st, a);
    else if (a.nsplit <= 16)
      hipLaunchKernelGGL((decode_combine_kernel<D, kF32Out, 16>), grid, dim3(D), 0, st, a);
    else
      hipLaunchKernelGGL((decode_combine_any_kernel<D, kF32Out>), grid, dim3(D), 0, st, a);
  }
}

}  // namespace

// Slots per split (a multiple of 4 waves x 32 slots) and the number of splits,
// chosen so that a step launches about kTargetBlocks workgroups.
static void decode_geometry(const Dims& d, int* spl, int* nsplit) {
  const int Bc = (int)d.budget();
  const long long pairs = (long long)d.b * d.Hkv;
  long long want = (kTargetBlocks + pairs - 1) / pairs;
  const int unit = kWaves * kBlk;
  const int max_split = (Bc + unit - 1) / unit;
  if (want < 1) want = 1;
  if (want > max_split) want = max_split;
  int per = (int)((Bc + want - 1) / want);
  per = ((per + unit - 1) / unit) * unit;
  *spl = per;
  *nsplit = (Bc + per - 1) / per;
}

int decode_splits(const Dims& d) {
  int spl, ns;
  decode_geometry(d, &spl, &ns);
  return ns;
}

size_t decode_ws_bytes(const Dims& d) {
  const int ns = decode_splits(d);
  return ns > 1 ? align256((size_t)d.b * d.Hq * ns * (d.D + 2) * 4) +
                      align256((size_t)d.nseg() * 4 * 4) + align256((size_t)d.nseg() * ns * 4 * 4)
                : 0;
}

hipError_t launch_decode(const Dims& d, const CacheArgs& c, const int* pos, const void* q,
                         const void* k_new, const void* v_new, const float* prio_leaving, void* o,
                         float* lse, void* ws, hipStream_t st) {
  int spl, nsplit;
  decode_geometry(d, &spl, &nsplit);
  DecArgs a;
  a.ck = c.k; a.cv = c.v; a.slot_pos = c.slot_pos; a.slot_prio = c.slot_prio; a.ring = c.ring;
  a.pos = pos; a.q = q; a.k_new = k_new; a.v_new = v_new; a.prio_leaving = prio_leaving;
  a.o = o; a.lse = lse;
  a.part = (float*)ws;
  a.dec = nsplit > 1 ? (int*)((char*)ws + align256((size_t)d.b * d.Hq * nsplit * (d.D + 2) * 4))
                     : nullptr;
  a.cand = nsplit > 1 ? a.dec + align256((size_t)d.nseg() * 4 * 4) / 4 : nullptr;
  a.state = c.state;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.s = d.s; a.w = d.w; a.k = d.k;
  a.Bc = (int)d.budget(); a.spl = spl; a.nsplit = nsplit;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  if (d.D == 128) {
    if (d.f32_in) {
      if (d.f32_out) launch_dec<128, true, true>(a, d.b, st);
      else launch_dec<128, true, false>(a, d.b, st);
    } else {
      if (d.f32_out) launch_dec<128, false, true>(a, d.b, st);
      else launch_dec<128, false, false>(a, d.b, st);
    }
  } else {
    if (d.f32_in) {
      if (d.f32_out) launch_dec<64, true, true>(a, d.b, st);
      else launch_dec<64, true, false>(a, d.b, st);
    } else {
      if (d.f32_out) launch_dec<64, false, true>(a, d.b, st);
      else launch_dec<64, false, false>(a, d.b, st);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- no-alloc
// Scratch of kvpop_decode_step_noalloc: the split-K partials and decision
// records that kvpop_decode_step keeps in the caller's workspace live here
// instead, one copy per GPU (each device holds the array from the library's
// first use on it until the process ends).  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the device
// address looked up once per device by hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KVPOP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t decode_noalloc_scratch_bytes() { return sizeof(scratch); }

hipError_t decode_noalloc_scratch(hipStream_t st, void** out) {
  *out = nullptr;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  hipDevice_t sdev = cur;
  e = hipStreamGetDevice(st, &sdev);
  if (e != hipSuccess) return e;
  // the address is looked up with the stream's device current; a stream of
  // another device is refused rather than switching devices under the caller
  if ((int)sdev != cur || cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[cur].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_addr[cur].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_addr[cur].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace kvpop
