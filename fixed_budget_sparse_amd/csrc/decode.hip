// kvpop_decode_step: one decode step over the compact fixed-size cache.
//
// KVpop reading notes §2.3: inference keeps only the compact cache; §2.2 and
// §2.4: at query q the token u = q - w leaves the protected window and is
// scored then (the delayed readout), competing for the k long-range slots;
// gist.science summary §2.1: B = s + w + k entries per KV head.
//
// Three kernels per step, all on the caller's stream:
//  1. decide (one workgroup per (sequence, KV head)): reads the slot metadata,
//     picks the slot token p takes (slot p while the cache fills; afterwards
//     the slot of u when u is dropped, or of the worst held long-range token
//     when u replaces it), updates slot_pos / slot_prio / ring and writes the
//     new K/V row into that slot.  The choice is exact integer/compare work.
//  2. attend (split-K): every wave streams 32-slot blocks of K and V from HBM
//     with coalesced loads, stages them in its own LDS region (V transposed)
//     and runs S^T = K Q^T and O^T = V^T P^T on MFMA with the G query heads of
//     the KV head as the 32 MFMA rows, keeping a per-wave online softmax; it
//     writes a partial (max, sum, unnormalised O).
//  3. combine: merges the partials of each query head into o and lse.
// The attention reads only K/V, so the metadata update of step 1 cannot race
// with it, and stream order makes the new row visible to step 2.
#include <type_traits>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBlk = 32;          // slots per wave iteration
constexpr int kTargetBlocks = 2048;

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
  float* part;          // [b, Hq, nparts, D + 2]: max (log2 units), sum, O
  int Hq, Hkv, G, s, w, k, Bc, spl, nparts;
  float scale_log2;
};

template <int D, bool kF32>
__global__ __launch_bounds__(kThreads) void decode_decide_kernel(DecArgs a) {
  __shared__ float r_prio[kThreads];
  __shared__ int r_pos[kThreads];
  __shared__ int r_slot[kThreads];
  __shared__ int s_new;
  const int tid = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int p = a.pos[b];
  if (p < 0) return;
  const int s = a.s, w = a.w, k = a.k, Bc = a.Bc;
  const size_t seg = (size_t)b * a.Hkv + h;
  int* spos = a.slot_pos + seg * Bc;
  float* sprio = a.slot_prio + seg * Bc;
  int* ring = a.ring + seg * w;
  const int u = p - w;
  int u_slot = -1;
  float pu = 0.0f;
  bool keep_u = false;     // u becomes (or stays) a long-range token in its own slot

  if (p < Bc) {
    // filling: token p takes slot p; u (if eligible) joins the long-range set
    if (tid == 0) s_new = p;
    if (p > 0 && u >= s) {
      u_slot = ring[p % w];
      pu = canonical_priority(a.prio_leaving[seg]);
      keep_u = true;
    }
  } else {
    // full: u = p - w >= s + k; it is kept iff it beats the worst long-range token
    u_slot = ring[p % w];
    pu = canonical_priority(a.prio_leaving[seg]);
    if (k == 0) {
      if (tid == 0) s_new = u_slot;
    } else {
      float bp = __builtin_huge_valf();
      int bpos = -1, bslot = -1;
      for (int j = tid; j < Bc; j += kThreads) {
        const int sp = spos[j];
        if (sp >= s && sp < u) {
          const float pr = sprio[j];
          if (pr < bp || (pr == bp && sp > bpos)) {
            bp = pr;
            bpos = sp;
            bslot = j;
          }
        }
      }
      r_prio[tid] = bp;
      r_pos[tid] = bpos;
      r_slot[tid] = bslot;
      __syncthreads();
      for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off) {
          const float op = r_prio[tid + off];
          const int opos = r_pos[tid + off];
          if (r_slot[tid + off] >= 0 &&
              (r_slot[tid] < 0 || op < r_prio[tid] || (op == r_prio[tid] && opos > r_pos[tid]))) {
            r_prio[tid] = op;
            r_pos[tid] = opos;
            r_slot[tid] = r_slot[tid + off];
          }
        }
        __syncthreads();
      }
      const int worst = r_slot[0];
      keep_u = worst >= 0 && pu > r_prio[0];
      if (tid == 0) s_new = keep_u ? worst : u_slot;
    }
  }
  __syncthreads();   // every read of the metadata precedes the updates below
  const int ns = s_new;
  if ((unsigned)ns >= (unsigned)Bc) return;   // inconsistent cache state: leave it untouched
  if (tid == 0) {
    if (keep_u && (unsigned)u_slot < (unsigned)Bc) sprio[u_slot] = pu;
    ring[p % w] = ns;
    spos[ns] = p;
    sprio[ns] = 0.0f;
  }
  // the new token's K/V row goes into its slot
  constexpr int kWords = D * (kF32 ? 4 : 2) / 4;
  if (tid < kWords) {
    const uint32_t* kn = (const uint32_t*)a.k_new + seg * kWords;
    const uint32_t* vn = (const uint32_t*)a.v_new + seg * kWords;
    uint32_t* kc = (uint32_t*)a.ck + (seg * Bc + ns) * kWords;
    uint32_t* vc = (uint32_t*)a.cv + (seg * Bc + ns) * kWords;
    kc[tid] = kn[tid];
    vc[tid] = vn[tid];
  }
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
};

template <int D, bool kF32>
__global__ __launch_bounds__(kThreads, 2) void decode_attend_kernel(DecArgs a) {
  using L = DecLds<D, kF32>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kWaves * L::waveBytes];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
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

  for (int blk = j_lo + wave * kBlk; blk < j_hi; blk += kWaves * kBlk) {
    // ---- stage 32 slots of K (row-major) and V into this wave's LDS
    if constexpr (!kF32) {
      const uint16_t* kg = (const uint16_t*)a.ck + cbase;
      const uint16_t* vg = (const uint16_t*)a.cv + cbase;
      uint16_t* kl = (uint16_t*)my;
      uint16_t* vl = (uint16_t*)(my + L::kBytes);
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < kBlk * PPR / 64; ++i) {
        const int pi = lane + 64 * i;
        const int row = pi / PPR, piece = pi % PPR;
        const int slot = blk + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (slot < j_hi) val = *(const uint4*)(kg + (size_t)slot * D + piece * 8);
        *(uint4*)(kl + row * L::KS + piece * 8) = val;
      }
#pragma unroll
      for (int i = 0; i < 4 * (D / 2) / 64; ++i) {
        const int task = lane + 64 * i;
        const int grp = task / (D / 2), dp = task % (D / 2);
        uint32_t x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int slot = blk + 16 * (grp >> 1) + 8 * (e >> 2) + 4 * (grp & 1) + (e & 3);
          x[e] = slot < j_hi ? *(const uint32_t*)(vg + (size_t)slot * D + 2 * dp) : 0u;
        }
        uint4 lo, hi;
        lo.x = (x[0] & 0xffffu) | (x[1] << 16);
        lo.y = (x[2] & 0xffffu) | (x[3] << 16);
        lo.z = (x[4] & 0xffffu) | (x[5] << 16);
        lo.w = (x[6] & 0xffffu) | (x[7] << 16);
        hi.x = (x[0] >> 16) | (x[1] & 0xffff0000u);
        hi.y = (x[2] >> 16) | (x[3] & 0xffff0000u);
        hi.z = (x[4] >> 16) | (x[5] & 0xffff0000u);
        hi.w = (x[6] >> 16) | (x[7] & 0xffff0000u);
        *(uint4*)(vl + (2 * dp) * L::VS + grp * 8) = lo;
        *(uint4*)(vl + (2 * dp + 1) * L::VS + grp * 8) = hi;
      }
    } else {
      const float* kg = (const float*)a.ck + cbase;
      const float* vg = (const float*)a.cv + cbase;
      float* kl = (float*)my;
      float* vl = (float*)(my + L::kBytes);
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < kBlk * PPR / 64; ++i) {
        const int pi = lane + 64 * i;
        const int row = pi / PPR, piece = pi % PPR;
        const int slot = blk + row;
        float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
        if (slot < j_hi) {
          kv4 = *(const float4*)(kg + (size_t)slot * D + piece * 4);
          vv4 = *(const float4*)(vg + (size_t)slot * D + piece * 4);
        }
        float* kd = kl + row * L::KS + piece * 4;
        kd[0] = kv4.x; kd[1] = kv4.y; kd[2] = kv4.z; kd[3] = kv4.w;
        *(float4*)(vl + row * L::VS + piece * 4) = vv4;
      }
    }
    wave_lds_fence();

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
    mc = fmaxf(mc, __shfl_xor(mc, 32));
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

  // ---- this wave's partial for each query head row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    float* pp = a.part + (((size_t)b * a.Hq + hq) * a.nparts + split * kWaves + wave) * (D + 2);
    if (hh == 0) {
      pp[0] = m_run;
      pp[1] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * hh;
#pragma unroll
        for (int r = 0; r < 4; ++r) pp[2 + d + r] = oacc[db][4 * j + r];
      }
  }
}

template <int D, bool kF32Out>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* pp = a.part + ((size_t)b * a.Hq + hq) * a.nparts * (D + 2);
  float M = kNegInf;
  for (int j = 0; j < a.nparts; ++j) M = fmaxf(M, pp[j * (D + 2)]);
  float Lsum = 0.0f, od = 0.0f;
  if (M != kNegInf) {
    for (int j = 0; j < a.nparts; ++j) {
      const float mj = pp[j * (D + 2)];
      const float wgt = exp2_fast(mj - M);        // 0 for empty partials (mj = -inf)
      Lsum += pp[j * (D + 2) + 1] * wgt;
      if (tid < D) od += pp[j * (D + 2) + 2 + tid] * wgt;
    }
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  if (tid < D) {
    const size_t oi = ((size_t)b * a.Hq + hq) * D + tid;
    if constexpr (kF32Out) ((float*)a.o)[oi] = od * inv;
    else ((__bf16*)a.o)[oi] = (__bf16)(od * inv);
  }
  if (tid == 0 && a.lse)
    a.lse[(size_t)b * a.Hq + hq] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : kNegInf;
}

template <int D, bool kF32, bool kF32Out>
void launch_dec(const DecArgs& a, int b, int nsplit, hipStream_t st) {
  hipLaunchKernelGGL((decode_decide_kernel<D, kF32>), dim3(a.Hkv, b), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((decode_attend_kernel<D, kF32>), dim3(nsplit, a.Hkv, b), dim3(kThreads), 0,
                     st, a);
  hipLaunchKernelGGL((decode_combine_kernel<D, kF32Out>), dim3(a.Hq, b), dim3(128), 0, st, a);
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
  return align256((size_t)d.b * d.Hq * ns * kWaves * (d.D + 2) * 4);
}

hipError_t launch_decode(const Dims& d, const CacheArgs& c, const int* pos, const void* q,
                         const void* k_new, const void* v_new, const float* prio_leaving, void* o,
                         float* lse, void* ws, hipStream_t st) {
  int spl, nsplit;
  decode_geometry(d, &spl, &nsplit);
  DecArgs a;
  a.ck = c.k; a.cv = c.v; a.slot_pos = c.slot_pos; a.slot_prio = c.slot_prio; a.ring = c.ring;
  a.pos = pos; a.q = q; a.k_new = k_new; a.v_new = v_new; a.prio_leaving = prio_leaving;
  a.o = o; a.lse = lse; a.part = (float*)ws;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.s = d.s; a.w = d.w; a.k = d.k;
  a.Bc = (int)d.budget(); a.spl = spl; a.nparts = nsplit * kWaves;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  if (d.D == 128) {
    if (d.f32_in) {
      if (d.f32_out) launch_dec<128, true, true>(a, d.b, nsplit, st);
      else launch_dec<128, true, false>(a, d.b, nsplit, st);
    } else {
      if (d.f32_out) launch_dec<128, false, true>(a, d.b, nsplit, st);
      else launch_dec<128, false, false>(a, d.b, nsplit, st);
    }
  } else {
    if (d.f32_in) {
      if (d.f32_out) launch_dec<64, true, true>(a, d.b, nsplit, st);
      else launch_dec<64, true, false>(a, d.b, nsplit, st);
    } else {
      if (d.f32_out) launch_dec<64, false, true>(a, d.b, nsplit, st);
      else launch_dec<64, false, false>(a, d.b, nsplit, st);
    }
  }
  return hipGetLastError();
}

}  // namespace kvpop
