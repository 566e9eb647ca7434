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
//  * A workgroup owns 128 key rows t (4 waves x 32) of one query head.  It
//    streams the future queries d in 64-column chunks staged in LDS, shared
//    by the 4 waves; each wave keeps its 32 key rows as the MFMA B operand in
//    registers, so X^T[d][t] = Q K^T leaves every lane owning one row t.
//  * Each score becomes exp2(x * scale log2 e - LSE_d log2 e) and is summed
//    directly: with the dense LSE every exponent is <= 0, so no running
//    maximum or rescaling is needed (3 VALU operations per score).
//  * Chunks wholly below a wave's first row + w are skipped; the d >= t + w
//    test runs only on the chunks that straddle the band.
#include <type_traits>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerTile = 128;
constexpr int kChunk = 64;

struct TgtArgs {
  const void* q;
  const void* k;
  const float* lse;
  float* target;
  int S, Hq, Hkv, G, w;
  float scale_log2;
};

template <int D, bool kF32In>
__global__ __launch_bounds__(kThreads, 2) void future_target_kernel(TgtArgs a) {
  constexpr int QS = kF32In ? D + 1 : D + 8;                 // LDS row stride (elements)
  constexpr int qBytes = kChunk * QS * (kF32In ? 4 : 2);
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[qBytes];
  __shared__ __attribute__((aligned(16))) float nlse[kChunk];  // -LSE_d * log2(e)

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int hh = lane >> 5, li = lane & 31;
  const int tile = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int S = a.S, w = a.w;
  const int h = hq / a.G;
  const int t0 = tile * kRowsPerTile;
  const int t = t0 + wave * 32 + li;              // this lane's key row
  const int t_first = t0 + wave * 32;
  const int t_last = min(t_first + 31, S - 1);
  float* out = a.target + ((size_t)b * a.Hq + hq) * S;

  const int d_start = t0 + w;                      // first query any row of the tile needs
  if (d_start > S - 1) {
    if (hh == 0 && t < S) out[t] = kNegInf;
    return;
  }

  // key operand (B of X^T = Q K^T): row t, dims [16ks + 8hh, +8)
  constexpr int NKS = kF32In ? D / 2 : D / 16;
  typedef typename std::conditional<kF32In, float, bf16x8>::type KOp;
  KOp kop[NKS];
  {
    const bool ok = t < S;
    const size_t krow = (((size_t)b * a.Hkv + h) * S + (ok ? t : 0)) * D;
    if constexpr (kF32In) {
      const float* kp = (const float*)a.k + krow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kop[ks] = ok ? kp[2 * ks + hh] : 0.0f;
    } else {
      const uint16_t* kp = (const uint16_t*)a.k + krow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (ok) u = *(const uint4*)(kp + 16 * ks + 8 * hh);
        kop[ks] = as_bf16x8(u);
      }
    }
  }

  const size_t qbase = ((size_t)b * a.Hq + hq) * S * D;
  const float* lse = a.lse + ((size_t)b * a.Hq + hq) * S;
  float sum = 0.0f;

  for (int d0 = d_start; d0 < S; d0 += kChunk) {
    // ---- stage Q rows d0 .. d0+63 and their -LSE
    if constexpr (!kF32In) {
      const uint16_t* qg = (const uint16_t*)a.q + qbase;
      uint16_t* ql = (uint16_t*)q_lds;
      constexpr int PPR = D / 8;
#pragma unroll
      for (int i = 0; i < kChunk * PPR / kThreads; ++i) {
        const int p = tid + i * kThreads;
        const int row = p / PPR, piece = p % PPR;
        const int d = d0 + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (d < S) val = *(const uint4*)(qg + (size_t)d * D + piece * 8);
        *(uint4*)(ql + row * QS + piece * 8) = val;
      }
    } else {
      const float* qg = (const float*)a.q + qbase;
      float* ql = (float*)q_lds;
      constexpr int PPR = D / 4;
#pragma unroll
      for (int i = 0; i < kChunk * PPR / kThreads; ++i) {
        const int p = tid + i * kThreads;
        const int row = p / PPR, piece = p % PPR;
        const int d = d0 + row;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (d < S) val = *(const float4*)(qg + (size_t)d * D + piece * 4);
        float* dst = ql + row * QS + piece * 4;
        dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
      }
    }
    if (tid < kChunk) {
      const int d = d0 + tid;
      nlse[tid] = d < S ? -lse[d] * kLog2e : kNegInf;
    }
    __syncthreads();

    // ---- this wave's rows need d >= t + w: skip chunks wholly below
    if (d0 + kChunk - 1 >= t_first + w) {
      const bool need_mask = d0 < t_last + w || d0 + kChunk - 1 > S - 1;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x16 acc = f32x16{};
        if constexpr (!kF32In) {
          const uint16_t* ql = (const uint16_t*)q_lds + (32 * cb + li) * QS + 8 * hh;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            acc = mfma32x32x16(as_bf16x8(*(const uint4*)(ql + 16 * ks)), kop[ks], acc);
        } else {
          const float* ql = (const float*)q_lds + (32 * cb + li) * QS + hh;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = mfma32x32x2(ql[2 * ks], kop[ks], acc);
        }
        // lane holds columns d = d0 + 32cb + 8j + 4hh + r for row t
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dl = 32 * cb + 8 * j + 4 * hh;
          const f32x4 bias = *(const f32x4*)(&nlse[dl]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float p = exp2_fast(fmaf(acc[4 * j + r], a.scale_log2, bias[r]));
            if (need_mask) {   // wave-uniform; the test itself is a select
              const int d = d0 + dl + r;
              p = ((d >= t + w) & (d < S)) ? p : 0.0f;
            }
            sum += p;
          }
        }
      }
    }
    __syncthreads();
  }

  const float tot = sum + __shfl_xor(sum, 32);
  if (hh == 0 && t < S) out[t] = tot > 0.0f ? log2f(tot) * kLn2 : kNegInf;
}

template <int D, bool kF32In>
void launch_tgt(const TgtArgs& a, int b, hipStream_t st) {
  const int ntiles = (a.S + kRowsPerTile - 1) / kRowsPerTile;
  hipLaunchKernelGGL((future_target_kernel<D, kF32In>), dim3(ntiles, a.Hq, b), dim3(kThreads), 0,
                     st, a);
}

}  // namespace

size_t target_ws_bytes(const Dims&) { return 0; }

hipError_t launch_future_target(const Dims& d, const void* q, const void* k, const float* lse,
                                float* target, void*, hipStream_t st) {
  TgtArgs a;
  a.q = q; a.k = k; a.lse = lse; a.target = target;
  a.S = d.S; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.w = d.w;
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

}  // namespace kvpop
