// kvpop_boundary_labels: the teacher's boundary labels of the retention loss.
//
// KVpop reading notes §2.2: the target score of token t is aged by
//   r(q, t) = r_t + floor((q - t) / n) * log(gamma_h),
// the teacher keeps the top-k of E(q) = [s, q - w] under r(q, .), the boundary
// token t_bnd is the lowest-scoring token it keeps, and the label of the
// newcomer t_new = q - w is y = +1 if the teacher keeps it, -1 if not.
//
// The decayed score is one rounded float32 product followed by one rounded
// sum (no fused multiply-add), NaN counts as -inf and -0 as +0; the teacher's
// order is (decayed score descending, index ascending) and it keeps the first
// min(k, |E(q)|) tokens.  Rows without a newcomer (q - w < s) get t_bnd = -1,
// y = 0; with k = 0 nothing is kept (t_bnd = -1, y = -1).
//
// Design (gfx950): the floor decay changes the order from query to query, so
// every query runs an exact selection of its own, one wave per query and no
// workgroup barrier after the scores are staged.  A workgroup of NW waves
// owns (sequence, KV head, chunk of queries) and keeps the head's scores in
// LDS; each wave owns a run of consecutive queries, a histogram of NB bins
// over the chunk's range of decayed scores, a small selection histogram and
// a candidate buffer.  Per query the wave
//   1. brings the histogram up to date: built once for the run's first query;
//      from query q-1 to q only the tokens with t = q (mod n), whose age
//      floor((q - t)/n) steps up, move to their new bin, and the newcomer is
//      added (the bin map is monotone, so the token ranked min(k, |E|) lies in
//      the bin where the count from the top first reaches it);
//   2. copies that bin's tokens, in index order, into its candidate buffer;
//   3. selects among the candidates exactly: a radix select over their
//      order-preserving keys (8 bits at a time from the top of their range)
//      and an index-ordered ballot scan over the tokens with the selected key.
// A bin too large for the buffer (heavy ties) runs step 3 over all of E(q)
// instead, computing the keys again on each pass.  Along each lane's tokens
// the age is carried incrementally.
#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int kSelBins = 256;   // bins of the exact selection (8-bit digits)
constexpr int kU = 8;           // tokens per lane in flight in the full passes

struct LabelArgs {
  const float* score;
  const float* log_gamma;
  int32_t* t_bnd;
  int32_t* y;
  int Hkv, S, s, w, k, n, chunk;
};

// Order-preserving unsigned key of a decayed score (larger score, larger key).
__device__ __forceinline__ uint32_t score_key(float r) {
  const uint32_t u = __float_as_uint(r == 0.0f ? 0.0f : r);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The decayed score: the product age * log(gamma) rounded to float32, then
// the sum rounded again.  Contraction into one fused multiply-add (one
// rounding) is switched off here.
__device__ __forceinline__ float decayed(float score, int age, float lg) {
#pragma clang fp contract(off)
  const float p = (float)age * lg;
  return score + p;
}

__device__ __forceinline__ int floor_div(int x, int n) {
  return x >= 0 ? x / n : -((-x + n - 1) / n);
}

// Lane-strided walk over E(q): the lane's tokens are t0, t0 + 64, ...; carries
// the age floor((q - t)/n) of its current token.
struct AgeWalk {
  int a, r, step_q, step_r, n;
  __device__ __forceinline__ void init(int q, int t0, int n_) {
    n = n_;
    a = floor_div(q - t0, n);
    r = (q - t0) - a * n;
    step_q = 64 / n;
    step_r = 64 % n;
  }
  __device__ __forceinline__ void next() {   // t += 64
    r -= step_r;
    a -= step_q;
    if (r < 0) { r += n; a -= 1; }
  }
};

// Histogram search from the top, one wave: lane l owns the NB/64 bins
// [NB - P (l + 1), NB - P l), read downwards (P = NB/64).  Returns the bin
// where the count from the top first reaches `need` (1 <= need <= total), the
// count above it and the count in it; with `clear` the histogram is left
// zeroed.
template <int NB>
__device__ __forceinline__ void wave_find_bin(int* hist, int need, bool clear, int& bin,
                                              int& above, int& count) {
  constexpr int kPer = NB / 64;
  const int lane = lane_id();
  const int hi = NB - kPer * lane;          // bins [hi - kPer, hi)
  int c[kPer];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = hist[hi - 1 - i];
    tot += c[i];
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  int before = incl - tot;
  int my_bin = -1, my_above = 0, my_count = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (before < need && need <= before + c[i]) {
      my_bin = hi - 1 - i;
      my_above = before;
      my_count = c[i];
    }
    before += c[i];
  }
  if (clear) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) hist[hi - 1 - i] = 0;
  }
  const uint64_t m = wave_ballot(my_bin >= 0);
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  bin = __shfl(my_bin, src);
  above = __shfl(my_above, src);
  count = __shfl(my_count, src);
  wave_lds_fence();
}

// Exact selection by one wave over `n` items (get(i, key, t) gives item i's
// key and token; t < 0 marks no item): the token of the need-th item in the
// order (key descending, token ascending) and its key.  With `ordered` the
// items come in increasing token order and equal keys are resolved by a scan;
// otherwise by ranking the equal items' tokens pairwise.  Uses `hist`
// (kSelBins bins, zero on entry and on return).
template <class Get>
__device__ __forceinline__ void wave_select(int* hist, int n, int need, bool ordered, Get get,
                                            int& t_out, uint32_t& key_out) {
  const int lane = lane_id();
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int base = 0; base < n; base += 64) {
    uint32_t key;
    int t;
    get(base + lane, key, t);
    if (t >= 0) {
      lo = min(lo, key);
      hi = max(hi, key);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
  }
  const uint32_t range = hi - lo;
  uint32_t prefix = 0;
  int top = range ? 32 - __builtin_clz(range) : 0;   // low bits of key - lo still open
  while (top > 0) {
    const int width = min(8, top), shift = top - width;
    for (int base = 0; base < n; base += 64) {
      uint32_t key;
      int t;
      get(base + lane, key, t);
      const uint32_t rel = key - lo;
      const uint32_t hb = top >= 32 ? 0u : rel >> top;
      if (t >= 0 && hb == prefix) atomicAdd(&hist[(rel >> shift) & ((1u << width) - 1u)], 1);
    }
    wave_lds_fence();
    int bin, above, count;
    wave_find_bin<kSelBins>(hist, need, true, bin, above, count);
    prefix = (prefix << width) | (uint32_t)bin;
    need -= above;
    top = shift;
  }
  const uint32_t xkey = lo + prefix;
  int found = -1;
  if (!ordered) {
    // the item with this key whose token has exactly need-1 smaller tokens
    // among the items with this key
    for (int base = 0; base < n && found < 0; base += 64) {
      uint32_t key;
      int t;
      get(base + lane, key, t);
      const bool eq = t >= 0 && key == xkey;
      int below = 0;
      if (wave_ballot(eq) != 0) {
        for (int j = 0; j < n; ++j) {
          uint32_t kj;
          int tj;
          get(j, kj, tj);
          below += (tj >= 0 && kj == xkey && tj < t) ? 1 : 0;
        }
      }
      const uint64_t hm = wave_ballot(eq && below == need - 1);
      if (hm) found = __shfl(t, (int)__builtin_ctzll(hm));
    }
    t_out = found;
    key_out = xkey;
    return;
  }
  // the need-th item with this key, in token order
  for (int base = 0; base < n && found < 0; base += 64) {
    uint32_t key;
    int t;
    get(base + lane, key, t);
    const bool eq = t >= 0 && key == xkey;
    const uint64_t m = wave_ballot(eq);
    const int c = __builtin_popcountll(m);
    if (need <= c) {
      const uint64_t hm = wave_ballot(eq && lanes_below(m) == need - 1);
      found = __shfl(t, (int)__builtin_ctzll(hm));
    } else {
      need -= c;
    }
  }
  t_out = found;
  key_out = xkey;
}

template <int NW, int NB, int NC>
__global__ __launch_bounds__(NW * 64) void boundary_labels_kernel(LabelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  int* hist_all = reinterpret_cast<int*>(dyn);                      // NW x NB
  int* sel_all = hist_all + NW * NB;                                // NW x kSelBins
  int* cand_t_all = sel_all + NW * kSelBins;                        // NW x NC
  uint32_t* cand_k_all = reinterpret_cast<uint32_t*>(cand_t_all + NW * NC);
  float* red = reinterpret_cast<float*>(cand_k_all + NW * NC);      // 2 x NW
  float* sc = red + 2 * NW;                                         // scores 0 .. t_last

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t seg = (size_t)b * a.Hkv + h;
  const int S = a.S, s = a.s, w = a.w, k = a.k, n = a.n;
  const int q_lo = blockIdx.x * a.chunk, q_hi = min(S, q_lo + a.chunk);
  int32_t* out_t = a.t_bnd + seg * S;
  int32_t* out_y = a.y + seg * S;

  // rows without a newcomer, and every row when nothing is kept
  const int q_first = max(q_lo, s + w);          // first row with t_new >= s
  for (int q = q_lo + tid; q < q_hi; q += NW * 64) {
    if (q < q_first || k == 0) {
      out_t[q] = -1;
      out_y[q] = q < s + w ? 0 : -1;
    }
  }
  if (k == 0 || q_first >= q_hi) return;

  // ---- stage the scores (canonical) and the chunk's range of finite scores
  const float lg = a.log_gamma[h];
  const int t_last = q_hi - 1 - w;
  const float* src = a.score + seg * S;
  const float kInf = __builtin_huge_valf();
  float mn = kInf, mx = -kInf;
  for (int t = tid; t <= t_last; t += NW * 64) {
    const float v = canonical_priority(src[t]);
    sc[t] = v;
    if (t >= s && v > -kInf && v < kInf) {
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
  for (int i = tid; i < NW * (NB + kSelBins); i += NW * 64) hist_all[i] = 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) {
    red[wave] = mn;
    red[NW + wave] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[NW];
  for (int wv = 1; wv < NW; ++wv) {
    mn = fminf(mn, red[wv]);
    mx = fmaxf(mx, red[NW + wv]);
  }
  // the chunk's decayed scores lie in [mn + min(0, A lg), mx + max(0, A lg)],
  // A the largest age; the bin map only needs to be monotone (infinite
  // scores fall into the end bins, an empty range puts everything in bin 0)
  const float aged = (float)floor_div(q_hi - 1 - s, n) * lg;
  const float vlo = mn + fminf(0.0f, aged), vhi = mx + fmaxf(0.0f, aged);
  const float inv_w = (vhi > vlo) ? (float)NB / (vhi - vlo) : 0.0f;
  auto bin_of = [&](float r) {
    const float x = fminf(fmaxf((r - vlo) * inv_w, 0.0f), (float)(NB - 1));
    return (int)x;
  };

  int* hist = hist_all + wave * NB;
  int* sel = sel_all + wave * kSelBins;
  int* cand_t = cand_t_all + wave * NC;
  uint32_t* cand_k = cand_k_all + wave * NC;

  // this wave's run of consecutive queries; the candidate list of the
  // previous query's bin is kept and patched when the bin stays the same
  const int per = (q_hi - q_first + NW - 1) / NW;
  const int qa = q_first + wave * per, qb = min(q_hi, qa + per);
  int cur_bin = -1, cur_count = 0;
  bool have_list = false;
  // removals and additions of a step, in the (then idle) selection histogram
  constexpr int kPatch = kSelBins / 4;
  int* rem_t = sel;
  int* add_t = sel + kPatch;
  uint32_t* add_k = (uint32_t*)(sel + 2 * kPatch);
  for (int q = qa; q < qb; ++q) {
    const int t_new = q - w;
    const int n_e = t_new - s + 1;
    const int kk = min(k, n_e);

    // ---- 1. histogram of the bins of the decayed scores
    int n_rem = 0, n_add = 0;
    if (q > qa) {
      // from q-1: tokens t = q (mod n) of E(q-1) age by one step, then the
      // newcomer joins (its age is floor(w / n)); changes to the kept list's
      // bin are recorded
      const int t0 = s + (((q - s) % n) + n) % n;      // first such token >= s
      const int m0 = (q - t0) / n;                      // its age at q
      const int n_age = t_new - 1 >= t0 ? (t_new - 1 - t0) / n + 1 : 0;
      for (int base = 0; base < n_age; base += 64) {
        const int i = base + lane;
        const bool ok = i < n_age;
        const int t = t0 + min(i, n_age - 1) * n;
        const float v = sc[t];
        const float ro = decayed(v, m0 - i - 1, lg), rn = decayed(v, m0 - i, lg);
        const int ob = bin_of(ro), nb = bin_of(rn);
        if (ok) {
          atomicAdd(&hist[ob], -1);
          atomicAdd(&hist[nb], 1);
        }
        if (have_list) {
          const bool rm = ok && ob == cur_bin, ad = ok && nb == cur_bin;
          const uint64_t mr = wave_ballot(rm), ma = wave_ballot(ad);
          if (rm && n_rem + lanes_below(mr) < kPatch) rem_t[n_rem + lanes_below(mr)] = t;
          if (ad && n_add + lanes_below(ma) < kPatch) {
            add_t[n_add + lanes_below(ma)] = t;
            add_k[n_add + lanes_below(ma)] = score_key(rn);
          }
          n_rem += __builtin_popcountll(mr);
          n_add += __builtin_popcountll(ma);
        }
      }
      const float r_new = decayed(sc[t_new], w / n, lg);
      const int b_new = bin_of(r_new);
      if (lane == 0) {
        atomicAdd(&hist[b_new], 1);
        if (have_list && b_new == cur_bin && n_add < kPatch) {
          add_t[n_add] = t_new;
          add_k[n_add] = score_key(r_new);
        }
      }
      if (have_list && b_new == cur_bin) ++n_add;
    } else {
      // the run's first query: every eligible token (kU per lane in flight;
      // loads past t_new are clamped and add nothing)
      AgeWalk ag;
      ag.init(q, s + lane, n);
      for (int base = s; base <= t_new; base += 64 * kU) {
        float v[kU];
        int age[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          v[u] = sc[min(base + 64 * u + lane, t_new)];
          age[u] = ag.a;
          ag.next();
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)   // branch-free: past t_new the increment is 0
          atomicAdd(&hist[bin_of(decayed(v[u], age[u], lg))], base + 64 * u + lane <= t_new ? 1 : 0);
      }
    }
    wave_lds_fence();
    int bin, above, count;
    wave_find_bin<NB>(hist, kk, false, bin, above, count);
    const int need = kk - above;        // rank of the sought token within its bin

    int t_sel;
    uint32_t key_sel;
    bool ordered = true;
    bool patched = false;
    if (count <= NC && have_list && bin == cur_bin && n_rem <= kPatch && n_add <= kPatch) {
      // ---- 2a. same bin as the previous query: drop the removed tokens from
      // the list (compacted in place) and append the additions
      int kept = 0;
      for (int base = 0; base < cur_count; base += 64) {
        const int i = base + lane;
        const bool okk = i < cur_count;
        const int tt = okk ? cand_t[i] : -1;
        const uint32_t kt = okk ? cand_k[i] : 0u;
        bool keep = okk;
        for (int r = 0; r < n_rem; ++r) keep &= tt != rem_t[r];
        const uint64_t m = wave_ballot(keep);
        if (keep) {
          cand_t[kept + lanes_below(m)] = tt;
          cand_k[kept + lanes_below(m)] = kt;
        }
        kept += __builtin_popcountll(m);
        wave_lds_fence();
      }
      if (kept + n_add == count) {
        for (int j = lane; j < n_add; j += 64) {
          cand_t[kept + j] = add_t[j];
          cand_k[kept + j] = add_k[j];
        }
        patched = true;
        ordered = false;
      }
    }
    // the selection histogram held the patch lists: clear it
    if (q > qa && have_list) {
      for (int j = lane; j < kSelBins; j += 64) sel[j] = 0;
    }
    wave_lds_fence();
    if (count <= NC && !patched) {
      // ---- 2b. the bin's tokens, in index order, into the candidate buffer
      int placed = 0;
      AgeWalk ag;
      ag.init(q, s + lane, n);
      for (int base = s; base <= t_new; base += 64 * kU) {
        float v[kU];
        int age[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          v[u] = sc[min(base + 64 * u + lane, t_new)];
          age[u] = ag.a;
          ag.next();
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int t = base + 64 * u + lane;
          const float r = decayed(v[u], age[u], lg);
          const bool in = t <= t_new && bin_of(r) == bin;
          const uint64_t m = wave_ballot(in);
          if (in) {
            const int j = placed + lanes_below(m);
            cand_t[j] = t;
            cand_k[j] = score_key(r);
          }
          placed += __builtin_popcountll(m);
        }
      }
      wave_lds_fence();
    }
    if (count <= NC) {
      // ---- 3. exact selection among the candidates
      wave_select(
          sel, count, need, ordered,
          [&](int i, uint32_t& key, int& t) {
            const bool ok = i < count;
            key = ok ? cand_k[i] : 0u;
            t = ok ? cand_t[i] : -1;
          },
          t_sel, key_sel);
    } else {
      // heavy ties: exact selection over all of E(q), keys computed per pass
      wave_select(
          sel, n_e, kk, true,
          [&](int i, uint32_t& key, int& t) {
            t = s + i;
            if (t > t_new) {
              t = -1;
              key = 0u;
              return;
            }
            key = score_key(decayed(sc[t], (q - t) / n, lg));
          },
          t_sel, key_sel);
    }
    wave_lds_fence();   // the buffers are rewritten for the wave's next query
    have_list = count <= NC;
    cur_bin = bin;
    cur_count = count;

    if (lane == 0) {
      const uint32_t key_new = score_key(decayed(sc[t_new], w / n, lg));
      out_t[q] = t_sel;
      out_y[q] = (key_new > key_sel || t_sel == t_new) ? 1 : -1;
    }
  }
}

template <int NW, int NB, int NC>
void launch_cfg(const LabelArgs& a, int nchunks, int b, hipStream_t st) {
  const size_t lds = (size_t)NW * (NB + kSelBins) * 4 + (size_t)NW * NC * 8 +
                     (size_t)2 * NW * 4 + (size_t)a.S * sizeof(float);
  // more than 64 KiB of dynamic LDS must be allowed explicitly (160 KiB per CU)
  (void)hipFuncSetAttribute((const void*)boundary_labels_kernel<NW, NB, NC>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((boundary_labels_kernel<NW, NB, NC>), dim3(nchunks, a.Hkv, b),
                     dim3(NW * 64), lds, st, a);
}

}  // namespace

int labels_max_seq() { return 32768; }

hipError_t launch_boundary_labels(const Dims& d, const float* score, const float* log_gamma,
                                  int decay_step, int32_t* t_bnd, int32_t* y, hipStream_t st) {
  LabelArgs a;
  a.score = score; a.log_gamma = log_gamma; a.t_bnd = t_bnd; a.y = y;
  a.Hkv = d.Hkv; a.S = d.S; a.s = d.s; a.w = d.w; a.k = d.k; a.n = decay_step;
  // about 256 workgroups in all (one per CU), at least 64 queries each
  const int segs = d.b * d.Hkv;
  const int want = (256 + segs - 1) / segs;
  const int nchunks = max(1, min((d.S + 63) / 64, want));
  a.chunk = (d.S + nchunks - 1) / nchunks;
  const int nch = (d.S + a.chunk - 1) / a.chunk;
  if (d.S <= 16384) launch_cfg<16, 512, 256>(a, nch, d.b, st);   // 80 KiB + S floats of LDS
  else launch_cfg<4, 512, 256>(a, nch, d.b, st);                // 20 KiB + S floats of LDS
  return hipGetLastError();
}

}  // namespace kvpop
