// Device-side helpers for the libkvpop kernels (CDNA4 / gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvpop {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kInt32Max = 0x7fffffff;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Wave index within the workgroup, in a scalar register: values derived from
// it are provably wave-uniform, so branches on them stay scalar branches
// instead of per-lane exec masking.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// Orders LDS accesses of this wave against each other: waits for its
// outstanding LDS operations and keeps the compiler from moving memory
// accesses across (used where lanes of one wave exchange data through LDS).
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier that hands over LDS only: each wave waits for its own
// LDS operations, then all waves meet.  Unlike __syncthreads, whose release
// fence also waits for every vector-memory operation in flight (direct loads
// into LDS included), it leaves this wave's direct loads running; the caller
// awaits the ones the other waves will read (s_waitcnt vmcnt) before it.  The
// memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct loads from global memory into LDS, 16 or 4 bytes per lane: lane L
// writes lds_base + 16 L (or 4 L), lds_base being the same for the whole
// wave.  Issued from inline asm, so the compiler does not see the LDS write
// and adds no wait for it of its own (it would otherwise wait, at the first
// LDS read it cannot prove disjoint, for every load in flight); the caller
// awaits these loads with s_waitcnt vmcnt before the barrier that hands the
// data to the other waves.  The compiler's own vmcnt waits stay correct: the
// counter drains in order, and loads it does not know of only make them
// wait longer.  The asm sets M0 itself: a kernel using these must not keep
// another value in M0 (no direct-load builtins, no indexed register access).
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void_t*)p);
}
__device__ __forceinline__ void dma_lds_x4(const void* g, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_address(lds_base))
               : "memory");
}
__device__ __forceinline__ void dma_lds_x1(const void* g, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_address(lds_base))
               : "memory");
}
// The 16-byte form with a wave-uniform 64-bit base and an unsigned 32-bit
// per-lane byte offset (one VGPR of address arithmetic per lane).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma_lds_x4_so(const void* base, uint32_t off, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(lds_address(lds_base))
               : "memory");
}

// Workgroups of a 1-D grid are dispatched round-robin over the 8 XCDs, each
// with its own L2.  This maps the hardware block id to a logical id such that
// every XCD receives a contiguous range of logical ids (a bijection on
// [0, n)), so neighbouring logical blocks, which share data, share an L2.
// The hardware block index a workgroup takes its work from: blockIdx.x, or
// counted from the end when the launch order is reversed (a testing aid: no
// result depends on the order in which workgroups run).
__device__ __forceinline__ int launch_block(int reversed) {
  return reversed ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
}

__device__ __forceinline__ int xcd_logical_block(int bid, int n) {
  constexpr int kXcds = 8;
  const int q = n / kXcds, r = n % kXcds;
  const int x = bid % kXcds, j = bid / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// max and sum of a lane's value with that of lane ^ 32: v_permlane32_swap
// (gfx950) returns, in every lane l, the values of lanes l & 31 and
// (l & 31) + 32 (checked on the device), so one VALU instruction replaces an
// LDS permute round trip; both operations commute, so the result is the same
// in both halves
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- numbers
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;   // round to nearest even (v_cvt_pk_bf16_f32)
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Priority with NaN mapped to -inf and -0 to +0.
__device__ __forceinline__ float canonical_priority(float p) {
  if (p != p) return kNegInf;
  if (p == 0.0f) return 0.0f;
  return p;
}

// Unsigned key whose ascending order is the priority order (priority
// descending); equal priorities give equal keys, so a stable sort by key keeps
// ties in index order.
__device__ __forceinline__ uint32_t priority_sort_key(float p) {
  uint32_t u = __float_as_uint(canonical_priority(p));
  uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].  Lane l supplies
// A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; it holds
// D[8*j + 4*(l/32) + r][l%32] in element 4*j + r (j, r in 0..3).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32];
// the D layout is the one above.
__device__ __forceinline__ f32x16 mfma32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  uint4 u;
  u.x = pack_bf16x2(p[0], p[1]);
  u.y = pack_bf16x2(p[2], p[3]);
  u.z = pack_bf16x2(p[4], p[5]);
  u.w = pack_bf16x2(p[6], p[7]);
  return as_bf16x8(u);
}

}  // namespace kvpop
