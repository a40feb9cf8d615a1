// Device-side helpers shared by the SwitchFFN kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, blocks dealt round-robin

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Routing order of two candidate experts (logit a of expert ia against logit b
// of expert ib): the larger fp32 logit goes first, a NaN counts as larger than
// every number, and equal values (two NaNs included) go to the lower index.
// This is numpy's argmax order, so an argmax that starts from (-inf, a
// sentinel index above every expert) always ends on an expert in [0, N),
// whatever a token's logits hold.
__device__ __forceinline__ bool route_before(float a, int ia, float b, int ib) {
  // Written without branches (selects only): it runs per candidate in the
  // routing loops.
  const bool an = __builtin_isnan(a), bn = __builtin_isnan(b), lt = ia < ib;
  const bool num = (a > b) | ((a == b) & lt);
  return (an & (!bn | lt)) | (!an & !bn & num);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest, ties to even; one v_cvt_pk_bf16_f32),
// lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// D = A(32x16) * B(16x32) + C on the matrix cores.  Lane l supplies
// A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32]; the 16 results of
// lane l are C[8*(v/4) + 4*(l/32) + v%4][l%32], v = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Map the hardware block id to a logical tile id so that each XCD receives a
// contiguous range of logical tiles (blocks are dealt to XCDs round-robin).
// Tiles that share operands then share one XCD's L2.
__device__ __forceinline__ int xcd_contiguous_tile(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int q = nblocks / kXcds;
  const int r = nblocks % kXcds;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

// Buffer resource over [base, base + bytes): loads past `bytes` return zero,
// which covers ragged row and k tails without branches.  dword3 = 0x00020000
// is the gfx9-family raw-buffer format word.
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource (sizes stay < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// Stores at offsets past the resource's size are dropped by the hardware's
// range check, like the loads above return zero: ragged tails need no branch.
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Workgroup barrier ordering LDS only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima, i.e. not waited for).  Loads that write LDS are not tracked
// by the compiler's wait insertion; kernels that issue them wait with this.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N < 0 ? 0 : (N > 63 ? 63 : N);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for kernels with loads that write LDS in flight.  An LDS
// fence would make the compiler wait for every such load (all pipeline steps
// in flight); those are waited for explicitly instead, so this only completes
// the wave's own LDS accesses and meets the other waves.  The memory clobber
// keeps the compiler from moving any memory access across it.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace sffn
