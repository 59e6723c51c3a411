// Device-side helpers shared by the gfx950 kernels of the H2O step:
// vector types for the CDNA4 bf16 MFMA operands, fragment loads, and the
// small math primitives (exp2 on v_exp_f32, packed bf16 conversion).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

typedef uint16_t bf16_t;  // storage type of bf16 tensors (bit pattern)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// v_mfma_f32_32x32x16_bf16 (CDNA4).  Lane l supplies A[row l%32][k 8(l/32)..+8]
// and B[k 8(l/32)..+8][col l%32]; the 16 accumulators of lane l hold
// C[8(r/4) + 4(l/32) + r%4][l%32], r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16 (gfx950) from a pointer into __shared__ memory: in each
// 16-lane group, lane i receives element i%4 of the 8-byte pieces addressed
// by lanes 4r + i/4, r = 0..3.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// LDS byte address of a __shared__ location, hidden from constant folding.
// A read at lds_addr(p) + a constant then carries the constant in its 16-bit
// offset field; without the barrier the compiler folds the array's own
// position into that constant, and for arrays above 64 KB of LDS it then
// spends one address add per read.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
  asm volatile("" : "+v"(a));
  return a;
}
// ds_read_b64_tr_b16 at LDS byte address a (see lds_read_tr16)
__device__ __forceinline__ bf16x4 lds_read_tr16_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(a));
}

// Raw buffer resource over [base, base + bytes) (gfx9 word 3): a load whose
// offset falls past `bytes` returns zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// buffer_load_dwordx4 ... lds: lane i copies the 16 bytes at voff + soff of
// the resource to LDS address lds_base + 16 i (lds_base wave-uniform, in M0).
// Issued from inline asm so that the compiler does not track the copy: its
// own tracking cannot tell one LDS destination array from another across a
// loop back-edge and would wait for copies just issued into other slots
// before an LDS read, draining the prefetch.  Every caller orders the copies
// itself: an explicit vmcnt wait and a barrier before any wave reads the
// destination, and a barrier after the last reads before a copy overwrites
// it.  The instruction has no register result, and copies issued here only
// make the compiler's own vmcnt waits stricter (loads retire in order).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voff,
                                      uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(lds_base)));
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
               : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Workgroup barrier for LDS traffic: waits for this wave's LDS accesses
// (lgkmcnt(0)) and meets the other waves.  Unlike __syncthreads, whose
// release fence waits for every outstanding global load -- copies into LDS
// still in flight included -- it leaves those copies running; their
// completion is waited for explicitly (vmcnt) where a stage is consumed.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store_u32x4(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 v) {
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return __builtin_convertvector(v, bf16x4);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Value of lane (l ^ 32): the other half of a 32x32 MFMA accumulator column.
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }

}  // namespace h2o
