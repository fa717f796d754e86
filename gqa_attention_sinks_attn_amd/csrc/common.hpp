// Device-side helpers shared by the sink-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Work-item and workgroup indices read straight from the hardware registers
// (the runtime's accessor functions are not inlined into kernels built
// without IEEE mode, and would cost a call at every kernel start).
__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int block_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int block_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// 16-byte global load of 8 bf16 values (kept as raw bits).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotation of one rotary pair (u, v) by the angle whose cosine and sine
// (both times the attention temperature) are c and s: (u c - v s, v c + u s).
// Each output is one rounded product and one fused multiply-add, written out
// with contraction off, so that every kernel that rotates a token rounds it
// identically (the decode step's fused append must reproduce the append
// kernel bit for bit).
__device__ __forceinline__ void rotate_pair(float& u, float& v, float c, float s) {
#pragma clang fp contract(off)
  const float uu = u, vv = v;
  const float vs = vv * s, us = uu * s;
  u = __builtin_fmaf(uu, c, -vs);
  v = __builtin_fmaf(vv, c, us);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return bf16_bits_to_float(w & 0xffffu); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return bf16_bits_to_float(w >> 16); }

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// A: lane l holds row l%16, eight k values; B: lane l holds column l%16,
// the same eight k values; D: lane l holds column l%16, rows 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32) += A(32x16) * B(16x32).  A: lane l holds row l%32, eight k
// values; B: column l%32, the same k values; D: lane l holds column l%32,
// rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// lane j receives element j % 4 of the 8-byte words that lanes 4 e + j / 4
// of the group point at, for e = 0..3.  So if lane s points at row
// (r0 + s / 4), columns (c0 + 4 (s % 4)) of a row-major bf16 matrix, lane
// j receives column c0 + j of rows r0 .. r0 + 3: a 4 x 16 block transposed.
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Two transposed reads forming one 8-value MFMA operand (slots 0-3 from
// `lo`, slots 4-7 from `hi`).
__device__ __forceinline__ u32x4 lds_tr16_pair(const uint16_t* lo, const uint16_t* hi) {
  const u32x2 a = lds_tr16(lo);
  const u32x2 b = lds_tr16(hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Wait until at most N vector memory operations of this wave are
// outstanding (the LDS-direct tile loads count among them).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4):
// lane l reads base + off and writes LDS bytes lds + 16 l .. lds + 16 l + 15
// (base and lds wave-uniform).  Written as assembly so that the compiler
// neither counts nor waits for these loads (it would otherwise wait for all
// of them before any LDS read): wait_vmem and the workgroup barrier order
// them against the LDS reads.  M0 carries the LDS address; the compiler
// keeps no value of its own in it (the clobber is declared, the warning
// about it silenced).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS offset of a __shared__ object.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global load); the empty assembly statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Cross-lane exchange with lane ^ mask (mask in {16, 32}) through
// ds_bpermute; wave-uniform control flow required.
__device__ __forceinline__ float xor_lane(float v, int mask) {
  int lane = __lane_id();
  int src = (lane ^ mask) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

}  // namespace sa
