// Device-side helpers shared by the gfx950 kernels of the MXFP4 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Largest top_k the kernels handle (the ABI limit).
constexpr int MAX_TOPK_DEV = 8;

// Compiler-only ordering point for memory operations (emits nothing).  It
// keeps the compiler from sinking loads towards their first use, so a batch
// of loads is in flight together, and from moving a load across an explicit
// vmcnt wait that counts the loads of one pipeline stage.
__device__ __forceinline__ void order_point() { __asm__ __volatile__("" ::: "memory"); }

// A value the compiler must treat as produced at this point: its uses (and
// the wait for the load that produced it) stay below it.  Keeps address
// arithmetic from being hoisted above loads that should go out first.
__device__ __forceinline__ void hold(uint32_t& v) { __asm__ __volatile__("" : "+v"(v)); }
__device__ __forceinline__ void hold(int& v) { __asm__ __volatile__("" : "+v"(v)); }
// All fields of a wave-uniform record in registers here (one load, before
// any branch on one of them).
__device__ __forceinline__ void hold_uniform(const int4& r) {
  __asm__ __volatile__("" ::"s"(r.x), "s"(r.y), "s"(r.z), "s"(r.w));
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  order_point();
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  order_point();
}

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }


// Two floats -> packed bf16 pair (lo in bits 0..15), rounded to nearest
// even by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// An e8m0 scale byte as the float whose exponent field is that byte; the
// scaled conversions read only the exponent, so byte 0 means 2^-127 and
// byte 255 means NaN.
__device__ __forceinline__ float e8m0_as_scale_operand(uint32_t s) { return __uint_as_float(s << 23); }

// float8_e4m3fn code of v (round to nearest even), saturating to +-448 first:
// the hardware conversion itself turns overflow into NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  v = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xFFu;
}

// Four floats -> four e4m3 codes packed little-endian in a dword.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  c = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
  d = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return uint32_t(r);
}

// ------------------------------------------------------------ FP4 decode

// Nibbles of byte `sel` of `w` -> two bf16 values code * 2^(s-127), packed.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// Eight nibbles (one dword, low nibble first) -> eight bf16 for an MFMA operand.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4_t v;
  v[0] = fp4x2_to_bf16x2<0>(w, scale);
  v[1] = fp4x2_to_bf16x2<1>(w, scale);
  v[2] = fp4x2_to_bf16x2<2>(w, scale);
  v[3] = fp4x2_to_bf16x2<3>(w, scale);
  return __builtin_bit_cast(bf16x8_t, v);
}

// ----------------------------------------------------------- buffer loads
//
// Raw buffer loads with hardware range checking: every dword at or past
// `bytes` reads as zero.  That turns the tails of the tiles (rows past the
// matrix, K past the contracting dimension, tokens past the expert's count)
// into unconditional loads, so the compiler can count outstanding loads
// exactly instead of draining all of them at each conditional one.  Buffers
// must be smaller than 2^31 bytes so that kOOB is out of range for all.

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// a + b for buffer offsets, staying out of range if either one is.
__device__ __forceinline__ uint32_t oob_add(uint32_t a, uint32_t b) { return ((a | b) & kOOB) ? kOOB : a + b; }

__device__ __forceinline__ uint4 buf_load_b128(rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Offset split into a per-lane part (voff, a VGPR) and a wave-uniform part
// (soff, an SGPR): the address arithmetic shared by the wave stays in
// scalar registers.  Range checking: a voff of kOOB (plus any small
// constant) reads zeros whatever soff is; otherwise voff + soff must lie
// inside the buffer.
__device__ __forceinline__ uint4 buf_load_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Buffer-to-LDS form of a 16-byte load: lane i's 16 bytes land at lds_dst +
// 16 i (1 KB per wave), with no registers held while it is in flight; it
// counts in vmcnt like any other load.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t off, const uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds_dst), 16, off, 0, 0, 0);
}

// ------------------------------------------- device-scope hand-off
//
// Rows that one workgroup hands to another workgroup of the same launch
// (which may run on another XCD, behind another L2) are stored and loaded
// at device scope: stores with the sc1 cache policy write through to the
// device's point of coherence, and loads with sc1 read from it, so a reader
// never sees a line its own L2 kept from earlier.  The producer waits for
// its stores (vmcnt 0) before it signals through a device-scope atomic
// counter; the consumer issues its loads only after it has read the
// signal.  (Plain stores would need a write-back of the producer's L2 and
// an invalidate of the consumer's.)

constexpr int kAuxDev = 16;  // cache-policy operand of buffer loads / stores: sc1

__device__ __forceinline__ void buf_store_dev_b64(rsrc_t r, uint32_t off, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kAuxDev);
}

__device__ __forceinline__ uint4 buf_load_dev_b128(rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxDev);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- misc

__device__ __forceinline__ float clamped_swiglu(float gate, float up) {
  // gate <= 7, up in [-7, 7], h = (up + 1) * gate * sigmoid(1.702 * gate)
  float g = __builtin_fminf(gate, 7.0f);
  float u = __builtin_fminf(__builtin_fmaxf(up, -7.0f), 7.0f);
  float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * g));  // v_rcp_f32 (1 ulp)
  return (u + 1.0f) * g * sig;
}

__device__ __forceinline__ float load_param(const void* p, int64_t i, int is_bf16) {
  return is_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

}  // namespace mxmoe
