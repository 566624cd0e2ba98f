// Shared device helpers for the gfx950 kernels: vector types, bf16 rounding,
// buffer resources and LDS-direct loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;                                            // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Buffer resource word 3 for raw (untyped, stride 0) buffers on gfx9-class parts.
#define TP_BUFFER_RSRC_WORD3 0x00020000

// Offsets at or beyond this are outside every buffer we build: loads return 0.
#define TP_OOB_OFFSET 0x80000000u

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float32 -> bf16 via the hardware pack instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           TP_BUFFER_RSRC_WORD3);
}

// 16 bytes per lane from a buffer straight into LDS.  The destination of lane
// L is lds_wave_base + 16 * L; lds_wave_base must be uniform across the wave.
// A voffset outside the buffer's range stores zeros.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds_wave_base), 16, voffset, 0, 0, 0);
}

// Same, with a wave-uniform byte offset added from a scalar register.  Lanes
// that must read zeros keep voffset itself out of range; for the others
// voffset + soffset must stay inside the buffer.
__device__ __forceinline__ void buffer_load_lds16_so(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base,
                                                     uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds_wave_base), 16, voffset, (int)soffset, 0, 0);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, 0, 0));
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ u32x4 lds_read16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 lds_read8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Transpose of a 4 x 4 block held by a quad of lanes (q = lane & 3): on
// entry a[e] is element (row e, column q); on exit a[c] is element (row q,
// column c).  Two butterfly rounds over lane bit 0 and lane bit 1, each a
// DPP quad permutation plus selects.
__device__ __forceinline__ float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(float (&a)[4], int q) {
  const bool b0 = (q & 1) != 0, b1 = (q & 2) != 0;
#pragma unroll
  for (int e = 0; e < 4; e += 2) {  // rows/columns differing in bit 0
    const float r = quad_xor1(b0 ? a[e] : a[e + 1]);
    if (b0) a[e] = r; else a[e + 1] = r;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {  // rows/columns differing in bit 1
    const float r = quad_xor2(b1 ? a[e] : a[e + 2]);
    if (b1) a[e] = r; else a[e + 2] = r;
  }
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }
// For bf16 outputs: the hardware reciprocal (about 1 ulp) instead of a
// correctly rounded division.  x -> -inf gives -0, x -> +inf gives x.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
