// Shared device helpers for the gfx950 kernels: element types, conversions,
// MFMA operand vectors and launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/mtgr.h"

namespace mtgr {

// Storage element types.  Conversions to float are exact; conversions from
// float round to nearest even.
typedef __bf16 bf16_t;
typedef _Float16 f16_t;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }

// Raw 16-bit pattern of a float rounded to T (T = bf16_t or f16_t).
template <typename T> __device__ __forceinline__ uint16_t bits16(float x) {
  T h = from_f32<T>(x);
  return __builtin_bit_cast(uint16_t, h);
}
template <typename T> __device__ __forceinline__ float from_bits16(uint16_t b) {
  return to_f32(__builtin_bit_cast(T, b));
}

// 8 x 16-bit MFMA operand (bf16 or f16) held as 4 dwords.
struct op8 {
  u32x4_t v;
};

// D += A * B on a 32x32 output tile with K = 16 (8 elements per lane each).
template <typename T> __device__ __forceinline__ f32x16_t mfma32(const op8& a, const op8& b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mfma32<bf16_t>(const op8& a, const op8& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mfma32<f16_t>(const op8& a, const op8& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a.v),
                                                __builtin_bit_cast(f16x8_t, b.v), c, 0, 0, 0);
}

// Pack two floats as 16-bit values of T into one dword (lo first), one
// v_cvt_pk_* instruction, round to nearest even.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Raw buffer resource over `bytes` bytes from `base`: 16-byte loads at
// offsets at or beyond `bytes` return zeros (hardware range check).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// Every resource built here is wave-uniform.  The base and size are passed
// through readfirstlane so that they stay in scalar registers even when the
// compiler has computed them in vector registers (under scalar register
// pressure it does); a resource it cannot prove uniform would otherwise be
// used inside a per-lane loop around every load and store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* b = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  i32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return __builtin_bit_cast(uint4, x);
}
// 16-byte store through a buffer resource: stores at offsets at or beyond
// the resource's size are dropped by the hardware range check.
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, off, 0, 0);
}

// Index of the calling wave in its workgroup, as a value the compiler knows
// to be the same on every lane (held in a scalar register, so branches on it
// are scalar branches and buffer resources built from it stay scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// LDS transpose read of gfx950: the 16 lanes of each quarter-wave together
// read a 4 (rows) x 16 (columns) block of 16-bit values, lane 4*r + c
// supplying the address of row r, columns 4c..4c+3; lane i then holds
// column i, rows 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds_addr) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(i16x4_t*)lds_addr);
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Sum over the 64 lanes of a wave, result in every lane: DPP moves inside
// each 16-lane row (quad swaps, then rotations by 4 and 8), then the four
// row sums are read into scalar registers and added.
__device__ __forceinline__ float warp_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

}  // namespace mtgr

#define MTGR_LAUNCH_CHECK()                                 \
  do {                                                      \
    hipError_t _e = hipGetLastError();                      \
    if (_e != hipSuccess) return MTGR_ERR_HIP;              \
  } while (0)
