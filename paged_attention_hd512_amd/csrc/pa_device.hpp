// Device-side helpers shared by every libpa kernel: vector types, element conversions,
// the paged address path and wave-level primitives.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Stored KV formats, as kernel template arguments.
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvFp4 = 2;

// ---------------------------------------------------------------- element conversions

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two fp32 -> two bf16 in one dword, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four FP8 E4M3FN codes (one dword) -> four fp32 values, exact.  gfx950's conversion
// instructions read the OCP E4M3FN encoding.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Four FP8 codes -> four bf16 values packed in two dwords.  Exact: every E4M3FN value has
// at most 4 significant bits and an exponent inside bf16's range, so the upper half of
// its fp32 image is the bf16 value.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t w) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  u32x2_t r;
  r[0] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
  r[1] = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
  return r;
}

// Eight E2M1 values (one dword; element 2i is the low nibble of byte i) -> eight fp32,
// exact.  v_cvt_scalef32_pk_f32_fp4 converts the byte `sel`, low nibble first.  Its f32
// scale operand acts through its exponent only (an E8M0 scale: 448 acts as 256), so it
// stays 1 here and E4M3 block scales are multiplied in separately.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float* out) {
  const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
  out[4] = c[0]; out[5] = c[1]; out[6] = d[0]; out[7] = d[1];
}

// Eight E2M1 values (one dword, element 2i in the low nibble of byte i) times a block
// scale, as eight fp16 values: the nibbles convert exactly at scale 1 and the products are
// exact in fp16 when the scale is an E4M3 value (at most 6 significant bits, magnitudes in
// [2^-10, 2688]).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8_t fp4x8_to_f16_scaled(uint32_t w, _Float16 bs) {
  const f16x2_t s2 = {bs, bs};
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Two E2M1 rows a and b (one dword each, element 2i in the low nibble of byte i), column
// by column as fp16 pairs: out[e] = (a[e], b[e]) for e = 0..7, exact.  The nibbles are
// interleaved first (byte i of lo holds a[2i] and b[2i], byte i of hi a[2i+1] and b[2i+1]),
// so each conversion yields one column of both rows.
__device__ __forceinline__ void fp4x8_pair_to_f16x2(uint32_t a, uint32_t b, f16x2_t* out) {
  const uint32_t lo = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
  const uint32_t hi = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 0);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 1);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 1);
  out[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 2);
  out[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 2);
  out[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 1.0f, 3);
  out[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 1.0f, 3);
}

// Two fp32 -> two fp16 in one dword, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One FP8 E4M3FN code (byte `sel` of w) -> fp32, exact.
template <int SEL>
__device__ __forceinline__ float fp8_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// LDS transpose load (ds_read_b64_tr_b16): within each block of 16 lanes, lane i = 4c + e
// receives element e of the 8-byte rows addressed by lanes c, c+4, c+8 and c+12.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// ---------------------------------------------------------------- paged address path
//
// Logical token t of a request whose page list starts at `pages` is slot t % P of page
// pages[t / P] (page table layout of the Triton page, section "Approach"); every kernel
// and the debug gather resolve keys through these two functions.

__device__ __forceinline__ void token_page_slot(const int32_t* __restrict__ pages, int32_t t,
                                                int32_t page_size, int32_t& page,
                                                int32_t& slot) {
  const int32_t j = t / page_size;
  page = pages[j];
  slot = t - j * page_size;
}

// Same, with the division replaced by a shift when page_size = 2^page_shift
// (page_shift < 0: any page size).
__device__ __forceinline__ void token_page_slot_fast(const int32_t* __restrict__ pages, int32_t t,
                                                     int32_t page_size, int32_t page_shift,
                                                     int32_t& page, int32_t& slot) {
  if (page_shift >= 0) {
    page = pages[t >> page_shift];
    slot = t & (page_size - 1);
  } else {
    token_page_slot(pages, t, page_size, page, slot);
  }
}

__device__ __forceinline__ int64_t row_elem_offset(int32_t page, int32_t head, int32_t slot,
                                                   int64_t stride_page, int64_t stride_head,
                                                   int64_t stride_token) {
  return (int64_t)page * stride_page + (int64_t)head * stride_head + (int64_t)slot * stride_token;
}

// Wave-uniform variant: reads the page table through the constant address space, so the
// index load is a scalar load (it is then counted apart from vector memory operations).
typedef const int32_t __attribute__((address_space(4))) * const_i32_ptr;
__device__ __forceinline__ void token_page_slot_uniform(const int32_t* pages, int32_t t,
                                                        int32_t page_size, int32_t page_shift,
                                                        int32_t& page, int32_t& slot) {
  const_i32_ptr cp = (const_i32_ptr)pages;
  t = __builtin_amdgcn_readfirstlane(t);
  int32_t j;
  if (page_shift >= 0) {
    j = t >> page_shift;
    slot = t & (page_size - 1);
  } else {
    j = t / page_size;
    slot = t - j * page_size;
  }
  page = cp[j];
}

// ---------------------------------------------------------------- wave primitives

// Orders this wave's LDS writes before its later LDS reads by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS accesses only: global loads in flight stay in flight
// (a full __syncthreads would first wait for every outstanding vector memory load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane max / sum with the lane 32 (or 16) apart, on the VALU: each swap returns, per
// lane, the lane's own value in one result and its partner's in the other.
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

__device__ __forceinline__ int shfl_i(int v, int src_lane) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ __forceinline__ int64_t shfl_i64(int64_t v, int src_lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
// The value of v in lane src (wave-uniform src), as a scalar.
__device__ __forceinline__ int64_t readlane_i64(int64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)((uint64_t)v >> 32), src);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace pa
