// Shared device helpers for the gfx950 kernels of libindexpool.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ip {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- cache layout
// Token t of sequence b: paged -> page_table[b][t / page_tokens] * page_tokens + t % page_tokens,
// contiguous -> b * seq_stride + t.  Pooled block j uses page_tokens / 4 and seq_stride / 4.
struct Layout {
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t page_tokens;
  int64_t seq_stride;

  // token positions and block indices are below 2^31 (int32 sequence lengths), so
  // the in-page split is a 32-bit unsigned division
  __device__ __forceinline__ int64_t tok_row(int b, int64_t t) const {
    if (page_table) {
      const uint32_t pt = (uint32_t)page_tokens, tt = (uint32_t)t;
      const uint32_t pi = tt / pt;
      const int64_t pg = page_table[(int64_t)b * max_pages + pi];
      return pg * page_tokens + (tt - pi * pt);
    }
    return (int64_t)b * seq_stride + t;
  }
  __device__ __forceinline__ int64_t pool_row(int b, int64_t j) const {
    if (page_table) {
      const uint32_t pr = (uint32_t)page_tokens >> 2, jj = (uint32_t)j;
      const uint32_t pi = jj / pr;
      const int64_t pg = page_table[(int64_t)b * max_pages + pi];
      return pg * pr + (jj - pi * pr);
    }
    return (int64_t)b * (seq_stride >> 2) + j;
  }
};

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even; inputs here are finite
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats -> packed bf16 pair (lo in the low half), round to nearest even, by
// gfx950's v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- fp8 e4m3fn
// Four codes (one dword, byte 0 first) -> four floats, by the hardware converter
// (gfx950 decodes the OCP e4m3fn format: bias 7, max 448).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

// Eight codes -> eight bf16 (exact: every e4m3fn value is a bf16 value, so the
// top half of the float is the bf16 pattern).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  float f[8];
  fp8x4_to_f32(w0, f);
  fp8x4_to_f32(w1, f + 4);
  u32x4_t p;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xFFFF0000u);
  return __builtin_bit_cast(bf16x8_t, p);
}

// The same widening by gfx950's v_cvt_scalef32_pk_bf16_fp8 with scale 1 (two codes
// per instruction; word_sel picks bytes 0-1 or 2-3, the lower byte to the lower half).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8_pk(uint32_t w0, uint32_t w1) {
  u32x4_t p;
  p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, p);
}

// float -> e4m3fn code, round to nearest even.  |x| must already be <= 448.
// Normal range (|x| >= 2^-6): round the float's mantissa to 3 bits, then rebias the
// exponent from 127 to 7.  Below 2^-6 the code is the nearest multiple of 2^-9
// (8 * 2^-9 = 2^-6 is code 0x08, so the two branches meet).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                       // < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // 8-bit exp + 3-bit mantissa
    code = r - (120u << 3);
  }
  return code | sign;
}

// ---------------------------------------------------------------- order-preserving keys
// float -> uint32 whose unsigned order is the float order (-0 folded into +0).
// Key 0 is never produced for a non-NaN float and marks "no element".
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding global
// loads (on gfx9 vmcnt counts loads too), so prefetches stay in flight across it.
// The "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace ip

namespace ip {
// ---------------------------------------------------------------- wave-level DPP
// Cross-lane steps on the VALU (DPP) instead of ds_bpermute: a reduction or scan
// over 64 lanes is six dependent VALU ops rather than six LDS round trips.
// DPP controls (GFX9): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_shr:n =
// 0x110+n, row_mirror = 0x140, row_half_mirror = 0x141, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.  Lanes whose source is masked off get `old`.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROW_MASK, 0xF,
                                                    BOUND_ZERO));
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111, 0xF, true>(0, x);
  x += dpp_i<0x112, 0xF, true>(0, x);
  x += dpp_i<0x114, 0xF, true>(0, x);
  x += dpp_i<0x118, 0xF, true>(0, x);
  x += dpp_i<0x142, 0xA>(0, x);
  x += dpp_i<0x143, 0xC>(0, x);
  return x;
}

// value of lane 63 (wave-uniform)
__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }
__device__ __forceinline__ float lane63f(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// sum / max / min over the 64 lanes of a wave, returned to every lane
__device__ __forceinline__ int wave_sum(int x) {
  x += dpp_i<0xB1>(0, x);
  x += dpp_i<0x4E>(0, x);
  x += dpp_i<0x141>(0, x);
  x += dpp_i<0x140>(0, x);
  x += dpp_i<0x142, 0xA>(0, x);
  x += dpp_i<0x143, 0xC>(0, x);
  return lane63(x);
}
__device__ __forceinline__ float wave_sum_f(float x) {
  x += dpp_f<0xB1>(0.f, x);
  x += dpp_f<0x4E>(0.f, x);
  x += dpp_f<0x141>(0.f, x);
  x += dpp_f<0x140>(0.f, x);
  x += dpp_f<0x142, 0xA>(0.f, x);
  x += dpp_f<0x143, 0xC>(0.f, x);
  return lane63f(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x4E>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x141>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x140>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x142, 0xA>(-INFINITY, x));
  x = fmaxf(x, dpp_f<0x143, 0xC>(-INFINITY, x));
  return lane63f(x);
}
__device__ __forceinline__ float wave_min(float x) {
  x = fminf(x, dpp_f<0xB1>(INFINITY, x));
  x = fminf(x, dpp_f<0x4E>(INFINITY, x));
  x = fminf(x, dpp_f<0x141>(INFINITY, x));
  x = fminf(x, dpp_f<0x140>(INFINITY, x));
  x = fminf(x, dpp_f<0x142, 0xA>(INFINITY, x));
  x = fminf(x, dpp_f<0x143, 0xC>(INFINITY, x));
  return lane63f(x);
}
}  // namespace ip
