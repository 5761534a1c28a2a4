// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_WAVE 64

typedef uint16_t bf16_t;                                          // raw bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));        // MFMA operand
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> f32 is exact: the bf16 bits are the top half of the f32.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two f32 -> bf16 (lo in bits 0..15), round to nearest, ties to even: one
// v_cvt_pk_bf16_f32.  On every non-NaN f32 it equals rounding the bits by
// hand, (u + 0x7FFF + ((u >> 16) & 1)) >> 16, denormals included (checked
// exhaustively on gfx950); a NaN stays a NaN.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// Logistic sigmoid from the hardware 2^x and reciprocal (v_exp_f32, v_rcp_f32,
// about 1 ulp each): 1 / (1 + 2^(-z*log2(e))).  Overflow of 2^x for very
// negative z gives 1/inf = 0, the correct limit.  Used where the result is
// rounded to bf16 or feeds a bf16 product.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}
__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_fast(z); }

// Splits two fp32 values a, b exactly into three bf16 parts each, v = hi +
// mid + lo, packed in pairs (a in the low half): hi = the top 16 bits
// (truncation, so v - hi is exact), mid = the top 16 bits of r1 = v - hi, lo
// = the top 16 bits of r2 = r1 - mid, which has at most 8 significant bits
// left and so is exact (8 + 8 + 8 bits hold the 24-bit fp32 significand, in
// the normal range).  Each pair is one byte permutation of the two words.
// Against a bf16 factor, each part's product is exact in fp32.
__device__ __forceinline__ void split3x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  constexpr uint32_t TOP = 0x07060302u;   // bytes 2, 3 of the second operand, then of the first
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  hi = __builtin_amdgcn_perm(ub, ua, TOP);
  const float ra = a - __uint_as_float(ua & 0xFFFF0000u), rb = b - __uint_as_float(ub & 0xFFFF0000u);
  const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
  mid = __builtin_amdgcn_perm(vb, va, TOP);
  const float sa = ra - __uint_as_float(va & 0xFFFF0000u), sb = rb - __uint_as_float(vb & 0xFFFF0000u);
  lo = __builtin_amdgcn_perm(__float_as_uint(sb), __float_as_uint(sa), TOP);
}

// Raw buffer resource over [base, base + bytes), bytes >= 0: loads at
// offsets past the end read zeros (offsets of 2^31 and up are always past it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Wave-uniform copies of values that are uniform by construction: a buffer
// resource the compiler cannot prove uniform costs a loop over the lanes at
// every load that uses it.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint32_t lo = uni((uint32_t)(uint64_t)v), hi = uni((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const void* uni(const void* ptr) {
  return reinterpret_cast<const void*>((uintptr_t)uni((int64_t)(uintptr_t)ptr));
}

// Lane mask of lanes strictly below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = threadIdx.x & (MOE_WAVE - 1);
  return l == 0 ? 0ull : (~0ull >> (MOE_WAVE - l));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// Host-side launch check: returns MOE_EHIP from the enclosing function.
#define MOE_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipPeekAtLastError() != hipSuccess) {                \
      (void)hipGetLastError();                               \
      return MOE_EHIP;                                       \
    }                                                        \
  } while (0)

static inline hipStream_t moe_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Runs MACRO(K) with K the compile-time value of runtime k in [1, MOE_MAX_TOPK]:
// per-token kernels keep their k row addresses in registers and issue all k
// row loads together, which a runtime-bounded loop would serialise.
#define MOE_DISPATCH_K(k, MACRO)                                             \
  switch (k) {                                                              \
    case 1: MACRO(1); break;   case 2: MACRO(2); break;                     \
    case 3: MACRO(3); break;   case 4: MACRO(4); break;                     \
    case 5: MACRO(5); break;   case 6: MACRO(6); break;                     \
    case 7: MACRO(7); break;   case 8: MACRO(8); break;                     \
    case 9: MACRO(9); break;   case 10: MACRO(10); break;                   \
    case 11: MACRO(11); break; case 12: MACRO(12); break;                   \
    case 13: MACRO(13); break; case 14: MACRO(14); break;                   \
    case 15: MACRO(15); break; case 16: MACRO(16); break;                   \
    default: return MOE_ENOTSUP;                                            \
  }

// Number of compute units of the current device (cached per device id).
int moe_num_cus();
