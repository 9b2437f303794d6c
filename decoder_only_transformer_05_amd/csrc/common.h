// common.h -- shared definitions for the gfx950 kernels and the host orchestration.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define GPT2_DEVICE_INLINE __device__ __forceinline__

// bf16 storage: the upper 16 bits of an IEEE fp32 value. Conversion to bf16 rounds to
// nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950).
typedef uint16_t bf16_t;
GPT2_DEVICE_INLINE float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
GPT2_DEVICE_INLINE bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Four consecutive elements of an activation tensor, fp32 or bf16 storage, as fp32
// (16- or 8-byte aligned accesses).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
GPT2_DEVICE_INLINE f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
GPT2_DEVICE_INLINE f32x4 ld4(const bf16_t* p) {
  const u32x2_t u = *reinterpret_cast<const u32x2_t*>(p);
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
               __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
}
// The same four elements kept as stored (fp32: 16 bytes, bf16: 8 bytes) until widened, so a
// prefetched bf16 row takes half the registers.
template <typename T> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<bf16_t> { typedef u32x2_t type; };
GPT2_DEVICE_INLINE f32x4 raw4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
GPT2_DEVICE_INLINE u32x2_t raw4(const bf16_t* p) { return *reinterpret_cast<const u32x2_t*>(p); }
GPT2_DEVICE_INLINE f32x4 widen4(f32x4 v) { return v; }
GPT2_DEVICE_INLINE f32x4 widen4(u32x2_t u) {
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
               __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
}
GPT2_DEVICE_INLINE void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
GPT2_DEVICE_INLINE void st4(bf16_t* p, f32x4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{lo, hi};
}
GPT2_DEVICE_INLINE float ld1(const float* p) { return *p; }
GPT2_DEVICE_INLINE float ld1(const bf16_t* p) { return bf16_to_f32(*p); }
GPT2_DEVICE_INLINE void st1(float* p, float v) { *p = v; }
GPT2_DEVICE_INLINE void st1(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// fp16 storage (IEEE binary16: 11 significant bits, largest finite 65504). Conversion from
// fp32 rounds to nearest, ties to even; values beyond the range become infinities.
typedef _Float16 f16_t;
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
GPT2_DEVICE_INLINE float f16_to_f32(f16_t h) { return (float)h; }
GPT2_DEVICE_INLINE f16_t f32_to_f16(float f) { return (f16_t)f; }
GPT2_DEVICE_INLINE f32x4 ld4(const f16_t* p) {
  return __builtin_convertvector(*reinterpret_cast<const f16x4_t*>(p), f32x4);
}
template <> struct Raw4<f16_t> { typedef f16x4_t type; };
GPT2_DEVICE_INLINE f16x4_t raw4(const f16_t* p) { return *reinterpret_cast<const f16x4_t*>(p); }
GPT2_DEVICE_INLINE f32x4 widen4(f16x4_t v) { return __builtin_convertvector(v, f32x4); }
GPT2_DEVICE_INLINE void st4(f16_t* p, f32x4 v) {
  *reinterpret_cast<f16x4_t*>(p) = __builtin_convertvector(v, f16x4_t);
}
GPT2_DEVICE_INLINE float ld1(const f16_t* p) { return f16_to_f32(*p); }
GPT2_DEVICE_INLINE void st1(f16_t* p, float v) { *p = f32_to_f16(v); }

// 16-bit storage formats of the mixed-precision steps, for kernels templated on them:
// the bits of two values rounded from fp32 packed into one word (a in the low half), and
// one value's bits widened to fp32.
template <typename TS> struct Half16;
template <> struct Half16<bf16_t> {
  static GPT2_DEVICE_INLINE uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  }
  static GPT2_DEVICE_INLINE float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static GPT2_DEVICE_INLINE float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
};
template <> struct Half16<f16_t> {
  static GPT2_DEVICE_INLINE uint32_t pack2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, f32_to_f16(a)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, f32_to_f16(b)) << 16);
  }
  static GPT2_DEVICE_INLINE float lo(uint32_t w) {
    return f16_to_f32(__builtin_bit_cast(f16_t, (uint16_t)(w & 0xFFFFu)));
  }
  static GPT2_DEVICE_INLINE float hi(uint32_t w) {
    return f16_to_f32(__builtin_bit_cast(f16_t, (uint16_t)(w >> 16)));
  }
};

// Exact split of fp32 values into three bf16 parts, x = hi + mid + lo: hi is x rounded to
// bf16 (8 significand bits), mid the remainder x - hi rounded to bf16, lo what remains.
// x - hi is exact in fp32 (hi is within a factor 2 of x) and, being a multiple of the last
// significand bit of x below 2^-8 |x|, has at most 16 significant bits; after mid at most 8
// are left, so lo is that remainder exactly (down to |x| ~ 2^-110, where lo leaves the
// normal bf16 range). |mid| <= 2^-8 |x| and |lo| <= 2^-16 |x|. Used by the kernels that form
// fp32 products as six bf16 MFMA products of the parts.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two values rounded to bf16 by one v_cvt_pk_bf16_f32 (a in the low half)
GPT2_DEVICE_INLINE uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// x0, x1 -> their packed (hi, mid, lo) pairs
GPT2_DEVICE_INLINE void split2(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_pair(x0, x1);
  const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
  mid = bf16_pair(r0, r1);
  const float s0 = r0 - __uint_as_float(mid << 16), s1 = r1 - __uint_as_float(mid & 0xFFFF0000u);
  lo = bf16_pair(s0, s1);
}
// eight values (two float4s) -> the three parts, 8 bf16 each in value order
GPT2_DEVICE_INLINE void split8(f32x4 x, f32x4 y, u32x4& hi, u32x4& mid, u32x4& lo) {
  uint32_t h0, h1, h2, h3, m0, m1, m2, m3, l0, l1, l2, l3;
  split2(x[0], x[1], h0, m0, l0);
  split2(x[2], x[3], h1, m1, l1);
  split2(y[0], y[1], h2, m2, l2);
  split2(y[2], y[3], h3, m3, l3);
  hi = u32x4{h0, h1, h2, h3};
  mid = u32x4{m0, m1, m2, m3};
  lo = u32x4{l0, l1, l2, l3};
}

// One wave64 MFMA: acc(32x32) += A(32x2) * B(2x32), fp32 in and out.
// Operand layout: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32].
// Result layout: acc[i] of lane l is element (row 8*(i/4) + 4*(l/32) + i%4, col l % 32).
GPT2_DEVICE_INLINE f32x16 mfma32x32x2(float a, float b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
}

// Workgroups of a launch are dealt to the 8 XCDs of the chip round-robin (hardware block i
// runs on XCD i % 8), and each XCD has its own L2. This maps the hardware block id to a
// logical id such that logical ids [x*n/8, (x+1)*n/8) all run on XCD x, so neighbouring
// logical tiles (which read the same operand panels) share one L2.
GPT2_DEVICE_INLINE int xcd_logical_block(int bid, int nblocks) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return xcd * per + min(xcd, rem) + idx;
}

GPT2_DEVICE_INLINE float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
GPT2_DEVICE_INLINE float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// tanh-form GELU ("llm.c 的中文注解", sections 1.9 and 1.10; "60 行 NumPy 代码实现一个 GPT",
// GELU): gelu(x) = 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated through s = sigmoid(2u), using 1 + tanh(u) = 2s and sech^2(u) = 4 s (1 - s), so
// neither the function nor its derivative subtracts nearly equal numbers for negative x
// (1 + tanh(u) computed directly loses all its bits there). u is clamped to +-30, where s
// is 0 or 1 to fp32 precision, so exp cannot overflow. The reciprocal is the hardware
// v_rcp_f32 (1 ulp) rather than an IEEE division, which costs about ten instructions in
// the GEMM epilogues that apply GELU to every output.
#define GPT2_GELU_S 0.7978845608028654f  // sqrt(2/pi)
GPT2_DEVICE_INLINE float gelu_u(float x) {
  return fminf(fmaxf(GPT2_GELU_S * (x + 0.044715f * x * x * x), -30.f), 30.f);
}
GPT2_DEVICE_INLINE float gelu_fwd(float x) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * gelu_u(x)));
  return x * s;
}
// d gelu / dx = s + 2 x s (1 - s) u'(x), u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2)
GPT2_DEVICE_INLINE float gelu_bwd(float x) {
  const float e = __expf(-2.0f * gelu_u(x));
  const float s = __builtin_amdgcn_rcpf(1.0f + e);
  const float one_minus_s = e * s;
  return s + 2.0f * x * s * one_minus_s * GPT2_GELU_S * (1.0f + 3.0f * 0.044715f * x * x);
}

// Error reporting shared by the translation units of the library.
namespace gpt2 {
void set_global_error(const char* fmt, ...);
}

#define GPT2_HIP_OK(expr)                                                                 \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) {                                                             \
      gpt2::set_global_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),     \
                             __FILE__, __LINE__);                                       \
      return -6;                                                                        \
    }                                                                                   \
  } while (0)
