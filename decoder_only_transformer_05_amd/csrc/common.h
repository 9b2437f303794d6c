// common.h -- shared definitions for the gfx950 kernels and the host orchestration.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define GPT2_DEVICE_INLINE __device__ __forceinline__

// One wave64 MFMA: acc(32x32) += A(32x2) * B(2x32), fp32 in and out.
// Operand layout: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32].
// Result layout: acc[i] of lane l is element (row 8*(i/4) + 4*(l/32) + i%4, col l % 32).
GPT2_DEVICE_INLINE f32x16 mfma32x32x2(float a, float b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
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

// tanh-form GELU ("llm.c 的中文注解", section 1.9; "60 行 NumPy 代码实现一个 GPT", GELU).
// tanh(u) is evaluated as 1 - 2/(exp(2u)+1), which saturates correctly for large |u|.
#define GPT2_GELU_S 0.7978845608028654f  // sqrt(2/pi)
GPT2_DEVICE_INLINE float gelu_tanh_arg(float x) { return GPT2_GELU_S * (x + 0.044715f * x * x * x); }
GPT2_DEVICE_INLINE float fast_tanh(float u) { return 1.0f - 2.0f / (__expf(2.0f * u) + 1.0f); }
GPT2_DEVICE_INLINE float gelu_fwd(float x) { return 0.5f * x * (1.0f + fast_tanh(gelu_tanh_arg(x))); }
// derivative of the tanh form (section 1.10), with sech^2 = 1 - tanh^2
GPT2_DEVICE_INLINE float gelu_bwd(float x) {
  float th = fast_tanh(gelu_tanh_arg(x));
  return 0.5f * (1.0f + th) +
         0.5f * x * (1.0f - th * th) * GPT2_GELU_S * (1.0f + 3.0f * 0.044715f * x * x);
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
