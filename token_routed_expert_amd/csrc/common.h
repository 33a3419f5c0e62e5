// Shared device helpers for the routed-expert MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace tre {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte access

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Packs two fp32 values into two bf16 (low half = a), round to nearest even,
// NaN stays NaN: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Element loads/stores by storage dtype (fp32 or bf16), used by the
// memory-bound kernels and by the fp32 GEMM.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// SiLU and the logistic function with gfx950's reciprocal (v_rcp_f32, about
// 1 ulp) in place of an IEEE division: the fused SwiGLU epilogues evaluate
// them for every output element, and the results are rounded to bf16 (or
// compared at 1e-4 in fp32) far above that error.  Measured on the Qwen3
// shape: fc2 dgrad 2 %, fc1 forward 0.5-1.3 % faster.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_f32(z); }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace tre

// Host-side launch helpers shared by the translation units of the library.
#define TRE_LAUNCH_CHECK()                                   \
  do {                                                       \
    hipError_t _e = hipGetLastError();                       \
    if (_e != hipSuccess) return MOE_ERR_HIP;                \
  } while (0)
