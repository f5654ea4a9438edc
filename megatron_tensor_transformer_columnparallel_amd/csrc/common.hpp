// Shared device helpers for the gfx950 kernels: bf16 storage conversion,
// 16-byte vector types, and host-side error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/tpshard.h"

namespace tps {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element-type traits: storage type and conversions to/from fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float load(const float* p) { return *p; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Store 4 consecutive values (fp32 in registers) to T storage, bounds-checked
// element-wise when `nvalid` < 4.  Aligned vector store when complete.
template <typename T>
__device__ __forceinline__ void store4(T* p, const float v[4], int nvalid);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float v[4], int nvalid) {
  if (nvalid >= 4) {
    f32x4_t x = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p) = x;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nvalid) p[i] = v[i];
  }
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float v[4], int nvalid) {
  if (nvalid >= 4) {
    u32x2_t x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2_t*>(p) = x;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nvalid) p[i] = f32_to_bf16(v[i]);
  }
}

// Load 4 consecutive elements as fp32 (element-wise when incomplete).
template <typename T>
__device__ __forceinline__ void load4(const T* p, float v[4], int nvalid);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float v[4], int nvalid) {
  if (nvalid >= 4) {
    f32x4_t x = *reinterpret_cast<const f32x4_t*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = i < nvalid ? p[i] : 0.f;
  }
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float v[4], int nvalid) {
  if (nvalid >= 4) {
    u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
    v[0] = bf16lo(x[0]); v[1] = bf16hi(x[0]); v[2] = bf16lo(x[1]); v[3] = bf16hi(x[1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = i < nvalid ? bf16_to_f32(p[i]) : 0.f;
  }
}

// 8 consecutive elements <-> fp32 (16-byte aligned for bf16, 32 for fp32),
// element-wise when fewer than 8 are valid.
template <typename T>
__device__ __forceinline__ void store8(T* p, const float v[8], int nvalid) {
  if (nvalid >= 8) {
    store4<T>(p, v, 4);
    store4<T>(p + 4, v + 4, 4);
  } else {
    store4<T>(p, v, nvalid);
    if (nvalid > 4) store4<T>(p + 4, v + 4, nvalid - 4);
  }
}
template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[8], int nvalid) {
  if (nvalid >= 8) {
    load4<T>(p, v, 4);
    load4<T>(p + 4, v + 4, 4);
  } else {
    load4<T>(p, v, nvalid);
    if (nvalid > 4) load4<T>(p + 4, v + 4, nvalid - 4);
    else { v[4] = v[5] = v[6] = v[7] = 0.f; }
  }
}
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float v[8], int nvalid) {
  if (nvalid >= 8) {
    u32x4_t x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
    *reinterpret_cast<u32x4_t*>(p) = x;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nvalid) p[i] = f32_to_bf16(v[i]);
  }
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float v[8], int nvalid) {
  if (nvalid >= 8) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) { v[2 * w] = bf16lo(x[w]); v[2 * w + 1] = bf16hi(x[w]); }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < nvalid ? bf16_to_f32(p[i]) : 0.f;
  }
}

// GELU with the erf form and its derivative (fp32): gelu(x) = x Phi(x) and
// gelu'(x) = Phi(x) + x phi(x), with Phi the standard normal CDF and phi its
// density.  Phi comes from the complementary error function,
// Phi(x) = erfc(-x / sqrt 2) / 2, evaluated with the Chebyshev-fitted formula
// of Numerical Recipes (2nd ed., section 6.2, "erfcc"):
//   t = 1 / (1 + z/2),  erfc(z) = t exp(-z^2 + poly(t)),  z >= 0,
// whose fractional error is below 1.2e-7 for every z >= 0.  With z = |x|/sqrt 2
// the tail mass c = erfc(z)/2 is Phi(x) for x < 0 and 1 - Phi(x) for x >= 0,
// so both tails keep that relative accuracy (far below bf16 rounding).  One
// reciprocal and one exponential per element for gelu, two for gelu'.
__device__ __forceinline__ float erfcc_poly(float t) {
  // -1.26551223 + t (1.00002368 + t (0.37409196 + ... + t 0.17087277))
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  return fmaf(p, t, -1.26551223f);
}
__device__ __forceinline__ float gelu_f(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));   // 1 + z/2 >= 1: hardware reciprocal, 1 ulp
  const float c = 0.5f * t * __expf(fmaf(-z, z, erfcc_poly(t)));   // erfc(z) / 2
  return x * (x >= 0.f ? 1.0f - c : c);
}
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));   // 1 + z/2 >= 1: hardware reciprocal, 1 ulp
  const float g = __expf(-z * z);                                   // exp(-x^2 / 2)
  const float c = 0.5f * t * g * __expf(erfcc_poly(t));             // erfc(z) / 2
  const float cdf = x >= 0.f ? 1.0f - c : c;
  return fmaf(x * 0.39894228040143268f, g, cdf);                    // Phi(x) + x phi(x)
}

// ---------------------------------------------------------------- host side

// Records a thread-local error message and returns `s`.
tps_status set_error(tps_status s, const std::string& msg);
tps_status check_launch(const char* what);

// Launch tracing (measurement support; see tps_trace_start in tpshard.h).
// ApiScope names the entry point that the launches of its lifetime belong
// to; TraceScope brackets one kernel launch with a pair of timing events on
// the launch's stream while tracing is on and the launch's name matches the
// filter.  Both cost one flag test when tracing is off.
extern bool g_trace_on;
struct ApiScope {
  const char* prev;
  explicit ApiScope(const char* api);
  ~ApiScope();
};
struct TraceScope {
  int slot = -1;
  hipStream_t stream = nullptr;
  TraceScope() = default;
  TraceScope(hipStream_t st, const char* kernel, const char* detail = nullptr) {
    if (g_trace_on) begin(st, kernel, detail);
  }
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;
  ~TraceScope() {
    if (slot >= 0) end();
  }
  void begin(hipStream_t st, const char* kernel, const char* detail);
  void end();
};

// "<v1,v2,...>" from the "[A = v1, B = v2, ...]" part of a template
// function's __PRETTY_FUNCTION__ (namespace and element-type spelled short).
std::string template_args(const char* pretty);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t elem_bytes(tps_dtype dt) { return dt == TPS_BF16 ? 2 : 4; }
inline int64_t vec_elems(tps_dtype dt) { return dt == TPS_BF16 ? 8 : 4; }

}  // namespace tps
