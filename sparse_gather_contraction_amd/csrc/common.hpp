// common.hpp — device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace disco {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef _Float16 f16_t;   // IEEE binary16

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays NaN (quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ float load_elem(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_elem(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(bf16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ float load_elem(const f16_t *p, int64_t i) { return (float)p[i]; }
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default rounding mode)
__device__ __forceinline__ void store_elem(f16_t *p, int64_t i, float v) { p[i] = (f16_t)v; }

}  // namespace disco
