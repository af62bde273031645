// Shared device/host helpers of the gfx950 FP8 block-scaled GEMM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;     // K-group / scale-block edge (fine-grained scaling granularity)
constexpr float kE4M3Max = 448.0f;

// Status codes mirror include/dg.h.
enum Status : int { kOk = 0, kInvalidArg = -1, kUnsupported = -2, kWorkspace = -3, kHip = -4 };

// Records a thread-local error message (implemented in api.cpp).
int set_error(int status, const char* fmt, ...);

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four fp32 values (already in [-448, 448]) -> four E4M3 bytes, packed little-endian.
// The hardware convert rounds to nearest even in the default round mode; the
// sign bit of every input is ORed in afterwards so that negative values that
// round to zero (and -0.0) give 0x80, whatever the converter does with them.
__device__ __forceinline__ uint32_t pack4_e4m3(float y0, float y1, float y2, float y3) {
  uint32_t w = 0;
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)w, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)w, true);
  const uint32_t sign = ((__float_as_uint(y0) >> 31) << 7) | ((__float_as_uint(y1) >> 31) << 15) |
                        ((__float_as_uint(y2) >> 31) << 23) | ((__float_as_uint(y3) >> 31) << 31);
  return w | sign;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); }

}  // namespace dg
