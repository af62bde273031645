// Shared device/host helpers of the gfx950 FP8 block-scaled GEMM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;     // K-group / scale-block edge (fine-grained scaling granularity)
constexpr int kKAlign = 16;     // K must be a multiple of this (16-byte rows); a last K group may be partial
constexpr float kE4M3Max = 448.0f;

// Status codes mirror include/dg.h.
enum Status : int { kOk = 0, kInvalidArg = -1, kUnsupported = -2, kWorkspace = -3, kHip = -4 };

// Records a thread-local error message (implemented in api.cpp).
int set_error(int status, const char* fmt, ...);

// DG_DEBUG set in the environment (read at every call): device-side layout checks and a log of
// each GEMM's plan on stderr (implemented in api.cpp).
bool debug_enabled();

// Two fp32 -> two bf16, round to nearest even (a NaN stays a NaN, made quiet), packed little-endian
// (lo in bits 0-15): one v_cvt_pk_bf16_f32.  On MI355X it equals the bit-level rounding
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 on every finite fp32 input, and (u >> 16) | 0x40 on NaNs
// (checked exhaustively over all 2^32 inputs).
__device__ __forceinline__ uint32_t pack2_bf16_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
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

// max over each 16-lane row of the wave, by DPP lane swaps (VALU, no LDS crossbar): xor 1 and
// xor 2 inside quads, then the half-row and row mirrors.  Every lane gets its row's maximum.
__device__ __forceinline__ float row16_max(float v) {
  auto dpp = [](float x, auto ctrl_c) {
    constexpr int ctrl = decltype(ctrl_c)::value;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xf, 0xf, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));   // row_mirror
  return v;
}

// max over each 32-lane half of the wave (lanes 0-31 and 32-63), returned to every lane of the half.
__device__ __forceinline__ float half_wave_max(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
}

// max over the whole wave, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Four consecutive activations as fp32: fp32 input as is, bf16 input widened exactly (a bf16
// value is the upper half of the fp32 word).  Streaming (nontemporal) loads: each is read once.
__device__ __forceinline__ v4f load4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ v4f load4(const uint16_t* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return v4f{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
             __uint_as_float(w.y & 0xffff0000u)};
}

// One 1 x 128 group held by a half-wave (4 consecutive values per lane; values past k are zero):
// s = amax / 448 (1 when amax = 0, IEEE division) into `s` on every lane, and the lane's 4 E4M3
// bytes of fl32(v / s), rounded to nearest even and saturated, as the return value.  Fine-grained
// scaling as proposed with DeepSeek-V3 (机器之心 DeepGEMM report, opening section).
__device__ __forceinline__ uint32_t quant_group4(v4f v, float& s) {
  const float amax = half_wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  s = amax == 0.0f ? 1.0f : amax / kE4M3Max;
  return pack4_e4m3(clamp448(v.x / s), clamp448(v.y / s), clamp448(v.z / s), clamp448(v.w / s));
}

}  // namespace dg
