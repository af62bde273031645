// Fine-grained FP8 quantizers for gfx950.
//
// Fine-grained scaling as proposed with DeepSeek-V3 (机器之心 DeepGEMM report,
// opening section), E4M3 data (ai.abqq.net DeepGEMM summary, section 3):
//   amax = max |x| over a group, s = amax / 448 (s = 1 for amax = 0),
//   q = E4M3 round-to-nearest-even (saturating) of fl32(x / s).
// Both divisions are IEEE fp32 divisions (the library is built without fast
// math), so bytes and scales are bit-exact with any correct implementation.
//
// Both kernels are HBM-bound streaming kernels (read 4 B, write 1 B + 1/32 B
// per element): 16-byte coalesced loads, several loads in flight per lane.
#include "common.hpp"

namespace dg {

// ---------------------------------------------------------------------------
// 1 x 128 groups along K (activations), for `groups` stacked (m, k) matrices.
// A half-wave (32 lanes x 4 floats) owns one 128-wide group; consecutive
// half-waves take consecutive rows of the same K group so that the MN-major
// scale stores are contiguous.  Group index gi = (g * KB + kb) * m + row.
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 256;
constexpr int kTokUnroll = 4;   // groups per lane per iteration (loads in flight)

__global__ __launch_bounds__(kTokThreads) void quant_token_group_kernel(
    const float* __restrict__ x, int64_t m, int64_t k, uint8_t* __restrict__ q,
    float* __restrict__ sa, int64_t ld_sa, int64_t groups) {
  const int lane = threadIdx.x & 31;
  const int64_t half_waves = ((int64_t)gridDim.x * kTokThreads) >> 5;
  const int64_t first = ((int64_t)blockIdx.x * kTokThreads + threadIdx.x) >> 5;

  for (int64_t base = first; base < groups; base += half_waves * kTokUnroll) {
    v4f v[kTokUnroll];
#pragma unroll
    for (int u = 0; u < kTokUnroll; ++u) {
      const int64_t gi = base + u * half_waves;
      if (gi < groups) {
        const int64_t gkb = gi / m, row = gi - gkb * m;      // gkb = g * KB + kb
        const int64_t kbc = k / kGroup, g = gkb / kbc, kb = gkb - g * kbc;
        v[u] = __builtin_nontemporal_load(
            reinterpret_cast<const v4f*>(x + (g * m + row) * k + kb * kGroup) + lane);
      }
    }
#pragma unroll
    for (int u = 0; u < kTokUnroll; ++u) {
      const int64_t gi = base + u * half_waves;
      if (gi >= groups) break;   // uniform across the half-wave
      const int64_t gkb = gi / m, row = gi - gkb * m;
      const int64_t kbc = k / kGroup, g = gkb / kbc, kb = gkb - g * kbc;
      float amax = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
      const float s = amax == 0.0f ? 1.0f : amax / kE4M3Max;
      const uint32_t packed = pack4_e4m3(clamp448(v[u].x / s), clamp448(v[u].y / s),
                                         clamp448(v[u].z / s), clamp448(v[u].w / s));
      reinterpret_cast<uint32_t*>(q + (g * m + row) * k + kb * kGroup)[lane] = packed;
      if (lane == 0) sa[gkb * ld_sa + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128 x 128 blocks (weights).  One workgroup per block: 256 threads, each
// holding 16 float4 (rows tid/32 + 8u, columns 4*(tid%32) .. +3).  Every load
// instruction reads one full 512-byte block row per half-wave.
// ---------------------------------------------------------------------------
constexpr int kBlkThreads = 256;

__global__ __launch_bounds__(kBlkThreads) void quant_block_kernel(
    const float* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ q,
    float* __restrict__ sb, int64_t nb_n) {
  const int64_t kbc = k / kGroup;
  const int64_t bid = blockIdx.x;
  const int64_t kb = bid % kbc;
  const int64_t t = bid / kbc;
  const int64_t nb = t % nb_n;
  const int64_t g = t / nb_n;
  const int64_t row0 = nb * kGroup;
  const int rows_here = (int)((n - row0) < kGroup ? (n - row0) : kGroup);

  const int tid = threadIdx.x;
  const int c4 = tid & 31;
  const int r0 = tid >> 5;
  const float* src = w + (g * n + row0) * k + kb * kGroup;
  uint8_t* dst = q + (g * n + row0) * k + kb * kGroup;

  v4f v[16];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 8 * u;
    if (r < rows_here) {
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + r * k) + c4);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float red[kBlkThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax == 0.0f ? 1.0f : amax / kE4M3Max;

#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 8 * u;
    if (r < rows_here) {
      reinterpret_cast<uint32_t*>(dst + r * k)[c4] =
          pack4_e4m3(clamp448(v[u].x / s), clamp448(v[u].y / s), clamp448(v[u].z / s),
                     clamp448(v[u].w / s));
    }
  }
  if (tid == 0) sb[(g * nb_n + nb) * kbc + kb] = s;
}

// ---------------------------------------------------------------------------
// Launchers (arguments already validated by the C ABI layer).
// ---------------------------------------------------------------------------
int launch_quant_token_group(const float* x, int64_t mats, int64_t m, int64_t k, uint8_t* q, float* sa,
                             int64_t ld_sa, hipStream_t stream, int num_cus) {
  const int64_t groups = mats * m * (k / kGroup);
  const int64_t groups_per_block = kTokThreads / 32;
  int64_t blocks = (groups + groups_per_block * kTokUnroll - 1) / (groups_per_block * kTokUnroll);
  const int64_t cap = (int64_t)num_cus * 16;   // enough resident waves to cover HBM latency
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quant_token_group_kernel, dim3((unsigned)blocks), dim3(kTokThreads), 0,
                     stream, x, m, k, q, sa, ld_sa, groups);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "quantize_per_token_group launch: %s", hipGetErrorString(e));
}

int launch_quant_block(const float* w, int64_t groups, int64_t n, int64_t k, uint8_t* q, float* sb,
                       hipStream_t stream) {
  const int64_t nb_n = (n + kGroup - 1) / kGroup;
  const int64_t blocks = groups * nb_n * (k / kGroup);
  if (blocks > 0x7fffffffLL) return set_error(kUnsupported, "quantize_per_block: too many blocks");
  hipLaunchKernelGGL(quant_block_kernel, dim3((unsigned)blocks), dim3(kBlkThreads), 0, stream, w,
                     n, k, q, sb, nb_n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "quantize_per_block launch: %s", hipGetErrorString(e));
}

}  // namespace dg
