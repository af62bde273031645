// Fine-grained FP8 quantizers for gfx950.
//
// Fine-grained scaling as proposed with DeepSeek-V3 (机器之心 DeepGEMM report,
// opening section), E4M3 data (ai.abqq.net DeepGEMM summary, section 3):
//   amax = max |x| over a group, s = amax / 448 (s = 1 for amax = 0),
//   q = E4M3 round-to-nearest-even (saturating) of fl32(x / s).
// Both divisions are IEEE fp32 divisions (the library is built without fast
// math), so bytes and scales are bit-exact with any correct implementation.
//
// Both kernels are HBM-bound streaming kernels (read 4 B - 2 B for bf16 activations -, write
// 1 B + 1/32 B per element): coalesced 16-byte (8-byte for bf16) loads, several in flight per
// lane.  Group maxima use DPP lane swaps and lane reads (no LDS crossbar).
#include "common.hpp"

namespace dg {

// ---------------------------------------------------------------------------
// 1 x 128 groups along K (activations), for `mats` stacked (m, k) matrices.
// A half-wave (32 lanes x 4 floats) owns one 128-wide group.  A 256-thread workgroup takes 8
// consecutive rows (of the stacked rows) x kTokKb consecutive K groups: grid (row blocks,
// K-group blocks), so each half-wave splits its row index once (32-bit) and the loads of its
// kTokKb groups are all in flight together.  The 8 half-waves of one K group store 8
// consecutive scales.
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 256;
constexpr int kTokRows = kTokThreads / 32;   // rows per workgroup
constexpr int kTokKb = 4;                    // K groups per workgroup (loads in flight per lane)

// Four consecutive activations of a lane as fp32: fp32 input as is, bf16 input widened exactly
// (a bf16 value is the upper half of the fp32 word).
__device__ __forceinline__ v4f load4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ v4f load4(const uint16_t* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return v4f{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
             __uint_as_float(w.y & 0xffff0000u)};
}

template <class T>
__global__ __launch_bounds__(kTokThreads) void quant_token_group_kernel(
    const T* __restrict__ x, int m, int k, uint8_t* __restrict__ q,
    float* __restrict__ sa, int64_t ld_sa, int total_rows) {
  const int lane = threadIdx.x & 31;
  const int row = blockIdx.x * kTokRows + (threadIdx.x >> 5);   // stacked row: g * m + r
  if (row >= total_rows) return;                                 // uniform per half-wave
  const int kbc = (k + kGroup - 1) / kGroup;   // a last group of k % 128 elements is partial
  const int kb0 = blockIdx.y * kTokKb;
  const int g = row / m, r = row - g * m;
  const T* src = x + (int64_t)row * k + kb0 * kGroup;
  uint8_t* dst = q + (int64_t)row * k + kb0 * kGroup;
  float* scl = sa + ((int64_t)g * kbc + kb0) * ld_sa + r;

  // lane columns past k (partial last group) read as zeros: the amax is that of the elements present
  v4f v[kTokKb];
#pragma unroll
  for (int u = 0; u < kTokKb; ++u)
    v[u] = (kb0 + u < kbc && (kb0 + u) * kGroup + 4 * lane < k) ? load4(src + u * kGroup + 4 * lane)
                                                                : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kTokKb; ++u) {
    if (kb0 + u >= kbc) break;   // uniform
    const float amax =
        half_wave_max(fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    const float s = amax == 0.0f ? 1.0f : amax / kE4M3Max;
    const uint32_t packed = pack4_e4m3(clamp448(v[u].x / s), clamp448(v[u].y / s),
                                       clamp448(v[u].z / s), clamp448(v[u].w / s));
    if ((kb0 + u) * kGroup + 4 * lane < k) reinterpret_cast<uint32_t*>(dst + u * kGroup)[lane] = packed;
    if (lane == 0) scl[(int64_t)u * ld_sa] = s;
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
  const int64_t kbc = (k + kGroup - 1) / kGroup;
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
  const bool col_ok = kb * kGroup + 4 * c4 < k;   // a partial last K block: columns past k are absent
  const float* src = w + (g * n + row0) * k + kb * kGroup;
  uint8_t* dst = q + (g * n + row0) * k + kb * kGroup;

  v4f v[16];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 8 * u;
    if (r < rows_here && col_ok) {
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + r * k) + c4);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
  }
  amax = wave_max(amax);
  __shared__ float red[kBlkThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax == 0.0f ? 1.0f : amax / kE4M3Max;

#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 8 * u;
    if (r < rows_here && col_ok) {
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
template <class T>
static int launch_token_group(const T* x, int64_t mats, int64_t m, int64_t k, uint8_t* q, float* sa,
                              int64_t ld_sa, hipStream_t stream) {
  const int64_t total_rows = mats * m;
  const int64_t kbc = (k + kGroup - 1) / kGroup;
  if (total_rows > 0x7fffffffLL || k > 0x7fffffffLL)
    return set_error(kUnsupported, "quantize_per_token_group: more than 2^31 rows or columns");
  const int64_t gx = (total_rows + kTokRows - 1) / kTokRows;
  const int64_t gy = (kbc + kTokKb - 1) / kTokKb;
  if (gx > 0x7fffffffLL || gy > 65535)
    return set_error(kUnsupported, "quantize_per_token_group: shape too large for the launch grid");
  hipLaunchKernelGGL(quant_token_group_kernel<T>, dim3((unsigned)gx, (unsigned)gy), dim3(kTokThreads), 0, stream,
                     x, (int)m, (int)k, q, sa, ld_sa, (int)total_rows);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "quantize_per_token_group launch: %s", hipGetErrorString(e));
}

int launch_quant_token_group(const float* x, int64_t mats, int64_t m, int64_t k, uint8_t* q, float* sa,
                             int64_t ld_sa, hipStream_t stream) {
  return launch_token_group(x, mats, m, k, q, sa, ld_sa, stream);
}

int launch_quant_token_group_bf16(const uint16_t* x, int64_t mats, int64_t m, int64_t k, uint8_t* q, float* sa,
                                  int64_t ld_sa, hipStream_t stream) {
  return launch_token_group(x, mats, m, k, q, sa, ld_sa, stream);
}

int launch_quant_block(const float* w, int64_t groups, int64_t n, int64_t k, uint8_t* q, float* sb,
                       hipStream_t stream) {
  const int64_t nb_n = (n + kGroup - 1) / kGroup;
  const int64_t blocks = groups * nb_n * ((k + kGroup - 1) / kGroup);
  if (blocks > 0x7fffffffLL) return set_error(kUnsupported, "quantize_per_block: too many blocks");
  hipLaunchKernelGGL(quant_block_kernel, dim3((unsigned)blocks), dim3(kBlkThreads), 0, stream, w,
                     n, k, q, sb, nb_n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "quantize_per_block launch: %s", hipGetErrorString(e));
}

}  // namespace dg
