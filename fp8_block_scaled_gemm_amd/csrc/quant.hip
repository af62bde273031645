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
// consecutive rows (of the stacked rows) x KB consecutive K groups: grid (K-group blocks, row
// blocks), so each half-wave splits its row index once (32-bit) and the loads of its KB groups
// are all in flight together.  The 8 half-waves of one K group store 8 consecutive scales.
// KB is 4, halved while the grid would have fewer than kTokMinBlocks workgroups: at large M,
// 2 to 8 groups per lane run at the same rate (4.2-4.5 TB/s on the V3 shapes), while at decode
// sizes the wider grid of 1 or 2 groups per lane is ~0.7 us faster per launch (measured).
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 256;
constexpr int kTokRows = kTokThreads / 32;   // rows per workgroup
constexpr int kTokMinBlocks = 1024;

template <class T, int KB>
__global__ __launch_bounds__(kTokThreads) void quant_token_group_kernel(
    const T* __restrict__ x, int m, int k, uint8_t* __restrict__ q,
    float* __restrict__ sa, int64_t ld_sa, int total_rows) {
  const int lane = threadIdx.x & 31;
  const int kbc = (k + kGroup - 1) / kGroup;   // a last group of k % 128 elements is partial
  const int kb0 = blockIdx.x * KB;
  // K blocks along x: the workgroups running side by side read neighbouring pieces of the same
  // rows (measured 5.0-5.1 TB/s instead of 4.4-4.5 with row blocks along x at K = 7168 and
  // 16384).  Row blocks along y, continued along z past 65535 of them.
  const int64_t row64 = ((int64_t)blockIdx.y + (int64_t)gridDim.y * blockIdx.z) * kTokRows + (threadIdx.x >> 5);
  if (row64 >= total_rows) return;   // uniform per half-wave
  {
    const int row = (int)row64;      // stacked row: g * m + r
    const int g = row / m, r = row - g * m;
    const T* src = x + (int64_t)row * k + kb0 * kGroup;
    uint8_t* dst = q + (int64_t)row * k + kb0 * kGroup;
    float* scl = sa + ((int64_t)g * kbc + kb0) * ld_sa + r;

    // lane columns past k (partial last group) read as zeros: the amax is that of the elements
    // present.  Every lane loads (an absent column from the row's first element, which exists),
    // so no load sits behind a branch and all KB of them are in flight together.
    v4f v[KB];
    bool ok[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      ok[u] = kb0 + u < kbc && (kb0 + u) * kGroup + 4 * lane < k;
      v[u] = load4(ok[u] ? src + u * kGroup + 4 * lane : src);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (!ok[u]) v[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (kb0 + u >= kbc) break;   // uniform
      float s;
      const uint32_t packed = quant_group4(v[u], s);
      if ((kb0 + u) * kGroup + 4 * lane < k) reinterpret_cast<uint32_t*>(dst + u * kGroup)[lane] = packed;
      if (lane == 0) scl[(int64_t)u * ld_sa] = s;
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
  // block index -> (matrix, 128-row block, K block) in 32-bit arithmetic (the launcher keeps the
  // block count, the K-block count and the row-block count below 2^31)
  const uint32_t kbc = (uint32_t)((k + kGroup - 1) / kGroup);
  const uint32_t bid = blockIdx.x;
  const uint32_t kb = bid % kbc;
  const uint32_t t = bid / kbc;
  const uint32_t nb = t % (uint32_t)nb_n;
  const int64_t g = t / (uint32_t)nb_n;
  const int64_t row0 = (int64_t)nb * kGroup;
  const int rows_here = (int)((n - row0) < kGroup ? (n - row0) : kGroup);

  const int tid = threadIdx.x;
  const int c4 = tid & 31;
  const int r0 = tid >> 5;
  const bool col_ok = kb * kGroup + 4 * c4 < k;   // a partial last K block: columns past k are absent
  const float* src = w + (g * n + row0) * k + kb * kGroup;
  uint8_t* dst = q + (g * n + row0) * k + kb * kGroup;

  // Every lane loads all 16 of its rows (an absent row or column from the block's first element,
  // which exists), so no load sits behind a branch and all 16 are in flight together; absent
  // values are zeroed before the maximum.
  v4f v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 8 * u;
    v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(r < rows_here && col_ok ? src + (int64_t)r * k + 4 * c4 : src));
  }
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if (!(r0 + 8 * u < rows_here && col_ok)) v[u] = v4f{0.f, 0.f, 0.f, 0.f};
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
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
      reinterpret_cast<uint32_t*>(dst + (int64_t)r * k)[c4] =
          pack4_e4m3(clamp448(v[u].x / s), clamp448(v[u].y / s), clamp448(v[u].z / s),
                     clamp448(v[u].w / s));
    }
  }
  if (tid == 0) sb[(g * nb_n + nb) * (int64_t)kbc + kb] = s;
}

// ---------------------------------------------------------------------------
// 128 x 1 groups (128 consecutive tokens of one column), output transposed: the operands of the
// weight-gradient GEMM dW = dY^T X, whose contraction runs over the tokens.  x is (m, k) per
// matrix; the codes go to qt (k, m), the scales to st[mb][col] (row stride ld_st), so that each
// output row is one column's tokens with their groups contiguous - the layout of an activation
// operand.  A workgroup takes 128 tokens x 64 columns: thread t loads 8 consecutive tokens of
// 4 consecutive columns (16 threads cover a 64-column row slice with coalesced loads), the column
// maxima are reduced across the 16 token octets (lanes 16 and 32 apart, then the 4 waves through
// LDS), and the codes are transposed through LDS so that every store is a 16-byte run of one
// output row.
// ---------------------------------------------------------------------------
constexpr int kChThreads = 256;
constexpr int kChCols = 64;   // columns (output rows) per workgroup

template <class T>
__global__ __launch_bounds__(kChThreads) void quant_channel_group_kernel(
    const T* __restrict__ x, int m, int k, uint8_t* __restrict__ qt, float* __restrict__ st, int64_t ld_st) {
  __shared__ float red[kChThreads / 64][kChCols];
  __shared__ float scl[kChCols];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kChCols][kGroup];
  const int tid = threadIdx.x;
  const int c4 = tid & 15, oct = tid >> 4;   // columns 4*c4 .. +3, tokens 8*oct .. +7 of the tile
  const int mat = blockIdx.z;
  const int col0 = blockIdx.x * kChCols, tok0 = blockIdx.y * kGroup;
  const int mbc = (m + kGroup - 1) / kGroup;
  const int col = col0 + 4 * c4;
  const bool col_ok = col < k;   // k % 4 == 0: the 4 columns are all present or all absent
  const T* src = x + ((int64_t)mat * m + tok0 + 8 * oct) * k + col;

  // tokens past m (a partial last group) read as zeros: the maxima are those of the tokens present
  // (every lane loads all 8 tokens - an absent one from the matrix's first element - so that no load
  // sits behind a branch; absent values are zeroed afterwards)
  const T* first = x + (int64_t)mat * m * k;
  v4f v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = load4(col_ok && tok0 + 8 * oct + u < m ? src + (int64_t)u * k : first);
  v4f amax = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (!(col_ok && tok0 + 8 * oct + u < m)) v[u] = v4f{0.f, 0.f, 0.f, 0.f};
    amax = v4f{fmaxf(amax.x, fabsf(v[u].x)), fmaxf(amax.y, fabsf(v[u].y)), fmaxf(amax.z, fabsf(v[u].z)),
               fmaxf(amax.w, fabsf(v[u].w))};
  }
#pragma unroll
  for (int sh = 16; sh <= 32; sh *= 2) {
    amax.x = fmaxf(amax.x, __shfl_xor(amax.x, sh));
    amax.y = fmaxf(amax.y, __shfl_xor(amax.y, sh));
    amax.z = fmaxf(amax.z, __shfl_xor(amax.z, sh));
    amax.w = fmaxf(amax.w, __shfl_xor(amax.w, sh));
  }
  if ((tid & 63) < 16) {
    float* r = &red[tid >> 6][4 * c4];
    r[0] = amax.x; r[1] = amax.y; r[2] = amax.z; r[3] = amax.w;
  }
  __syncthreads();
  if (tid < kChCols) {
    const float a = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    const float s = a == 0.0f ? 1.0f : a / kE4M3Max;
    scl[tid] = s;
    if (col0 + tid < k) st[((int64_t)mat * mbc + blockIdx.y) * ld_st + col0 + tid] = s;
  }
  __syncthreads();
  const float s0 = scl[4 * c4], s1 = scl[4 * c4 + 1], s2 = scl[4 * c4 + 2], s3 = scl[4 * c4 + 3];
  // column c of this thread: its 8 tokens are 8 consecutive bytes of output row 4*c4 + c
  const uint32_t c0lo = pack4_e4m3(clamp448(v[0].x / s0), clamp448(v[1].x / s0), clamp448(v[2].x / s0), clamp448(v[3].x / s0));
  const uint32_t c0hi = pack4_e4m3(clamp448(v[4].x / s0), clamp448(v[5].x / s0), clamp448(v[6].x / s0), clamp448(v[7].x / s0));
  const uint32_t c1lo = pack4_e4m3(clamp448(v[0].y / s1), clamp448(v[1].y / s1), clamp448(v[2].y / s1), clamp448(v[3].y / s1));
  const uint32_t c1hi = pack4_e4m3(clamp448(v[4].y / s1), clamp448(v[5].y / s1), clamp448(v[6].y / s1), clamp448(v[7].y / s1));
  const uint32_t c2lo = pack4_e4m3(clamp448(v[0].z / s2), clamp448(v[1].z / s2), clamp448(v[2].z / s2), clamp448(v[3].z / s2));
  const uint32_t c2hi = pack4_e4m3(clamp448(v[4].z / s2), clamp448(v[5].z / s2), clamp448(v[6].z / s2), clamp448(v[7].z / s2));
  const uint32_t c3lo = pack4_e4m3(clamp448(v[0].w / s3), clamp448(v[1].w / s3), clamp448(v[2].w / s3), clamp448(v[3].w / s3));
  const uint32_t c3hi = pack4_e4m3(clamp448(v[4].w / s3), clamp448(v[5].w / s3), clamp448(v[6].w / s3), clamp448(v[7].w / s3));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(&tile[4 * c4 + 0][8 * oct]) = u32x2{c0lo, c0hi};
  *reinterpret_cast<u32x2*>(&tile[4 * c4 + 1][8 * oct]) = u32x2{c1lo, c1hi};
  *reinterpret_cast<u32x2*>(&tile[4 * c4 + 2][8 * oct]) = u32x2{c2lo, c2hi};
  *reinterpret_cast<u32x2*>(&tile[4 * c4 + 3][8 * oct]) = u32x2{c3lo, c3hi};
  __syncthreads();
  // 64 output rows x 128 tokens = 512 chunks of 16 bytes, two per thread (m % 16 == 0: a chunk
  // is all present or all absent)
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int chunk = tid + h * kChThreads;
    const int orow = chunk >> 3, piece = chunk & 7;
    const int tok = tok0 + 16 * piece;
    if (col0 + orow < k && tok < m)
      *reinterpret_cast<u32x4*>(qt + ((int64_t)mat * k + col0 + orow) * m + tok) =
          *reinterpret_cast<const u32x4*>(&tile[orow][16 * piece]);
  }
}

// ---------------------------------------------------------------------------
// Transpose of block-quantized codes and their block scales: (groups, r, c) codes ->
// (groups, c, r), (groups, ceil(r/128), ceil(c/128)) scales -> (groups, ceil(c/128),
// ceil(r/128)).  A 128 x 128 block is square, so this is the block quantization of the
// transposed matrix (the weight operand of dX = dY W).  64 x 64-byte tiles through LDS; the
// workgroup whose tile opens a 128 x 128 block moves that block's scale.
// ---------------------------------------------------------------------------
constexpr int kTrTile = 64;

__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                               int r, int c, uint8_t* __restrict__ qt,
                                                               float* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTrTile][kTrTile + 4];
  const int tid = threadIdx.x;
  const int g = blockIdx.z;
  const int c0 = blockIdx.x * kTrTile, r0 = blockIdx.y * kTrTile;
  const int row = tid >> 2, piece = tid & 3;   // 64 rows x 4 chunks of 16 bytes
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  // r % 16 == 0 and c % 16 == 0: a 16-byte chunk is all present or all absent
  if (r0 + row < r && c0 + 16 * piece < c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(q + ((int64_t)g * r + r0 + row) * c + c0 + 16 * piece);
    *reinterpret_cast<unsigned*>(&tile[row][16 * piece + 0]) = v.x;
    *reinterpret_cast<unsigned*>(&tile[row][16 * piece + 4]) = v.y;
    *reinterpret_cast<unsigned*>(&tile[row][16 * piece + 8]) = v.z;
    *reinterpret_cast<unsigned*>(&tile[row][16 * piece + 12]) = v.w;
  }
  __syncthreads();
  // output row c0 + row (an input column), bytes r0 + 16*piece .. +15 (input rows)
  if (c0 + row < c && r0 + 16 * piece < r) {
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = (uint32_t)tile[16 * piece + 4 * u][row] | ((uint32_t)tile[16 * piece + 4 * u + 1][row] << 8) |
             ((uint32_t)tile[16 * piece + 4 * u + 2][row] << 16) | ((uint32_t)tile[16 * piece + 4 * u + 3][row] << 24);
    *reinterpret_cast<u32x4*>(qt + ((int64_t)g * c + c0 + row) * r + r0 + 16 * piece) = u32x4{w[0], w[1], w[2], w[3]};
  }
  if (tid == 0 && (blockIdx.x & 1) == 0 && (blockIdx.y & 1) == 0) {
    const int rb = (r + kGroup - 1) / kGroup, cb = (c + kGroup - 1) / kGroup;
    const int br = r0 / kGroup, bc = c0 / kGroup;
    st[((int64_t)g * cb + bc) * rb + br] = s[((int64_t)g * rb + br) * cb + bc];
  }
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
  const int64_t row_blocks = (total_rows + kTokRows - 1) / kTokRows;
  int kb = 4;
  while (kb > 1 && row_blocks * ((kbc + kb - 1) / kb) < kTokMinBlocks) kb /= 2;
  const int64_t gx = (kbc + kb - 1) / kb;                       // K blocks
  const int64_t gy = row_blocks < 65535 ? row_blocks : 65535;   // row blocks, continued along z
  const int64_t gz = (row_blocks + gy - 1) / gy;
  if (gx > 0x7fffffffLL || gz > 65535)
    return set_error(kUnsupported, "quantize_per_token_group: shape too large for the launch grid");
  auto fn = kb == 4 ? quant_token_group_kernel<T, 4> : kb == 2 ? quant_token_group_kernel<T, 2>
                                                               : quant_token_group_kernel<T, 1>;
  hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy, (unsigned)gz), dim3(kTokThreads), 0, stream, x, (int)m,
                     (int)k, q, sa, ld_sa, (int)total_rows);
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

template <class T>
static int launch_channel_group(const T* x, int64_t mats, int64_t m, int64_t k, uint8_t* qt, float* st,
                                int64_t ld_st, hipStream_t stream) {
  if (m > 0x7fffffffLL || k > 0x7fffffffLL || mats > 65535)
    return set_error(kUnsupported, "quantize_per_channel_group: shape too large");
  const int64_t gx = (k + kChCols - 1) / kChCols, gy = (m + kGroup - 1) / kGroup;
  if (gx > 0x7fffffffLL || gy > 65535)
    return set_error(kUnsupported, "quantize_per_channel_group: shape too large for the launch grid");
  hipLaunchKernelGGL(quant_channel_group_kernel<T>, dim3((unsigned)gx, (unsigned)gy, (unsigned)mats), dim3(kChThreads),
                     0, stream, x, (int)m, (int)k, qt, st, ld_st);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "quantize_per_channel_group launch: %s", hipGetErrorString(e));
}

int launch_quant_channel_group(const float* x, int64_t mats, int64_t m, int64_t k, uint8_t* qt, float* st,
                               int64_t ld_st, hipStream_t stream) {
  return launch_channel_group(x, mats, m, k, qt, st, ld_st, stream);
}

int launch_quant_channel_group_bf16(const uint16_t* x, int64_t mats, int64_t m, int64_t k, uint8_t* qt, float* st,
                                    int64_t ld_st, hipStream_t stream) {
  return launch_channel_group(x, mats, m, k, qt, st, ld_st, stream);
}

int launch_transpose_blocks(const uint8_t* q, const float* s, int64_t groups, int64_t r, int64_t c, uint8_t* qt,
                            float* st, hipStream_t stream) {
  if (r > 0x7fffffffLL || c > 0x7fffffffLL || groups > 65535)
    return set_error(kUnsupported, "transpose_blocks: shape too large");
  const int64_t gx = (c + kTrTile - 1) / kTrTile, gy = (r + kTrTile - 1) / kTrTile;
  if (gx > 0x7fffffffLL || gy > 65535) return set_error(kUnsupported, "transpose_blocks: shape too large for the grid");
  hipLaunchKernelGGL(transpose_blocks_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)groups), dim3(256), 0, stream,
                     q, s, (int)r, (int)c, qt, st);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "transpose_blocks launch: %s", hipGetErrorString(e));
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
