// FP8 block-scaled GEMM for gfx950 (CDNA4): D = A * B^T with two-level accumulation.
//
// Method (DeepGEMM pages): E4M3 operands with fine-grained scales - one fp32
// scale per 1x128 activation group and per 128x128 weight block - and FP32
// promotion of the matrix-core partials (机器之心 report, opening section;
// ai.abqq.net summary, sections 1 and 3; 3loumao explainer, section 03).  Three
// forms share one main loop: normal, contiguous-grouped and masked-grouped
// (机器之心 report, "quick start"; 3loumao explainer, section 03).
//
// Design for gfx950 (none of the Hopper-specific structure of the pages):
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 covers a whole 128-deep K block of a
//    16x16 output fragment, so the level-1 partial of a K block is exactly one
//    MFMA into a zero accumulator, and the level-2 promotion is one VALU FMA per
//    output element:  acc += P * fl32(sa * sb).  The promotion of one fragment
//    overlaps the next fragments' MFMAs.  The MFMA's own E8M0 block scales are
//    left neutral (2^0): the fine-grained scales are arbitrary fp32 values.
//  * MFMA operand A is the weight tile (rows n), operand B the activation tile
//    (rows m): each lane then holds 4 consecutive n of one row m, so the bf16
//    epilogue stores 8 contiguous bytes per lane and the promotion scale is one
//    value per lane and fragment.
//  * Operand tiles (BN x 128 and BM x 128 bytes per K block) are staged in LDS
//    with 16-byte coalesced global loads, double-buffered, with an XOR swizzle of
//    the 16-byte chunks (chunk c of row r lives at slot c ^ (r & 7)) so the
//    fragment reads are free of bank conflicts.
//  * A persistent grid (at most the CU cap x occupancy) walks work items
//    (group, m-block, n-block, k-split) - the contiguous layout reads each
//    m-block's expert from m_indices, the masked layout reads masked_m on the
//    device and skips empty m-blocks - with an XCD-aware item order so that
//    workgroups sharing a weight panel run on the same XCD (same L2).
//  * Small-m shapes split K over workgroups; the last-arriving workgroup of a
//    tile sums the fp32 partials in fixed split order (deterministic) and stores
//    bf16.
#include <cstdio>

#include "common.hpp"

namespace dg {

enum Layout : int { kDense = 0, kContiguous = 1, kMasked = 2 };

struct GemmParams {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  uint16_t* d;
  const int32_t* m_indices;   // contiguous: expert per row
  const int32_t* masked_m;    // masked: valid rows per group
  float* ws;                  // split-K partials
  unsigned* counters;         // split-K arrival counters, one per tile
  int64_t ld_sa;
  int64_t a_gstride, sa_gstride, b_gstride, sb_gstride, d_gstride;   // per-group strides (elements)
  int m;            // rows per group (dense: M, contiguous: M_total, masked: M_max)
  int n, k;
  int num_groups;
  int kb_total;     // k / 128
  int tiles_m;      // ceil(m / BM)
  int tiles_n;      // ceil(n / BN)
  int splits;       // K splits (1 = none)
  int kb_per_split;
  int nb128;        // ceil(n / 128): weight-scale rows per group
};

template <int BN, int BM, int WN, int WM>
struct TileCfg {
  static constexpr int kWavesN = BN / WN;
  static constexpr int kWavesM = BM / WM;
  static constexpr int kThreads = 64 * kWavesN * kWavesM;
  static constexpr int kFragN = WN / 16;
  static constexpr int kFragM = WM / 16;
  static constexpr int kStageBytes = (BN + BM) * kGroup;
  static constexpr int kChunksB = BN * 8;          // 16-byte chunks per K block
  static constexpr int kChunksA = BM * 8;
  static constexpr int kLoadsB = kChunksB / kThreads;
  static constexpr int kLoadsA = kChunksA / kThreads;
  static_assert(kChunksB % kThreads == 0 && kChunksA % kThreads == 0, "tile/threads mismatch");
  static_assert(WN % 16 == 0 && WM % 16 == 0 && 128 % WN == 0, "wave tile must be 16-aligned, WN | 128");
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i make_v8i(u32x4 lo, u32x4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kGroup + ((chunk ^ (row & 7)) << 4); }

// Work item -> tile coordinates.  Returns false when the item maps to nothing.
struct Tile {
  int g, mb, nbt, split;
  int m_valid;      // rows of this group that may be stored (dense: m; masked: masked count)
  int tile_id;      // index of the (g, mb, nbt) tile for split-K bookkeeping
};

template <int BN, int BM, int WN, int WM, int LAYOUT>
__global__ __launch_bounds__(64 * (BN / WN) * (BM / WM)) void gemm_fp8_kernel(GemmParams p) {
  using C = TileCfg<BN, BM, WN, WM>;
  constexpr int NT = C::kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][C::kStageBytes];
  __shared__ int s_prefix[LAYOUT == kMasked ? 1025 : 1];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave % C::kWavesN;
  const int wave_m = wave / C::kWavesN;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- total work items -------------------------------------------------------
  int total_items;
  if constexpr (LAYOUT == kMasked) {
    // prefix over groups of the number of (m-block, n-block) tiles, from device counts
    if (tid == 0) {
      int acc = 0;
      s_prefix[0] = 0;
      for (int g = 0; g < p.num_groups; ++g) {
        int mv = p.masked_m[g];
        mv = mv < 0 ? 0 : (mv > p.m ? p.m : mv);
        acc += ((mv + BM - 1) / BM) * p.tiles_n;
        s_prefix[g + 1] = acc;
      }
    }
    __syncthreads();
    total_items = s_prefix[p.num_groups] * p.splits;
  } else {
    // contiguous: the expert comes from m_indices, not from the item index
    total_items = p.tiles_m * p.tiles_n * (LAYOUT == kDense ? p.num_groups : 1) * p.splits;
  }

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of items in every round of the persistent loop.
  const int grid = gridDim.x;
  int wg = blockIdx.x;
  if ((grid & 7) == 0) wg = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  for (int item = wg; item < total_items; item += grid) {
    // ---- decode the item ------------------------------------------------------
    Tile t;
    t.split = item % p.splits;
    int rest = item / p.splits;
    if constexpr (LAYOUT == kMasked) {
      int g = 0;
      while (s_prefix[g + 1] <= rest) ++g;
      rest -= s_prefix[g];
      t.g = g;
      t.mb = rest % ((s_prefix[g + 1] - s_prefix[g]) / p.tiles_n);
      t.nbt = rest / ((s_prefix[g + 1] - s_prefix[g]) / p.tiles_n);
      int mv = p.masked_m[g];
      t.m_valid = mv < 0 ? 0 : (mv > p.m ? p.m : mv);
      t.tile_id = (g * p.tiles_m + t.mb) * p.tiles_n + t.nbt;
    } else {
      t.mb = rest % p.tiles_m;
      rest /= p.tiles_m;
      t.nbt = rest % p.tiles_n;
      t.g = rest / p.tiles_n;
      t.m_valid = p.m;
      t.tile_id = (t.g * p.tiles_m + t.mb) * p.tiles_n + t.nbt;
    }
    const int m0 = t.mb * BM;
    const int n0 = t.nbt * BN;
    int expert = t.g;
    if constexpr (LAYOUT == kContiguous) {
      expert = p.m_indices[m0];
      if (expert < 0 || expert >= p.num_groups) continue;   // uniform: skip unmapped block
    }
    const int kb_begin = t.split * p.kb_per_split;
    int kb_end = kb_begin + p.kb_per_split;
    if (kb_end > p.kb_total) kb_end = p.kb_total;

    const uint8_t* a_g = p.a + (LAYOUT == kMasked ? (int64_t)t.g * p.a_gstride : 0);
    const float* sa_g = p.sa + (LAYOUT == kMasked ? (int64_t)t.g * p.sa_gstride : 0);
    const uint8_t* b_g = p.b + (int64_t)expert * p.b_gstride;
    const float* sb_g = p.sb + (int64_t)expert * p.sb_gstride;
    const int m_last = p.m - 1;   // clamp target for edge rows (rows per group)

    // ---- global -> register staging (thread t: chunk t % 8 of rows t / 8 + u * NT / 8) ----
    // 32-bit offsets: every operand matrix of one group is < 2^31 bytes (checked on the host).
    constexpr int kRowStep = NT / 8;
    const int ch = tid & 7;
    const int rbase = tid >> 3;
    int offB[C::kLoadsB], offA[C::kLoadsA];
#pragma unroll
    for (int u = 0; u < C::kLoadsB; ++u) {
      int grow = n0 + rbase + u * kRowStep;
      grow = grow < p.n ? grow : p.n - 1;
      offB[u] = grow * p.k + ch * 16;
    }
#pragma unroll
    for (int u = 0; u < C::kLoadsA; ++u) {
      int grow = m0 + rbase + u * kRowStep;
      grow = grow <= m_last ? grow : m_last;
      offA[u] = grow * p.k + ch * 16;
    }
    const int lds_st = swz(rbase, ch);   // + u * kRowStep * 128 (kRowStep is a multiple of 8)
    // per-lane activation-scale rows and the wave's weight-scale block
    int sa_row[C::kFragM];
#pragma unroll
    for (int j = 0; j < C::kFragM; ++j) {
      const int r = m0 + wave_m * WM + 16 * j + l16;
      sa_row[j] = r <= m_last ? r : m_last;
    }
    const int nb_w = (n0 + wave_n * WN) >> 7;
    const float* sb_row = sb_g + (int64_t)(nb_w < p.nb128 ? nb_w : p.nb128 - 1) * p.kb_total;

    v4f acc[C::kFragN][C::kFragM];
#pragma unroll
    for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    u32x4 regB[C::kLoadsB], regA[C::kLoadsA];
    float sa_cur[C::kFragM], sa_next[C::kFragM];
    float sb_cur, sb_next;

#define DG_LOAD_STAGE(KB)                                                                     \
  do {                                                                                        \
    const uint8_t* gb = b_g + (int64_t)(KB) * kGroup;                                         \
    const uint8_t* ga = a_g + (int64_t)(KB) * kGroup;                                         \
    _Pragma("unroll") for (int u = 0; u < C::kLoadsB; ++u) regB[u] =                         \
        *reinterpret_cast<const u32x4*>(gb + offB[u]);                                        \
    _Pragma("unroll") for (int u = 0; u < C::kLoadsA; ++u) regA[u] =                         \
        *reinterpret_cast<const u32x4*>(ga + offA[u]);                                        \
    _Pragma("unroll") for (int j = 0; j < C::kFragM; ++j) sa_next[j] =                       \
        sa_g[(int64_t)(KB) * p.ld_sa + sa_row[j]];                                            \
    sb_next = sb_row[(KB)];                                                                   \
  } while (0)
#define DG_STORE_STAGE(STG)                                                                   \
  do {                                                                                        \
    uint8_t* sdst = smem[(STG)] + lds_st;                                                     \
    _Pragma("unroll") for (int u = 0; u < C::kLoadsB; ++u)                                    \
        *reinterpret_cast<u32x4*>(sdst + u * kRowStep * kGroup) = regB[u];                    \
    _Pragma("unroll") for (int u = 0; u < C::kLoadsA; ++u)                                    \
        *reinterpret_cast<u32x4*>(sdst + BN * kGroup + u * kRowStep * kGroup) = regA[u];      \
  } while (0)

    __syncthreads();   // previous tile's readers are done with both stages
    DG_LOAD_STAGE(kb_begin);
    DG_STORE_STAGE(0);
#pragma unroll
    for (int j = 0; j < C::kFragM; ++j) sa_cur[j] = sa_next[j];
    sb_cur = sb_next;
    __syncthreads();

    int stage = 0;
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      const bool more = kb + 1 < kb_end;
      if (more) DG_LOAD_STAGE(kb + 1);

      const uint8_t* sB = smem[stage];
      const uint8_t* sA = smem[stage] + BN * kGroup;
      // activation fragments (MFMA operand B), all of the wave's m-fragments
      v8i bop[C::kFragM];
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) {
        const int row = wave_m * WM + 16 * j + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + swz(row, 2 * g4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + swz(row, 2 * g4 + 1));
        bop[j] = make_v8i(lo, hi);
      }
      float scale[C::kFragM];
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) scale[j] = sa_cur[j] * sb_cur;   // fl32(sa * sb)

#pragma unroll
      for (int i = 0; i < C::kFragN; ++i) {
        const int row = wave_n * WN + 16 * i + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sB + swz(row, 2 * g4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sB + swz(row, 2 * g4 + 1));
        const v8i aop = make_v8i(lo, hi);
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop, bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], scale[j], acc[i][j][r]);
        }
      }

      if (more) {
        DG_STORE_STAGE(stage ^ 1);
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j) sa_cur[j] = sa_next[j];
        sb_cur = sb_next;
      }
      __syncthreads();
      stage ^= 1;
    }
#undef DG_LOAD_STAGE
#undef DG_STORE_STAGE

    // ---- split-K: last arriving workgroup sums partials in split order ---------
    // The hand-off avoids device-scope fences (on a multi-XCD part they write back and
    // invalidate whole L2 caches): partials are written with agent-scope stores, which
    // write through the XCD's L2, completion is awaited with s_waitcnt before the
    // arrival counter is bumped, and the last workgroup reads them back with
    // agent-scope loads, which miss in its own (non-coherent) L2.
    if (p.splits > 1) {
      constexpr int kVals = C::kFragN * C::kFragM * 4;
      float* mine = p.ws + ((int64_t)t.tile_id * p.splits + t.split) * (int64_t)(kVals * NT);
#pragma unroll
      for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __hip_atomic_store(mine + ((i * C::kFragM + j) * 4 + r) * NT + tid, acc[i][j][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);   // every partial store of this thread has completed
      __syncthreads();
      if (tid == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(p.counters + t.tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = (prev == (unsigned)(p.splits - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (!s_flag) continue;
      const float* base = p.ws + (int64_t)t.tile_id * p.splits * (int64_t)(kVals * NT);
      // fixed order: sum = p_0 + p_1 + ... + p_{S-1}; this workgroup's own partial comes from registers
      v4f red[C::kFragN][C::kFragM];
      for (int s = 0; s < p.splits; ++s) {
        v4f v[C::kFragN][C::kFragM];
        if (s == t.split) {
#pragma unroll
          for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
            for (int j = 0; j < C::kFragM; ++j) v[i][j] = acc[i][j];
        } else {
          const float* src = base + (int64_t)s * (kVals * NT) + tid;
#pragma unroll
          for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
            for (int j = 0; j < C::kFragM; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                v[i][j][r] = __hip_atomic_load(src + ((i * C::kFragM + j) * 4 + r) * NT, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
          for (int j = 0; j < C::kFragM; ++j) red[i][j] = (s == 0) ? v[i][j] : red[i][j] + v[i][j];
      }
#pragma unroll
      for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j) acc[i][j] = red[i][j];
      if (tid == 0)   // leave the counter zeroed for the next call
        __hip_atomic_store(p.counters + t.tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: fp32 -> bf16 (RNE), row-major store, edge masking ------------
    uint16_t* d_g = p.d + (LAYOUT == kMasked ? (int64_t)t.g * p.d_gstride : 0);
    const bool vec_ok = (p.n & 3) == 0;
#pragma unroll
    for (int j = 0; j < C::kFragM; ++j) {
      const int mrow = m0 + wave_m * WM + 16 * j + l16;
      if (mrow >= t.m_valid) continue;
      uint16_t* drow = d_g + (int64_t)mrow * p.n;
#pragma unroll
      for (int i = 0; i < C::kFragN; ++i) {
        const int ncol = n0 + wave_n * WN + 16 * i + 4 * g4;
        const uint16_t h0 = f32_to_bf16_rne(acc[i][j][0]);
        const uint16_t h1 = f32_to_bf16_rne(acc[i][j][1]);
        const uint16_t h2 = f32_to_bf16_rne(acc[i][j][2]);
        const uint16_t h3 = f32_to_bf16_rne(acc[i][j][3]);
        if (vec_ok && ncol + 3 < p.n) {
          uint2 v;
          v.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
          v.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
          *reinterpret_cast<uint2*>(drow + ncol) = v;
        } else {
          if (ncol + 0 < p.n) drow[ncol + 0] = h0;
          if (ncol + 1 < p.n) drow[ncol + 1] = h1;
          if (ncol + 2 < p.n) drow[ncol + 2] = h2;
          if (ncol + 3 < p.n) drow[ncol + 3] = h3;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: tile configurations, occupancy, split-K choice and launch.
// ---------------------------------------------------------------------------
struct LaunchInfo {
  int bn, bm, threads;
  const void* fn;
};

template <int BN, int BM, int WN, int WM, int LAYOUT>
static LaunchInfo info() {
  return LaunchInfo{BN, BM, TileCfg<BN, BM, WN, WM>::kThreads,
                    reinterpret_cast<const void*>(&gemm_fp8_kernel<BN, BM, WN, WM, LAYOUT>)};
}

// Tile configurations (BN x BM, wave tile WN x WM).
enum Cfg : int { kCfgLarge = 0, kCfgSmallM = 1, kNumCfg = 2 };

template <int LAYOUT>
static LaunchInfo cfg_info(int cfg) {
  switch (cfg) {
    case kCfgSmallM: return info<128, 64, 64, 32, LAYOUT>();
    default: return info<128, 128, 64, 64, LAYOUT>();
  }
}

static int occupancy(const LaunchInfo& li) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, li.fn, li.threads, 0) != hipSuccess || blocks < 1)
    blocks = 1;
  return blocks;
}

struct Plan {
  int cfg;
  int splits;
  int kb_per_split;
  int tiles_m, tiles_n;
  size_t ws_bytes;   // needed workspace for this plan (0 when splits == 1)
};

// Pick the tile config and the K split for a problem with `tiles` output tiles per group.
static Plan make_plan(int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, bool allow_split) {
  Plan pl{};
  pl.cfg = (m <= 64) ? kCfgSmallM : kCfgLarge;
  const int bn = 128, bm = (pl.cfg == kCfgSmallM) ? 64 : 128;
  pl.tiles_m = (int)((m + bm - 1) / bm);
  pl.tiles_n = (int)((n + bn - 1) / bn);
  const int kb_total = (int)(k / kGroup);
  const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n * groups;
  pl.splits = 1;
  if (allow_split && tiles < num_cus) {
    int want = (int)((num_cus + tiles - 1) / tiles);
    const int max_split = kb_total / 4 > 0 ? kb_total / 4 : 1;   // keep >= 4 K blocks per split
    if (want > max_split) want = max_split;
    if (want > 1) pl.splits = want;
  }
  pl.kb_per_split = (kb_total + pl.splits - 1) / pl.splits;
  pl.splits = (kb_total + pl.kb_per_split - 1) / pl.kb_per_split;   // no empty split
  pl.ws_bytes = 0;
  if (pl.splits > 1) {
    const size_t counters = ((size_t)tiles * 4 + 255) & ~(size_t)255;
    pl.ws_bytes = counters + (size_t)tiles * pl.splits * (size_t)bn * bm * 4;
  }
  return pl;
}

void gemm_config_name(int layout, int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, char* buf,
                      size_t len) {
  const Plan pl = make_plan(m, n, k, layout == kMasked ? groups : 1, num_cus, layout != kContiguous);
  const LaunchInfo li = cfg_info<kDense>(pl.cfg);
  const int waves = li.threads / 64;
  snprintf(buf, len, "%dx%d/%dwaves/split%d", li.bn, li.bm, waves, pl.splits);
}

size_t gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus) {
  return make_plan(m, n, k, groups, num_cus, true).ws_bytes;
}

template <int LAYOUT>
static int launch_layout(GemmParams p, const Plan& pl, hipStream_t stream, int num_cus) {
  const LaunchInfo li = cfg_info<LAYOUT>(pl.cfg);
  const int occ = occupancy(li);
  int64_t items = (int64_t)pl.tiles_m * pl.tiles_n * (LAYOUT == kContiguous ? 1 : p.num_groups) * pl.splits;
  if (items > 0x7fffffffLL) return set_error(kUnsupported, "gemm: too many work items");
  int64_t grid = (int64_t)num_cus * occ;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(li.fn, dim3((unsigned)grid), dim3(li.threads), args, 0, stream);
  return e == hipSuccess ? kOk : set_error(kHip, "gemm launch: %s", hipGetErrorString(e));
}

int launch_gemm(int layout, const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                const float* sb, uint16_t* d, const int32_t* m_indices, const int32_t* masked_m,
                int64_t groups, int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                hipStream_t stream, int num_cus) {
  if (n * k > 0x7fffffffLL || m * k > 0x7fffffffLL)
    return set_error(kUnsupported, "gemm: one group's operand must be < 2^31 bytes (m=%lld n=%lld k=%lld)",
                     (long long)m, (long long)n, (long long)k);
  const bool can_split = (layout != kContiguous) && ws != nullptr;
  Plan pl = make_plan(m, n, k, layout == kMasked ? groups : 1, num_cus, can_split);
  if (pl.splits > 1 && ws_bytes < pl.ws_bytes) pl = make_plan(m, n, k, layout == kMasked ? groups : 1, num_cus, false);

  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.m_indices = m_indices; p.masked_m = masked_m;
  p.ld_sa = ld_sa;
  p.m = (int)m; p.n = (int)n; p.k = (int)k;
  p.num_groups = (int)(layout == kDense ? 1 : groups);
  p.kb_total = (int)(k / kGroup);
  p.nb128 = (int)((n + kGroup - 1) / kGroup);
  p.tiles_m = pl.tiles_m; p.tiles_n = pl.tiles_n;
  p.splits = pl.splits; p.kb_per_split = pl.kb_per_split;
  p.a_gstride = m * k;
  p.sa_gstride = (k / kGroup) * ld_sa;
  p.b_gstride = n * k;
  p.sb_gstride = (int64_t)p.nb128 * p.kb_total;
  p.d_gstride = m * n;
  if (pl.splits > 1) {
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n * p.num_groups;
    const size_t counters = ((size_t)tiles * 4 + 255) & ~(size_t)255;
    p.counters = static_cast<unsigned*>(ws);
    p.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + counters);
  }
  if (layout == kMasked && groups > 1024) return set_error(kUnsupported, "masked gemm: at most 1024 groups");
  switch (layout) {
    case kContiguous: return launch_layout<kContiguous>(p, pl, stream, num_cus);
    case kMasked: return launch_layout<kMasked>(p, pl, stream, num_cus);
    default: return launch_layout<kDense>(p, pl, stream, num_cus);
  }
}

}  // namespace dg
