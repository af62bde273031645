// Definitions shared by the GEMM kernel and its host-side planner.
#pragma once

#include "common.hpp"

namespace dg {

// kDenseRowB: the dense form whose B operand carries one scale per row per 128-wide K group,
// in the activation-scale layout sb[kb * ld_sb + row] (both operands per-row: the weight-gradient
// GEMM of a linear layer), instead of one per 128 x 128 block.
enum Layout : int { kDense = 0, kContiguous = 1, kMasked = 2, kDenseRowB = 3 };

// Kernel arguments (one struct, passed by value).  Sizes are per group; the
// strides step from one group's operand to the next (masked layout, weights of
// the grouped layouts).
struct GemmParams {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  uint16_t* d;
  const int32_t* m_indices;   // contiguous: expert per row
  const int32_t* masked_m;    // masked: valid rows per group
  float* ws;                  // split-K partials
  unsigned* counters;         // split-K arrival counters, one per split output tile
  int64_t ld_sa;
  int64_t ld_sb;             // kDenseRowB: row stride of the per-row B scales
  int ld_ab;                 // kDenseRowB: row stride (bytes) of both operands (k, or larger for K slices)
  int64_t a_gstride, sa_gstride, b_gstride, sb_gstride, d_gstride;   // per-group strides (elements)
  int m;            // rows per group (dense: M, contiguous: M_total, masked: M_max)
  int n, k;
  int num_groups;
  int kb_total;     // k / 128
  int tiles_m;      // ceil(m / BM)
  int tiles_n;      // ceil(n / BN)
  int splits;       // K splits of the split tiles (1 = none)
  int kb_per_split;
  int tail_start;   // work items [0, tail_start) are whole tiles; every later tile is split in `splits`
  int nb128;        // ceil(n / 128): weight-scale rows per group
  // Activation quantization inside the launch (dense layout): the unquantized activations
  // (m x k row-major, fp32 or bf16) that the workgroups quantize into a / sa before the GEMM,
  // and the three counters of that step (chunks taken, chunks finished, workgroups past the wait).
  const void* fq_x;
  unsigned* fq_sync;
  int fq_bf16;
  int fq_max_polls; // bound of the wait for every chunk (polls of the finished-chunk counter)
  int debug;        // DG_DEBUG: run the layout checks and report through the diagnostics words
};

// Flag bits of the device diagnostics word (sticky until read with clearing).
enum DiagFlag : unsigned {
  kDiagMixedBlock = 1u,    // contiguous layout: a 128-row block whose rows name different experts
  kDiagExpertRange = 2u,   // contiguous layout: an expert index outside [0, num_groups) other than a
                           // whole block of -1
  kDiagFqTimeout = 4u,     // in-launch activation quantization: the bounded wait gave up
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// Buffer resource word 3 for raw (untyped, stride 0) buffer accesses on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy bit of buffer accesses that makes them coherent at device (agent) scope on
// gfx950: the access bypasses the non-coherent per-XCD L2.
constexpr int kCpolSc1 = 16;

// Raw buffer resource over [base, base + bytes): accesses at offsets >= bytes read zeros and
// drop writes (the hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferWord3);
}

// Masked layout: per-group work-item prefix s_prefix[0..groups] (s_prefix[g] = items before group
// g), where group g has ceil(clamp(masked_m[g], 0, m) / bm) * per_mblock items.  Threads 0..255 of
// the workgroup (at least 256 threads) count 4 groups each and scan in LDS; ends with a barrier.
__device__ __forceinline__ void masked_item_prefix(const int32_t* masked_m, int groups, int m, int bm,
                                                   int per_mblock, int* s_prefix, int* s_scan) {
  const int tid = threadIdx.x;
  const bool counts = tid < 256;
  int cnt[4];
  int local = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = 4 * tid + u;
    int mv = (counts && g < groups) ? masked_m[g] : 0;
    mv = mv < 0 ? 0 : (mv > m ? m : mv);
    cnt[u] = ((mv + bm - 1) / bm) * per_mblock;
    local += cnt[u];
  }
  if (counts) s_scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {   // inclusive Hillis-Steele scan over the 256 sums
    const int v = (counts && tid >= off) ? s_scan[tid - off] : 0;
    __syncthreads();
    if (counts) s_scan[tid] += v;
    __syncthreads();
  }
  if (counts) {
    int run = s_scan[tid] - local;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = 4 * tid + u;
      if (g <= groups) s_prefix[g] = run;
      run += cnt[u];
    }
    if (tid == 255 && groups == 1024) s_prefix[1024] = run;
  }
  __syncthreads();
}

// Group of work item `item` under that prefix: the g with s_prefix[g] <= item < s_prefix[g + 1].
__device__ __forceinline__ int masked_group_of(const int* s_prefix, int groups, int item) {
  int lo = 0, hi = groups;   // invariant: s_prefix[lo] <= item < s_prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_prefix[mid] <= item) lo = mid;
    else hi = mid;
  }
  return lo;
}

constexpr int kMaxSplits = 16;   // K splits of one output tile at most
// Split-K workspace: a fixed 64 KiB prefix of per-tile arrival counters (so that the partials of
// one call never land where another call's counters are), then the fp32 partials.  Shapes with
// more output tiles than counters do not split (they have plenty of tiles anyway).
// The last 16 words of the prefix are not tile counters: the in-launch activation quantization
// keeps its three counters there.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kFqSyncWord = kCounterBytes / 4 - 16;
constexpr int64_t kMaxCounterTiles = kFqSyncWord;

// Scratch the library holds per device for the normal GEMM that allocates nothing: the counter
// prefix and the split-K partials of every plan of the DeepSeek-V3 shapes on 256 CUs (the largest,
// 4096 x 7168 x 16384, needs ~41 MB).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

}  // namespace dg
