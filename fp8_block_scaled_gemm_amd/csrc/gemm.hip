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
//    16x16 output fragment, so the level-1 partial of a K block is one MFMA into a
//    zero accumulator and the level-2 promotion is one VALU FMA per output:
//    acc += P * fl32(sa * sb).  The MFMA's own E8M0 block scales stay neutral
//    (2^0): the fine-grained scales are arbitrary fp32 values.  The library is
//    built with MFMA results in VGPRs (no AGPR round trip before the FMA), and the
//    large tiles run two waves per SIMD so that one wave's promotion FMAs overlap
//    the other's MFMAs.
//  * MFMA operand A is the weight tile (rows n), operand B the activation tile
//    (rows m): each lane holds 4 consecutive n of one row m, so the promotion
//    scale is one value per lane and fragment and the bf16 epilogue stores 8
//    contiguous bytes per lane.
//  * Operand tiles (BN x 128 and BM x 128 bytes per K block) go straight from
//    global memory into LDS (buffer_load_dwordx4 ... lds: a 32-bit per-lane offset,
//    the K-block offset in an SGPR, no staging registers) in a
//    ring of STAGES buffers, each its own __shared__ object so that the compiler's
//    wait insertion can tell them apart.  On the 8-wave tiles one wave per SIMD issues
//    a stage's DMAs (it stalls while the DMA path drains them) and its SIMD partner
//    starts its MFMAs meanwhile.  Row r's 16-byte chunk c lives at slot
//    c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1): the 8 lanes of a DMA that fill one
//    row write one contiguous 128-byte line, and a fragment read (16 consecutive
//    rows, one logical chunk) touches 16 distinct 16-byte bank groups.
//  * A persistent grid (at most CU cap x occupancy) walks work items (group,
//    m-block, n-block, k-split) - the contiguous layout reads each m-block's
//    expert from m_indices, the masked layout reads masked_m on the device and
//    skips empty m-blocks - in an XCD-aware order (workgroups of one XCD take
//    neighbouring items, so they share weight panels in their L2).
//  * Small-m shapes split K over workgroups; the last-arriving workgroup of a
//    tile sums the fp32 partials in fixed split order (deterministic) and stores
//    bf16.
//  * The normal form can also take unquantized activations (the FQ flag): a prologue
//    quantizes them once into the workspace, shared by all workgroups through a work
//    queue, before the unchanged main loop.  It costs one device-scope atomic per
//    workgroup and one L2 invalidation per wave, which on this 8-XCD part exceed what
//    a separate quantizer launch costs in a HIP graph; the two-launch path stays the
//    faster one.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "gemm_common.hpp"

namespace dg {

typedef __attribute__((address_space(3))) void lds_void;

// LDS DMA: every active lane copies 16 (4) bytes from rsrc + voff + soff into lds + lane * 16 (4)
// (buffer_load_dword{,x4} ... lds; out-of-range offsets read zeros).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 4, voff, soff, 0, 0);
}
template <int V>
using IC = std::integral_constant<int, V>;

// Sticky diagnostics raised by the device code, one copy per device: word 0 holds DiagFlag bits,
// word 1 the first 128-row block (+1) a contiguous-layout check found wrong.  Only atomics
// write them; the host reads (and clears) them through read_diag after a synchronisation.
__device__ unsigned g_diag[4];

__device__ __forceinline__ void raise_diag(unsigned flag, unsigned detail_plus1) {
  atomicOr(&g_diag[0], flag);
  if (detail_plus1) atomicCAS(&g_diag[1], 0u, detail_plus1);
}

// DG_DEBUG check of one m-block of the contiguous layout: every row of a 128-row block must name
// the expert of the block's first row, and that expert must be in [0, groups) - or the whole block
// -1, the documented skip.  Reports through g_diag; the kernel goes on as without the check.
template <int NT, int BM>
__device__ __forceinline__ void check_contiguous_block(const int32_t* m_indices, int m, int groups, int m0) {
  for (int i = threadIdx.x; i < BM; i += NT) {
    const int row = m0 + i;
    if (row >= m) break;
    const int head = m_indices[row & ~(kGroup - 1)];
    const int v = m_indices[row];
    const unsigned blk = (unsigned)(row / kGroup) + 1u;
    if (v != head) raise_diag(kDiagMixedBlock, blk);
    else if ((v < 0 || v >= groups) && v != -1) raise_diag(kDiagExpertRange, blk);
  }
}

template <int BN_, int BM_, int WN_, int WM_, int STAGES_, bool HALF_ISSUE_ = false, bool PIPE_ = false>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, STAGES = STAGES_;
  // PIPE: the two-slot main loop that overlaps every K block's operand reads and DMA issue with
  // the previous block's MFMAs (one barrier per K block, placed two fragment rows before its end)
  static constexpr bool PIPE = PIPE_;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWaves = kWavesN * kWavesM;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kFragN = WN / 16;
  static constexpr int kFragM = WM / 16;
  static constexpr int kSaOffset = (BN + BM) * kGroup;         // BM activation scales follow the tiles
  static constexpr int kSbOffset = kSaOffset + BM * 4;          // then the weight scales (adjacent)
  static constexpr int kSbCount = (BN + 127) / 128;             // 128-row weight blocks of a tile
  static constexpr int kSbWaveBytes = 16 * ((kSbCount * 4 + 15) / 16);   // one copy per issuing wave
  // Waves that issue the stage DMAs: all of them, or (half issue) the upper half, one wave per
  // SIMD.  An issuing wave stalls until the DMA path takes its instructions (~64 B/clk/CU); with
  // half issue the other wave on its SIMD starts its MFMAs meanwhile.
  static constexpr int kIssuers = HALF_ISSUE_ ? kWaves / 2 : kWaves;
  // per-row B scales (kDenseRowB): BN floats = BN/4 16-byte chunks, spread over the issuers' lanes
  static constexpr int kSbRowLanesPerWave = (BN / 4 + kIssuers - 1) / kIssuers;
  static constexpr int kDmaRows = 8;                          // one DMA instruction = 8 rows x 128 B
  static constexpr int kDmaB = BN / kDmaRows;                 // DMA instructions per stage, weights
  static constexpr int kDma = (BN + BM) / kDmaRows;           // ... weights + activations
  static constexpr int kDmaPerWave = kDma / kIssuers;         // per issuing wave
  // activation scales: BM floats = BM/4 16-byte chunks, spread over the issuers' lanes
  static constexpr int kSaLanesPerWave = (BM / 4 + kIssuers - 1) / kIssuers;
  // vector-memory instructions an issuing thread issues per stage: operand DMAs + the two scale DMAs
  static constexpr int kVmPerStage = kDmaPerWave + 2;
  // PIPE stage: the operand tiles, then per wave 64 activation scales (256 B) and, after all of
  // those, per wave 64 copies of its weight block's scale (256 B)
  static constexpr int kPipeSaOffset = (BN + BM) * kGroup;
  static constexpr int kPipeSbOffset = kPipeSaOffset + kWaves * 256;
  static_assert(kDma % kIssuers == 0 && kDmaB % kIssuers == 0, "DMA instructions must split evenly over waves");
  static_assert(kIssuers % 2 == 0, "a DMA band must span a multiple of 16 rows (the swizzle period)");
  static_assert(WN % 16 == 0 && WM % 16 == 0 && 128 % WN == 0, "wave tile must be 16-aligned, WN | 128");
  static_assert(STAGES >= 2 && STAGES <= 4, "2..4 stages");
  static_assert(kVmPerStage * (STAGES - 1) < 64, "vmcnt range");
  static_assert(!PIPE || (STAGES == 2 && WN / 16 >= 3 && !HALF_ISSUE_), "PIPE: two slots, >= 3 fragment rows, all waves issue");
  // every issuing wave issues exactly kVmPerStage instructions per stage (lane 0 of each scale DMA
  // is active), which the vmcnt waits count on
  static_assert(kSaLanesPerWave <= 64 && BM % 4 == 0 && (kIssuers - 1) * kSaLanesPerWave < BM / 4,
                "scale DMA shape");
  static_assert(kSbRowLanesPerWave <= 64 && BN % 4 == 0 && (kIssuers - 1) * kSbRowLanesPerWave < BN / 4,
                "row-scale DMA shape");
};

// Bytes of one LDS stage: the operand tiles, the activation scales, then the B scales (per-wave
// copies of the tile's block scales, or BN per-row scales for kDenseRowB).
template <class C, int LAYOUT>
constexpr int stage_bytes() {
  if constexpr (C::PIPE) return C::kPipeSbOffset + C::kWaves * 256;
  return C::kSbOffset + (LAYOUT == kDenseRowB ? C::BN * 4 : C::kIssuers * C::kSbWaveBytes);
}

// LDS slot of 16-byte chunk c of tile row r.  f depends on r mod 16 only, so every fragment
// of a lane shares one pattern and fragment addresses differ by immediates.
__device__ __forceinline__ int swz_row(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kGroup + ((c ^ swz_row(r)) << 4); }

__device__ __forceinline__ v8i make_v8i(u32x4 lo, u32x4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most `younger` stage groups of PER vector-memory instructions remain outstanding.
template <int PER, int MAXG>
__device__ __forceinline__ void wait_groups(int younger) {
  if constexpr (MAXG >= 3) {
    if (younger >= 3) { wait_vmcnt<3 * PER>(); return; }
  }
  if constexpr (MAXG >= 2) {
    if (younger >= 2) { wait_vmcnt<2 * PER>(); return; }
  }
  if constexpr (MAXG >= 1) {
    if (younger >= 1) { wait_vmcnt<PER>(); return; }
  }
  wait_vmcnt<0>();
}

struct TileCoord {
  int g, mb, nbt, split;
  int m_lo, m_valid;   // the tile's output rows are those in [m_lo, m_valid)
};

// ---- activation quantization inside the GEMM launch (dense layout) ---------------------------
// The 1 x 128 groups of x, numbered in row-major order (r * KB + kb), are cut into chunks of
// kFqGroupsPerLane groups per half-wave.  Workgroups take chunks from a counter until none is
// left, quantize them into a / sa with the per-token-group rule (quant_group4) through stores
// that write through the XCD's L2 (the agent-scope stores of the split-K partials), wait for
// those stores, and count the chunk as finished.  Every workgroup then waits until all chunks
// are finished, and every wave acquires at device scope (its CU's L1 and its XCD's L2 drop
// non-coherent lines), so the GEMM's ordinary loads read the quantized operand.  Nothing waits
// inside a chunk and only a running workgroup takes one, so the wait ends however many of the
// grid's workgroups are resident.
constexpr int kFqGroupsPerLane = 4;   // groups per half-wave per chunk (loads in flight per lane)
constexpr int kFqMaxPolls = 1 << 20;  // default bound of the wait (on the order of a second)

template <int NT, class T>
__device__ __forceinline__ void fq_chunk(const GemmParams& p, const T* x, int c, int groups,
                                         __amdgpu_buffer_rsrc_t rs_q, __amdgpu_buffer_rsrc_t rs_s) {
  constexpr int kHalfWaves = NT / 32;
  constexpr int kChunkGroups = kHalfWaves * kFqGroupsPerLane;
  const int hw = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  int e[kFqGroupsPerLane], sidx[kFqGroupsPerLane];
  bool ok[kFqGroupsPerLane];
  v4f v[kFqGroupsPerLane];
  // every lane loads (an absent group or column from x's first element), so the loads of all
  // kFqGroupsPerLane groups are in flight together; absent values are zeroed afterwards
#pragma unroll
  for (int u = 0; u < kFqGroupsPerLane; ++u) {
    const int gid = c * kChunkGroups + u * kHalfWaves + hw;
    const bool present = gid < groups;
    const int r = present ? gid / p.kb_total : 0;
    const int kb = present ? gid - r * p.kb_total : 0;
    const int col = kb * kGroup + 4 * l32;
    ok[u] = present && col < p.k;
    e[u] = r * p.k + col;
    sidx[u] = present ? kb * (int)p.ld_sa + r : -1;
    v[u] = load4(x + (ok[u] ? e[u] : 0));
  }
#pragma unroll
  for (int u = 0; u < kFqGroupsPerLane; ++u)
    if (!ok[u]) v[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kFqGroupsPerLane; ++u) {
    float s;
    const uint32_t packed = quant_group4(v[u], s);
    if (ok[u]) __builtin_amdgcn_raw_buffer_store_b32(packed, rs_q, e[u], 0, kCpolSc1);
    if (l32 == 0 && sidx[u] >= 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), rs_s, sidx[u] * 4, 0, kCpolSc1);
  }
}

template <int NT>
__device__ __forceinline__ void fused_act_quant(const GemmParams& p, int* s_bcast) {
  constexpr int kChunkGroups = (NT / 32) * kFqGroupsPerLane;
  const int tid = threadIdx.x;
  const int groups = p.m * p.kb_total;   // m * k < 2^31 (host check)
  const int chunks = (groups + kChunkGroups - 1) / kChunkGroups;
  unsigned* const take = p.fq_sync;
  unsigned* const done = p.fq_sync + 1;
  const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(p.a, (int64_t)p.m * p.k);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(p.sa, (int64_t)p.kb_total * p.ld_sa * 4);
  // One thread-0 region per iteration, between two barriers: it counts the previous chunk as
  // finished (every thread waited for its stores of it, then reached the first barrier) and
  // takes the next.  (Two thread-0 regions next to each other across the loop's back edge are
  // merged by the compiler into one with a divergent latch, and the loop then never ends.)  The
  // taken index is read as a wave-uniform scalar, so the loop's exit is a scalar branch.
  bool had_chunk = false;
  for (;;) {
    __syncthreads();   // the previous chunk's stores are complete; the previous broadcast was read
    if (tid == 0) {
      if (had_chunk) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_bcast = (int)__hip_atomic_fetch_add(take, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int c = __builtin_amdgcn_readfirstlane(*s_bcast);
    if (c >= chunks) break;
    if (p.fq_bf16) fq_chunk<NT>(p, static_cast<const uint16_t*>(p.fq_x), c, groups, rs_q, rs_s);
    else fq_chunk<NT>(p, static_cast<const float*>(p.fq_x), c, groups, rs_q, rs_s);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's stores of the chunk have completed
    had_chunk = true;
  }
  // Once every chunk is taken, the wait lasts about one chunk's time.  It gives up after
  // p.fq_max_polls polls (kFqMaxPolls: on the order of a second) so that counters left non-zero
  // by a misuse of the workspace give a wrong result, flagged in the device diagnostics, instead
  // of a wait that never ends.
  if (tid == 0) {
    bool finished = false;
    for (int poll = 0; poll < p.fq_max_polls; ++poll) {
      if (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)chunks) {
        finished = true;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    if (!finished) raise_diag(kDiagFqTimeout, 0u);   // the result of this call is not valid
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Leaving the kernel: the last workgroup out zeroes the counters of the quantization step for the
// next call (every workgroup is past its wait by then).  Done here, after the persistent loop,
// rather than right after the wait: a store there costs the main loop ~40 VGPRs.
__device__ __forceinline__ void fused_act_quant_exit(const GemmParams& p) {
  if (threadIdx.x != 0) return;
  const unsigned prev = __hip_atomic_fetch_add(p.fq_sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (prev == gridDim.x - 1) {
    __hip_atomic_store(p.fq_sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.fq_sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.fq_sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


template <class C, int LAYOUT, bool FQ = false>
__global__ __launch_bounds__(C::kThreads) void gemm_fp8_kernel(GemmParams p) {
  constexpr int NT = C::kThreads;
  constexpr int S = C::STAGES;
  constexpr bool kRowB = LAYOUT == kDenseRowB;
  constexpr int kStage = stage_bytes<C, LAYOUT>();
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? kStage : 16];
  __shared__ int s_prefix[LAYOUT == kMasked ? 1025 : 1];
  __shared__ int s_scan[LAYOUT == kMasked ? 256 : 1];
  __shared__ int s_flag;
  static_assert(NT >= 256, "the masked-layout prefix needs 256 threads");
  static_assert(!FQ || LAYOUT == kDense, "activation quantization in the launch: dense layout only");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) from here on
  const int wave_n = wave % C::kWavesN;
  const int wave_m = wave / C::kWavesN;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int wn0 = wave_n * C::WN;
  const int wm0 = wave_m * C::WM;

  if constexpr (FQ) fused_act_quant<NT>(p, &s_flag);

  // ---- total work items -------------------------------------------------------
  int total_items;
  if constexpr (LAYOUT == kMasked) {
    // prefix over groups of the number of (m-block, n-block) tiles, from device counts
    masked_item_prefix(p.masked_m, p.num_groups, p.m, C::BM, p.tiles_n, s_prefix, s_scan);
    total_items = s_prefix[p.num_groups] * p.splits;
  } else {
    // contiguous: the expert comes from m_indices, not from the item index.  The first tail_start
    // tiles are whole work items, each later tile is `splits` items (a K split that fills the last,
    // partial round of the persistent grid)
    const int tiles = p.tiles_m * p.tiles_n * (LAYOUT == kDense ? p.num_groups : 1);
    total_items = p.tail_start + (tiles - p.tail_start) * p.splits;
  }

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of items in every round of the persistent loop.
  const int grid = gridDim.x;
  int wg = blockIdx.x;
  if ((grid & 7) == 0) wg = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);

  // The contiguous layout on 256-row tiles: a tile whose two 128-row halves belong to different
  // experts runs twice (pass 0 with the first half's expert, pass 1 with the second's), each pass
  // storing only its own half.  Every other tile runs once.
  constexpr bool kTwoPass = LAYOUT == kContiguous && C::BM > kGroup;
  int step = grid, next_pass = 0;
  for (int item = wg, pass = 0; item < total_items; item += step, pass = next_pass) {
    step = grid;
    next_pass = 0;
    // ---- decode the item ------------------------------------------------------
    TileCoord t;
    t.m_lo = 0;
    // whole tile (item < tail_start) or split `t.split` of split tile `sidx`
    const bool split_item = item >= p.tail_start;
    const int sidx = (item - p.tail_start) / p.splits;
    t.split = split_item ? (item - p.tail_start) % p.splits : 0;
    int rest = split_item ? p.tail_start + sidx : item;
    if constexpr (LAYOUT == kMasked) {
      const int g = masked_group_of(s_prefix, p.num_groups, rest);
      rest -= s_prefix[g];
      const int mblocks = (s_prefix[g + 1] - s_prefix[g]) / p.tiles_n;
      t.g = g;
      t.mb = rest % mblocks;
      t.nbt = rest / mblocks;
      int mv = p.masked_m[g];
      t.m_valid = mv < 0 ? 0 : (mv > p.m ? p.m : mv);
    } else {
      // grouped order: runs of kGroupM m-tiles x all n-tiles, m fastest inside a run, so the
      // grid/8 consecutive items one XCD takes per round cover ~8 activation panels and a few
      // weight panels (both reused from that XCD's L2)
      constexpr int kGroupM = 8;
      const int per_group = p.tiles_m * p.tiles_n;
      t.g = rest / per_group;
      const int tl = rest - t.g * per_group;
      const int run = tl / (kGroupM * p.tiles_n);
      const int first_m = run * kGroupM;
      const int run_m = (p.tiles_m - first_m) < kGroupM ? (p.tiles_m - first_m) : kGroupM;
      const int in_run = tl - run * (kGroupM * p.tiles_n);
      t.mb = first_m + in_run % run_m;
      t.nbt = in_run / run_m;
      t.m_valid = p.m;
    }
    const int m0 = t.mb * C::BM;
    const int n0 = t.nbt * C::BN;
    int expert = t.g;
    if constexpr (LAYOUT == kContiguous) {
      expert = p.m_indices[m0];
      if (p.debug && pass == 0) check_contiguous_block<NT, C::BM>(p.m_indices, p.m, p.num_groups, m0);
      if constexpr (kTwoPass) {
        static_assert(C::BM == 2 * kGroup, "a contiguous tile spans one or two 128-row expert blocks");
        const int e1 = m0 + kGroup < p.m ? p.m_indices[m0 + kGroup] : expert;
        if (e1 != expert) {   // uniform: the halves name different experts (or one is unmapped)
          if (pass == 0) {
            step = 0;          // the same item again, as pass 1
            next_pass = 1;
            t.m_valid = m0 + kGroup;
          } else {
            expert = e1;
            t.m_lo = m0 + kGroup;
          }
        }
      }
      if (expert < 0 || expert >= p.num_groups) continue;   // uniform: skip an unmapped block or half
    }
    const int kb_begin = split_item ? t.split * p.kb_per_split : 0;
    int kb_end = split_item ? kb_begin + p.kb_per_split : p.kb_total;
    if (kb_end > p.kb_total) kb_end = p.kb_total;
    const int nk = kb_end - kb_begin;

    const uint8_t* a_g = p.a + (LAYOUT == kMasked ? (int64_t)t.g * p.a_gstride : 0);
    const float* sa_g = p.sa + (LAYOUT == kMasked ? (int64_t)t.g * p.sa_gstride : 0);
    const uint8_t* b_g = p.b + (int64_t)expert * p.b_gstride;
    const float* sb_g = p.sb + (int64_t)expert * p.sb_gstride;

    // DMA instruction u of this wave fills tile rows [8q, 8q+8) of a stage, q = wave + kWaves*u:
    // weights for u < kDmaB / kWaves, activations after.  Lane i writes slot i of that 1 KB (tile
    // row 8q + i/8, slot i%8), so it loads logical chunk (i%8) ^ f(row).  Each operand has one
    // buffer resource based at the tile's first row and sized to the rows that exist (for the
    // masked layout: the group's valid rows, so its padding rows cost no memory traffic): the
    // hardware range check returns zeros for rows past the N or M edge (those outputs are never
    // stored).
    constexpr int kBandRows = 8 * C::kIssuers;
    constexpr int kBandsB = C::kDmaB / C::kIssuers;
    const int iw = wave - (C::kWaves - C::kIssuers);   // index among the issuing waves (< 0: not one)
    const bool issuer = iw >= 0;                      // wave-uniform
    const int dma_row = 8 * iw + (lane >> 3);   // tile-local row within band 0 (f(row) is band-invariant)
    const int dma_chunk = ((lane & 7) ^ swz_row(dma_row)) << 4;   // byte offset of this lane's chunk in the K block
    // Operand rows are ld bytes apart: k, except for kDenseRowB on a K slice of wider matrices
    // (the per-expert token ranges of the grouped weight gradient).  A resource ends after the last
    // present row's k bytes, so rows past the edge read zeros.
    const int ld = kRowB ? p.ld_ab : p.k;
    const uint32_t dma_off = (uint32_t)dma_row * (uint32_t)ld + (uint32_t)dma_chunk;
    const uint32_t band_step = (uint32_t)kBandRows * (uint32_t)ld;
    const __amdgpu_buffer_rsrc_t rs_b =
        make_rsrc(b_g + (int64_t)n0 * ld, p.n > n0 ? (int64_t)(p.n - n0 - 1) * ld + p.k : 0);
    const __amdgpu_buffer_rsrc_t rs_a =
        make_rsrc(a_g + (int64_t)m0 * ld, t.m_valid > m0 ? (int64_t)(t.m_valid - m0 - 1) * ld + p.k : 0);
    // activation scales: lanes [kSaLanesPerWave*wave, +kSaLanesPerWave) of the BM/4 16-byte chunks
    // of sa[kb][m0 .. m0+BM); chunks are clamped to the caller's ld_sa row (rows >= m are never stored)
    const int sa_lane = iw * C::kSaLanesPerWave + lane;
    const bool sa_active = issuer && lane < C::kSaLanesPerWave && sa_lane < C::BM / 4;
    int sa_src_row = m0 + 4 * sa_lane;
    sa_src_row = sa_src_row + 4 <= p.ld_sa ? sa_src_row : (int)p.ld_sa - 4;
    const uint32_t sa_src = (uint32_t)sa_src_row * 4u;   // byte offset within the kb row
    // B scales.  Block scales: lane i < kSbCount of every wave fetches the scale of weight block
    // n0/128 + i into the wave's own copy (keeps the per-wave vmcnt accounting uniform).  Per-row
    // scales (kDenseRowB): as the activation scales, lanes of every wave fetch the BN/4 16-byte
    // chunks of sb[kb][n0 .. n0+BN), clamped to the caller's ld_sb row.
    const int sbr_lane = iw * C::kSbRowLanesPerWave + lane;
    const bool sb_active =
        issuer && (kRowB ? (lane < C::kSbRowLanesPerWave && sbr_lane < C::BN / 4) : lane < C::kSbCount);
    int sb_blk = (n0 >> 7) + lane;
    sb_blk = sb_blk < p.nb128 ? sb_blk : p.nb128 - 1;
    int sbr_row = n0 + 4 * sbr_lane;
    sbr_row = sbr_row + 4 <= p.ld_sb ? sbr_row : (int)p.ld_sb - 4;
    const uint32_t sb_src = kRowB ? (uint32_t)sbr_row * 4u : (uint32_t)sb_blk * (uint32_t)p.kb_total * 4u;
    const int sb_idx = ((n0 + wn0) >> 7) - (n0 >> 7);   // this wave's block within the tile
    const __amdgpu_buffer_rsrc_t rs_sa = make_rsrc(sa_g, (int64_t)p.kb_total * p.ld_sa * 4);
    const __amdgpu_buffer_rsrc_t rs_sb =
        make_rsrc(sb_g, kRowB ? (int64_t)p.kb_total * p.ld_sb * 4 : (int64_t)p.nb128 * p.kb_total * 4);

    v4f acc[C::kFragN][C::kFragM];
#pragma unroll
    for (int i = 0; i < C::kFragN; ++i)
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Issue the stage group of local K block tk (absolute kb_begin + tk) into ring slot SLOT:
    // kDmaPerWave operand DMAs and the activation- and weight-scale DMAs (the vmcnt accounting
    // counts kVmPerStage per group).
    auto issue = [&](int tk, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      if (!issuer) return;
      const int kb = kb_begin + tk;
      uint8_t* sbase = slot == 0 ? st0 : slot == 1 ? st1 : slot == 2 ? st2 : st3;
      // the per-band offsets are recomputed at every issue (one add each) from an opaque copy
      // of the band-0 offset, rather than kept live in a register per band across the main loop
      uint32_t base_off = dma_off;
      asm volatile("" : "+v"(base_off));
      // a partial last K block (k % 128 != 0): chunks past k take an out-of-range offset, so the
      // range check writes zeros instead of reading the next row's bytes
      const bool tail = (kb + 1) * kGroup > p.k;   // wave-uniform
      const bool chunk_out = tail && kb * kGroup + dma_chunk >= p.k;
#pragma unroll
      for (int u = 0; u < C::kDmaPerWave; ++u) {
        const int q = iw + C::kIssuers * u;
        const bool is_b = u < kBandsB;
        const uint32_t voff = base_off + (uint32_t)(is_b ? u : u - kBandsB) * band_step;
        lds_dma16(is_b ? rs_b : rs_a, sbase + q * (C::kDmaRows * kGroup), chunk_out ? 0xFFFFFFF0u : voff,
                  kb * kGroup);
      }
      if (sa_active)
        lds_dma16(rs_sa, sbase + C::kSaOffset + 16 * iw * C::kSaLanesPerWave, sa_src, kb * (int)p.ld_sa * 4);
      if (sb_active) {
        if constexpr (kRowB)
          lds_dma16(rs_sb, sbase + C::kSbOffset + 16 * iw * C::kSbRowLanesPerWave, sb_src, kb * (int)p.ld_sb * 4);
        else
          lds_dma4(rs_sb, sbase + C::kSbOffset + iw * C::kSbWaveBytes, sb_src, kb * 4);
      }
    };
    auto issue_rt = [&](int tk, int slot) {
      if (slot == 0) issue(tk, IC<0>{});
      else if (slot == 1) issue(tk, IC<1>{});
      else if (slot == 2) issue(tk, IC<(S > 2 ? 2 : 0)>{});
      else issue(tk, IC<(S > 3 ? 3 : 0)>{});
    };

    // Level-1 MFMA partials of the K block in ring slot SLOT and their level-2 promotion.
    // The B fragments (activations) and scales of the K block are read from LDS once; the A
    // fragments (weights) are streamed, fragment i+1 being read while fragment i's MFMAs run.
    // Over the flat sequence q = (i, j) the MFMA of q is issued before the promotion FMAs of
    // q-1, so the matrix core does not wait for a partial the VALU is about to consume.
    auto compute = [&](auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      const uint8_t* sbase = slot == 0 ? st0 : slot == 1 ? st1 : slot == 2 ? st2 : st3;
      // A operand (weights) rows wn0 + 16i + l16, B operand (activations) rows wm0 + 16j + l16; a lane
      // reads logical chunks 2*g4 and 2*g4+1 (K bytes 32*g4 .. 32*g4+31) of its row.  The second
      // chunk's slot differs from the first's in bit 0 only: address ^ 16.
      const int lane_off = lds_off(l16, 2 * g4);   // == lds_off(16x + l16, 2*g4) - 16x*128
      auto read_a = [&](int i) {
        const int off = (wn0 + 16 * i) * kGroup + lane_off;
        return make_v8i(*reinterpret_cast<const u32x4*>(sbase + off),
                        *reinterpret_cast<const u32x4*>(sbase + (off ^ 16)));
      };
      v8i bop[C::kFragM];
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) {
        const int off = (C::BN + wm0 + 16 * j) * kGroup + lane_off;
        bop[j] = make_v8i(*reinterpret_cast<const u32x4*>(sbase + off),
                          *reinterpret_cast<const u32x4*>(sbase + (off ^ 16)));
      }
      const float* sa_l = reinterpret_cast<const float*>(sbase + C::kSaOffset);
      // block scales: scale[j] = fl32(sa * sb) of the lane's row, the wave's weight block; per-row
      // B scales: scale[j] = sa, and the 4 scales of the lane's 4 B rows of fragment i in sbr[i]
      float scale[C::kFragM];
      v4f sbr[kRowB ? C::kFragN : 1];
      if constexpr (kRowB) {
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j) scale[j] = sa_l[wm0 + 16 * j + l16];
#pragma unroll
        for (int i = 0; i < C::kFragN; ++i)
          sbr[i] = *reinterpret_cast<const v4f*>(sbase + C::kSbOffset + 4 * (wn0 + 16 * i + 4 * g4));
      } else {
        const float sbv = sa_l[C::BM + (wave % C::kIssuers) * (C::kSbWaveBytes / 4) + sb_idx];   // an issuer's copy
#pragma unroll
        for (int j = 0; j < C::kFragM; ++j) scale[j] = sa_l[wm0 + 16 * j + l16] * sbv;   // fl32(sa * sb)
      }

      constexpr int Q = C::kFragN * C::kFragM;
      v8i aop[2];
      aop[0] = read_a(0);
      v4f part[2];
#pragma unroll
      for (int q = 0; q <= Q; ++q) {
        if (q < Q) {
          const int i = q / C::kFragM, j = q % C::kFragM;
          // fragment row i: nothing of a later row may be scheduled above this point, so at most
          // two weight fragments are live (the one in use and the one being read)
          if (j == 0) __builtin_amdgcn_sched_barrier(0);
          if (j == 0 && i + 1 < C::kFragN) aop[(i + 1) & 1] = read_a(i + 1);
          part[q & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop[i & 1], bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        }
        if (q > 0) {
          const int i = (q - 1) / C::kFragM, j = (q - 1) % C::kFragM;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = __builtin_fmaf(part[(q - 1) & 1][r], kRowB ? scale[j] * sbr[kRowB ? i : 0][r] : scale[j],
                                          acc[i][j][r]);   // kRowB: fl32(sa * sb) per element
        }
        if (q > 0 && q < Q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA of q
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // FMAs of q-1
        }
      }
    };

    // ---- main loop ---------------------------------------------------------------
    if constexpr (C::PIPE) {
      // Two slots; a K block's operands come from slot tk & 1.  A wave's A fragments (weight rows)
      // are read two fragment rows ahead of their MFMAs, its B fragments (activation rows) and
      // scales one block ahead: every LDS read has two rows of MFMAs to return, the block
      // boundaries included.  Two rows before the end of block tk every wave has read all it reads
      // of slot tk & 1 and waits for its own DMAs of block tk+1; one barrier then makes both hold
      // for every wave.  After it, block tk+2's DMAs go into slot tk & 1, and block tk+1's scales,
      // first two A fragments and (each as soon as the last row's MFMA has consumed its
      // predecessor) B fragments are read from the other slot while the last two rows of block tk
      // run.  Every DMA of a block thus has one block's compute to land.  The block body has no
      // branch (a branch there lets the compiler sink the MFMAs below the barrier): past the last
      // K block the DMAs take out-of-range offsets and write zeros that nothing reads, and the
      // scales come by two all-lane DMAs per wave into the wave's own copy.
      static_assert(!kRowB, "per-row B scales run on the three-stage loop");
      constexpr int kFN = C::kFragN, kFM = C::kFragM;
      constexpr int kBarRow = kFN - 2;   // the rows after the barrier: kBarRow and the last one
      static_assert(kBarRow >= 1, "PIPE: at least three fragment rows");
      constexpr uint32_t kOut = 0xFFFFFFF0u;   // an offset past every resource: the DMA writes zeros
      using SlotPtr = const uint8_t*;
      // slot 0 (blocks 0, 2, ...) is the buffer the epilogue's strips do not use
      uint8_t* const slot0 = st1;
      uint8_t* const slot1 = st0;
      const int lane_off = lds_off(l16, 2 * g4);
      // this wave's activation-scale rows m0 + wm0 + lane (64 of them, the wave's WM first) and the
      // scale of its weight block, as byte offsets within a K block's scale row
      const int sa_row = m0 + wm0 + lane;
      const uint32_t sa_lane_off = sa_row < (int)p.ld_sa ? (uint32_t)sa_row * 4u : kOut;
      int sb_blk_w = (n0 + wn0) >> 7;
      sb_blk_w = sb_blk_w < p.nb128 ? sb_blk_w : p.nb128 - 1;
      const uint32_t sb_wave_off = (uint32_t)sb_blk_w * (uint32_t)p.kb_total * 4u;
      // The DMAs of one stage, issued one at a time (DMA d < kDmaPerWave: operand rows; then the
      // activation scales and the weight-block scale), so that the issue can be spread over MFMAs.
      constexpr int kStageDmas = C::kDmaPerWave + 2;
      struct DmaCtx {
        uint8_t* sbase;
        int kb;
        uint32_t base_off, out_mask, inv_mask;
      };
      auto dma_ctx = [&](int tk, auto slot_c, bool valid) {
        constexpr int slot = decltype(slot_c)::value;
        DmaCtx c;
        c.sbase = slot == 0 ? slot0 : slot1;
        c.kb = kb_begin + tk;
        c.base_off = dma_off;
        asm volatile("" : "+v"(c.base_off));
        // bitwise, not short-circuit: a branch here would split the block body
        const uint32_t out = (uint32_t)(!valid) | ((uint32_t)((c.kb + 1) * kGroup > p.k) &
                                                   (uint32_t)(c.kb * kGroup + dma_chunk >= p.k));
        c.out_mask = 0u - out;                   // all ones: out of range
        c.inv_mask = 0u - (uint32_t)(!valid);
        return c;
      };
      auto dma_one = [&](const DmaCtx& c, int d) {
        if (d < C::kDmaPerWave) {
          const int q = iw + C::kIssuers * d;
          const bool is_b = d < kBandsB;
          const uint32_t voff = c.base_off + (uint32_t)(is_b ? d : d - kBandsB) * band_step;
          lds_dma16(is_b ? rs_b : rs_a, c.sbase + q * (C::kDmaRows * kGroup), voff | (c.out_mask & kOut),
                    c.kb * kGroup);
        } else if (d == C::kDmaPerWave) {
          // (readfirstlane: the offset is uniform; keeps the compiler from computing it per lane)
          lds_dma4(rs_sa, c.sbase + C::kPipeSaOffset + wave * 256, sa_lane_off | (c.inv_mask & kOut),
                   __builtin_amdgcn_readfirstlane(c.kb * (int)p.ld_sa * 4));
        } else {
          lds_dma4(rs_sb, c.sbase + C::kPipeSbOffset + wave * 256, sb_wave_off | (c.inv_mask & kOut),
                   __builtin_amdgcn_readfirstlane(c.kb * 4));
        }
      };
      auto issue_pipe = [&](int tk, auto slot_c, bool valid) {
        const DmaCtx c = dma_ctx(tk, slot_c, valid);
#pragma unroll
        for (int d = 0; d < kStageDmas; ++d) dma_one(c, d);
      };
      auto read_a = [&](SlotPtr sbase, int i) {
        const int off = (wn0 + 16 * i) * kGroup + lane_off;
        return make_v8i(*reinterpret_cast<const u32x4*>(sbase + off),
                        *reinterpret_cast<const u32x4*>(sbase + (off ^ 16)));
      };
      auto read_b = [&](SlotPtr sbase, int j) {
        const int off = (C::BN + wm0 + 16 * j) * kGroup + lane_off;
        return make_v8i(*reinterpret_cast<const u32x4*>(sbase + off),
                        *reinterpret_cast<const u32x4*>(sbase + (off ^ 16)));
      };
      // the scales of the block in slot sbase: the lane's activation scale of each B fragment in
      // raw[0, kFM), the wave's weight-block scale in raw[kFM] (multiplied where first used, so
      // that nothing waits for these reads)
      auto read_scales = [&](SlotPtr sbase, float* raw) {
        const float* sa_w = reinterpret_cast<const float*>(sbase + C::kPipeSaOffset + wave * 256);
#pragma unroll
        for (int j = 0; j < kFM; ++j) raw[j] = sa_w[16 * j + l16];
        raw[kFM] = *reinterpret_cast<const float*>(sbase + C::kPipeSbOffset + wave * 256);
      };
      // Fragment rows [R0, R1) of the block in slot cur; the rows from 0 first form the promotion
      // scales sc[j] = fl32(sa * sb) from the raw ones.  Row i takes its A fragment from a[i % 3]
      // and, at its start, requests row i+2's (rows kFN and kFN+1 are the next block's rows 0 and
      // 1, from slot nxt: only the rows after the barrier reach them).  In the last row, B fragment
      // j is replaced by the next block's as soon as that row's MFMA j has been issued.  The
      // promotion FMAs run one MFMA behind (flushed at the end).  Rows ahead of a barrier pin their
      // accumulators at the end, so that no MFMA of theirs can move below it.
      auto rows = [&](auto r0_c, auto r1_c, SlotPtr cur, SlotPtr nxt, v8i* a, v8i* bop, float* sc, const float* raw,
                      const DmaCtx* dc) {
        constexpr int R0 = decltype(r0_c)::value, R1 = decltype(r1_c)::value;
        if constexpr (R0 == 0) {
#pragma unroll
          for (int j = 0; j < kFM; ++j) sc[j] = raw[j] * raw[kFM];   // fl32(sa * sb)
        }
        constexpr int T = (R1 - R0) * kFM;   // MFMAs of these rows; with dc, the stage's DMAs spread over them
        v4f part[2];
#pragma unroll
        for (int q = R0 * kFM; q <= R1 * kFM; ++q) {
          if (q < R1 * kFM) {
            const int i = q / kFM, j = q % kFM;
            if (j == 0) {
              __builtin_amdgcn_sched_barrier(0);
              const int r = i + 2;
              a[r % 3] = r < kFN ? read_a(cur, r) : read_a(nxt, r - kFN);
            }
            part[q & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[i % 3], bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            if (i == kFN - 1) bop[j] = read_b(nxt, j);
          }
          if (q > R0 * kFM) {
            const int i = (q - 1) / kFM, j = (q - 1) % kFM;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[(q - 1) & 1][r], sc[j], acc[i][j][r]);
          }
          if (q > R0 * kFM && q < R1 * kFM) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA of q
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // FMAs of q-1
          }
          if (dc != nullptr && q < R1 * kFM) {
            // after MFMA t of these rows: DMAs [t * D / T, (t + 1) * D / T)
            const int t = q - R0 * kFM;
            const int d0 = t * kStageDmas / T, d1 = (t + 1) * kStageDmas / T;
            for (int d = d0; d < d1; ++d) dma_one(*dc, d);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (R1 == kBarRow) {
#pragma unroll
          for (int q = R0 * kFM; q < R1 * kFM; ++q) asm volatile("" : "+v"(acc[q / kFM][q % kFM]));
        }
      };
      // The barrier of block tk (slot CUR; the next block in slot NXT) and its last two rows.  A
      // loop iteration starts here: it waits for every DMA in flight, so what the compiler's wait
      // insertion cannot track across the loop's back edge costs nothing.  On return a[0], a[1]
      // hold the next block's first two A fragments, bop its B fragments, rn its raw scales.
      auto bar_tail = [&](int tk, auto cur_c, auto nxt_c, v8i* a, v8i* bop, float* sc, float* rn) {
        constexpr int cur_slot = decltype(cur_c)::value;
        constexpr int nxt_slot = decltype(nxt_c)::value;
        const SlotPtr cur = cur_slot == 0 ? slot0 : slot1;
        const SlotPtr nxt = nxt_slot == 0 ? slot0 : slot1;
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of slot CUR are done
        wait_vmcnt<0>();                      // its DMAs of block tk+1 have landed
        __syncthreads();                      // ... and every wave's
        const DmaCtx dc = dma_ctx(tk + 2, cur_c, tk + 2 < nk);
        read_scales(nxt, rn);
        rows(IC<kBarRow>{}, IC<kFN>{}, cur, nxt, a, bop, sc, nullptr, &dc);
        const v8i n0a = a[kFN % 3], n1a = a[(kFN + 1) % 3];
        a[0] = n0a;
        a[1] = n1a;
      };
      // Block 0's DMAs go out before the first wait, so that their latency overlaps the draining
      // of the previous tile's output stores.  Every wave is past its last read of slot 0 (the
      // previous tile's epilogue and K-split hand-off each begin with a barrier), and slot 1
      // holds the epilogue's strips until the barrier below.
      if (nk > 0) issue_pipe(0, IC<0>{}, true);   // (k = 0: no K block, the accumulators stay zero)
      wait_vmcnt<0>();
      __syncthreads();   // block 0 landed for every wave; every wave is done with the strips
      if (nk > 0) {
      issue_pipe(1, IC<1>{}, nk > 1);
      v8i bop[kFM], a[3];
      float sc[kFM], r0[kFM + 1], r1[kFM + 1];
#pragma unroll
      for (int j = 0; j < kFM; ++j) bop[j] = read_b(slot0, j);
      read_scales(slot0, r0);
      a[0] = read_a(slot0, 0);
      a[1] = read_a(slot0, 1);
      // block 0 up to its barrier row
      rows(IC<0>{}, IC<kBarRow>{}, slot0, slot1, a, bop, sc, r0, nullptr);
      // two blocks per iteration (the slots alternate), while a block tk+2 follows; then the rest
      int tk = 0;
      for (; tk + 2 < nk; tk += 2) {
        bar_tail(tk, IC<0>{}, IC<1>{}, a, bop, sc, r1);
        rows(IC<0>{}, IC<kBarRow>{}, slot1, slot0, a, bop, sc, r1, nullptr);
        bar_tail(tk + 1, IC<1>{}, IC<0>{}, a, bop, sc, r0);
        rows(IC<0>{}, IC<kBarRow>{}, slot0, slot1, a, bop, sc, r0, nullptr);
      }
      bar_tail(tk, IC<0>{}, IC<1>{}, a, bop, sc, r1);
      if (tk + 1 < nk) {
        rows(IC<0>{}, IC<kBarRow>{}, slot1, slot0, a, bop, sc, r1, nullptr);
        bar_tail(tk + 1, IC<1>{}, IC<0>{}, a, bop, sc, r0);
      }
      wait_vmcnt<0>();   // the zero-filling DMAs past the last K block
      }
    } else {
    __syncthreads();   // the previous tile's readers are done with every stage
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue_rt(s, s);
    for (int t0 = 0; t0 < nk; t0 += S) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int tk = t0 + s;
        if (tk >= nk) break;
        // K block tk landed for this thread (groups tk+1 .. min(tk+S-2, nk-1) may still fly) ...
        const int younger = (nk - 1 - tk) < (S - 2) ? (nk - 1 - tk) : (S - 2);
        wait_groups<C::kVmPerStage, S - 2>(younger);
        // ... and for every thread; also everyone finished computing tk-1, whose slot is refilled next
        __syncthreads();
        if (tk + S - 1 < nk) issue_rt(tk + S - 1, (s + S - 1) % S);
        if (s == 0) compute(IC<0>{});
        else if (s == 1) compute(IC<1>{});
        else if (s == 2) compute(IC<(S > 2 ? 2 : 0)>{});
        else compute(IC<(S > 3 ? 3 : 0)>{});
      }
    }
    }

    // ---- split-K: last arriving workgroup sums partials in split order ---------
    // The hand-off avoids device-scope fences (on a multi-XCD part they write back and
    // invalidate whole L2 caches): partials are written with agent-scope stores, which
    // write through the XCD's L2, completion is awaited with s_waitcnt before the
    // arrival counter is bumped, and the last workgroup reads them back with
    // agent-scope loads, which miss in its own (non-coherent) L2.
    if (split_item && p.splits > 1) {
      // partial layout: [fragment][thread][4] - 16 bytes per thread and fragment (coalesced)
      constexpr int kFrags = C::kFragN * C::kFragM;
      constexpr int kSplitBytes = kFrags * NT * 16;
      float* ws_tile = p.ws + (int64_t)sidx * p.splits * (int64_t)(kSplitBytes / 4);
      const __amdgpu_buffer_rsrc_t rs_ws = make_rsrc(ws_tile, (int64_t)p.splits * kSplitBytes);
      const int own = t.split * kSplitBytes + tid * 16;
#pragma unroll
      for (int f = 0; f < kFrags; ++f)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[f / C::kFragM][f % C::kFragM]), rs_ws,
                                               own + f * NT * 16, 0, kCpolSc1);
      __builtin_amdgcn_s_waitcnt(0);   // every partial store of this thread has completed
      __syncthreads();
      if (tid == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(p.counters + sidx, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = (prev == (unsigned)(p.splits - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (!s_flag) continue;
      // fixed order acc = p_0 + p_1 + ... + p_{S-1}, every partial (this workgroup's own
      // included) read back from the workspace, so the sum does not depend on who arrived last.
      // Up to kBatch splits of kChunk fragments are loaded together (all in flight) before they are
      // added (at most 32 fragments' worth of registers; 16 on tiles whose accumulators take 128).
      constexpr int kChunk = kFrags >= 32 ? 16 : kFrags;
      constexpr int kBatch = kFrags >= 32 ? 1 : 32 / kFrags;
      static_assert(kFrags % kChunk == 0, "fragment chunks");
#pragma unroll
      for (int f0 = 0; f0 < kFrags; f0 += kChunk) {
        for (int s0 = 0; s0 < p.splits; s0 += kBatch) {
          v4f v[kBatch][kChunk];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int sp = s0 + u < p.splits ? s0 + u : s0;
#pragma unroll
            for (int f = 0; f < kChunk; ++f)
              v[u][f] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs_ws, sp * kSplitBytes + tid * 16 + (f0 + f) * NT * 16, 0, kCpolSc1));
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if (s0 + u >= p.splits) break;
#pragma unroll
            for (int f = 0; f < kChunk; ++f) {
              v4f& dst = acc[(f0 + f) / C::kFragM][(f0 + f) % C::kFragM];
              dst = (s0 + u == 0) ? v[u][f] : dst + v[u][f];
            }
          }
        }
      }
      if (tid == 0)   // leave the counter zeroed for the next call
        __hip_atomic_store(p.counters + sidx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: fp32 -> bf16 (RNE), row-major store, edge masking ------------
    uint16_t* d_g = p.d + (LAYOUT == kMasked ? (int64_t)t.g * p.d_gstride : 0);
    if ((p.n & 7) == 0) {
      // Through LDS: a lane's fragment values are 16 rows x 8 bytes apart, so storing them as they
      // are makes every store instruction touch 16 rows (measured 4.0 TB/s for a bf16 output,
      // against 6.5 TB/s for row-contiguous 16-byte stores).  Each wave writes one 16-row strip of
      // its tile (WN columns) into its own padded LDS area of the first ring buffer, reads it back
      // as 16-byte chunks, and stores whole row segments of WN * 2 bytes.  N % 8 == 0 keeps every
      // chunk 16-byte aligned and either inside or outside the N edge.
      constexpr int kPitch = C::WN * 2 + 16;           // padded strip row (bytes)
      constexpr int kChunksRow = C::WN / 8;            // 16-byte chunks per strip row
      constexpr int kChunksLane = 16 * kChunksRow / 64;
      static_assert(kChunksLane * 64 == 16 * kChunksRow, "a strip is a whole number of chunks per lane");
      static_assert(C::kWaves * 16 * kPitch <= kStage, "the strips fit in one ring buffer");
      uint8_t* strip = st0 + wave * (16 * kPitch);
      __syncthreads();   // every wave is done with the ring (the last K block's operands)
#pragma unroll
      for (int j = 0; j < C::kFragM; ++j) {
#pragma unroll
        for (int i = 0; i < C::kFragN; ++i) {
          uint2 v;
          v.x = pack2_bf16_rne(acc[i][j][0], acc[i][j][1]);
          v.y = pack2_bf16_rne(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(strip + l16 * kPitch + (16 * i + 4 * g4) * 2) = v;
        }
        // the wave reads back what its own lanes wrote (LDS operations of one wave complete in order)
#pragma unroll
        for (int u = 0; u < kChunksLane; ++u) {
          const int c = lane + 64 * u;
          const int row = c / kChunksRow, cc = c % kChunksRow;
          const u32x4 val = *reinterpret_cast<const u32x4*>(strip + row * kPitch + cc * 16);
          const int mrow = m0 + wm0 + 16 * j + row;
          const int ncol = n0 + wn0 + 8 * cc;
          if ((!kTwoPass || mrow >= t.m_lo) && mrow < t.m_valid && ncol < p.n)
            *reinterpret_cast<u32x4*>(d_g + (int64_t)mrow * p.n + ncol) = val;
        }
      }
      continue;
    }
    const bool vec_ok = (p.n & 3) == 0;
    __syncthreads();   // every wave is done with the ring (the next tile's first DMAs may follow at once)
#pragma unroll
    for (int j = 0; j < C::kFragM; ++j) {
      const int mrow = m0 + wm0 + 16 * j + l16;
      if ((kTwoPass && mrow < t.m_lo) || mrow >= t.m_valid) continue;
      uint16_t* drow = d_g + (int64_t)mrow * p.n;
#pragma unroll
      for (int i = 0; i < C::kFragN; ++i) {
        const int ncol = n0 + wn0 + 16 * i + 4 * g4;
        const uint32_t lo = pack2_bf16_rne(acc[i][j][0], acc[i][j][1]);
        const uint32_t hi = pack2_bf16_rne(acc[i][j][2], acc[i][j][3]);
        const uint16_t h0 = (uint16_t)lo, h1 = (uint16_t)(lo >> 16), h2 = (uint16_t)hi, h3 = (uint16_t)(hi >> 16);
        if (vec_ok && ncol + 3 < p.n) {
          uint2 v;
          v.x = lo;
          v.y = hi;
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
  if constexpr (FQ) fused_act_quant_exit(p);
}

// ---------------------------------------------------------------------------
// Host side: tile configurations, occupancy, split-K choice and launch.
// ---------------------------------------------------------------------------
struct LaunchInfo {
  int bn, bm, threads, stages;
  const void* fn;
  int lds_bytes;   // the kernel's static LDS: its __shared__ arrays
};

template <class C, int LAYOUT, bool FQ = false>
static LaunchInfo info() {
  void (*fn)(GemmParams) = gemm_fp8_kernel<C, LAYOUT, FQ>;
  constexpr int kStage = stage_bytes<C, LAYOUT>();
  constexpr int kLds = 2 * kStage + (C::STAGES > 2 ? kStage : 16) + (C::STAGES > 3 ? kStage : 16) +
                       4 * (LAYOUT == kMasked ? 1025 + 256 + 1 : 3);
  return LaunchInfo{C::BN, C::BM, C::kThreads, C::STAGES, reinterpret_cast<const void*>(fn), kLds};
}

// Tile configurations: BN x BM workgroup tile, WN x WM wave tile, LDS stages.
//  kCfgLarge   256x128, 8 waves of 64x64, 3 stages (~147 KB LDS), the three-stage loop: the per-row
//              B scales of the weight-gradient GEMM (no room for them in the pipelined loop).
//  kCfgRows128 256x128, 8 waves of 64x64, two slots (~104 KB LDS), the pipelined main loop: the
//              256x128 choice of the dense, masked and contiguous forms (a contiguous tile of it
//              lies in one 128-row expert block).
//  kCfgWide    256x192, 8 waves of 128x48, two slots (~120 KB LDS), the pipelined main loop: 1.5x
//              the work per tile and ~1/6 less operand traffic per flop than kCfgLarge.
//  kCfgSquare  256x256, 8 waves of 128x64, two slots (~136 KB LDS), the pipelined main loop: 2x the
//              work per tile, 1/4 less operand traffic per flop than kCfgLarge and 1/6 fewer LDS
//              reads per MFMA than kCfgWide.  The planner picks whichever of the three needs the
//              least time in rounds of the persistent grid (wave quantisation decides most shapes).
//              In the contiguous form a tile spans two 128-row expert blocks and runs once per
//              expert when they differ.
//  kCfgDec*    m <= 128 rows: 64 weight rows x 64 or 128 activation rows, 4 waves, a two-stage
//              ring: HBM-bound shapes (for 65..128 rows the planner's model picks one 128-row or
//              two 64-row activation tiles).  Each barrier waits for every DMA in flight, so a
//              workgroup has one stage in flight whatever the ring's depth; two stages leave LDS
//              for four (64x64) or three (64x128) workgroups per CU, against two with the
//              four- and three-stage rings (the twelve M = 64 / 128 DeepSeek-V3 shapes 5% faster
//              at their best plans).  (Measured against 128-row weight
//              tiles on all twelve M = 64 / 128 DeepSeek-V3 shapes: the 64-row weight tile, with
//              K split to fill the grid, is faster on every one.)
enum CfgId : int { kCfgLarge = 0, kCfgRows128, kCfgWide, kCfgDec64, kCfgDec128, kCfgSquare, kNumCfg };
using CfgLarge = Cfg<256, 128, 64, 64, 3, true>;
using CfgRows128 = Cfg<256, 128, 64, 64, 2, false, true>;
using CfgWide = Cfg<256, 192, 128, 48, 2, false, true>;
using CfgSquare = Cfg<256, 256, 128, 64, 2, false, true>;
using CfgDec64 = Cfg<64, 64, 32, 32, 2>;
using CfgDec128 = Cfg<64, 128, 32, 64, 2>;

template <int LAYOUT, bool FQ = false>
static LaunchInfo cfg_info(int cfg) {
  switch (cfg) {
    // per-row B scales hold one float4 per weight fragment row: the 256x192 tile's registers
    // have no room for them, so kDenseRowB runs its large shapes on 256x128
    case kCfgWide:
      if constexpr (LAYOUT == kDenseRowB) return info<CfgLarge, LAYOUT>();
      // 192-row tiles would cut 128-row expert blocks: the contiguous form has no such tile
      else if constexpr (LAYOUT == kContiguous) return info<CfgRows128, LAYOUT>();
      else return info<CfgWide, LAYOUT, FQ>();
    case kCfgSquare:
      if constexpr (LAYOUT == kDenseRowB) return info<CfgLarge, LAYOUT>();
      else return info<CfgSquare, LAYOUT, FQ>();
    case kCfgDec64: return info<CfgDec64, LAYOUT, FQ>();
    case kCfgDec128: return info<CfgDec128, LAYOUT, FQ>();
    case kCfgRows128:
      if constexpr (LAYOUT == kDenseRowB) return info<CfgLarge, LAYOUT>();
      else return info<CfgRows128, LAYOUT, FQ>();
    default: return info<CfgLarge, LAYOUT, FQ>();
  }
}

// Workgroups per CU.  Without a device to ask (planning queries on a host without a GPU), the
// LDS bound: 160 KB per CU over the kernel's static LDS, which is what limits every tile
// configuration here (two 64-row tiles or one 256-row tile per CU).
static int occupancy(const LaunchInfo& li) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, li.fn, li.threads, 0) != hipSuccess || blocks < 1) {
    (void)hipGetLastError();
    blocks = 160 * 1024 / li.lds_bytes;
    blocks = blocks < 1 ? 1 : blocks;
  }
  return blocks;
}

struct Plan {
  int cfg;
  int bn, bm;
  int splits;        // K splits of each split tile
  int kb_per_split;
  int tail_start;    // tiles [0, tail_start) run whole; the rest are split (0: every tile)
  int tiles_m, tiles_n;
  int64_t tiles;     // output tiles
  size_t ws_bytes;   // needed workspace for this plan (0 when splits == 1)
};

static void finish_plan(Plan& pl, int64_t m, int64_t n, int64_t k, int64_t groups) {
  const LaunchInfo li = cfg_info<kDense>(pl.cfg);
  pl.bn = li.bn;
  pl.bm = li.bm;
  pl.tiles_m = (int)((m + li.bm - 1) / li.bm);
  pl.tiles_n = (int)((n + li.bn - 1) / li.bn);
  pl.tiles = (int64_t)pl.tiles_m * pl.tiles_n * groups;
  if (pl.tail_start > pl.tiles) pl.tail_start = 0;
  const int64_t split_tiles = pl.tiles - pl.tail_start;
  if (split_tiles > kMaxCounterTiles) {   // one arrival counter per split tile must fit the counter prefix
    pl.splits = 1;
    pl.tail_start = 0;
    pl.kb_per_split = (int)((k + kGroup - 1) / kGroup);
  }
  if (pl.splits == 1) pl.tail_start = 0;
  pl.ws_bytes = 0;
  if (pl.splits > 1)
    pl.ws_bytes = kCounterBytes + (size_t)(pl.tiles - pl.tail_start) * pl.splits * (size_t)li.bn * li.bm * 4;
}

// K splits of the tiles in the partial last round of the persistent grid (1: none).  That round
// holds tiles % grid tiles; split in K over the idle workgroups, it takes 1/splits of a round.  The
// split's hand-off (partials out and back, ~20 us) must cost less than the part of a round it
// saves: every piece keeps >= 24 K blocks (measured on MI355X: 4096 x 7168 x 16384 13% faster;
// with 4-8 K blocks per piece, K = 1536 and 2048, 3-6% slower).
static int last_round_splits(int64_t tiles, int64_t grid, int kb_total) {
  if (tiles <= grid || tiles % grid == 0 || 2 * (tiles % grid) > grid) return 1;
  int want = (int)(grid / (tiles % grid));
  if (want > kb_total / 24) want = kb_total / 24;
  if (want > kMaxSplits) want = kMaxSplits;
  return want > 1 ? want : 1;
}

// Large-m tile choice: estimated time = rounds of the persistent grid x time per tile round.  A
// round of 256x192 tiles takes ~1.45x and a round of 256x256 tiles ~1.85x a round of 256x128
// tiles (1.5x and 2x the MFMA work, less operand traffic per flop; measured on MI355X over
// DeepSeek-V3 shapes with M = 2048 .. 16384, all three on the pipelined main loop).  A partial
// last round with a fraction f of the CUs busy costs ~0.3 + 0.7 f of a full one (fewer workgroups
// share the L2s and HBM), a split last round 1/splits + 0.1 (the hand-off).  The larger tiles win
// where they save rounds, e.g. 4096 x 4096 (256 tiles of 256x256: one round, against two).
static double tile_rounds(int64_t tiles, int num_cus, int splits) {
  // every large-tile configuration runs one workgroup per CU
  const double full = (double)(tiles / num_cus);
  const int64_t rest = tiles % num_cus;
  if (rest == 0) return full;
  if (splits > 1) return full + 1.0 / splits + 0.1;
  return full + 0.3 + 0.7 * (double)rest / (double)num_cus;
}

static int choose_large(int64_t m, int64_t n, int64_t groups, int num_cus, int kb_total, bool split_tail) {
  auto rounds = [&](int bn, int bm) {
    const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn) * groups;
    return tile_rounds(tiles, num_cus, split_tail ? last_round_splits(tiles, num_cus, kb_total) : 1);
  };
  const double t_large = (double)rounds(CfgRows128::BN, CfgRows128::BM);
  const double t_wide = 1.45 * (double)rounds(CfgWide::BN, CfgWide::BM);
  const double t_square = 1.85 * (double)rounds(CfgSquare::BN, CfgSquare::BM);
  if (t_square < t_large && t_square < t_wide) return kCfgSquare;
  return t_wide < t_large ? kCfgWide : kCfgRows128;
}

// Contiguous-layout tile choice between 256x128 (one 128-row expert block per tile) and 256x256
// (two blocks; a tile whose blocks name different experts runs once per block), by the same
// rounds estimate.  The host does not see m_indices: the 256x256 estimate counts one extra tile
// per expert boundary in each n-tile column (experts - 1 of them, at most one per 256-row block),
// as if every boundary fell inside a tile.  Large experts (a few thousand rows each) take
// 256x256; many small ones (e.g. 64 experts of a few hundred rows) keep 256x128.
static int choose_contiguous(int64_t m, int64_t n, int64_t experts, int num_cus) {
  const int64_t tiles_n = (n + CfgSquare::BN - 1) / CfgSquare::BN;
  const int64_t blocks = (m + CfgSquare::BM - 1) / CfgSquare::BM;
  int64_t boundaries = experts - 1 < blocks ? experts - 1 : blocks;
  if (boundaries < 0) boundaries = 0;
  const double t_rows = tile_rounds(((m + CfgRows128::BM - 1) / CfgRows128::BM) * tiles_n, num_cus, 1);
  const double t_square = 1.85 * tile_rounds((blocks + boundaries) * tiles_n, num_cus, 1);
  return t_square < t_rows ? kCfgSquare : kCfgRows128;
}

// Few-row plan (m <= 128 rows per group): the tile and K split from a model of the streaming regime,
// fitted to timings of every tile and split on MI355X.  Work items spread evenly over the CUs; a
// workgroup has one stage in flight per K block (the barrier waits for every DMA in flight) and
// takes ~0.6 us per K block, and a CU runs c of them side by side; the whole grid is further bound
// by HBM (~5 TB/s for the weights, read once) and by L2-to-CU delivery (both tiles: the activation
// tile is re-read by every weight tile); a split's hand-off costs ~2 us plus the last workgroup's
// read of every partial at ~50 GB/s.  Returns the estimated time in microseconds.
static double decode_estimate(const LaunchInfo& li, int occ, int64_t m, int64_t n, int kb_total, int64_t groups,
                              int num_cus, int splits, int kbps) {
  const int64_t tiles = ((m + li.bm - 1) / li.bm) * ((n + li.bn - 1) / li.bn) * groups;
  const int64_t items = tiles * splits;
  const int64_t per_cu = (items + num_cus - 1) / num_cus;
  const double conc = (double)(per_cu < occ ? per_cu : occ);
  const double stage = (double)(li.bn + li.bm) * kGroup;
  double t = (double)per_cu * kbps * 0.6 / conc;
  const double l2 = (double)items * stage * kbps / 16.0e6;
  const double hbm = (double)tiles * li.bn * kGroup * kb_total / 5.0e6;
  if (t < l2) t = l2;
  if (t < hbm) t = hbm;
  if (splits > 1) t += 2.0 + (double)splits * li.bn * li.bm * 4 / 5.0e4;
  return t;
}

static Plan make_decode_plan(int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, bool allow_split) {
  const int kb_total = (int)((k + kGroup - 1) / kGroup);
  Plan pl{};
  pl.cfg = m <= 64 ? kCfgDec64 : kCfgDec128;
  pl.splits = 1;
  pl.tail_start = 0;
  pl.kb_per_split = kb_total;
  int max_split = kb_total / 2 < kMaxSplits ? kb_total / 2 : kMaxSplits;
  if (!allow_split || max_split < 1) max_split = 1;
  // 65..128 rows: either one 128-row activation tile or two 64-row ones, whichever the model rates
  // faster (the 64-row tile moves less per K block and wins where the split count matters, e.g.
  // 128 x 7168 x 2048 unsplit on 64-row tiles: 9.8 us against 11.9 us on 128-row tiles, split 2)
  const int cfgs[2] = {kCfgDec64, kCfgDec128};
  double best_t = 1e30;
  for (int c = 0; c < (m <= 64 ? 1 : 2); ++c) {
    const LaunchInfo li = cfg_info<kDense>(cfgs[c]);
    const int occ = occupancy(li);
    for (int want = 1; want <= max_split; ++want) {
      const int kbps = (kb_total + want - 1) / want;
      const int splits = (kb_total + kbps - 1) / kbps;
      if (splits != want) continue;   // the same split as a smaller request
      const double t = decode_estimate(li, occ, m, n, kb_total, groups, num_cus, splits, kbps);
      if (t < best_t) {
        best_t = t;
        pl.cfg = cfgs[c];
        pl.splits = splits;
        pl.kb_per_split = kbps;
      }
    }
  }
  finish_plan(pl, m, n, k, groups);
  return pl;
}

static Plan make_plan_auto(int layout, int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus,
                           bool allow_split);

// DG_PLAN: a measurement override of the planner's choice, "tile=BNxBM" and / or "splits=S"
// (comma-separated; e.g. "tile=64x128,splits=4").  The tile must be one the planner could pick for
// the form and size (64x64 or 64x128 for m <= 128; 256x128, 256x192 or 256x256 above, 256x128 or
// 256x256 for the contiguous form, 256x128 for the row-scaled one); anything else is ignored.  Splits apply where the call may split K, as a
// split of every tile.  Read at every call, like DG_DEBUG; the workspace queries see the same plan.
static void apply_plan_override(Plan& pl, int layout, int64_t m, int kb_total, bool allow_split) {
  const char* e = std::getenv("DG_PLAN");
  if (e == nullptr || e[0] == '\0') return;
  int bn = 0, bm = 0, want = 0;
  for (const char* q = e; *q;) {
    if (std::sscanf(q, "tile=%dx%d", &bn, &bm) == 2 || std::sscanf(q, "splits=%d", &want) == 1) {}
    const char* c = std::strchr(q, ',');
    if (c == nullptr) break;
    q = c + 1;
  }
  if (bn > 0) {
    static const int kDecCfgs[] = {kCfgDec64, kCfgDec128};
    static const int kLargeCfgs[] = {kCfgRows128, kCfgWide, kCfgSquare};
    const bool few = layout != kContiguous && m <= 128;
    const int* list = few ? kDecCfgs : kLargeCfgs;
    const int count = few ? 2 : (layout == kDenseRowB ? 1 : 3);
    for (int i = 0; i < count; ++i) {
      if (layout == kContiguous && list[i] == kCfgWide) continue;
      const LaunchInfo li = cfg_info<kDense>(list[i]);
      if (li.bn == bn && li.bm == bm) pl.cfg = layout == kDenseRowB && !few ? kCfgLarge : list[i];
    }
  }
  if (want > 0 && allow_split && layout != kContiguous) {
    if (want > kMaxSplits) want = kMaxSplits;
    pl.kb_per_split = (kb_total + want - 1) / want;
    pl.splits = (kb_total + pl.kb_per_split - 1) / pl.kb_per_split;
    pl.tail_start = 0;
  }
}

// Pick the tile config and the K split.  `groups`: the call's groups (masked: they multiply the
// tile count; contiguous: the experts, which the tile choice weighs; otherwise 1).
static Plan make_plan(int layout, int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, bool allow_split) {
  Plan pl = make_plan_auto(layout, m, n, k, groups, num_cus, allow_split);
  if (const char* e = std::getenv("DG_PLAN"); e != nullptr && e[0] != '\0') {
    apply_plan_override(pl, layout, m, (int)((k + kGroup - 1) / kGroup), allow_split);
    finish_plan(pl, m, n, k, layout == kMasked ? groups : 1);
  }
  return pl;
}

// The planner's own choice.
static Plan make_plan_auto(int layout, int64_t m, int64_t n, int64_t k, int64_t call_groups, int num_cus,
                           bool allow_split) {
  const int64_t groups = layout == kMasked ? call_groups : 1;   // tiles per (m-block, n-block)
  if (layout != kContiguous && m <= 128) return make_decode_plan(m, n, k, groups, num_cus, allow_split);
  Plan pl{};
  const int kb_total = (int)((k + kGroup - 1) / kGroup);
  pl.cfg = layout == kContiguous ? choose_contiguous(m, n, call_groups, num_cus)
           : layout == kDenseRowB ? kCfgLarge
                                  : choose_large(m, n, groups, num_cus, kb_total, allow_split && layout == kDense);
  // (the 256x128 tile of the dense and masked forms is the pipelined one, kCfgRows128; kCfgLarge,
  // the three-stage loop, serves the per-row B scales)
  const LaunchInfo li = cfg_info<kDense>(pl.cfg);
  pl.splits = 1;
  pl.tail_start = 0;
  // few tiles and a long K (e.g. 256 x 512 x 8192): split K so that every CU gets work
  const int64_t tiles = ((m + li.bm - 1) / li.bm) * ((n + li.bn - 1) / li.bn) * groups;
  const int max_split = kb_total / 4 > 0 ? kb_total / 4 : 1;   // keep >= 4 K blocks per split
  const int64_t grid = (int64_t)num_cus * occupancy(li);
  if (allow_split && 2 * tiles <= num_cus) {
    int want = (int)(num_cus / tiles);
    if (want > max_split) want = max_split;
    if (want > kMaxSplits) want = kMaxSplits;
    if (want > 1) pl.splits = want;
  } else if (allow_split && (layout == kDense || layout == kDenseRowB)) {
    // e.g. 616 tiles of 4096 x 7168 on 256 CUs: two full rounds, and the last round's 104 tiles
    // split in K
    const int want = last_round_splits(tiles, grid, kb_total);
    if (want > 1) {
      pl.splits = want;
      pl.tail_start = (int)(tiles - tiles % grid);
    }
  }
  pl.kb_per_split = (kb_total + pl.splits - 1) / pl.splits;
  pl.splits = (kb_total + pl.kb_per_split - 1) / pl.kb_per_split;   // no empty split
  finish_plan(pl, m, n, k, groups);
  return pl;
}

void gemm_config_name(int layout, int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, char* buf,
                      size_t len) {
  const Plan pl = make_plan(layout, m, n, k, layout == kDense || layout == kDenseRowB ? 1 : groups, num_cus,
                            layout != kContiguous);
  const LaunchInfo li = cfg_info<kDense>(pl.cfg);
  if (pl.tail_start > 0)   // whole tiles, then a split last round
    snprintf(buf, len, "%dx%d/%dwaves/split1+tail%d", li.bn, li.bm, li.threads / 64, pl.splits);
  else
    snprintf(buf, len, "%dx%d/%dwaves/split%d", li.bn, li.bm, li.threads / 64, pl.splits);
}

size_t gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus) {
  if (groups > 1) return make_plan(kMasked, m, n, k, groups, num_cus, true).ws_bytes;
  // one group: enough for the dense plan and for the per-row-B-scale plan of the same shape
  const size_t dense = make_plan(kDense, m, n, k, 1, num_cus, true).ws_bytes;
  const size_t rowb = make_plan(kDenseRowB, m, n, k, 1, num_cus, true).ws_bytes;
  return dense > rowb ? dense : rowb;
}

template <int LAYOUT, bool FQ = false>
static int launch_layout(GemmParams p, const Plan& pl, hipStream_t stream, int num_cus) {
  const LaunchInfo li = cfg_info<LAYOUT, FQ>(pl.cfg);
  const int occ = occupancy(li);
  const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n * (LAYOUT == kContiguous ? 1 : p.num_groups);
  const int64_t items = pl.tail_start + (tiles - pl.tail_start) * pl.splits;
  if (items > 0x7fffffffLL) return set_error(kUnsupported, "gemm: too many work items");
  int64_t grid = (int64_t)num_cus * occ;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(li.fn, dim3((unsigned)grid), dim3(li.threads), args, 0, stream);
  return e == hipSuccess ? kOk : set_error(kHip, "gemm launch: %s", hipGetErrorString(e));
}

static GemmParams make_params(int layout, const Plan& pl, const uint8_t* a, const float* sa, int64_t ld_sa,
                              const uint8_t* b, const float* sb, int64_t ld_sb, int64_t ld, uint16_t* d,
                              const int32_t* m_indices, const int32_t* masked_m, int64_t groups, int64_t m, int64_t n,
                              int64_t k) {
  GemmParams p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.m_indices = m_indices; p.masked_m = masked_m;
  p.ld_sa = ld_sa;
  p.ld_sb = ld_sb;
  p.ld_ab = (int)ld;
  p.m = (int)m; p.n = (int)n; p.k = (int)k;
  p.num_groups = (int)(layout == kDense || layout == kDenseRowB ? 1 : groups);
  p.kb_total = (int)((k + kGroup - 1) / kGroup);
  p.nb128 = (int)((n + kGroup - 1) / kGroup);
  p.tiles_m = pl.tiles_m; p.tiles_n = pl.tiles_n;
  p.splits = pl.splits; p.kb_per_split = pl.kb_per_split;
  p.tail_start = pl.tail_start;
  p.a_gstride = m * k;
  p.sa_gstride = (int64_t)p.kb_total * ld_sa;
  p.b_gstride = n * k;
  p.sb_gstride = (int64_t)p.nb128 * p.kb_total;
  p.d_gstride = m * n;
  p.debug = debug_enabled() ? 1 : 0;
  return p;
}

// DG_DEBUG: one line per GEMM launch with the plan the host chose.
static void log_plan(int layout, const Plan& pl, int64_t m, int64_t n, int64_t k, int64_t groups, size_t ws_bytes) {
  static const char* const kNames[] = {"normal", "contiguous", "masked", "row-scaled"};
  const LaunchInfo li = cfg_info<kDense>(pl.cfg);
  std::fprintf(stderr,
               "[dg] gemm %s m=%lld n=%lld k=%lld groups=%lld: %dx%d/%dwaves splits=%d%s kb_per_split=%d "
               "tiles=%lld workspace=%zu/%zu bytes\n",
               kNames[layout & 3], (long long)m, (long long)n, (long long)k, (long long)groups, li.bn, li.bm,
               li.threads / 64, pl.splits, pl.tail_start > 0 ? " (last round only)" : "", pl.kb_per_split,
               (long long)pl.tiles, pl.ws_bytes, ws_bytes);
}

int launch_gemm(int layout, const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                const float* sb, int64_t ld_sb, int64_t ld_ab, uint16_t* d, const int32_t* m_indices,
                const int32_t* masked_m, int64_t groups, int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                hipStream_t stream, int num_cus) {
  const int64_t ld = ld_ab > 0 ? ld_ab : k;   // operand row stride (bytes)
  if (n * ld > 0x7fffffffLL || m * ld > 0x7fffffffLL)
    return set_error(kUnsupported, "gemm: one group's operand must be < 2^31 bytes (m=%lld n=%lld k=%lld ld=%lld)",
                     (long long)m, (long long)n, (long long)k, (long long)ld);
  if (layout == kMasked && groups > 1024) return set_error(kUnsupported, "masked gemm: at most 1024 groups");
  const int64_t plan_groups = layout == kDense || layout == kDenseRowB ? 1 : groups;
  const bool can_split = (layout != kContiguous) && ws != nullptr;
  Plan pl = make_plan(layout, m, n, k, plan_groups, num_cus, can_split);
  if (pl.splits > 1 && ws_bytes < pl.ws_bytes) pl = make_plan(layout, m, n, k, plan_groups, num_cus, false);

  GemmParams p = make_params(layout, pl, a, sa, ld_sa, b, sb, ld_sb, ld, d, m_indices, masked_m, groups, m, n, k);
  if (pl.splits > 1) {
    p.counters = static_cast<unsigned*>(ws);
    p.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes);
  }
  if (p.debug) log_plan(layout, pl, m, n, k, groups, ws_bytes);
  switch (layout) {
    case kContiguous: return launch_layout<kContiguous>(p, pl, stream, num_cus);
    case kMasked: return launch_layout<kMasked>(p, pl, stream, num_cus);
    case kDenseRowB: return launch_layout<kDenseRowB>(p, pl, stream, num_cus);
    default: return launch_layout<kDense>(p, pl, stream, num_cus);
  }
}

// ---- normal GEMM with the activation quantization inside the launch --------------------------
// Workspace: the counter prefix (split-K arrival counters, the quantization step's counters in
// its last words), then the E4M3 activations (m x k), their scales (KB x ld_sa, ld_sa = m
// rounded up to 4), then the split-K partials of the same plan as the normal GEMM's.
static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct FqLayout {
  Plan pl;
  int64_t ld_sa;
  size_t q_off, s_off, partial_off, bytes;
};

static FqLayout fq_layout(int64_t m, int64_t n, int64_t k, int num_cus) {
  FqLayout f;
  f.pl = make_plan(kDense, m, n, k, 1, num_cus, true);
  f.ld_sa = (m + 3) / 4 * 4;
  const int64_t kb_total = (k + kGroup - 1) / kGroup;
  f.q_off = kCounterBytes;
  f.s_off = f.q_off + align256((size_t)(m * k));
  f.partial_off = f.s_off + align256((size_t)(kb_total * f.ld_sa * 4));
  f.bytes = f.partial_off + (f.pl.splits > 1 ? f.pl.ws_bytes - kCounterBytes : 0);
  return f;
}

size_t gemm_fq_workspace_size(int64_t m, int64_t n, int64_t k, int num_cus) { return fq_layout(m, n, k, num_cus).bytes; }

int launch_gemm_fq(const void* x, bool x_bf16, const uint8_t* b, const float* sb, uint16_t* d, int64_t m, int64_t n,
                   int64_t k, void* ws, size_t ws_bytes, hipStream_t stream, int num_cus) {
  if (n * k > 0x7fffffffLL || m * k > 0x7fffffffLL)
    return set_error(kUnsupported, "gemm: one operand must be < 2^31 bytes (m=%lld n=%lld k=%lld)", (long long)m,
                     (long long)n, (long long)k);
  const FqLayout f = fq_layout(m, n, k, num_cus);
  if (ws == nullptr || ws_bytes < f.bytes)
    return set_error(kWorkspace, "gemm with activation quantization: workspace of %zu bytes, %zu needed", ws_bytes,
                     f.bytes);
  uint8_t* w = static_cast<uint8_t*>(ws);
  GemmParams p = make_params(kDense, f.pl, w + f.q_off, reinterpret_cast<const float*>(w + f.s_off), f.ld_sa, b, sb, 0,
                             k, d, nullptr, nullptr, 1, m, n, k);
  p.counters = static_cast<unsigned*>(ws);
  if (f.pl.splits > 1) p.ws = reinterpret_cast<float*>(w + f.partial_off);
  p.fq_x = x;
  p.fq_sync = static_cast<unsigned*>(ws) + kFqSyncWord;
  p.fq_bf16 = x_bf16 ? 1 : 0;
  // DG_FQ_MAX_POLLS lowers the wait's bound (a test of the give-up path forces it from the host)
  p.fq_max_polls = kFqMaxPolls;
  if (const char* e = std::getenv("DG_FQ_MAX_POLLS")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v < kFqMaxPolls) p.fq_max_polls = (int)v;
  }
  if (p.debug) log_plan(kDense, f.pl, m, n, k, 1, ws_bytes);
  return launch_layout<kDense, true>(p, f.pl, stream, num_cus);
}

// bf16 zero fill of count elements (count % 8 == 0, 16-byte aligned): the weight gradient of an
// expert that received no tokens.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* d, int64_t chunks) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256)
    reinterpret_cast<u32x4*>(d)[i] = u32x4{0u, 0u, 0u, 0u};
}

int launch_fill_zero_bf16(uint16_t* d, int64_t count, hipStream_t stream) {
  const int64_t chunks = count / 8;
  if (chunks <= 0) return kOk;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, d, chunks);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : set_error(kHip, "zero fill launch: %s", hipGetErrorString(e));
}

// ---- normal GEMM that allocates nothing: split-K scratch in the library's own device array ------
// For callers that cannot allocate (graph capture, tight serving loops): the split-K counters
// and partials live in `scratch`, one copy per device, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not a device address):
// the device address comes from hipGetSymbolAddress once per device, with that device current.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchDevices];

// The current device's scratch address; on the first call for a device also clears the counter
// prefix (with a fill kernel on `stream`: no memset node if the caller is capturing a graph).
static int scratch_for_device(void** out, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(kHip, "no-alloc gemm: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices) return set_error(kUnsupported, "no-alloc gemm: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return set_error(kHip, "no-alloc gemm: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int r = launch_fill_zero_bf16(static_cast<uint16_t*>(ptr), (int64_t)(kCounterBytes / 2), stream);
    if (r != kOk) return r;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return kOk;
}

int launch_gemm_no_alloc(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b, const float* sb,
                         uint16_t* d, int64_t m, int64_t n, int64_t k, hipStream_t stream, int num_cus) {
  const Plan pl = make_plan(kDense, m, n, k, 1, num_cus, true);
  if (pl.ws_bytes > kNoAllocScratchBytes)
    return set_error(kWorkspace, "no-alloc gemm: the plan %dx%d split %d needs %zu bytes of scratch, the library "
                     "holds %zu", pl.bn, pl.bm, pl.splits, pl.ws_bytes, (size_t)kNoAllocScratchBytes);
  void* ws = nullptr;
  const int r = scratch_for_device(&ws, stream);
  if (r != kOk) return r;
  return launch_gemm(kDense, a, sa, ld_sa, b, sb, 0, 0, d, nullptr, nullptr, 1, m, n, k, ws, kNoAllocScratchBytes,
                     stream, num_cus);
}

// The device diagnostics words of the current device, after every queued kernel on it has
// finished; optionally cleared.
int read_diag(unsigned out[4], bool clear) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_diag), 4 * sizeof(unsigned), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const unsigned zero[4] = {0u, 0u, 0u, 0u};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_diag), zero, sizeof(zero), 0, hipMemcpyHostToDevice);
  }
  return e == hipSuccess ? kOk : set_error(kHip, "reading the device diagnostics: %s", hipGetErrorString(e));
}

}  // namespace dg
