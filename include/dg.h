/*
 * dg.h - C ABI of the MI355X (gfx950) FP8 block-scaled GEMM library (libdg.so).
 *
 * The method: FP8 (E4M3) matrix multiplication with DeepSeek-V3 style
 * fine-grained scaling and two-level (promoted) FP32 accumulation, in three
 * forms - a normal GEMM, a contiguous-grouped MoE GEMM and a masked-grouped
 * MoE GEMM.  Sources (DeepGEMM news/blog pages):
 *   - 机器之心 DeepGEMM report, opening section: fine-grained scaling as in
 *     DeepSeek-V3; normal and MoE grouped GEMMs; two-level accumulation on
 *     the general-purpose cores because FP8 tensor-core accumulation is
 *     imprecise.  Same report, "quick start": the three GEMM forms.
 *   - ai.abqq.net summary, section 3 "core functions and features": E4M3
 *     data (4-bit exponent, 3-bit mantissa); contiguous and masked layouts.
 *   - 3loumao explainer, section 03 "how DeepSeek innovated": the contiguous
 *     layout joins every expert's rows into one block; the masked layout marks
 *     which rows to compute and skips the rest at run time.
 *   - CSDN "DeepGEMM: concise, efficient ..." article, "utilities": maximum
 *     number of compute units used, the contiguous-layout alignment, and the
 *     aligned column-major activation-scale tensor.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after it returns.  All pointers must be 16-byte
 *     aligned.
 *   - E4M3 means the OCP E4M3FN encoding (largest finite value 448).  FP8
 *     operands are passed as uint8_t bytes; bf16 outputs as uint16_t bits.
 *   - K (the reduction length) must be a positive multiple of 16 (16-byte rows).
 *     KB = ceil(K / 128) scale groups cover it; when K % 128 != 0 the last group
 *     holds the K % 128 elements present, its scale is their amax / 448, and the
 *     GEMM treats the absent positions as zeros (the pages ask for irregular
 *     shapes - ai.abqq.net summary, section 1 - without fixing this case).
 *   - Activation scales `sa` are stored K-group-major ("MN-major"):
 *     sa[kb * ld_sa + row] is the scale of row `row`, columns
 *     [128*kb, min(128*kb+128, K)).  ld_sa >= rows and ld_sa % 4 == 0
 *     (dg_get_scale_ld gives the smallest such value).
 *   - Weight scales `sb` are stored block-row-major: sb[nb * KB + kb] is the
 *     scale of rows [128*nb, 128*nb+128) (a partial last block is allowed),
 *     columns [128*kb, min(128*kb+128, K)).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) without any host synchronisation: device-resident counts
 *     (m_indices, masked_m) are read by the kernels only.
 *   - Return value: DG_OK, or a negative dg_status.  Argument errors are
 *     detected synchronously, before anything is launched.  A failed launch
 *     returns DG_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  A zero-sized problem (m == 0, num_groups == 0) is a
 *     successful no-op.  No C++ exception crosses this interface.
 *   - Entry points are reentrant; dg_set_num_cus is process-wide.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* dg_stream_t; /* hipStream_t */

enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1, /* a pointer, size, stride or alignment is invalid */
  DG_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
  DG_ERR_WORKSPACE = -3,   /* workspace too small where one is required (the GEMMs that take an
                              optional workspace skip split-K instead) */
  DG_ERR_HIP = -4          /* a HIP runtime call failed */
};

/* Human-readable name of a status code (static string). */
const char* dg_status_string(int status);

/* Detail of the last non-OK return on the calling thread (thread-local, static storage). */
const char* dg_last_error_message(void);

/*
 * Per-token-group activation quantizer (1 x 128), for num_groups stacked (m, k)
 * matrices (num_groups = 1 for a plain activation matrix; the masked MoE layout
 * uses one group per expert).
 * Fine-grained scaling as in DeepSeek-V3 (机器之心 report, opening section),
 * E4M3 data (ai.abqq.net summary, section 3).  For each row r and K group kb:
 *   amax = max |x[r, 128kb .. 128kb+127]|
 *   s    = amax / 448 (IEEE fp32 division; s = 1 when amax == 0)
 *   q    = E4M3 round-to-nearest-even, saturating, of fl32(x / s) (IEEE division)
 * x  : fp32 (num_groups, m, k) row-major, read only.
 * q  : E4M3 bytes (num_groups, m, k) row-major, written.
 * sa : fp32 scales, MN-major per group: written at sa[(g * KB + kb) * ld_sa + r]
 *      for r < m; entries r >= m are untouched.
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers, m < 0, num_groups < 0,
 * k % 16 != 0, ld_sa < m or ld_sa % 4 != 0.  Output is bit-exact (the result is unique).
 */
int dg_quantize_per_token_group(const float* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* q,
                                float* sa, int64_t ld_sa, dg_stream_t stream);

/*
 * The same per-token-group quantizer for bf16 activations (x : bf16 bits, (num_groups,
 * m, k) row-major).  A bf16 value widens to fp32 exactly, so the bytes and scales are those
 * dg_quantize_per_token_group gives for the widened values.  Activations of this path are
 * commonly bf16 (the GEMM's own output format: 机器之心 report, "quick start"); reading them
 * directly halves the quantizer's input traffic (2 B instead of 4 B per element).
 * Same layouts, errors and guarantees as dg_quantize_per_token_group.
 */
int dg_quantize_per_token_group_bf16(const uint16_t* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* q,
                                     float* sa, int64_t ld_sa, dg_stream_t stream);

/*
 * Per-block weight quantizer (128 x 128), for num_groups stacked (n, k) matrices.
 * Same rule as above with the amax over each 128 x 128 block (a partial last
 * block at the N edge takes its amax over the rows present).
 * w  : fp32 (num_groups, n, k) row-major, read only.
 * q  : E4M3 bytes (num_groups, n, k), written.
 * sb : fp32 (num_groups, ceil(n/128), KB), written.
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers, n < 0, num_groups < 0,
 * k % 16 != 0.  Output is bit-exact.
 */
int dg_quantize_per_block(const float* w, int64_t num_groups, int64_t n, int64_t k, uint8_t* q,
                          float* sb, dg_stream_t stream);

/*
 * Normal FP8 GEMM  D = A * B^T  with two-level accumulation (机器之心 report,
 * opening section and "quick start"; 3loumao explainer, section 03).
 * After every 128-deep K block the MFMA partial P is promoted into FP32
 * accumulators:  acc += P * fl32(sa[row, kb] * sb[n/128, kb]);  D = bf16_rne(acc).
 * a  : E4M3 (m, k) row-major.        sa : fp32, MN-major with stride ld_sa (see above).
 * b  : E4M3 (n, k) row-major.        sb : fp32 (ceil(n/128), KB).
 * d  : bf16 (m, n) row-major, written.
 * workspace : optional device scratch for K splits: every tile of a small-m shape, or the
 *   tiles of a large shape's partial last round of the persistent grid (long K only).
 *   Its first 64 KiB hold per-tile arrival counters: they must be zero before the first
 *   use (e.g. a zero-filled allocation), and every call leaves them zero; the
 *   rest holds fp32 partials.  Calls sharing one workspace must be ordered on
 *   one stream (concurrent calls race).  NULL or too small (see
 *   dg_gemm_workspace_size) => no split: still correct, slower (the rounding of
 *   the split tiles' outputs may differ in the last bit: partials are summed in
 *   fixed split order).
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers, negative sizes,
 * k % 16 != 0, ld_sa < m or ld_sa % 4 != 0.  Deterministic: the same inputs
 * give bit-identical outputs.
 */
int dg_gemm_fp8_nt(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                   const float* sb, uint16_t* d, int64_t m, int64_t n, int64_t k, void* workspace,
                   size_t workspace_bytes, dg_stream_t stream);

/*
 * Normal FP8 GEMM on unquantized activations: D = A * B^T where A, sa are the per-token-group
 * quantization of x (the rule of dg_quantize_per_token_group: 机器之心 report, opening section;
 * ai.abqq.net summary, section 3), computed inside the GEMM launch instead of by a launch of
 * its own.  The pages leave where the quantization runs open; the result is defined by the
 * two steps it replaces.
 * x  : fp32 (dg_gemm_fp8_nt_act_quant) or bf16 bits (..._bf16), (m, k) row-major, read only.
 * b, sb, d, m, n, k : as dg_gemm_fp8_nt.
 * workspace : required, at least dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k) bytes.  It
 *   holds the counters (its first 64 KiB: zero before the first use, e.g. a zero-filled
 *   allocation, and left zero by every call), the quantized activations and their scales, and
 *   the split-K partials.  Calls sharing one workspace must be ordered on one stream
 *   (concurrent calls race); x and d must not overlap it.  The workgroups of one call wait
 *   for each other once (after the quantization); that wait is bounded, so counters that
 *   are not zero on entry (a misuse of the workspace) give a wrong result, not a hang.
 * Performance: on MI355X this form is slower than the two launches it replaces (the wait
 *   across all workgroups costs more than a kernel boundary); it serves callers that need
 *   a single launch.
 * Result: bit-identical to dg_quantize_per_token_group(_bf16) of x (ld_sa = dg_get_scale_ld(m))
 *   followed by dg_gemm_fp8_nt with a workspace of at least dg_gemm_workspace_size(m, n, k, 1)
 *   bytes (the same tile plan and K split).
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers (16 bytes), negative sizes,
 * k % 16 != 0; DG_ERR_WORKSPACE when the workspace is smaller than required;
 * DG_ERR_UNSUPPORTED when m * k or n * k reaches 2^31.  Deterministic.
 */
int dg_gemm_fp8_nt_act_quant(const float* x, const uint8_t* b, const float* sb, uint16_t* d, int64_t m, int64_t n,
                             int64_t k, void* workspace, size_t workspace_bytes, dg_stream_t stream);
int dg_gemm_fp8_nt_act_quant_bf16(const uint16_t* x, const uint8_t* b, const float* sb, uint16_t* d, int64_t m,
                                  int64_t n, int64_t k, void* workspace, size_t workspace_bytes, dg_stream_t stream);

/*
 * The normal GEMM for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same operation, arguments, layouts and
 * result as dg_gemm_fp8_nt (the same tile plan and K split as with a large enough workspace, so
 * the output is bit-identical to it), but the split-K counters and partials live in scratch
 * memory the library holds itself: DG_NO_ALLOC_SCRATCH_BYTES of device memory per GPU it runs
 * on, from the first call on that GPU until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).
 * Every call on one GPU shares that GPU's scratch: calls must be ordered on one stream (calls
 * that overlap on one GPU race).  The counters are cleared on the first call on a GPU (a fill
 * kernel on `stream`) and every call leaves them zero.
 * Errors: as dg_gemm_fp8_nt, plus DG_ERR_WORKSPACE (before any launch) when the plan of the
 * shape needs more scratch than DG_NO_ALLOC_SCRATCH_BYTES (no DeepSeek-V3 shape does on 256 CUs);
 * DG_ERR_HIP if the scratch address cannot be obtained.
 */
#define DG_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dg_gemm_fp8_nt_no_alloc(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b, const float* sb,
                            uint16_t* d, int64_t m, int64_t n, int64_t k, dg_stream_t stream);

/* Workspace bytes dg_gemm_fp8_nt_act_quant(_bf16) needs for a shape (0 for invalid sizes). */
size_t dg_gemm_fp8_nt_act_quant_workspace_size(int64_t m, int64_t n, int64_t k);

/*
 * Contiguous-grouped MoE GEMM (3loumao explainer, section 03: every expert's
 * rows joined into one block; ai.abqq.net summary, section 3).
 * Rows of A are grouped in blocks of dg_get_m_alignment_for_contiguous_layout()
 * (128) rows; every row of one block carries the same expert index
 * m_indices[row] in [0, num_groups).  Row r of D is A[r] * B[m_indices[r]]^T.
 * A block whose index is outside [0, num_groups) (e.g. -1 padding) is skipped
 * and its D rows are left unwritten.
 * a  : E4M3 (m_total, k);  sa : fp32 MN-major, stride ld_sa >= m_total.
 * b  : E4M3 (num_groups, n, k);  sb : fp32 (num_groups, ceil(n/128), KB).
 * m_indices : int32 (m_total,), DEVICE memory, read by the kernel only.
 * d  : bf16 (m_total, n).
 * Errors: as dg_gemm_fp8_nt, plus m_total % 128 != 0.
 */
int dg_gemm_fp8_grouped_contiguous(const uint8_t* a, const float* sa, int64_t ld_sa,
                                   const uint8_t* b, const float* sb, const int32_t* m_indices,
                                   int64_t num_groups, uint16_t* d, int64_t m_total, int64_t n,
                                   int64_t k, dg_stream_t stream);

/*
 * Masked-grouped MoE GEMM (3loumao explainer, section 03: mark which rows to
 * compute and skip invalid work such as empty decode tokens at run time).
 * For expert g only rows r < min(max(masked_m[g], 0), m_max) are computed and
 * written; rows at or past that count are never written.
 * a  : E4M3 (num_groups, m_max, k);  sa : fp32 (num_groups, KB, ld_sa), ld_sa >= m_max.
 * b  : E4M3 (num_groups, n, k);      sb : fp32 (num_groups, ceil(n/128), KB).
 * d  : bf16 (num_groups, m_max, n).
 * masked_m : int32 (num_groups,), DEVICE memory, read by the kernel only.
 * workspace : as dg_gemm_fp8_nt (used for split-K when m_max is small).
 * Errors: as dg_gemm_fp8_nt.
 */
int dg_gemm_fp8_grouped_masked(const uint8_t* a, const float* sa, int64_t ld_sa,
                               const uint8_t* b, const float* sb, uint16_t* d,
                               const int32_t* masked_m, int64_t num_groups, int64_t m_max,
                               int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                               dg_stream_t stream);

/*
 * Training-side layouts: the backward GEMMs of a linear layer Y = X * W^T.  The pages say the
 * library serves DeepSeek-V3/R1 training as well as inference (机器之心 report, opening section;
 * 3loumao explainer, section 03; ai.abqq.net summary, section 3 "application scenarios") but
 * describe no backward pass.  These entry points keep the fine-grained recipe with the scale
 * groups along each backward GEMM's own contraction dimension:
 *   dgrad  dX = dY * W       = dg_gemm_fp8_nt(dY per-token groups, W^T blocks)
 *          (W^T's 128 x 128 block quantization is W's transposed: dg_transpose_blocks);
 *   wgrad  dW = dY^T * X     = dg_gemm_fp8_nt_row_scaled(dY^T, X^T), both operands in
 *          groups of 128 tokens per column (dg_quantize_per_channel_group);
 *          per expert over the contiguous MoE layout: dg_gemm_fp8_k_grouped_row_scaled.
 */

/*
 * Per-channel-group quantizer (128 x 1: 128 consecutive tokens of one column), transposed
 * output, for num_groups stacked (m, k) matrices.  Same rule as the per-token quantizer with
 * the amax over x[128mb .. 128mb+127, col] (a last group of m % 128 tokens takes its amax over
 * the tokens present).
 * x  : fp32 (num_groups, m, k) row-major, read only.
 * qt : E4M3 bytes (num_groups, k, m) row-major, written: qt[g, col, tok] encodes x[g, tok, col].
 * st : fp32 scales in the activation-scale layout of the transposed matrix: written at
 *      st[(g * MB + mb) * ld_st + col] for col < k, MB = ceil(m / 128); other entries untouched.
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers, negative sizes, m % 16 != 0,
 * k % 4 != 0, ld_st < k or ld_st % 4 != 0.  Output is bit-exact.
 */
int dg_quantize_per_channel_group(const float* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* qt, float* st,
                                  int64_t ld_st, dg_stream_t stream);

/* The per-channel-group quantizer for bf16 input (exact widening, as
 * dg_quantize_per_token_group_bf16).  Same layouts, errors and guarantees. */
int dg_quantize_per_channel_group_bf16(const uint16_t* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* qt,
                                       float* st, int64_t ld_st, dg_stream_t stream);

/*
 * Transpose of block-quantized matrices: codes q (num_groups, rows, cols) -> qt (num_groups,
 * cols, rows), block scales s (num_groups, ceil(rows/128), ceil(cols/128)) -> st (num_groups,
 * ceil(cols/128), ceil(rows/128)).  A 128 x 128 block is square, so (qt, st) is exactly what
 * dg_quantize_per_block gives for the transposed matrix: the weight operand of the dgrad GEMM.
 * Errors: DG_ERR_INVALID_ARG for null/misaligned code pointers, negative sizes, rows or cols not
 * a multiple of 16, q == qt (no in-place transpose).  Bit-exact.
 */
int dg_transpose_blocks(const uint8_t* q, const float* s, int64_t num_groups, int64_t rows, int64_t cols, uint8_t* qt,
                        float* st, dg_stream_t stream);

/*
 * FP8 GEMM D = A * B^T where both operands carry per-row group scales (the weight-gradient
 * GEMM): after every 128-deep K block, acc += P * fl32(sa[row, kb] * sb[col, kb]);
 * D = bf16_rne(acc).
 * a  : E4M3 (m, k) row-major.   sa : fp32, sa[kb * ld_sa + row], ld_sa >= m.
 * b  : E4M3 (n, k) row-major.   sb : fp32, sb[kb * ld_sb + col], ld_sb >= n.
 * d  : bf16 (m, n) row-major, written.
 * workspace : as dg_gemm_fp8_nt (dg_gemm_workspace_size covers this form too).
 * Errors: as dg_gemm_fp8_nt, plus ld_sb < n or ld_sb % 4 != 0.  Deterministic.
 */
int dg_gemm_fp8_nt_row_scaled(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                              const float* sb, int64_t ld_sb, uint16_t* d, int64_t m, int64_t n, int64_t k,
                              void* workspace, size_t workspace_bytes, dg_stream_t stream);

/*
 * MoE weight gradients over the contiguous layout (the layout the pages name for MoE training
 * forward: 3loumao explainer, section 03): expert g's tokens are columns [start_g, start_g + T_g)
 * of both operands, start_g = T_0 + ... + T_{g-1}, and D[g] = A_g * B_g^T with per-row group
 * scales on both (dW_g = dY_g^T X_g from dg_quantize_per_channel_group of the whole dY and X:
 * every T_g is a multiple of 128, so no 128-token group straddles two experts).
 * a  : E4M3 (m, tokens_total) row-major;  sa : fp32 sa[tb * ld_sa + row], tb = token group.
 * b  : E4M3 (n, tokens_total) row-major;  sb : fp32 sb[tb * ld_sb + col].
 * d  : bf16 (num_groups, m, n), written; an expert with T_g = 0 gets zeros.
 * group_tokens : int64 (num_groups,), HOST memory, each a multiple of 128, summing to tokens_total.
 * workspace : as dg_gemm_fp8_nt, shared by the experts' GEMMs (run in order on `stream`).
 * Errors: DG_ERR_INVALID_ARG for null/misaligned pointers, negative sizes, a count that is not a
 * multiple of 128, counts not summing to tokens_total, ld_sa < m, ld_sb < n, m * n % 8 != 0.
 */
int dg_gemm_fp8_k_grouped_row_scaled(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                                     const float* sb, int64_t ld_sb, uint16_t* d, const int64_t* group_tokens,
                                     int64_t num_groups, int64_t m, int64_t n, int64_t tokens_total, void* workspace,
                                     size_t workspace_bytes, dg_stream_t stream);

/*
 * Utilities (CSDN article, "utilities": cap on the compute units used,
 * contiguous-layout alignment, aligned column-major scale tensor).
 */

/* Current cap on the compute units the persistent GEMM grid uses (default: all
 * CUs of the current device; queries the device on first use, returns < 0 on a
 * HIP error). */
int dg_get_num_cus(void);

/* Set that cap (1 <= n); n larger than the device's CU count is clamped.  Process-wide.
 * With no device visible, the cap stands in for the device's CU count in the planning
 * queries below (dg_gemm_workspace_size, dg_gemm_config_name, ...), so that plans can be
 * inspected on a host without a GPU.  Returns DG_OK or DG_ERR_INVALID_ARG. */
int dg_set_num_cus(int n);

/* Row alignment required of each group in the contiguous layout: 128. */
int dg_get_m_alignment_for_contiguous_layout(void);

/* Smallest valid ld_sa for `rows` rows: rows rounded up to a multiple of 4 (16 bytes). */
int64_t dg_get_scale_ld(int64_t rows);

/* Workspace bytes that let dg_gemm_fp8_nt / dg_gemm_fp8_nt_row_scaled /
 * dg_gemm_fp8_grouped_masked use split-K for the given shape (m = rows per group; num_groups = 1 for the
 * normal GEMM).  0 means split-K is never used for that shape. */
size_t dg_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t num_groups);

/* Name of the tile configuration and K split the GEMM picks for a shape, as
 * "BNxBM/Wwaves/splitS", or "BNxBM/Wwaves/split1+tailS" when only the last round's
 * tiles are split in S (static thread-local string), assuming a large enough
 * workspace.  layout: 0 normal, 1 contiguous-grouped, 2 masked-grouped (m = rows
 * per group), 3 row-scaled normal.  For profiling and reports; returns "" for invalid arguments. */
const char* dg_gemm_config_name(int layout, int64_t m, int64_t n, int64_t k, int64_t num_groups);

/*
 * Debug facility (the analogue of the pages' debug switch among the environment variables,
 * CSDN article, "environment variables").  With DG_DEBUG set to a value other than "" or "0"
 * in the environment (read at every call):
 *   - every GEMM launch logs its plan (tile configuration, K split, tiles, workspace) on stderr;
 *   - the contiguous-grouped GEMM checks m_indices on the device: each 128-row block must carry
 *     one expert index, in [0, num_groups) or -1 for the whole block.  A violation sets
 *     DG_DIAG_MIXED_BLOCK or DG_DIAG_EXPERT_RANGE; the GEMM itself proceeds as without the check
 *     (no trap, no fault: the rows of a mixed block are computed with the block's first expert).
 * Independently of DG_DEBUG, the in-launch activation quantization sets DG_DIAG_FQ_TIMEOUT when
 * its bounded wait gives up (a workspace whose counters were not zero): that call's output is
 * not valid.
 * The flags are sticky, one set per device, shared by every call on it.
 *
 * Planner override for measurement (DG_PLAN, read at every call): "tile=BNxBM" and / or
 * "splits=S", comma-separated (e.g. "tile=64x128,splits=4").  The tile replaces the planner's
 * choice when it is one the planner could pick for the form and size (64x64 or 64x128 for
 * m <= 128 rows; 256x128, 256x192 or 256x256 above; 256x128 or 256x256 for the contiguous form,
 * 256x128 for the row-scaled one); splits
 * (1..16) split every tile's K range where the call may split K.  Anything else is ignored.
 * dg_gemm_config_name and dg_gemm_workspace_size report the overridden plan; results stay within
 * the GEMM tolerance (a different K split changes the fp32 summation order).  For measuring the
 * alternatives the planner weighs, not for production use.
 */
enum dg_diag_flag {
  DG_DIAG_MIXED_BLOCK = 1,
  DG_DIAG_EXPERT_RANGE = 2,
  DG_DIAG_FQ_TIMEOUT = 4
};

/* Reads the diagnostics flags of the current device into *flags, and into *block (if not NULL)
 * the index of the first 128-row block a contiguous-layout check found wrong (-1 if none).
 * SYNCHRONISES the device first (a debugging call, not for the hot path).  clear != 0 resets
 * the flags afterwards.  Returns DG_OK, DG_ERR_INVALID_ARG (flags NULL) or DG_ERR_HIP. */
int dg_get_debug_status(uint32_t* flags, int64_t* block, int clear);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
