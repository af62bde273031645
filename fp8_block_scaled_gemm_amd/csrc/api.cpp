// C ABI of libdg.so: argument validation, device queries and dispatch to the
// gfx950 kernels.  Declarations and the contract of every entry point are in
// include/dg.h.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/dg.h"
#include "common.hpp"

namespace dg {

int launch_quant_token_group(const float* x, int64_t groups, int64_t m, int64_t k, uint8_t* q, float* sa,
                             int64_t ld_sa, hipStream_t stream);
int launch_quant_token_group_bf16(const uint16_t* x, int64_t groups, int64_t m, int64_t k, uint8_t* q, float* sa,
                                  int64_t ld_sa, hipStream_t stream);
int launch_quant_block(const float* w, int64_t groups, int64_t n, int64_t k, uint8_t* q, float* sb,
                       hipStream_t stream);
int launch_quant_channel_group(const float* x, int64_t mats, int64_t m, int64_t k, uint8_t* qt, float* st,
                               int64_t ld_st, hipStream_t stream);
int launch_quant_channel_group_bf16(const uint16_t* x, int64_t mats, int64_t m, int64_t k, uint8_t* qt, float* st,
                                    int64_t ld_st, hipStream_t stream);
int launch_transpose_blocks(const uint8_t* q, const float* s, int64_t groups, int64_t r, int64_t c, uint8_t* qt,
                            float* st, hipStream_t stream);
int launch_fill_zero_bf16(uint16_t* d, int64_t count, hipStream_t stream);
int launch_gemm(int layout, const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                const float* sb, int64_t ld_sb, int64_t ld_ab, uint16_t* d, const int32_t* m_indices,
                const int32_t* masked_m,
                int64_t groups, int64_t m, int64_t n, int64_t k, void* ws, size_t ws_bytes,
                hipStream_t stream, int num_cus);
size_t gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus);
int launch_gemm_fq(const void* x, bool x_bf16, const uint8_t* b, const float* sb, uint16_t* d, int64_t m, int64_t n,
                   int64_t k, void* ws, size_t ws_bytes, hipStream_t stream, int num_cus);
size_t gemm_fq_workspace_size(int64_t m, int64_t n, int64_t k, int num_cus);
void gemm_config_name(int layout, int64_t m, int64_t n, int64_t k, int64_t groups, int num_cus, char* buf,
                      size_t len);
int read_diag(unsigned out[4], bool clear);
int launch_gemm_no_alloc(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b, const float* sb,
                         uint16_t* d, int64_t m, int64_t n, int64_t k, hipStream_t stream, int num_cus);

static thread_local char g_msg[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  if (debug_enabled()) std::fprintf(stderr, "[dg] %s\n", g_msg);
  return status;
}

bool debug_enabled() {
  const char* v = std::getenv("DG_DEBUG");
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

// ---- compute-unit cap (process-wide) ----------------------------------------
static std::atomic<int> g_cu_cap{0};      // 0 = not set: use every CU of the device
constexpr int kMaxDevices = 64;
static std::atomic<int> g_dev_cus[kMaxDevices];

// CUs of the current device (cached per device), or a negative status.
static int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return set_error(kHip, "hipGetDevice failed");
  if (dev < kMaxDevices) {
    const int cached = g_dev_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  const hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) return set_error(kHip, "CU count query failed: %s", hipGetErrorString(e));
  if (dev < kMaxDevices) g_dev_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The CU count the planner uses: the device's, capped by dg_set_num_cus.  With no device
// visible, a set cap stands in for it, so that the planning queries (configuration names,
// workspace sizes) also answer on a host without a GPU; launches still fail there.
static int effective_cus() {
  const int cap = g_cu_cap.load(std::memory_order_relaxed);
  const int cus = device_cus();
  if (cus < 0) return cap > 0 ? cap : cus;
  return (cap > 0 && cap < cus) ? cap : cus;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace dg

using namespace dg;

#define DG_REQUIRE(cond, ...)                           \
  do {                                                  \
    if (!(cond)) return set_error(kInvalidArg, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
    case DG_ERR_WORKSPACE: return "DG_ERR_WORKSPACE";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    default: return "DG_ERR_UNKNOWN";
  }
}

const char* dg_last_error_message(void) { return g_msg; }

int dg_get_num_cus(void) { return effective_cus(); }

int dg_set_num_cus(int n) {
  DG_REQUIRE(n >= 1, "dg_set_num_cus: n must be >= 1 (got %d)", n);
  g_cu_cap.store(n, std::memory_order_relaxed);
  return DG_OK;
}

int dg_get_m_alignment_for_contiguous_layout(void) { return kGroup; }

int64_t dg_get_scale_ld(int64_t rows) { return rows <= 0 ? 0 : (rows + 3) / 4 * 4; }

size_t dg_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t num_groups) {
  if (m <= 0 || n <= 0 || k <= 0 || k % kKAlign || num_groups <= 0) return 0;
  const int cus = effective_cus();
  if (cus < 0) return 0;
  return gemm_workspace_size(m, n, k, num_groups, cus);
}

static int check_token_group(const void* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* q, float* sa,
                             int64_t ld_sa) {
  DG_REQUIRE(num_groups >= 0 && m >= 0 && k > 0 && k % kKAlign == 0,
             "quantize_per_token_group: need groups >= 0, m >= 0, k > 0, k %% 16 == 0 (m=%lld k=%lld)",
             (long long)m, (long long)k);
  DG_REQUIRE(ld_sa >= m && ld_sa % 4 == 0, "quantize_per_token_group: need ld_sa >= m and ld_sa %% 4 == 0 (ld_sa=%lld)",
             (long long)ld_sa);
  if (m == 0 || num_groups == 0) return DG_OK;
  DG_REQUIRE(x && q && sa, "quantize_per_token_group: null pointer");
  DG_REQUIRE(aligned16(x) && aligned16(q) && aligned16(sa), "quantize_per_token_group: pointers must be 16-byte aligned");
  return 1;   // proceed
}

int dg_quantize_per_token_group(const float* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* q,
                                float* sa, int64_t ld_sa, dg_stream_t stream) {
  const int c = check_token_group(x, num_groups, m, k, q, sa, ld_sa);
  if (c <= 0) return c;
  return launch_quant_token_group(x, num_groups, m, k, q, sa, ld_sa, static_cast<hipStream_t>(stream));
}

int dg_quantize_per_token_group_bf16(const uint16_t* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* q,
                                     float* sa, int64_t ld_sa, dg_stream_t stream) {
  const int c = check_token_group(x, num_groups, m, k, q, sa, ld_sa);
  if (c <= 0) return c;
  return launch_quant_token_group_bf16(x, num_groups, m, k, q, sa, ld_sa, static_cast<hipStream_t>(stream));
}

int dg_quantize_per_block(const float* w, int64_t num_groups, int64_t n, int64_t k, uint8_t* q,
                          float* sb, dg_stream_t stream) {
  DG_REQUIRE(num_groups >= 0 && n >= 0 && k > 0 && k % kKAlign == 0,
             "quantize_per_block: need groups >= 0, n >= 0, k > 0, k %% 16 == 0");
  if (num_groups == 0 || n == 0) return DG_OK;
  DG_REQUIRE(w && q && sb, "quantize_per_block: null pointer");
  DG_REQUIRE(aligned16(w) && aligned16(q) && aligned16(sb), "quantize_per_block: pointers must be 16-byte aligned");
  return launch_quant_block(w, num_groups, n, k, q, sb, static_cast<hipStream_t>(stream));
}

static int check_gemm_common(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                             const float* sb, uint16_t* d, int64_t rows, int64_t n, int64_t k) {
  DG_REQUIRE(rows >= 0 && n >= 0 && k > 0 && k % kKAlign == 0, "gemm: need m >= 0, n >= 0, k > 0, k %% 16 == 0 (m=%lld n=%lld k=%lld)",
             (long long)rows, (long long)n, (long long)k);
  DG_REQUIRE(ld_sa >= rows && ld_sa % 4 == 0, "gemm: need ld_sa >= m and ld_sa %% 4 == 0 (ld_sa=%lld m=%lld)",
             (long long)ld_sa, (long long)rows);
  DG_REQUIRE(rows <= 0x7fffffffLL && n <= 0x7fffffffLL && k <= 0x7fffffffLL, "gemm: dimension too large");
  if (rows == 0 || n == 0) return DG_OK;
  DG_REQUIRE(a && sa && b && sb && d, "gemm: null pointer");
  DG_REQUIRE(aligned16(a) && aligned16(sa) && aligned16(b) && aligned16(sb) && aligned16(d),
             "gemm: pointers must be 16-byte aligned");
  return 1;   // proceed
}

int dg_gemm_fp8_nt(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                   const float* sb, uint16_t* d, int64_t m, int64_t n, int64_t k, void* workspace,
                   size_t workspace_bytes, dg_stream_t stream) {
  const int c = check_gemm_common(a, sa, ld_sa, b, sb, d, m, n, k);
  if (c <= 0) return c;
  DG_REQUIRE(workspace == nullptr || aligned16(workspace), "gemm: workspace must be 16-byte aligned");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm(0, a, sa, ld_sa, b, sb, 0, 0, d, nullptr, nullptr, 1, m, n, k, workspace,
                     workspace ? workspace_bytes : 0, static_cast<hipStream_t>(stream), cus);
}

int dg_gemm_fp8_nt_no_alloc(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b, const float* sb,
                            uint16_t* d, int64_t m, int64_t n, int64_t k, dg_stream_t stream) {
  const int c = check_gemm_common(a, sa, ld_sa, b, sb, d, m, n, k);
  if (c <= 0) return c;
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm_no_alloc(a, sa, ld_sa, b, sb, d, m, n, k, static_cast<hipStream_t>(stream), cus);
}

size_t dg_gemm_fp8_nt_act_quant_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % kKAlign) return 0;
  const int cus = effective_cus();
  if (cus < 0) return 0;
  return gemm_fq_workspace_size(m, n, k, cus);
}

static int gemm_act_quant(const void* x, bool bf16, const uint8_t* b, const float* sb, uint16_t* d, int64_t m,
                          int64_t n, int64_t k, void* workspace, size_t workspace_bytes, dg_stream_t stream) {
  DG_REQUIRE(m >= 0 && n >= 0 && k > 0 && k % kKAlign == 0,
             "gemm_act_quant: need m >= 0, n >= 0, k > 0, k %% 16 == 0 (m=%lld n=%lld k=%lld)", (long long)m,
             (long long)n, (long long)k);
  DG_REQUIRE(m <= 0x7fffffffLL && n <= 0x7fffffffLL && k <= 0x7fffffffLL, "gemm_act_quant: dimension too large");
  if (m == 0 || n == 0) return DG_OK;
  DG_REQUIRE(x && b && sb && d && workspace, "gemm_act_quant: null pointer");
  DG_REQUIRE(aligned16(x) && aligned16(b) && aligned16(sb) && aligned16(d) && aligned16(workspace),
             "gemm_act_quant: pointers must be 16-byte aligned");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm_fq(x, bf16, b, sb, d, m, n, k, workspace, workspace_bytes, static_cast<hipStream_t>(stream), cus);
}

int dg_gemm_fp8_nt_act_quant(const float* x, const uint8_t* b, const float* sb, uint16_t* d, int64_t m, int64_t n,
                             int64_t k, void* workspace, size_t workspace_bytes, dg_stream_t stream) {
  return gemm_act_quant(x, false, b, sb, d, m, n, k, workspace, workspace_bytes, stream);
}

int dg_gemm_fp8_nt_act_quant_bf16(const uint16_t* x, const uint8_t* b, const float* sb, uint16_t* d, int64_t m,
                                  int64_t n, int64_t k, void* workspace, size_t workspace_bytes, dg_stream_t stream) {
  return gemm_act_quant(x, true, b, sb, d, m, n, k, workspace, workspace_bytes, stream);
}

int dg_gemm_fp8_grouped_contiguous(const uint8_t* a, const float* sa, int64_t ld_sa,
                                   const uint8_t* b, const float* sb, const int32_t* m_indices,
                                   int64_t num_groups, uint16_t* d, int64_t m_total, int64_t n,
                                   int64_t k, dg_stream_t stream) {
  DG_REQUIRE(num_groups >= 0, "contiguous gemm: num_groups must be >= 0");
  if (num_groups == 0) return DG_OK;
  DG_REQUIRE(m_total % kGroup == 0, "contiguous gemm: m_total must be a multiple of 128 (got %lld)", (long long)m_total);
  const int c = check_gemm_common(a, sa, ld_sa, b, sb, d, m_total, n, k);
  if (c <= 0) return c;
  DG_REQUIRE(m_indices != nullptr, "contiguous gemm: m_indices is null");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm(1, a, sa, ld_sa, b, sb, 0, 0, d, m_indices, nullptr, num_groups, m_total, n, k,
                     nullptr, 0, static_cast<hipStream_t>(stream), cus);
}

int dg_gemm_fp8_grouped_masked(const uint8_t* a, const float* sa, int64_t ld_sa,
                               const uint8_t* b, const float* sb, uint16_t* d,
                               const int32_t* masked_m, int64_t num_groups, int64_t m_max,
                               int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                               dg_stream_t stream) {
  DG_REQUIRE(num_groups >= 0, "masked gemm: num_groups must be >= 0");
  if (num_groups == 0) return DG_OK;
  DG_REQUIRE(num_groups <= 1024, "masked gemm: at most 1024 groups (got %lld)", (long long)num_groups);
  const int c = check_gemm_common(a, sa, ld_sa, b, sb, d, m_max, n, k);
  if (c <= 0) return c;
  DG_REQUIRE(masked_m != nullptr, "masked gemm: masked_m is null");
  DG_REQUIRE(workspace == nullptr || aligned16(workspace), "gemm: workspace must be 16-byte aligned");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm(2, a, sa, ld_sa, b, sb, 0, 0, d, nullptr, masked_m, num_groups, m_max, n, k,
                     workspace, workspace ? workspace_bytes : 0, static_cast<hipStream_t>(stream), cus);
}

int dg_gemm_fp8_nt_row_scaled(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                              const float* sb, int64_t ld_sb, uint16_t* d, int64_t m, int64_t n, int64_t k,
                              void* workspace, size_t workspace_bytes, dg_stream_t stream) {
  const int c = check_gemm_common(a, sa, ld_sa, b, sb, d, m, n, k);
  if (c <= 0) return c;
  DG_REQUIRE(ld_sb >= n && ld_sb % 4 == 0, "row-scaled gemm: need ld_sb >= n and ld_sb %% 4 == 0 (ld_sb=%lld n=%lld)",
             (long long)ld_sb, (long long)n);
  DG_REQUIRE(workspace == nullptr || aligned16(workspace), "gemm: workspace must be 16-byte aligned");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  return launch_gemm(3, a, sa, ld_sa, b, sb, ld_sb, 0, d, nullptr, nullptr, 1, m, n, k, workspace,
                     workspace ? workspace_bytes : 0, static_cast<hipStream_t>(stream), cus);
}

int dg_gemm_fp8_k_grouped_row_scaled(const uint8_t* a, const float* sa, int64_t ld_sa, const uint8_t* b,
                                     const float* sb, int64_t ld_sb, uint16_t* d, const int64_t* group_tokens,
                                     int64_t num_groups, int64_t m, int64_t n, int64_t tokens_total, void* workspace,
                                     size_t workspace_bytes, dg_stream_t stream) {
  DG_REQUIRE(num_groups >= 0 && m >= 0 && n >= 0 && tokens_total >= 0,
             "k-grouped gemm: negative size (groups=%lld m=%lld n=%lld tokens=%lld)", (long long)num_groups,
             (long long)m, (long long)n, (long long)tokens_total);
  if (num_groups == 0 || m == 0 || n == 0) return DG_OK;
  DG_REQUIRE(group_tokens != nullptr, "k-grouped gemm: group_tokens is null");
  int64_t total = 0;
  for (int64_t g = 0; g < num_groups; ++g) {
    DG_REQUIRE(group_tokens[g] >= 0 && group_tokens[g] % kGroup == 0,
               "k-grouped gemm: group %lld has %lld tokens (need a multiple of 128)", (long long)g,
               (long long)group_tokens[g]);
    total += group_tokens[g];
  }
  DG_REQUIRE(total == tokens_total, "k-grouped gemm: group tokens sum to %lld, tokens_total is %lld", (long long)total,
             (long long)tokens_total);
  DG_REQUIRE(a && sa && b && sb && d, "k-grouped gemm: null pointer");
  DG_REQUIRE(aligned16(a) && aligned16(sa) && aligned16(b) && aligned16(sb) && aligned16(d),
             "k-grouped gemm: pointers must be 16-byte aligned");
  DG_REQUIRE(ld_sa >= m && ld_sa % 4 == 0 && ld_sb >= n && ld_sb % 4 == 0,
             "k-grouped gemm: need ld_sa >= m, ld_sb >= n, both multiples of 4");
  DG_REQUIRE((m * n) % 8 == 0, "k-grouped gemm: m * n must be a multiple of 8 (16-byte output blocks)");
  DG_REQUIRE(workspace == nullptr || aligned16(workspace), "gemm: workspace must be 16-byte aligned");
  const int cus = effective_cus();
  if (cus < 0) return cus;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t start = 0;
  for (int64_t g = 0; g < num_groups; ++g) {
    const int64_t tk = group_tokens[g];
    uint16_t* dg_ = d + g * m * n;
    const int r = tk == 0 ? launch_fill_zero_bf16(dg_, m * n, s)
                          : launch_gemm(3, a + start, sa + (start / kGroup) * ld_sa, ld_sa, b + start,
                                        sb + (start / kGroup) * ld_sb, ld_sb, tokens_total, dg_, nullptr, nullptr, 1,
                                        m, n, tk, workspace, workspace ? workspace_bytes : 0, s, cus);
    if (r != kOk) return r;
    start += tk;
  }
  return DG_OK;
}

static int check_channel_group(const void* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* qt, float* st,
                               int64_t ld_st) {
  DG_REQUIRE(num_groups >= 0 && m >= 0 && m % kKAlign == 0 && k >= 0 && k % 4 == 0,
             "quantize_per_channel_group: need groups >= 0, m >= 0, m %% 16 == 0, k >= 0, k %% 4 == 0 "
             "(m=%lld k=%lld)", (long long)m, (long long)k);
  DG_REQUIRE(ld_st >= k && ld_st % 4 == 0, "quantize_per_channel_group: need ld_st >= k and ld_st %% 4 == 0 (ld_st=%lld)",
             (long long)ld_st);
  if (m == 0 || k == 0 || num_groups == 0) return DG_OK;
  DG_REQUIRE(x && qt && st, "quantize_per_channel_group: null pointer");
  DG_REQUIRE(aligned16(x) && aligned16(qt) && aligned16(st), "quantize_per_channel_group: pointers must be 16-byte aligned");
  return 1;   // proceed
}

int dg_quantize_per_channel_group(const float* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* qt, float* st,
                                  int64_t ld_st, dg_stream_t stream) {
  const int c = check_channel_group(x, num_groups, m, k, qt, st, ld_st);
  if (c <= 0) return c;
  return launch_quant_channel_group(x, num_groups, m, k, qt, st, ld_st, static_cast<hipStream_t>(stream));
}

int dg_quantize_per_channel_group_bf16(const uint16_t* x, int64_t num_groups, int64_t m, int64_t k, uint8_t* qt,
                                       float* st, int64_t ld_st, dg_stream_t stream) {
  const int c = check_channel_group(x, num_groups, m, k, qt, st, ld_st);
  if (c <= 0) return c;
  return launch_quant_channel_group_bf16(x, num_groups, m, k, qt, st, ld_st, static_cast<hipStream_t>(stream));
}

int dg_transpose_blocks(const uint8_t* q, const float* s, int64_t num_groups, int64_t rows, int64_t cols, uint8_t* qt,
                        float* st, dg_stream_t stream) {
  DG_REQUIRE(num_groups >= 0 && rows >= 0 && cols >= 0 && rows % kKAlign == 0 && cols % kKAlign == 0,
             "transpose_blocks: need groups >= 0 and rows, cols >= 0 multiples of 16 (rows=%lld cols=%lld)",
             (long long)rows, (long long)cols);
  if (num_groups == 0 || rows == 0 || cols == 0) return DG_OK;
  DG_REQUIRE(q && s && qt && st, "transpose_blocks: null pointer");
  DG_REQUIRE(aligned16(q) && aligned16(qt), "transpose_blocks: code pointers must be 16-byte aligned");
  DG_REQUIRE(q != qt, "transpose_blocks: in-place transpose is not supported");
  return launch_transpose_blocks(q, s, num_groups, rows, cols, qt, st, static_cast<hipStream_t>(stream));
}

int dg_get_debug_status(uint32_t* flags, int64_t* block, int clear) {
  DG_REQUIRE(flags != nullptr, "dg_get_debug_status: flags is null");
  unsigned w[4] = {0u, 0u, 0u, 0u};
  const int r = read_diag(w, clear != 0);
  if (r != kOk) return r;
  *flags = w[0];
  if (block) *block = (int64_t)w[1] - 1;
  return DG_OK;
}

const char* dg_gemm_config_name(int layout, int64_t m, int64_t n, int64_t k, int64_t num_groups) {
  static thread_local char buf[96];
  buf[0] = 0;
  if (layout < 0 || layout > 3 || m <= 0 || n <= 0 || k <= 0 || k % kKAlign || num_groups <= 0) return buf;
  const int cus = effective_cus();
  if (cus < 0) return buf;
  gemm_config_name(layout, m, n, k, num_groups, cus, buf, sizeof(buf));
  return buf;
}

}  // extern "C"
