// C-ABI entry points: argument validation on the host, launch shaping, kernel launches.
// Nothing here allocates device memory or synchronizes; every check runs before any HIP call.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/mla_nvfp4.h"
#include "mla_internal.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_timing_start = nullptr;
thread_local hipEvent_t g_timing_stop = nullptr;

mla_status fail(mla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error[0] = '\0';
    return MLA_OK;
  }
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kComputeUnits = 256;                 // MI355X: 8 XCDs x 32 CUs
constexpr int64_t kMaxCacheBytes = int64_t(1) << 36;   // row offsets kept in 16-byte units (u32)

mla_status check_cache(const void* kv_cache, int64_t page_stride, int64_t cache_bytes,
                       int64_t row_bytes = MLA_ROW_BYTES) {
  if (!kv_cache) return fail(MLA_ERR_INVALID_ARG, "kv_cache is null");
  if (!aligned(kv_cache, 16)) return fail(MLA_ERR_INVALID_ARG, "kv_cache must be 16-byte aligned");
  if (page_stride < (int64_t)MLA_PAGE_ROWS * row_bytes || page_stride % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG, "page_stride_bytes %lld must be >= %lld and a multiple of 16",
                (long long)page_stride, (long long)(MLA_PAGE_ROWS * row_bytes));
  if (cache_bytes < row_bytes || cache_bytes > kMaxCacheBytes)
    return fail(MLA_ERR_INVALID_ARG, "cache_bytes %lld out of range [%lld, 2^36]", (long long)cache_bytes,
                (long long)row_bytes);
  return MLA_OK;
}

// ---- opt-in content checks (MLA_DEBUG_CHECKS) ------------------------------------------------
// -1 = not decided yet (the environment is read at the first call), 0 = off, 1 = on.
std::atomic<int> g_debug_checks{-1};

bool debug_checks_on() {
  int v = g_debug_checks.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("MLA_DEBUG_CHECKS");
    v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug_checks.compare_exchange_strong(expected, v);
    v = g_debug_checks.load(std::memory_order_relaxed);
  }
  return v == 1;
}

// Copies n elements of a device array to the host, synchronizing `stream` (debug checks only).
template <class T>
mla_status debug_copy(std::vector<T>& v, const T* dev, size_t n, hipStream_t stream, const char* what) {
  v.resize(n);
  if (n == 0) return MLA_OK;
  hipError_t e = hipMemcpyAsync(v.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "debug checks: copy of %s: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// Decode workgroups resident at once: one per compute unit (768 threads, up to 160 KB of LDS).
int waves_capacity(int32_t) { return kComputeUnits; }

size_t ws_bytes(int64_t T, int64_t H, int64_t S) {
  if (S <= 1) return 0;
  // FP16 partial outputs (512 per head) followed by FP32 partial log-sum-exp (1 per head)
  const size_t b = (size_t)(T * S * H) * (MLA_LATENT_DIM * 2 + sizeof(float));
  return (b + 255) & ~(size_t)255;
}

mla_status check_decode_common(const void* q, mla_dtype q_dtype, const void* kv_cache,
                               int64_t page_stride, int64_t cache_bytes,
                               const int32_t* block_table, int32_t max_pages, int32_t B,
                               int32_t q_len, int32_t H, float softmax_scale, int32_t num_splits,
                               float* out, float* lse, void* workspace, size_t workspace_bytes,
                               int64_t row_bytes = MLA_ROW_BYTES) {
  if (!q || !block_table || !out) return fail(MLA_ERR_INVALID_ARG, "null q / block_table / out");
  if (q_dtype != MLA_BF16 && q_dtype != MLA_FP32) return fail(MLA_ERR_UNSUPPORTED, "q_dtype must be bf16 or fp32");
  mla_status st = check_cache(kv_cache, page_stride, cache_bytes, row_bytes);
  if (st != MLA_OK) return st;
  if (B < 1 || q_len < 1) return fail(MLA_ERR_INVALID_ARG, "B and q_len must be >= 1");
  if (H < 16 || H % 16 != 0) return fail(MLA_ERR_UNSUPPORTED, "H=%d must be a positive multiple of 16", H);
  if (max_pages < 1) return fail(MLA_ERR_INVALID_ARG, "max_pages must be >= 1");
  if ((int64_t)max_pages * MLA_PAGE_ROWS > (int64_t)1 << 30) return fail(MLA_ERR_INVALID_ARG, "max_pages too large");
  if (!isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(MLA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(MLA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (num_splits < 1 || num_splits > 4096) return fail(MLA_ERR_INVALID_ARG, "num_splits %d out of range", num_splits);
  const int64_t T = (int64_t)B * q_len;
  if (T * num_splits * (H / 16) > (int64_t)1 << 28) return fail(MLA_ERR_INVALID_ARG, "launch too large");
  if (num_splits > 1) {
    if (!workspace) return fail(MLA_ERR_WORKSPACE, "num_splits > 1 needs a workspace");
    if (!aligned(workspace, 256)) return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < ws_bytes(T, H, num_splits))
      return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes,
                  ws_bytes(T, H, num_splits));
  }
  return MLA_OK;
}

// Workgroups per token (all launches together) for H heads.
int32_t head_groups(int32_t H) {
  const int32_t nb = H / 16;
  return nb / 4 + (nb % 4 != 0 ? 1 : 0);
}

mla_status run_decode(mla::DecodeArgs a, int32_t H, bool dense, bool fp8, hipStream_t stream) {
  const int64_t T = (int64_t)a.B * a.q_len;
  const int32_t S = a.n_split;
  const int32_t T32 = (int32_t)T;
  const int32_t nb = H / 16;
  const int32_t full = nb / 4, tail = nb % 4;
  // launch 1: groups of 64 heads; launch 2: the remaining 16..48 heads. The timing events (if
  // set) are recorded at the start of the first decode kernel and the end of the last.
  const int first = full > 0 ? 0 : 1, last = tail > 0 ? 1 : 0;
  for (int part = 0; part < 2; ++part) {
    const int32_t nh = part == 0 ? 4 : tail;
    const int32_t groups = part == 0 ? full : (tail ? 1 : 0);
    if (groups == 0) continue;
    a.head_begin = part == 0 ? 0 : full * 64;
    a.n_hg = groups;
    a.total_items = T32 * groups * S;
    // Whole tokens per XCD (workgroup i runs on XCD i % 8) whenever that keeps the busiest XCD
    // at the same number of rounds of its 32 compute units: the splits of a token then write
    // their partials into one L2, and the merge reads them there (launch_combine deals tokens
    // the same way). Otherwise an even split of the items.
    const int32_t even = (a.total_items + 7) / 8;
    const int32_t aligned = ((T32 + 7) / 8) * groups * S;
    a.items_per_xcd = ((aligned + 31) / 32 == (even + 31) / 32) ? aligned : even;
    hipError_t e = mla::launch_decode(a, nh, dense, fp8, stream, part == first ? g_timing_start : nullptr,
                                      part == last ? g_timing_stop : nullptr);
    if (e != hipSuccess) return hip_status(e, "decode kernel launch");
  }
  if (S > 1) {
    hipError_t e = mla::launch_combine(T32, H, S, a.ws_o, a.ws_lse, a.out, a.lse, stream);
    if (e != hipSuccess) return hip_status(e, "combine kernel launch");
  }
  return hip_status(hipSuccess, "");
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error; }

mla_status mla_set_debug_checks(int32_t enabled) {
  g_debug_checks.store(enabled ? 1 : 0, std::memory_order_relaxed);
  return MLA_OK;
}

int32_t mla_debug_checks_enabled(void) { return debug_checks_on() ? 1 : 0; }

mla_status mla_check_sparse_indices(const int32_t* topk_idx, int32_t B, int32_t q_len,
                                    int32_t topk, const int32_t* block_table, int32_t max_pages,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    int64_t row_bytes) {
  if (!topk_idx || !block_table || B < 1 || q_len < 1 || topk < 1 || max_pages < 1)
    return fail(MLA_ERR_INVALID_ARG, "check_sparse_indices: null array or empty shape");
  const int64_t limit = (int64_t)max_pages * MLA_PAGE_ROWS;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t t = 0; t < q_len; ++t)
      for (int32_t s = 0; s < topk; ++s) {
        const int64_t e = ((int64_t)b * q_len + t) * topk + s;
        const int32_t j = topk_idx[e];
        if (j == -1) continue;
        if (j < 0)
          return fail(MLA_ERR_INVALID_ARG, "topk_idx[%d][%d][%d] = %d: negative and not -1", b, t, s, j);
        if (j >= limit)
          return fail(MLA_ERR_INVALID_ARG, "topk_idx[%d][%d][%d] = %d: beyond the block table (%lld positions)",
                      b, t, s, j, (long long)limit);
        const int32_t pg = block_table[(int64_t)b * max_pages + j / MLA_PAGE_ROWS];
        if (pg < 0)
          return fail(MLA_ERR_INVALID_ARG, "topk_idx[%d][%d][%d] = %d: block_table[%d][%d] = %d is unmapped",
                      b, t, s, j, b, j / MLA_PAGE_ROWS, pg);
        const int64_t off = (int64_t)pg * page_stride_bytes + (int64_t)(j % MLA_PAGE_ROWS) * row_bytes;
        if (pg > cache_bytes / page_stride_bytes || off + row_bytes > cache_bytes)
          return fail(MLA_ERR_INVALID_ARG, "topk_idx[%d][%d][%d] = %d: page %d puts the row at byte %lld, "
                      "outside the %lld-byte cache", b, t, s, j, pg, (long long)off, (long long)cache_bytes);
      }
  return MLA_OK;
}

mla_status mla_check_dense_tables(const int32_t* seq_lens, int32_t B, int32_t q_len,
                                  const int32_t* block_table, int32_t max_pages,
                                  int64_t page_stride_bytes, int64_t cache_bytes,
                                  int64_t row_bytes) {
  if (!seq_lens || !block_table || B < 1 || q_len < 1 || max_pages < 1)
    return fail(MLA_ERR_INVALID_ARG, "check_dense_tables: null array or empty shape");
  const int64_t limit = (int64_t)max_pages * MLA_PAGE_ROWS;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = seq_lens[b];
    if (n < 0) return fail(MLA_ERR_INVALID_ARG, "seq_lens[%d] = %lld is negative", b, (long long)n);
    if (n > limit)
      return fail(MLA_ERR_INVALID_ARG, "seq_lens[%d] = %lld exceeds the block table (%lld positions)",
                  b, (long long)n, (long long)limit);
    for (int64_t p = 0; p * MLA_PAGE_ROWS < n; ++p) {
      const int32_t pg = block_table[(int64_t)b * max_pages + p];
      if (pg < 0)
        return fail(MLA_ERR_INVALID_ARG, "block_table[%d][%lld] = %d is unmapped inside seq_lens[%d] = %lld",
                    b, (long long)p, pg, b, (long long)n);
      const int64_t rows = n - p * MLA_PAGE_ROWS < MLA_PAGE_ROWS ? n - p * MLA_PAGE_ROWS : MLA_PAGE_ROWS;
      const int64_t end = (int64_t)pg * page_stride_bytes + rows * row_bytes;
      if (pg > cache_bytes / page_stride_bytes || end > cache_bytes)
        return fail(MLA_ERR_INVALID_ARG, "block_table[%d][%lld] = %d: rows end at byte %lld, outside the "
                    "%lld-byte cache", b, (long long)p, pg, (long long)end, (long long)cache_bytes);
    }
  }
  return MLA_OK;
}

mla_status mla_check_slots(const int64_t* slots, int64_t n, int64_t page_stride_bytes,
                           int64_t cache_bytes, int64_t row_bytes) {
  if (n < 0 || (n > 0 && !slots)) return fail(MLA_ERR_INVALID_ARG, "check_slots: null array or negative n");
  for (int64_t i = 0; i < n; ++i) {
    const int64_t s = slots[i];
    if (s == -1) continue;
    if (s < 0) return fail(MLA_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld: negative and not -1", (long long)i, (long long)s);
    const int64_t pg = s / MLA_PAGE_ROWS;
    if (pg > (cache_bytes / page_stride_bytes) + 1 ||
        pg * page_stride_bytes + (s % MLA_PAGE_ROWS) * row_bytes + row_bytes > cache_bytes)
      return fail(MLA_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld: the row falls outside the %lld-byte cache",
                  (long long)i, (long long)s, (long long)cache_bytes);
  }
  return MLA_OK;
}

mla_status mla_set_timing_events(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(MLA_ERR_INVALID_ARG, "timing events must be both set or both null");
  g_timing_start = start;
  g_timing_stop = stop;
  return MLA_OK;
}

mla_status mla_nvfp4_quantize_append(const void* latent, int64_t latent_row_stride,
                                     const void* rope, int64_t rope_row_stride,
                                     const int64_t* slot_mapping, int64_t n_rows, void* kv_cache,
                                     int64_t page_stride_bytes, int64_t cache_bytes,
                                     hipStream_t stream) {
  if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0");
  mla_status st = check_cache(kv_cache, page_stride_bytes, cache_bytes);
  if (st != MLA_OK) return st;
  if (n_rows == 0) return hip_status(hipSuccess, "");
  if (!latent || !rope || !slot_mapping) return fail(MLA_ERR_INVALID_ARG, "null latent / rope / slot_mapping");
  if (!aligned(latent, 16) || latent_row_stride < MLA_LATENT_DIM || latent_row_stride % 8 != 0)
    return fail(MLA_ERR_INVALID_ARG, "latent must be 16-byte aligned with a row stride >= 512 and a multiple of 8");
  if (!aligned(rope, 2) || rope_row_stride < MLA_ROPE_DIM)
    return fail(MLA_ERR_INVALID_ARG, "rope must be 2-byte aligned with a row stride >= 64");
  if (!aligned(slot_mapping, 8)) return fail(MLA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  if (debug_checks_on()) {
    std::vector<int64_t> hs;
    if ((st = debug_copy(hs, slot_mapping, (size_t)n_rows, stream, "slot_mapping")) != MLA_OK) return st;
    if ((st = mla_check_slots(hs.data(), n_rows, page_stride_bytes, cache_bytes, MLA_ROW_BYTES)) != MLA_OK) return st;
  }
  return hip_status(mla::launch_quantize_append(latent, latent_row_stride, rope, rope_row_stride,
                                                slot_mapping, n_rows, kv_cache, page_stride_bytes,
                                                cache_bytes, stream),
                    "quantize_append launch");
}

size_t mla_decode_workspace_size(int32_t num_tokens, int32_t H, int32_t num_splits) {
  if (num_tokens < 1 || H < 1) return 0;
  return ws_bytes(num_tokens, H, num_splits);
}

int32_t mla_sparse_decode_num_splits(int32_t num_tokens, int32_t H, int32_t topk, int32_t max_splits) {
  if (num_tokens < 1 || H < 16 || topk < 1) return 1;
  const int32_t cap_by_rows = topk >= 64 ? topk / 64 : 1;    // keep >= 64 rows per split
  if (max_splits > 0) return max_splits < cap_by_rows ? max_splits : cap_by_rows;
  const int64_t groups = head_groups(H);
  const int64_t items = (int64_t)num_tokens * groups;
  const int64_t cap = waves_capacity(H);
  // Smallest split count whose items fill ~90% of one wave of workgroups.
  int64_t s = (cap * 9 / 10 + items - 1) / items;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  if (s > cap_by_rows) s = cap_by_rows;
  return (int32_t)s;
}

int32_t mla_dense_decode_split_tokens(int32_t num_tokens, int32_t H, int32_t max_pages) {
  if (num_tokens < 1 || H < 16 || max_pages < 1) return 4096;
  const int64_t items = (int64_t)num_tokens * head_groups(H);
  int64_t s = waves_capacity(H) / items;                 // splits per token that fit one wave
  if (s < 1) s = 1;
  const int64_t rows = (int64_t)max_pages * MLA_PAGE_ROWS;
  int64_t st = (rows + s - 1) / s;
  st = (st + MLA_PAGE_ROWS - 1) / MLA_PAGE_ROWS * MLA_PAGE_ROWS;
  const int64_t lo = MLA_PAGE_ROWS, hi = (int64_t)mla::kMaxDensePages * MLA_PAGE_ROWS;
  return (int32_t)(st < lo ? lo : (st > hi ? hi : st));
}

int32_t mla_dense_decode_num_splits(int32_t max_pages, int32_t split_tokens) {
  if (max_pages < 1 || split_tokens < 64) return 1;
  const int64_t n = (int64_t)max_pages * MLA_PAGE_ROWS;
  return (int32_t)((n + split_tokens - 1) / split_tokens);
}

}  // extern "C"

namespace {

// The new rows of a fused append + sparse decode (mla_sparse_decode_append).
struct AppendIn {
  const void* latent;
  int64_t latent_stride;
  const void* rope;
  int64_t rope_stride;
  const int64_t* slots;
  void* cache;
};

mla_status sparse_decode_impl(bool fp8, const void* q, mla_dtype q_dtype, const void* kv_cache,
                              int64_t page_stride_bytes, int64_t cache_bytes,
                              const int32_t* block_table, int32_t max_pages,
                              const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                              int32_t H, float softmax_scale, int32_t num_splits, float* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const AppendIn* ap = nullptr) {
  mla_status st = check_decode_common(q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                                      block_table, max_pages, B, q_len, H, softmax_scale,
                                      num_splits, out, lse, workspace, workspace_bytes,
                                      fp8 ? MLA_FP8_ROW_BYTES : MLA_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (ap) {
    if (q_len > mla::kApMaxRows) return fail(MLA_ERR_UNSUPPORTED, "fused append: q_len %d > %d", q_len, mla::kApMaxRows);
    if (!ap->latent || !ap->rope || !ap->slots) return fail(MLA_ERR_INVALID_ARG, "null latent / rope / slot_mapping");
    if (!aligned(ap->latent, 16) || ap->latent_stride < MLA_LATENT_DIM || ap->latent_stride % 8 != 0)
      return fail(MLA_ERR_INVALID_ARG, "latent must be 16-byte aligned with a row stride >= 512 and a multiple of 8");
    if (!aligned(ap->rope, 2) || ap->rope_stride < MLA_ROPE_DIM)
      return fail(MLA_ERR_INVALID_ARG, "rope must be 2-byte aligned with a row stride >= 64");
    if (!aligned(ap->slots, 8)) return fail(MLA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  }
  if (!topk_idx) return fail(MLA_ERR_INVALID_ARG, "topk_idx is null");
  if (topk < 1 || topk > MLA_MAX_TOPK) return fail(MLA_ERR_UNSUPPORTED, "topk %d outside [1, 2048]", topk);
  if (!aligned(topk_idx, 4) || !aligned(block_table, 4)) return fail(MLA_ERR_INVALID_ARG, "index arrays must be 4-byte aligned");
  const int64_t T = (int64_t)B * q_len;
  int32_t split_rows = (topk + num_splits - 1) / num_splits;
  split_rows = (split_rows + 63) & ~63;
  mla::DecodeArgs a{};
  a.q = q;
  a.q_fp32 = (q_dtype == MLA_FP32);
  a.cache = (const uint8_t*)kv_cache;
  a.page_stride = page_stride_bytes;
  a.cache_bytes = cache_bytes;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.B = B;
  a.q_len = q_len;
  a.H = H;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.n_split = num_splits;
  a.split_rows = split_rows;
  a.out = out;
  a.lse = lse;
  if (num_splits > 1) {
    a.ws_o = (_Float16*)workspace;
    a.ws_lse = (float*)(a.ws_o + T * num_splits * H * MLA_LATENT_DIM);
  }
  if (debug_checks_on()) {
    std::vector<int32_t> hi, hb;
    if ((st = debug_copy(hi, topk_idx, (size_t)(T * topk), stream, "topk_idx")) != MLA_OK) return st;
    if ((st = debug_copy(hb, block_table, (size_t)B * max_pages, stream, "block_table")) != MLA_OK) return st;
    st = mla_check_sparse_indices(hi.data(), B, q_len, topk, hb.data(), max_pages, page_stride_bytes,
                                  cache_bytes, fp8 ? MLA_FP8_ROW_BYTES : MLA_ROW_BYTES);
    if (st != MLA_OK) return st;
    if (ap) {
      std::vector<int64_t> hs;
      if ((st = debug_copy(hs, ap->slots, (size_t)T, stream, "slot_mapping")) != MLA_OK) return st;
      if ((st = mla_check_slots(hs.data(), T, page_stride_bytes, cache_bytes, MLA_ROW_BYTES)) != MLA_OK) return st;
    }
  }
  if (ap) {
    a.ap_latent = (const uint16_t*)ap->latent;
    a.ap_latent_stride = ap->latent_stride;
    a.ap_rope = (const uint16_t*)ap->rope;
    a.ap_rope_stride = ap->rope_stride;
    a.ap_slots = ap->slots;
    a.ap_cache = (uint8_t*)ap->cache;
  }
  return run_decode(a, H, false, fp8, stream);
}

mla_status dense_decode_impl(bool fp8, const void* q, mla_dtype q_dtype, const void* kv_cache,
                             int64_t page_stride_bytes, int64_t cache_bytes,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H,
                             float softmax_scale, int32_t split_tokens, int32_t num_splits,
                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  mla_status st = check_decode_common(q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                                      block_table, max_pages, B, q_len, H, softmax_scale,
                                      num_splits, out, lse, workspace, workspace_bytes,
                                      fp8 ? MLA_FP8_ROW_BYTES : MLA_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (!seq_lens) return fail(MLA_ERR_INVALID_ARG, "seq_lens is null");
  if (split_tokens < 64 || split_tokens % 64 != 0 || split_tokens > mla::kMaxDensePages * MLA_PAGE_ROWS)
    return fail(MLA_ERR_UNSUPPORTED, "split_tokens %d must be a multiple of 64 in [64, 8192]", split_tokens);
  if (num_splits != mla_dense_decode_num_splits(max_pages, split_tokens))
    return fail(MLA_ERR_INVALID_ARG, "num_splits %d != ceil(max_pages*64/split_tokens) = %d", num_splits,
                mla_dense_decode_num_splits(max_pages, split_tokens));
  const int64_t T = (int64_t)B * q_len;
  mla::DecodeArgs a{};
  a.q = q;
  a.q_fp32 = (q_dtype == MLA_FP32);
  a.cache = (const uint8_t*)kv_cache;
  a.page_stride = page_stride_bytes;
  a.cache_bytes = cache_bytes;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.B = B;
  a.q_len = q_len;
  a.H = H;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.n_split = num_splits;
  a.split_rows = split_tokens;
  a.out = out;
  a.lse = lse;
  if (num_splits > 1) {
    a.ws_o = (_Float16*)workspace;
    a.ws_lse = (float*)(a.ws_o + T * num_splits * H * MLA_LATENT_DIM);
  }
  if (debug_checks_on()) {
    std::vector<int32_t> hs, hb;
    if ((st = debug_copy(hs, seq_lens, (size_t)B, stream, "seq_lens")) != MLA_OK) return st;
    if ((st = debug_copy(hb, block_table, (size_t)B * max_pages, stream, "block_table")) != MLA_OK) return st;
    st = mla_check_dense_tables(hs.data(), B, q_len, hb.data(), max_pages, page_stride_bytes,
                                cache_bytes, fp8 ? MLA_FP8_ROW_BYTES : MLA_ROW_BYTES);
    if (st != MLA_OK) return st;
  }
  return run_decode(a, H, true, fp8, stream);
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Staged-path workspace: FP8 rows, staged index list, staged block table, decode partials.
struct StagedLayout {
  size_t rows, idx, bt, dec, total;
};

StagedLayout staged_layout(int64_t T, int32_t H, int32_t topk, int32_t num_splits) {
  const int64_t topk_pad = (topk + 63) & ~63;
  StagedLayout l;
  l.rows = 0;
  l.idx = round256((size_t)(T * topk_pad * MLA_FP8_ROW_BYTES));
  l.bt = l.idx + round256((size_t)(T * topk) * 4);
  l.dec = l.bt + round256((size_t)(T * (topk_pad / 64)) * 4);
  l.total = l.dec + ws_bytes(T, H, num_splits);
  return l;
}

// Shared-row decode workspace: union positions, token masks, union sizes, split partials.
struct SharedLayout {
  int32_t groups, stride, S;
  size_t mask, count, part, total;
};

SharedLayout shared_layout(int32_t B, int32_t q_len, int32_t H, int32_t topk) {
  SharedLayout l;
  l.groups = B * ((q_len + 3) / 4);
  l.stride = 4 * topk;
  // at least enough splits to keep every split's share of a union within the row list a
  // workgroup holds, then enough to fill ~90% of one wave of workgroups (at most 16)
  const int32_t min_s = (4 * topk + mla::kMaxSplitRows - 1) / mla::kMaxSplitRows;
  const int64_t items = (int64_t)l.groups * (H / 16);
  int64_t s = (kComputeUnits * 9 / 10 + items - 1) / items;
  if (s > 16) s = 16;
  if (s < min_s) s = min_s;
  if (s < 1) s = 1;
  l.S = (int32_t)s;
  const size_t n = (size_t)l.groups * mla::kUnionParts * (size_t)l.stride;
  l.mask = round256(n * sizeof(int32_t));
  l.count = l.mask + round256(n);
  l.part = l.count + round256((size_t)l.groups * mla::kUnionParts * sizeof(int32_t));
  l.total = l.part + ws_bytes((int64_t)B * q_len, H, l.S);
  return l;
}

}  // namespace

extern "C" {

mla_status mla_sparse_decode(const void* q, mla_dtype q_dtype, const void* kv_cache,
                             int64_t page_stride_bytes, int64_t cache_bytes,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                             int32_t H, float softmax_scale, int32_t num_splits, float* out,
                             float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return sparse_decode_impl(false, q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                            block_table, max_pages, topk_idx, topk, B, q_len, H, softmax_scale,
                            num_splits, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_sparse_decode_append(const void* q, mla_dtype q_dtype, void* kv_cache,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                                    int32_t H, float softmax_scale, int32_t num_splits,
                                    const void* latent, int64_t latent_row_stride,
                                    const void* rope, int64_t rope_row_stride,
                                    const int64_t* slot_mapping, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const AppendIn ap{latent, latent_row_stride, rope, rope_row_stride, slot_mapping, kv_cache};
  return sparse_decode_impl(false, q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                            block_table, max_pages, topk_idx, topk, B, q_len, H, softmax_scale,
                            num_splits, out, lse, workspace, workspace_bytes, stream, &ap);
}

size_t mla_shared_decode_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t topk) {
  if (B < 1 || q_len < 1 || H < 16 || topk < 1 || topk > MLA_MAX_TOPK) return 0;
  return shared_layout(B, q_len, H, topk).total;
}

int32_t mla_shared_decode_num_splits(int32_t B, int32_t q_len, int32_t H, int32_t topk) {
  if (B < 1 || q_len < 1 || H < 16 || topk < 1 || topk > MLA_MAX_TOPK) return 1;
  return shared_layout(B, q_len, H, topk).S;
}

mla_status mla_sparse_decode_shared(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                                    int32_t H, float softmax_scale, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mla_status st = check_decode_common(q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                                      block_table, max_pages, B, q_len, H, softmax_scale, 1, out,
                                      lse, nullptr, 0);
  if (st != MLA_OK) return st;
  if (!topk_idx) return fail(MLA_ERR_INVALID_ARG, "topk_idx is null");
  if (topk < 1 || topk > MLA_MAX_TOPK) return fail(MLA_ERR_UNSUPPORTED, "topk %d outside [1, 2048]", topk);
  if (!aligned(topk_idx, 4) || !aligned(block_table, 4)) return fail(MLA_ERR_INVALID_ARG, "index arrays must be 4-byte aligned");
  if ((int64_t)max_pages * MLA_PAGE_ROWS > mla::kUnionMaxPos)
    return fail(MLA_ERR_UNSUPPORTED, "shared rows: max_pages*64 = %lld positions > %d",
                (long long)max_pages * MLA_PAGE_ROWS, mla::kUnionMaxPos);
  const SharedLayout l = shared_layout(B, q_len, H, topk);
  if ((int64_t)l.groups * (H / 16) * l.S > (int64_t)1 << 28) return fail(MLA_ERR_INVALID_ARG, "launch too large");
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < l.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed", l.total);
  if (debug_checks_on()) {
    const int64_t T = (int64_t)B * q_len;
    std::vector<int32_t> hi, hb;
    if ((st = debug_copy(hi, topk_idx, (size_t)(T * topk), stream, "topk_idx")) != MLA_OK) return st;
    if ((st = debug_copy(hb, block_table, (size_t)B * max_pages, stream, "block_table")) != MLA_OK) return st;
    st = mla_check_sparse_indices(hi.data(), B, q_len, topk, hb.data(), max_pages, page_stride_bytes,
                                  cache_bytes, MLA_ROW_BYTES);
    if (st != MLA_OK) return st;
  }
  uint8_t* ws = (uint8_t*)workspace;
  mla::DecodeArgs a{};
  a.q = q;
  a.q_fp32 = (q_dtype == MLA_FP32);
  a.cache = (const uint8_t*)kv_cache;
  a.page_stride = page_stride_bytes;
  a.cache_bytes = cache_bytes;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.B = B;
  a.q_len = q_len;
  a.H = H;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.n_split = l.S;
  a.split_rows = 0;                             // each group's union is split evenly in the kernel
  a.head_begin = 0;
  a.n_hg = H / 16;
  a.total_items = l.groups * a.n_hg * l.S;
  a.items_per_xcd = (a.total_items + 7) / 8;
  a.out = out;
  a.lse = lse;
  a.u_pos = (const int32_t*)ws;
  a.u_mask = ws + l.mask;
  a.u_count = (const int32_t*)(ws + l.count);
  a.u_stride = l.stride;
  a.groups_per_req = (q_len + 3) / 4;
  const int64_t T = (int64_t)B * q_len;
  if (l.S > 1) {
    a.ws_o = (_Float16*)(ws + l.part);
    a.ws_lse = (float*)(a.ws_o + T * l.S * H * MLA_LATENT_DIM);
  }
  hipError_t e = mla::launch_union(topk_idx, topk, B, q_len, max_pages * MLA_PAGE_ROWS, (int32_t*)ws,
                                   ws + l.mask, (int32_t*)(ws + l.count), l.stride, stream);
  if (e != hipSuccess) return hip_status(e, "union kernel launch");
  // the timing hook brackets the decode kernel only
  e = mla::launch_decode_shared(a, stream, g_timing_start, g_timing_stop);
  if (e != hipSuccess) return hip_status(e, "shared decode kernel launch");
  if (l.S > 1) {
    e = mla::launch_combine((int32_t)T, H, l.S, a.ws_o, a.ws_lse, out, lse, stream);
    if (e != hipSuccess) return hip_status(e, "combine kernel launch");
  }
  return hip_status(hipSuccess, "");
}

mla_status mla_fp8_sparse_decode(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                 int64_t page_stride_bytes, int64_t cache_bytes,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                                 int32_t H, float softmax_scale, int32_t num_splits, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return sparse_decode_impl(true, q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                            block_table, max_pages, topk_idx, topk, B, q_len, H, softmax_scale,
                            num_splits, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_dense_decode(const void* q, mla_dtype q_dtype, const void* kv_cache,
                            int64_t page_stride_bytes, int64_t cache_bytes,
                            const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                            int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                            int32_t split_tokens, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dense_decode_impl(false, q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                           block_table, max_pages, seq_lens, B, q_len, H, softmax_scale,
                           split_tokens, num_splits, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_fp8_dense_decode(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                int64_t page_stride_bytes, int64_t cache_bytes,
                                const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t H,
                                float softmax_scale, int32_t split_tokens, int32_t num_splits,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return dense_decode_impl(true, q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                           block_table, max_pages, seq_lens, B, q_len, H, softmax_scale,
                           split_tokens, num_splits, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_fp8_append(const void* latent, int64_t latent_row_stride, const void* rope,
                          int64_t rope_row_stride, const int64_t* slot_mapping, int64_t n_rows,
                          void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                          hipStream_t stream) {
  if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0");
  mla_status st = check_cache(kv_cache, page_stride_bytes, cache_bytes, MLA_FP8_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (n_rows == 0) return hip_status(hipSuccess, "");
  if (!latent || !rope || !slot_mapping) return fail(MLA_ERR_INVALID_ARG, "null latent / rope / slot_mapping");
  if (!aligned(latent, 16) || latent_row_stride < MLA_LATENT_DIM || latent_row_stride % 8 != 0)
    return fail(MLA_ERR_INVALID_ARG, "latent must be 16-byte aligned with a row stride >= 512 and a multiple of 8");
  if (!aligned(rope, 2) || rope_row_stride < MLA_ROPE_DIM)
    return fail(MLA_ERR_INVALID_ARG, "rope must be 2-byte aligned with a row stride >= 64");
  if (!aligned(slot_mapping, 8)) return fail(MLA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  if (debug_checks_on()) {
    std::vector<int64_t> hs;
    if ((st = debug_copy(hs, slot_mapping, (size_t)n_rows, stream, "slot_mapping")) != MLA_OK) return st;
    if ((st = mla_check_slots(hs.data(), n_rows, page_stride_bytes, cache_bytes, MLA_FP8_ROW_BYTES)) != MLA_OK) return st;
  }
  return hip_status(mla::launch_fp8_append(latent, latent_row_stride, rope, rope_row_stride,
                                           slot_mapping, n_rows, kv_cache, page_stride_bytes,
                                           cache_bytes, stream),
                    "fp8_append launch");
}

mla_status mla_nvfp4_stage_fp8(const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                               const int32_t* block_table, int32_t max_pages,
                               const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                               void* staged_rows, int32_t* staged_idx, int32_t* staged_block_table,
                               hipStream_t stream) {
  mla_status st = check_cache(kv_cache, page_stride_bytes, cache_bytes);
  if (st != MLA_OK) return st;
  if (!block_table || !topk_idx || !staged_rows || !staged_idx || !staged_block_table)
    return fail(MLA_ERR_INVALID_ARG, "null block_table / topk_idx / staged buffers");
  if (B < 1 || q_len < 1) return fail(MLA_ERR_INVALID_ARG, "B and q_len must be >= 1");
  if (max_pages < 1 || (int64_t)max_pages * MLA_PAGE_ROWS > (int64_t)1 << 30)
    return fail(MLA_ERR_INVALID_ARG, "max_pages out of range");
  if (topk < 1 || topk > MLA_MAX_TOPK) return fail(MLA_ERR_UNSUPPORTED, "topk %d outside [1, 2048]", topk);
  if (!aligned(staged_rows, 16) || !aligned(staged_idx, 4) || !aligned(staged_block_table, 4) ||
      !aligned(topk_idx, 4) || !aligned(block_table, 4))
    return fail(MLA_ERR_INVALID_ARG, "misaligned staged buffers or index arrays");
  const int64_t T = (int64_t)B * q_len;
  if (T > (int64_t)1 << 20) return fail(MLA_ERR_INVALID_ARG, "too many query tokens");
  if (debug_checks_on()) {
    std::vector<int32_t> hi, hb;
    if ((st = debug_copy(hi, topk_idx, (size_t)(T * topk), stream, "topk_idx")) != MLA_OK) return st;
    if ((st = debug_copy(hb, block_table, (size_t)B * max_pages, stream, "block_table")) != MLA_OK) return st;
    st = mla_check_sparse_indices(hi.data(), B, q_len, topk, hb.data(), max_pages, page_stride_bytes,
                                  cache_bytes, MLA_ROW_BYTES);
    if (st != MLA_OK) return st;
  }
  return hip_status(mla::launch_stage_fp8(kv_cache, page_stride_bytes, cache_bytes, block_table,
                                          max_pages, topk_idx, topk, (int32_t)T, q_len, staged_rows,
                                          staged_idx, staged_block_table, stream),
                    "stage_fp8 launch");
}

size_t mla_staged_workspace_size(int32_t num_tokens, int32_t H, int32_t topk, int32_t num_splits) {
  if (num_tokens < 1 || H < 1 || topk < 1) return 0;
  return staged_layout(num_tokens, H, topk, num_splits).total;
}

mla_status mla_staged_sparse_decode(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk, int32_t B,
                                    int32_t q_len, int32_t H, float softmax_scale,
                                    int32_t num_splits, float* out, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  mla_status st = check_decode_common(q, q_dtype, kv_cache, page_stride_bytes, cache_bytes,
                                      block_table, max_pages, B, q_len, H, softmax_scale,
                                      num_splits, out, lse, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  if (!topk_idx) return fail(MLA_ERR_INVALID_ARG, "topk_idx is null");
  if (topk < 1 || topk > MLA_MAX_TOPK) return fail(MLA_ERR_UNSUPPORTED, "topk %d outside [1, 2048]", topk);
  const int64_t T = (int64_t)B * q_len;
  const int64_t staged_bytes = T * ((topk + 63) & ~63) * MLA_FP8_ROW_BYTES;
  if (staged_bytes > kMaxCacheBytes) return fail(MLA_ERR_INVALID_ARG, "staged rows exceed 2^36 bytes");
  const StagedLayout l = staged_layout(T, H, topk, num_splits);
  if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_WORKSPACE, "the staged path needs a 256-byte aligned workspace");
  if (workspace_bytes < l.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, l.total);
  uint8_t* ws = (uint8_t*)workspace;
  const int32_t topk_pad = (topk + 63) & ~63;
  st = mla_nvfp4_stage_fp8(kv_cache, page_stride_bytes, cache_bytes, block_table, max_pages,
                           topk_idx, topk, B, q_len, ws + l.rows, (int32_t*)(ws + l.idx),
                           (int32_t*)(ws + l.bt), stream);
  if (st != MLA_OK) return st;
  // every query token is its own "request" over its staged rows
  return sparse_decode_impl(true, q, q_dtype, ws + l.rows, (int64_t)MLA_PAGE_ROWS * MLA_FP8_ROW_BYTES,
                            (int64_t)T * topk_pad * MLA_FP8_ROW_BYTES, (const int32_t*)(ws + l.bt),
                            topk_pad / 64, (const int32_t*)(ws + l.idx), topk, (int32_t)T, 1, H,
                            softmax_scale, num_splits, out, lse, ws + l.dec, l.total - l.dec, stream);
}

mla_status mla_copy_kv_blocks(const void* src_pool, int64_t src_pool_bytes, void* dst_pool,
                              int64_t dst_pool_bytes, mla_kv_layout layout, int32_t n_layers,
                              int64_t page_bytes, const int32_t* src_blocks,
                              const int32_t* dst_blocks, int32_t n_blocks, hipStream_t stream) {
  if (layout != MLA_LAYOUT_BLOCK_MAJOR && layout != MLA_LAYOUT_LAYER_MAJOR)
    return fail(MLA_ERR_INVALID_ARG, "unknown layout %d", (int)layout);
  if (n_layers < 1 || page_bytes < 16 || page_bytes % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG, "n_layers must be >= 1 and page_bytes a positive multiple of 16");
  if (n_blocks < 0) return fail(MLA_ERR_INVALID_ARG, "n_blocks must be >= 0");
  const int64_t block_bytes = (int64_t)n_layers * page_bytes;
  if (src_pool_bytes < block_bytes || dst_pool_bytes < block_bytes ||
      src_pool_bytes % block_bytes != 0 || dst_pool_bytes % block_bytes != 0)
    return fail(MLA_ERR_INVALID_ARG, "pool sizes must be whole multiples of n_layers * page_bytes");
  if (n_blocks == 0) return hip_status(hipSuccess, "");
  if (!src_pool || !dst_pool || !src_blocks || !dst_blocks)
    return fail(MLA_ERR_INVALID_ARG, "null pool or block list");
  if (!aligned(src_pool, 16) || !aligned(dst_pool, 16) || !aligned(src_blocks, 4) || !aligned(dst_blocks, 4))
    return fail(MLA_ERR_INVALID_ARG, "pools must be 16-byte and block lists 4-byte aligned");
  return hip_status(mla::launch_copy_pages(src_pool, src_pool_bytes / block_bytes, dst_pool,
                                           dst_pool_bytes / block_bytes, (int32_t)layout, n_layers,
                                           page_bytes, src_blocks, dst_blocks, n_blocks, stream),
                    "copy_kv_blocks launch");
}

int64_t mla_kv_transfer_regions(mla_kv_layout layout, int32_t n_layers, int64_t page_bytes,
                                int64_t pool_blocks, const int32_t* blocks, int32_t n_blocks) {
  if ((layout != MLA_LAYOUT_BLOCK_MAJOR && layout != MLA_LAYOUT_LAYER_MAJOR) || n_layers < 1 ||
      page_bytes < 1 || pool_blocks < 1 || n_blocks < 0 || (n_blocks > 0 && !blocks))
    return -1;
  const int64_t n = (int64_t)n_blocks * n_layers;
  if (n == 0) return 0;
  int64_t* starts = (int64_t*)malloc(sizeof(int64_t) * n);
  if (!starts) return -1;
  for (int32_t i = 0; i < n_blocks; ++i) {
    if (blocks[i] < 0 || blocks[i] >= pool_blocks) { free(starts); return -1; }
    for (int32_t l = 0; l < n_layers; ++l) {
      const int64_t page = layout == MLA_LAYOUT_BLOCK_MAJOR ? (int64_t)blocks[i] * n_layers + l
                                                             : (int64_t)l * pool_blocks + blocks[i];
      starts[(int64_t)i * n_layers + l] = page * page_bytes;
    }
  }
  qsort(starts, (size_t)n, sizeof(int64_t), [](const void* x, const void* y) {
    const int64_t a = *(const int64_t*)x, b = *(const int64_t*)y;
    return (a > b) - (a < b);
  });
  int64_t regions = 0, end = -1;
  for (int64_t k = 0; k < n; ++k) {
    if (starts[k] != end) ++regions;        // a page that does not continue the previous range
    end = starts[k] + page_bytes;
  }
  free(starts);
  return regions;
}

size_t mla_topk_workspace_size(int32_t num_tokens, int64_t n_max, int32_t k) {
  if (num_tokens < 1 || n_max < 1 || k < 1) return 0;
  return mla::topk_ws_bytes(num_tokens, n_max, k);
}

mla_status mla_topk_indices(const float* scores, int64_t n_max, const int32_t* seq_lens, int32_t B,
                            int32_t q_len, int32_t k, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!scores || !seq_lens || !out_idx) return fail(MLA_ERR_INVALID_ARG, "null scores / seq_lens / out_idx");
  if (B < 1 || q_len < 1) return fail(MLA_ERR_INVALID_ARG, "B and q_len must be >= 1");
  if (k < 1 || k > mla::kTopkMaxK) return fail(MLA_ERR_UNSUPPORTED, "k %d outside [1, %d]", k, mla::kTopkMaxK);
  if (n_max < 1 || n_max > mla::kTopkMaxN)
    return fail(MLA_ERR_UNSUPPORTED, "n_max %lld outside [1, %lld]", (long long)n_max,
                (long long)mla::kTopkMaxN);
  const int64_t T = (int64_t)B * q_len;
  if (T > (int64_t)1 << 20) return fail(MLA_ERR_INVALID_ARG, "too many query tokens");
  if (!aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(out_idx, 4))
    return fail(MLA_ERR_INVALID_ARG, "misaligned scores / seq_lens / out_idx");
  const size_t need = mla::topk_ws_bytes(T, n_max, k);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed", need);
  return hip_status(mla::launch_topk(scores, n_max, seq_lens, (int32_t)T, q_len, k, workspace,
                                     out_idx, stream),
                    "topk launch");
}

mla_status mla_indexer_scores(const void* q_fp8, const float* head_weights, const void* k_cache,
                              int64_t page_stride_bytes, int64_t cache_bytes,
                              const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, int32_t B, int32_t q_len, int64_t n_max,
                              float* scores, hipStream_t stream) {
  if (!q_fp8 || !head_weights || !block_table || !seq_lens || !scores)
    return fail(MLA_ERR_INVALID_ARG, "null q_fp8 / head_weights / block_table / seq_lens / scores");
  if (!k_cache) return fail(MLA_ERR_INVALID_ARG, "k_cache is null");
  if (!aligned(k_cache, 16)) return fail(MLA_ERR_INVALID_ARG, "k_cache must be 16-byte aligned");
  if (page_stride_bytes < MLA_INDEXER_PAGE_BYTES || page_stride_bytes % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG, "page_stride_bytes %lld must be >= %d and a multiple of 16",
                (long long)page_stride_bytes, MLA_INDEXER_PAGE_BYTES);
  if (cache_bytes < MLA_INDEXER_PAGE_BYTES || cache_bytes > kMaxCacheBytes)
    return fail(MLA_ERR_INVALID_ARG, "cache_bytes %lld out of range", (long long)cache_bytes);
  if (B < 1 || B > 65535 || q_len < 1) return fail(MLA_ERR_INVALID_ARG, "B must be in [1, 65535], q_len >= 1");
  if (max_pages < 1) return fail(MLA_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (n_max < 1 || n_max > mla::kTopkMaxN)
    return fail(MLA_ERR_INVALID_ARG, "n_max %lld outside [1, %lld]", (long long)n_max, (long long)mla::kTopkMaxN);
  if ((int64_t)B * q_len > (int64_t)1 << 20) return fail(MLA_ERR_INVALID_ARG, "too many query tokens");
  if (!aligned(q_fp8, 16) || !aligned(head_weights, 16))
    return fail(MLA_ERR_INVALID_ARG, "q_fp8 and head_weights must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(scores, 4))
    return fail(MLA_ERR_INVALID_ARG, "misaligned block_table / seq_lens / scores");
  mla::IndexerArgs a;
  a.q = (const uint8_t*)q_fp8;
  a.weights = head_weights;
  a.cache = (const uint8_t*)k_cache;
  a.page_stride = page_stride_bytes;
  a.cache_bytes = cache_bytes;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.B = B;
  a.q_len = q_len;
  a.n_max = n_max;
  a.scores = scores;
  return hip_status(mla::launch_indexer(a, stream), "indexer launch");
}

mla_status mla_nvfp4_dequantize_rows(const void* kv_cache, int64_t page_stride_bytes,
                                     int64_t cache_bytes, const int64_t* slots, int64_t n,
                                     float* out, hipStream_t stream) {
  mla_status st = check_cache(kv_cache, page_stride_bytes, cache_bytes);
  if (st != MLA_OK) return st;
  if (n < 0) return fail(MLA_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return hip_status(hipSuccess, "");
  if (!slots || !out) return fail(MLA_ERR_INVALID_ARG, "null slots / out");
  if (!aligned(slots, 8) || !aligned(out, 4)) return fail(MLA_ERR_INVALID_ARG, "misaligned slots / out");
  return hip_status(mla::launch_dequantize_rows(kv_cache, page_stride_bytes, cache_bytes, slots, n,
                                                out, stream),
                    "dequantize_rows launch");
}

}  // extern "C"

// ---- allocation-free sparse decode -----------------------------------------------------------
// For callers that cannot call hipMalloc (code under HIP graph capture, tight serving loops,
// harnesses that forbid it). The split partials that mla_sparse_decode keeps in a caller-provided
// workspace live here in `scratch`, a file-scope device array of kNoallocScratchBytes. Each GPU
// the library runs on holds its own copy, at its own address, until the process ends; that
// address is looked up once per device with hipGetSymbolAddress (in host code the array's name
// is only a host-side stand-in) and kept. Every call on a GPU shares that GPU's array, so calls
// that overlap on one GPU (two streams, two host threads) race on it. The decode kernels write
// every partial they later read, so nothing in the array has to start at zero.
namespace {

constexpr size_t kNoallocScratchBytes = size_t(32) << 20;    // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first call on the device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t mla_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

mla_status mla_sparse_decode_noalloc(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                     int64_t page_stride_bytes, int64_t cache_bytes,
                                     const int32_t* block_table, int32_t max_pages,
                                     const int32_t* topk_idx, int32_t topk, int32_t B,
                                     int32_t q_len, int32_t H, float softmax_scale,
                                     int32_t num_splits, float* out, float* lse,
                                     hipStream_t stream) {
  size_t need = 0;
  if (B >= 1 && q_len >= 1 && H >= 16 && num_splits >= 1 && (int64_t)B * q_len <= INT32_MAX) {
    need = ws_bytes((int64_t)B * q_len, H, num_splits);
    if (need > kNoallocScratchBytes)
      return fail(MLA_ERR_WORKSPACE,
                  "the allocation-free decode keeps its split partials in a %zu-byte scratch "
                  "array; this call needs %zu bytes (fewer splits or query tokens per call)",
                  kNoallocScratchBytes, need);
  }
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch address (hipGetSymbolAddress)");
  }
  // invalid shapes fall through to mla_sparse_decode's own argument checks
  return mla_sparse_decode(q, q_dtype, kv_cache, page_stride_bytes, cache_bytes, block_table,
                           max_pages, topk_idx, topk, B, q_len, H, softmax_scale, num_splits, out,
                           lse, ws, need > 0 ? kNoallocScratchBytes : 0, stream);
}

}  // extern "C"
