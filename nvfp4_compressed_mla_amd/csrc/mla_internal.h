// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace mla {

// Arguments of the fused decode kernel (one struct, passed by value).
struct DecodeArgs {
  const void* q;            // [T, H, 576] bf16 or fp32, T = B*q_len
  int32_t q_fp32;
  const uint8_t* cache;
  int64_t page_stride;      // bytes
  int64_t cache_bytes;
  const int32_t* block_table;   // [B, max_pages]
  int32_t max_pages;
  const int32_t* seq_lens;      // [B] (dense)
  const int32_t* topk_idx;      // [T, topk] (sparse)
  int32_t topk;
  int32_t B, q_len, H;
  float scale_log2;         // softmax_scale * log2(e)
  int32_t n_split;          // row splits per (token, head group)
  int32_t split_rows;       // list entries (sparse) or positions (dense) per split, multiple of 64
  int32_t head_begin;       // first head handled by this launch
  int32_t n_hg;             // head groups (of 16*nh heads) handled by this launch
  int32_t total_items;      // T * n_hg * n_split
  int32_t items_per_xcd;    // ceil(total_items / 8)
  float* out;               // [T, H, 512] (n_split == 1)
  float* lse;               // [T, H] or null (n_split == 1)
  _Float16* ws_o;           // [T, n_split, H/16, 16, 64, 2, 4] FP16 partial outputs (n_split > 1)
  float* ws_lse;            // [T, n_split, H] partial log-sum-exp (log2 units)
  // Shared-row mode (the rows selected by a group of up to 4 consecutive query tokens of one
  // request, deduplicated): workgroup = (group, 16-head block, split), head block u of the
  // workgroup = token 4g+u of the group.
  const int32_t* u_pos;     // [n_groups, kUnionParts, u_stride] union positions, ascending
  const uint8_t* u_mask;    // same layout; bit u: token 4g+u selected the position
  const int32_t* u_count;   // [n_groups, kUnionParts] entries of each part
  int32_t u_stride;
  int32_t groups_per_req;   // ceil(q_len / 4)
  // Fused append (sparse NVFP4 rows only; ap_slots != null selects it): every workgroup of a
  // request encodes the request's q_len new rows (row b*q_len + t: bf16 latent and rope, cache
  // slot) and writes them to their cache slots before its first gather.
  const uint16_t* ap_latent;    // [T, ap_latent_stride] bf16
  int64_t ap_latent_stride;
  const uint16_t* ap_rope;      // [T, ap_rope_stride] bf16
  int64_t ap_rope_stride;
  const int64_t* ap_slots;      // [T] flat cache slots (page * 64 + row), -1 = not written
  uint8_t* ap_cache;            // the cache (written)
};

constexpr int kApMaxRows = 16;                                  // q_len limit of the fused append

constexpr int kMaxSplitRows = 2048;   // sparse rows per split held in LDS
constexpr int kMaxDensePages = 128;   // dense pages per split held in LDS (8192 positions)

hipError_t launch_quantize_append(const void* latent, int64_t latent_stride, const void* rope,
                                  int64_t rope_stride, const int64_t* slots, int64_t n_rows,
                                  void* cache, int64_t page_stride, int64_t cache_bytes,
                                  hipStream_t stream);

hipError_t launch_dequantize_rows(const void* cache, int64_t page_stride, int64_t cache_bytes,
                                  const int64_t* slots, int64_t n, float* out, hipStream_t stream);

// nh = heads per workgroup / 16 (1..4); dense selects implicit positions; fp8 selects 576-byte
// FP8 rows instead of 352-byte NVFP4 rows. ev_start / ev_stop (may be null) are recorded at the
// kernel's start and end.
hipError_t launch_decode(const DecodeArgs& a, int nh, bool dense, bool fp8, hipStream_t stream,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Shared-row decode (NVFP4 rows, 4 tokens x 16 heads per workgroup) over the unions built by
// launch_union.
hipError_t launch_decode_shared(const DecodeArgs& a, hipStream_t stream,
                                hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Union of the index lists of each group of up to 4 consecutive query tokens of a request:
// ascending distinct positions in [0, n_pos) and their 4-bit token masks, in kUnionParts parts
// (equal position ranges) of u_stride entries each, u_count[group * kUnionParts + part] entries
// used. n_pos <= kUnionMaxPos, topk <= kUnionMaxTopk.
constexpr int kUnionMaxPos = 1 << 20;
constexpr int kUnionParts = 16;
constexpr int kUnionMaxTopk = 2048;
hipError_t launch_union(const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                        int32_t n_pos, int32_t* u_pos, uint8_t* u_mask, int32_t* u_count,
                        int32_t u_stride, hipStream_t stream);

hipError_t launch_fp8_append(const void* latent, int64_t latent_stride, const void* rope,
                             int64_t rope_stride, const int64_t* slots, int64_t n_rows, void* cache,
                             int64_t page_stride, int64_t cache_bytes, hipStream_t stream);

// Staged NVFP4 -> FP8 rows of the selected entries: staged [T, ceil64(topk), 576] bytes,
// staged_idx int32 [T, topk], staged_bt int32 [T, ceil64(topk)/64].
hipError_t launch_stage_fp8(const void* cache, int64_t page_stride, int64_t cache_bytes,
                            const int32_t* block_table, int32_t max_pages, const int32_t* topk_idx,
                            int32_t topk, int32_t T, int32_t q_len, void* staged,
                            int32_t* staged_idx, int32_t* staged_bt, hipStream_t stream);

hipError_t launch_combine(int32_t T, int32_t H, int32_t n_split, const _Float16* ws_o,
                          const float* ws_lse, float* out, float* lse, hipStream_t stream);

// Pages of n_blocks blocks (all layers) from one multi-layer pool to another; layout 0 =
// block-major, 1 = layer-major.
hipError_t launch_copy_pages(const void* src, int64_t src_pool_blocks, void* dst,
                             int64_t dst_pool_blocks, int32_t layout, int32_t n_layers,
                             int64_t page_bytes, const int32_t* src_blocks,
                             const int32_t* dst_blocks, int32_t n_blocks, hipStream_t stream);

// Top-k position selection (scores fp32 [T, n_max], T = B*q_len, k <= kTopkMaxK). A token's
// positions are cut into n_slices slices of `slice` positions (one filter workgroup each, eight
// wave segments of slice / 8); each segment lists at most cap_seg candidates.
constexpr int kTopkMaxK = 2048;
constexpr int64_t kTopkMaxN = 1 << 20;
constexpr int kTopkTakeAll = 8192;            // rows this short are selected directly in LDS
constexpr int kTopkCandCap = 8192;            // candidates the merge holds in LDS
constexpr int kTopkSample = 2048;             // sample size of the cut
constexpr int kTopkMaxSlices = 16;
struct TopkPlan {
  int64_t slice;
  int32_t n_slices;
  int32_t cap_seg;
};
inline TopkPlan topk_plan(int64_t T, int64_t n_max) {
  // at most 512 filter workgroups (two per compute unit: one round), at most 16 per token
  const int64_t g = std::min<int64_t>(kTopkMaxSlices, std::max<int64_t>(1, 512 / T));
  TopkPlan p;
  p.slice = (((n_max + g - 1) / g) + 2047) / 2048 * 2048;
  p.n_slices = (int32_t)((n_max + p.slice - 1) / p.slice);
  p.cap_seg = (int32_t)std::min<int64_t>(p.slice / 8, std::min<int64_t>(4096, std::max<int64_t>(256, 32768 / (8 * p.n_slices))));
  return p;
}
inline size_t topk_ws_bytes(int64_t T, int64_t n_max, int64_t /*k*/) {
  const TopkPlan p = topk_plan(T, n_max);
  const int64_t segs = T * p.n_slices * 8;
  return (size_t)(segs * p.cap_seg * 8 + segs * 4);
}
hipError_t launch_topk(const float* scores, int64_t n_max, const int32_t* seq_lens, int32_t T,
                       int32_t q_len, int32_t k, void* workspace, int32_t* out, hipStream_t stream);

// Indexer scoring pass (FP8 scores of every visible position, the input of top-k selection).
constexpr int kIndexerHeads = 64;
constexpr int kIndexerDim = 128;
constexpr int kIndexerPageBytes = 64 * kIndexerDim + 64 * 4;   // 64 E4M3 keys, 64 fp32 scales
struct IndexerArgs {
  const uint8_t* q;            // [T, 64, 128] E4M3 indexer queries, T = B*q_len
  const float* weights;        // [T, 64] head weights
  const uint8_t* cache;        // indexer pages
  int64_t page_stride;         // bytes
  int64_t cache_bytes;
  const int32_t* block_table;  // [B, max_pages]
  int32_t max_pages;
  const int32_t* seq_lens;     // [B]
  int32_t B, q_len;
  int64_t n_max;
  float* scores;               // [T, n_max]; visible positions written
  int32_t block_rows;          // positions per workgroup (set by launch_indexer)
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream);

}  // namespace mla
