/*
 * mla_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4-compressed sparse-MLA decode library.
 *
 * What the library computes follows the page "Prime Inference: Fast, Reliable Serving for
 * Frontier Open Models" (Prime Intellect):
 *   - section "Making room for low-latency decode": each MLA cache row stores the 512-value
 *     latent as 4-bit E2M1 values with one FP8 (E4M3) scale per 16 values, and the 64-value rope
 *     part as FP8: 352 bytes per row instead of 576;
 *   - section "Native NVFP4 sparse MLA decode kernel": decode attention reads the rows selected
 *     by the sparse indexer, unpacks them on chip (no intermediate buffer in device memory), and
 *     computes with FP16 operands and FP32 accumulation; one query token's rows are split across
 *     cooperating workgroups whose partial results are merged; entries of -1 in the 2048-entry
 *     index list are empty and are not loaded;
 *   - section "Changing the layout to reduce fragmentation": the cache is paged in 64-token
 *     blocks; a page may belong to a block-major multi-layer layout, hence the page byte stride.
 *
 * Row layout (352 bytes): bytes [0,256) element codes, element 2k in the low nibble of byte k;
 * bytes [256,288) the E4M3 scale of group g (elements 16g..16g+15); bytes [288,352) the E4M3 rope
 * values. Scale = E4M3(amax/6) rounded to nearest even and saturated at 448; element code =
 * nearest E2M1 value of x/scale, ties to the even code, saturated at 6; a zero scale zeroes the
 * magnitudes and keeps the signs.
 *
 * Addressing: physical slot p = page*64 + offset lives at byte page*page_stride_bytes +
 * offset*352. Logical position j of request b lives at slot block_table[b*max_pages + j/64]*64 +
 * j%64.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library never frees,
 *     allocates persistent memory, or synchronizes the stream. All work is enqueued on `stream`.
 *   - Argument errors (null pointers, unsupported shapes, misalignment, a too-small workspace)
 *     are detected on the host before any HIP call and returned as MLA_ERR_INVALID_ARG /
 *     MLA_ERR_UNSUPPORTED / MLA_ERR_WORKSPACE; nothing is enqueued in that case.
 *   - A failing kernel launch returns MLA_ERR_HIP. mla_last_error() gives a per-thread text.
 *   - Content (index values, page ids, slots) is the caller's contract, but kernels never read or
 *     write outside [kv_cache, kv_cache + cache_bytes): a row that would fall outside, a page id
 *     that is negative, or a position beyond the block table is treated as an empty slot (not
 *     loaded / not written).
 *   - Inputs must be finite; queries must be representable in FP16 (|q| < 65504), since the
 *     contractions use FP16 operands.
 */
#ifndef MLA_NVFP4_H
#define MLA_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE = 3,
  MLA_ERR_HIP = 4
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_FP32 = 1 } mla_dtype;

#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_ROW_BYTES 352
#define MLA_PAGE_ROWS 64
#define MLA_MAX_TOPK 2048
#define MLA_FP8_ROW_BYTES 576
#define MLA_INDEXER_HEADS 64
#define MLA_INDEXER_DIM 128
#define MLA_INDEXER_PAGE_BYTES 8448   /* 64 E4M3 keys of 128 bytes, then 64 fp32 scales */

/* Quantize-on-append (page section "Making room for low-latency decode": the latent is stored
 * as NVFP4, the rope part as FP8).
 *   latent        bf16 [n_rows, 512], row i at latent + i*latent_row_stride elements.
 *   rope          bf16 [n_rows, 64],  row i at rope + i*rope_row_stride elements.
 *   slot_mapping  int64 [n_rows]: destination physical slot of row i; -1 = skip the row.
 *   kv_cache      byte buffer of cache_bytes bytes; page_stride_bytes >= 64*352 and a multiple
 *                 of 16; kv_cache 16-byte aligned.
 * Writes exactly the 352 bytes of each non-skipped row. n_rows == 0 is a no-op. Rows whose slot
 * falls outside the cache are not written. Two rows with the same slot race (last writer wins). */
mla_status mla_nvfp4_quantize_append(const void* latent, int64_t latent_row_stride,
                                     const void* rope, int64_t rope_row_stride,
                                     const int64_t* slot_mapping, int64_t n_rows,
                                     void* kv_cache, int64_t page_stride_bytes,
                                     int64_t cache_bytes, hipStream_t stream);

/* Bytes of workspace mla_sparse_decode / mla_dense_decode need for `num_splits` row splits of
 * `num_tokens` (= B*q_len) query tokens with H heads: num_tokens*num_splits*H*(512*2 + 4) rounded
 * up to 256 (each split keeps its normalised partial output in FP16 and its log-sum-exp in FP32;
 * the merge runs in FP32). Zero when num_splits <= 1 (no partials are kept). */
size_t mla_decode_workspace_size(int32_t num_tokens, int32_t H, int32_t num_splits);

/* Number of row splits mla_sparse_decode will use for this shape when `max_splits` = 0 (auto,
 * sized so that the launch covers one wave of the 256 compute units), or min(max_splits, topk/64)
 * otherwise (each split keeps at least 64 list entries). The caller sizes the workspace with this number. */
int32_t mla_sparse_decode_num_splits(int32_t num_tokens, int32_t H, int32_t topk,
                                     int32_t max_splits);

/* Number of row splits mla_dense_decode uses: ceil(max_pages*64 / split_tokens). */
int32_t mla_dense_decode_num_splits(int32_t max_pages, int32_t split_tokens);

/* A split size for mla_dense_decode that puts the whole launch in one wave of workgroups: the
 * largest split count s with num_tokens * ceil(H/64) * s <= 256 (one workgroup per compute
 * unit), then split_tokens = ceil(max_pages*64 / s) rounded up to a multiple of 64 and clamped
 * to [64, 8192]. Returns 4096 for invalid arguments. (A fixed 4096-token split can leave a short
 * second wave: 8 tokens x 37 splits = 296 workgroups at 149,504 positions.) */
int32_t mla_dense_decode_split_tokens(int32_t num_tokens, int32_t H, int32_t max_pages);

/* Sparse decode (page section "Native NVFP4 sparse MLA decode kernel").
 *   q          [B, q_len, H, 576] contiguous, bf16 or fp32 (q_dtype): absorbed queries, latent
 *              part first (512), rope part last (64).
 *   kv_cache   cache_bytes bytes of 352-byte rows in 64-row pages of page_stride_bytes.
 *   block_table int32 [B, max_pages] physical page ids.
 *   topk_idx   int32 [B, q_len, topk]: logical positions selected for each query token, shared
 *              by all heads; -1 marks an empty entry, anywhere in the list. 1 <= topk <= 2048.
 *   H          multiple of 16 (heads are processed in groups of up to 64).
 *   softmax_scale  scores are softmax_scale * (q . [latent; rope]).
 *   out        fp32 [B, q_len, H, 512]: softmax-weighted sum of the selected latents.
 *   lse        fp32 [B, q_len, H] natural-log sum of exp(scores), or NULL. A token whose list is
 *              empty gets out = 0 and lse = -inf.
 *   num_splits row splits per token (from mla_sparse_decode_num_splits); > 1 needs a workspace
 *              of mla_decode_workspace_size(B*q_len, H, num_splits) bytes, 256-byte aligned.
 * Results are deterministic: partials are merged in split order. */
mla_status mla_sparse_decode(const void* q, mla_dtype q_dtype,
                             const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* topk_idx, int32_t topk,
                             int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                             int32_t num_splits, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Quantize-append fused into the sparse decode (page section "Making room for low-latency
 * decode": the new latent rows are stored as NVFP4; section "Native NVFP4 sparse MLA decode
 * kernel": the decode reads the selected rows, which in a decode step include the rows the step
 * itself appends). One call does what mla_nvfp4_quantize_append(latent, rope, slot_mapping,
 * B*q_len) followed by mla_sparse_decode(...) does, in one decode launch (plus the split merge):
 *   latent, rope, latent_row_stride, rope_row_stride   as mla_nvfp4_quantize_append, with
 *              B*q_len rows: row b*q_len + t is the new row of query token t of request b;
 *   slot_mapping int64 [B*q_len] its physical slot; -1 = not appended;
 *   kv_cache   written: each appended row's 352 bytes, as mla_nvfp4_quantize_append writes them
 *              (the same encoder); every other argument, the workspace included, as
 *              mla_sparse_decode.
 * Every decode workgroup of request b encodes that request's q_len new rows and stores them to
 * their slots before it gathers any row, so whatever it reads of those rows is the new bytes
 * (other workgroups store the same bytes at the same time).
 * Requirements beyond mla_sparse_decode's: q_len <= 16; the slots of one call are distinct; no
 * request's list resolves to a row appended for another request in the same call (such an entry
 * may read the row before or after the append). */
mla_status mla_sparse_decode_append(const void* q, mla_dtype q_dtype, void* kv_cache,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                                    int32_t H, float softmax_scale, int32_t num_splits,
                                    const void* latent, int64_t latent_row_stride,
                                    const void* rope, int64_t rope_row_stride,
                                    const int64_t* slot_mapping, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sparse decode with rows shared across query tokens (page section "Native NVFP4 sparse MLA
 * decode kernel": a launch carries several query tokens of a request, 15 in the page's figure).
 * Same arguments and result as mla_sparse_decode; the work is split differently: the lists of
 * each group of up to 4 consecutive query tokens of a request are merged into their union
 * (distinct positions, ascending, with a 4-bit mask of the tokens that selected each), and one
 * workgroup serves 16 heads of each of the group's tokens over that union, gathering and
 * decoding each distinct row once and masking, per token, the rows it did not select. Pays when
 * the tokens' lists overlap (the union is much shorter than the lists together) and the
 * per-token launch is compute-bound, e.g. 16 heads per token; at 64 heads every tile already
 * serves 64 query rows, and the plain entry point is faster.
 * Requirements beyond mla_sparse_decode's: max_pages*64 <= 1,048,576 (the union is built over
 * the request's positions in on-chip memory, in 16 position ranges), and no position twice in one
 * token's list (a repeated position counts once here, twice in mla_sparse_decode).
 *   workspace  mla_shared_decode_workspace_size(B, q_len, H, topk) bytes, 256-byte aligned:
 *              union lists, masks and sizes, then the split partials.
 * Launches: the union pass, the decode, then the split merge when
 * mla_shared_decode_num_splits(...) > 1. Deterministic. */
size_t mla_shared_decode_workspace_size(int32_t B, int32_t q_len, int32_t H, int32_t topk);
int32_t mla_shared_decode_num_splits(int32_t B, int32_t q_len, int32_t H, int32_t topk);
mla_status mla_sparse_decode_shared(const void* q, mla_dtype q_dtype, const void* kv_cache,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                                    int32_t H, float softmax_scale, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense decode over the whole cache of each request (no indexer): query token t of request b
 * attends to logical positions 0 .. seq_lens[b]-q_len+t (causal inside the step), split into
 * chunks of split_tokens positions (a multiple of 64, at most 8192) merged by log-sum-exp.
 *   seq_lens   int32 [B] device array; values above max_pages*64 are clamped.
 *   Other arguments as mla_sparse_decode; num_splits from mla_dense_decode_num_splits. */
mla_status mla_dense_decode(const void* q, mla_dtype q_dtype,
                            const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                            const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                            int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                            int32_t split_tokens, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free sparse decode, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Arguments, results
 * and num_splits as mla_sparse_decode; the split partials live in a library-owned device array of
 * mla_noalloc_scratch_bytes() bytes (32 MiB), one per GPU, held until the process ends. The call
 * allocates nothing. It returns MLA_ERR_WORKSPACE when mla_decode_workspace_size(B*q_len, H,
 * num_splits) exceeds that size (the library's own split choice needs at most about 17 MB).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two streams or
 * two host threads) race and must not be issued. */
size_t mla_noalloc_scratch_bytes(void);
mla_status mla_sparse_decode_noalloc(const void* q, mla_dtype q_dtype,
                                     const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                                     const int32_t* block_table, int32_t max_pages,
                                     const int32_t* topk_idx, int32_t topk,
                                     int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                                     int32_t num_splits, float* out, float* lse, hipStream_t stream);

/* ---- FP8 baseline and the staged path ------------------------------------------------------
 * Page section "Making room for low-latency decode": before the NVFP4 change a row held the 512
 * latent and the 64 rope values as FP8, 576 bytes. Section "Native NVFP4 sparse MLA decode
 * kernel" compares the fused NVFP4 kernel with the FP8 kernel on such rows and with a staged path
 * that first unpacks the selected NVFP4 rows into a temporary FP8 buffer, then runs the FP8
 * kernel. FP8 row layout (576 bytes): latent element i at byte i, rope element j at byte 512+j,
 * each the nearest E4M3 value (ties to even, saturated at 448, unit scale). Addressing as for the
 * NVFP4 cache with 576 in place of 352; page_stride_bytes >= 64*576. */

/* Append FP8 rows; arguments and behaviour as mla_nvfp4_quantize_append. */
mla_status mla_fp8_append(const void* latent, int64_t latent_row_stride,
                          const void* rope, int64_t rope_row_stride,
                          const int64_t* slot_mapping, int64_t n_rows,
                          void* kv_cache, int64_t page_stride_bytes,
                          int64_t cache_bytes, hipStream_t stream);

/* Sparse / dense decode over an FP8 cache: arguments, splits, workspace and results as
 * mla_sparse_decode / mla_dense_decode (the same fused kernel with 576-byte rows converted to
 * FP16 operands instead of 352-byte NVFP4 rows). */
mla_status mla_fp8_sparse_decode(const void* q, mla_dtype q_dtype,
                                 const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* topk_idx, int32_t topk,
                                 int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                                 int32_t num_splits, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

mla_status mla_fp8_dense_decode(const void* q, mla_dtype q_dtype,
                                const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                                const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                                int32_t split_tokens, int32_t num_splits, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Staging pass of the staged path: for every query token tok = b*q_len + t and list entry e,
 * the NVFP4 row topk_idx[tok][e] of request b is converted to a 576-byte FP8 row (each element's
 * exact NVFP4 value rounded to E4M3, ties to even, saturated at 448; rope bytes copied) and
 * written at staged_rows + (tok*P + e)*576, P = topk rounded up to a multiple of 64;
 * staged_idx[tok][e] = e, or -1 for an empty entry (-1, or a position whose row is outside the
 * table or the cache, as the decode kernels treat it); staged_block_table[tok][p] = tok*P/64 + p.
 * The FP8 kernel then reads token tok as request tok of a cache with pages of 64*576 bytes.
 *   staged_rows  B*q_len*P*576 bytes, 16-byte aligned (rows of empty entries are not written).
 *   staged_idx   int32 [B*q_len, topk];  staged_block_table  int32 [B*q_len, P/64]. */
mla_status mla_nvfp4_stage_fp8(const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                               const int32_t* block_table, int32_t max_pages,
                               const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                               void* staged_rows, int32_t* staged_idx, int32_t* staged_block_table,
                               hipStream_t stream);

/* Workspace bytes of mla_staged_sparse_decode: staged rows, staged index list and block table,
 * and the decode partials of `num_splits` splits, each part 256-byte aligned. */
size_t mla_staged_workspace_size(int32_t num_tokens, int32_t H, int32_t topk, int32_t num_splits);

/* The staged path: mla_nvfp4_stage_fp8 into the workspace, then mla_fp8_sparse_decode over the
 * staged rows. Arguments as mla_sparse_decode over the NVFP4 cache; the workspace (always needed)
 * comes from mla_staged_workspace_size. */
mla_status mla_staged_sparse_decode(const void* q, mla_dtype q_dtype,
                                    const void* kv_cache, int64_t page_stride_bytes, int64_t cache_bytes,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* topk_idx, int32_t topk,
                                    int32_t B, int32_t q_len, int32_t H, float softmax_scale,
                                    int32_t num_splits, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Multi-layer page pools and block transfer --------------------------------------------
 * Page section "Changing the layout to reduce fragmentation": a layer-major pool (LBHNC) stores
 * each layer's pages on their own, so a 64-token block spans one region per layer; a block-major
 * pool (BLHNC) keeps the pages of all layers of a block side by side. A pool holds pool_blocks
 * blocks x n_layers pages of page_bytes bytes (64 * 352 for one layer of NVFP4 rows):
 *   block-major: page (b, l) at byte (b * n_layers + l) * page_bytes;
 *   layer-major: page (b, l) at byte (l * pool_blocks + b) * page_bytes.
 * Layer l of a block-major pool is the paged cache at pool + l * page_bytes with
 * page_stride_bytes = n_layers * page_bytes (layer-major: pool + l * pool_blocks * page_bytes,
 * page_stride_bytes = page_bytes), as the decode entry points take it. */
typedef enum { MLA_LAYOUT_BLOCK_MAJOR = 0, MLA_LAYOUT_LAYER_MAJOR = 1 } mla_kv_layout;

/* Copy every layer's page of block src_blocks[i] of src_pool to block dst_blocks[i] of dst_pool,
 * for i < n_blocks, in one launch. Both pools have the given layout; their block counts are
 * pool_bytes / (n_layers * page_bytes) (the sizes must be whole multiples). src_blocks and
 * dst_blocks are int32 device arrays; a block id outside its pool skips that pair. Pools 16-byte
 * aligned, page_bytes a multiple of 16. Overlapping source and destination pages race. */
mla_status mla_copy_kv_blocks(const void* src_pool, int64_t src_pool_bytes,
                              void* dst_pool, int64_t dst_pool_bytes,
                              mla_kv_layout layout, int32_t n_layers, int64_t page_bytes,
                              const int32_t* src_blocks, const int32_t* dst_blocks,
                              int32_t n_blocks, hipStream_t stream);

/* Host helper: the number of contiguous byte ranges (transfer descriptors) that cover all pages
 * of the given blocks (int32 HOST array) in a pool of pool_blocks blocks, touching ranges merged.
 * Returns -1 for invalid arguments or a block id outside the pool. */
int64_t mla_kv_transfer_regions(mla_kv_layout layout, int32_t n_layers, int64_t page_bytes,
                                int64_t pool_blocks, const int32_t* blocks, int32_t n_blocks);

/* ---- Top-k position selection (the indexer step before the path) ------------------------------
 * Page section "Native NVFP4 sparse MLA decode kernel": the sparse indexer picks, for each query
 * token, the positions attention reads (2048 per token); unused list entries are -1. The page
 * does not define the indexer's scores; they are an input here.
 *   scores   fp32 [B, q_len, n_max] device array: score of every position for every query token.
 *   seq_lens int32 [B] device array; token t of request b may pick positions
 *            0 .. seq_lens[b] - q_len + t (clamped to [0, n_max)).
 *   out_idx  int32 [B, q_len, k]: the k positions with the largest scores, in ascending order,
 *            then -1 when fewer than k positions are visible. Scores are ordered by the IEEE-754
 *            total order of the float32 value (-0 below +0), equal scores by position (smaller
 *            first); they must be finite. 1 <= k <= 2048, 1 <= n_max <= 1,048,576.
 *   workspace mla_topk_workspace_size(B*q_len, n_max, k) bytes, 256-byte aligned (candidate
 *            lists of the position segments, about 256 KiB per token at most).
 * The result is exact and deterministic: the same list for the same scores. */
size_t mla_topk_workspace_size(int32_t num_tokens, int64_t n_max, int32_t k);

mla_status mla_topk_indices(const float* scores, int64_t n_max, const int32_t* seq_lens,
                            int32_t B, int32_t q_len, int32_t k, int32_t* out_idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Indexer scores (the FP8 scoring pass that top-k selects from) ------------------------------
 * Page section "Native NVFP4 sparse MLA decode kernel": attention reads the positions a sparse
 * indexer selected; section "Making room for low-latency decode" keeps the indexer's cache beside
 * the MLA rows. The page does not define the indexer's scores. This library's reading (synthetic
 * inputs, no trained weights): position s holds a 128-dim E4M3 key k_s and a positive fp32 scale
 * c_s; query token t has 64 E4M3 heads q_{t,j} and fp32 head weights w_{t,j};
 *     scores[t, s] = c_s * sum_j w_{t,j} * max(0, q_{t,j} . k_s)
 * accumulated in fp32 (E4M3 products are exact).
 *   q_fp8        E4M3 bytes [B, q_len, 64, 128], 16-byte aligned.
 *   head_weights fp32 [B, q_len, 64], 16-byte aligned.
 *   k_cache      indexer pages: page p at k_cache + p*page_stride_bytes holds the keys of its 64
 *                positions (128 bytes each) and then their 64 fp32 scales; page_stride_bytes >=
 *                MLA_INDEXER_PAGE_BYTES, a multiple of 16; cache_bytes as for the MLA cache.
 *   block_table  int32 [B, max_pages]: position s of request b lives in page block_table[b][s/64]
 *                (the same table as the MLA rows; an unmapped or out-of-cache page scores as 0).
 *   seq_lens     int32 [B]; token t scores positions 0 .. seq_lens[b] - q_len + t (clamped to
 *                n_max and max_pages*64), the window mla_topk_indices selects from.
 *   scores       fp32 [B, q_len, n_max]: those positions are written; the rest are left as they
 *                are. 1 <= n_max <= 1,048,576; B <= 65,535.
 * Errors: MLA_ERR_INVALID_ARG for null or misaligned pointers and sizes out of range (checked on
 * the host, before any launch). */
mla_status mla_indexer_scores(const void* q_fp8, const float* head_weights, const void* k_cache,
                              int64_t page_stride_bytes, int64_t cache_bytes,
                              const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, int32_t B, int32_t q_len, int64_t n_max,
                              float* scores, hipStream_t stream);

/* Test hook, off the hot path: decode the rows at `slots` (int64 [n]) into fp32 [n, 576]
 * (latent then rope), through the same on-chip decoder the attention kernels use. Values are
 * exact. Slots outside the cache produce zeros. */
mla_status mla_nvfp4_dequantize_rows(const void* kv_cache, int64_t page_stride_bytes,
                                     int64_t cache_bytes, const int64_t* slots, int64_t n,
                                     float* out, hipStream_t stream);

/* Profiling hook, off the hot path: when `start`/`stop` are non-null, every later
 * mla_sparse_decode / mla_dense_decode call on this host thread records `start` on its stream
 * at the start of the (first) fused decode kernel and `stop` at the end of the (last) one, before
 * the split-combine kernel (hipExtLaunchKernel's kernel-boundary events), so hipEventElapsedTime
 * gives the fused kernel's own duration. Pass nulls to turn it off. The events are owned by the
 * caller; they must not be recorded inside a graph capture. */
mla_status mla_set_timing_events(hipEvent_t start, hipEvent_t stop);

const char* mla_status_string(mla_status s);
const char* mla_last_error(void);

/* ---- Opt-in content checks (MLA_DEBUG_CHECKS) ------------------------------------------------
 * Index values, page ids, slots and sequence lengths are the caller's contract: the kernels treat
 * a bad entry as an empty slot (nothing loaded or written) and report nothing. With the checks on
 * -- mla_set_debug_checks(1), or the environment variable MLA_DEBUG_CHECKS set to anything but
 * "0" when the library makes its first decision -- every append, decode and staging entry point
 * first copies its index arrays to the host (synchronizing `stream`; not usable under graph
 * capture, where the copy fails with MLA_ERR_HIP) and returns MLA_ERR_INVALID_ARG, with the first
 * offending entry in mla_last_error(), instead of launching when an entry would be skipped:
 *   - a topk_idx entry below -1, at or past max_pages*64, in an unmapped (negative) page, or whose
 *     row [page*page_stride + (j%64)*row_bytes, +row_bytes) is not inside [0, cache_bytes);
 *   - a seq_lens value below 0 or above max_pages*64, or a page among the first ceil(seq_len/64)
 *     that is unmapped or whose used rows fall outside the cache;
 *   - a slot_mapping entry below -1 or whose row falls outside the cache.
 * Off by default: the hot path then neither copies nor synchronizes. */
mla_status mla_set_debug_checks(int32_t enabled);
int32_t mla_debug_checks_enabled(void);

/* The same checks on HOST arrays (no HIP call; usable without a GPU). row_bytes is 352 for NVFP4
 * rows and 576 for FP8 rows. Return MLA_OK or MLA_ERR_INVALID_ARG with mla_last_error() set. */
mla_status mla_check_sparse_indices(const int32_t* topk_idx, int32_t B, int32_t q_len,
                                    int32_t topk, const int32_t* block_table, int32_t max_pages,
                                    int64_t page_stride_bytes, int64_t cache_bytes,
                                    int64_t row_bytes);
mla_status mla_check_dense_tables(const int32_t* seq_lens, int32_t B, int32_t q_len,
                                  const int32_t* block_table, int32_t max_pages,
                                  int64_t page_stride_bytes, int64_t cache_bytes,
                                  int64_t row_bytes);
mla_status mla_check_slots(const int64_t* slots, int64_t n, int64_t page_stride_bytes,
                           int64_t cache_bytes, int64_t row_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MLA_NVFP4_H */
