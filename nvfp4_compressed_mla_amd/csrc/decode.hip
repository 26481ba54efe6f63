// Fused NVFP4 sparse / dense MLA decode for gfx950, plus the split log-sum-exp combine.
//
// Source of the computation: page "Prime Inference: Fast, Reliable Serving for Frontier Open
// Models", section "Native NVFP4 sparse MLA decode kernel": the kernel takes the positions the
// sparse indexer selected, loads the compressed 352-byte rows, unpacks them on chip right before
// use (no intermediate buffer in device memory) and computes attention with FP16 operands and
// FP32 accumulation; a query token's rows are split across cooperating blocks whose partial
// results are merged; -1 entries of the index list are skipped instead of being loaded.
//
// MI355X design (not the page's Blackwell design). On gfx950 an MFMA and a VALU instruction of
// the same wave do not overlap, while those of two waves sharing a SIMD do. The workgroup is
// therefore split by role (per SIMD one math wave and two producer waves), and software-pipelined
// so that each SIMD runs one wave's MFMAs while the other wave's VALU work issues. Rows are
// gathered 32 at a time into a 3-slot LDS ring with direct-to-LDS 16-byte loads, three tiles
// ahead: the producers issue tiles 0..2 in the prologue, the math waves tile i+3 after the
// softmax of tile i.
//  * 4 math waves own one 16-head block each (up to 64 heads per workgroup). QK(i) runs
//    v_mfma_f32_16x16x32_f16 with the decoded rows as the A operand and the block's queries
//    (all 576 dims, FP16, in registers) as B, so each lane holds 8 rows of one head; then the
//    online softmax (FP32, base 2, lazily moved running max) runs in registers and writes FP16
//    probabilities to LDS.
//  * 8 producer waves (two per SIMD) decode tile i+1 once from the ring into FP16 MFMA fragments
//    (VALU, while the math waves run QK(i)), then run PV(i-1) on their 64 output dims for every
//    head (MFMA, while the math waves run softmax(i)); V comes from the decoded tile through
//    ds_read_b64_tr_b16 transposing reads. Empty and out-of-range list entries never reach the
//    ring: the index list is compacted up front, and padding rows read a zero row.
// One barrier per 32-row tile; three decoded-tile buffers and two probability buffers.
//
// Decoded tile layout ("fragment-major"): for row block rb (16 rows) and K-chunk c (32 dims),
// 1 KB holds 64 slots of 16 bytes; row r, dims 8*dg..8*dg+7 of the chunk sit in slot
// 16*dg + (r ^ 4*(dg & 1)). QK fragment reads are then whole 1 KB blocks, and the XOR keeps the
// transposing V reads free of LDS bank conflicts; the QK lanes take the 8-dim groups in the order
// 0, 2, 1, 3, which keeps their reads conflict-free too (measured per access pattern).
//
// Splits write normalised partial outputs (in the producers' register order, 16-byte stores) and
// their log-sum-exp; combine_kernel merges them in split order (deterministic). With a single
// split the kernel writes the final output.
// Workgroup i is placed on XCD i % 8 by the hardware; items are remapped so that the splits of
// one token are consecutive on one XCD and share its L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "codec_device.h"
#include "mla_internal.h"
#include "nvfp4_device.h"

#define LDS_AS __attribute__((address_space(3)))

namespace mla {

typedef short short4v __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 32;
constexpr int kRawTileBytes = kTileRows * kRowBytes;        // 11264
constexpr int kRawPieces = kRawTileBytes / 16;                // 704 16-byte pieces
constexpr int kRawSlots = 3;
constexpr int kChunks = kQkDim / 32;                          // 18 K-chunks of 32 dims
constexpr int kFragBytes = 1024;                              // one 16 x 32 FP16 fragment
constexpr int kDecTileBytes = 2 * kChunks * kFragBytes;       // 36864
constexpr int kPStride = 64;                                  // bytes per head row of P
// P row h holds the tile's 32 probabilities of one head; its four 16-byte columns (8 rows each)
// are stored at column c ^ ((h >> 1) & 3), which keeps the PV reads of P free of LDS bank
// conflicts (measured per access pattern).
__device__ __forceinline__ int p_col(int h, int c) { return 16 * (c ^ ((h >> 1) & 3)); }
constexpr int kThreads = 768;
constexpr uint32_t kInvalid = 0xFFFFFFFFu;

// Source of every load that has no row behind it (padding rows, padding pieces, bad pages).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kFp8RowBytes] = {0};

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS traffic only: unlike __syncthreads() it does not drain the
// direct-to-LDS prefetches of later tiles (their completion is tracked with wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Eight query values times `scale`, rounded to FP16.
__device__ __forceinline__ half8v q_to_half8(const void* q, int64_t off, bool fp32, float scale) {
  float f[8];
  if (fp32) {
    const float4v a = *(const float4v*)((const float*)q + off);
    const float4v b = *(const float4v*)((const float*)q + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
  } else {
    const uint4v u = *(const uint4v*)((const uint16_t*)q + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  half8v h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)(f[i] * scale);
  return h;
}

// Max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48), with the gfx950
// lane-swap instructions (VALU, no LDS round trip).
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float4v mfma16(half8v a, half8v b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Byte offset of (row 0..31 of the tile, K-chunk, 8-dim group dg 0..3) in a decoded tile.
__device__ __forceinline__ int frag_off(int row, int chunk, int dg) {
  const int rb = row >> 4, r = row & 15;
  return (rb * kChunks + chunk) * kFragBytes + (((dg << 4) + (r ^ ((dg & 1) << 2))) << 4);
}

// Direct-to-LDS 16-byte gather: every lane's 16 bytes at `src` land at lds_base + 16*lane.
// Issued as inline assembly so that the compiler does not order later LDS reads of other
// buffers behind it (it cannot tell the target apart); completion is tracked explicitly with
// wait_vmcnt before the barrier that publishes the data.
__device__ __forceinline__ void gather16_to_lds(const void* src, const uint8_t* lds_base) {
  // lds_base is the same for every lane of the wave
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const LDS_AS uint8_t*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ half4v lds_tr16(const uint8_t* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4v*)p);
  return __builtin_bit_cast(half4v, v);
}

constexpr int kDecSlots = 3;
constexpr int kStreamPartialSplits = 8;                       // see the epilogue
constexpr int kProducers = 8;                                 // producer waves (2 per SIMD)

// FP8 selects 576-byte FP8 rows (the baseline format): they need no group scales, so the
// producer waves load their bytes straight into registers two tiles ahead and convert them,
// and the math waves issue no gathers.
// SH (shared rows, NVFP4 sparse with NH = 4 only): the workgroup serves 16 heads of each of up
// to 4 consecutive query tokens of one request over the union of their lists (a.u_pos), so a
// row that several of them selected is gathered and decoded once; head block u belongs to token
// 4g+u and its softmax masks the rows token 4g+u did not select (a.u_mask).
// AP (fused append, NVFP4 sparse): while the producer waves compact the list (and note which of
// the request's new rows its entries resolve to), the math waves load the request's q_len new
// rows. A workgroup whose list reads new rows encodes them with the quantize-append encoder and
// writes them to their cache slots; its stores complete before it gathers those rows, so it
// reads the new bytes. One workgroup per request (token 0, split 0, first head group) encodes
// and writes all of them, which is the append itself. Concurrent stores of several workgroups
// write the same bytes, so no workgroup depends on another.
template <int NH, bool DENSE, bool FP8, bool SH = false, bool AP = false>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const DecodeArgs a) {
  static_assert(!SH || (NH == 4 && !DENSE && !FP8), "shared rows: NVFP4 sparse, 4 tokens");
  static_assert(!AP || (!SH && !DENSE && !FP8), "fused append: NVFP4 sparse");
  constexpr int RB = FP8 ? kFp8RowBytes : kRowBytes;     // bytes per cache row
  __shared__ __attribute__((aligned(16))) uint8_t raw[FP8 ? 1 : kRawSlots][FP8 ? 16 : kRawTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t dec[kDecSlots][kDecTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][NH * 16 * kPStride];
  __shared__ __attribute__((aligned(16))) float alpha_s[2][NH * 16];
  __shared__ __attribute__((aligned(16))) int32_t flag_s[2][4];
  __shared__ uint32_t rowoff[DENSE ? kMaxDensePages : kMaxSplitRows];
  __shared__ __attribute__((aligned(4))) uint8_t rowmask[SH ? kMaxSplitRows : 4];   // SH: token bits
  __shared__ int32_t cnt_s[4][kProducers];
  __shared__ __attribute__((aligned(16))) int32_t ap_hit_s[AP ? kProducers : 4];   // AP: per producer wave
  __shared__ __attribute__((aligned(16))) int32_t ap_early_s[AP ? kProducers : 4];

  // With two or more head blocks the wave index goes through a scalar register, so that what
  // derives from it (role, head block, query and output addresses) is known to be wave-uniform:
  // fewer VALU instructions and VGPRs, batched step 27.67 -> 27.23 us. The one-head-block
  // kernels measured 0.2 us slower that way and keep the plain form.
  const int tid = threadIdx.x, w = NH >= 2 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const bool math = w < 4;
  const int pw = w - 4;                                  // producer wave index (0..7)
  const int ptid = tid - 256;                            // producer thread index (0..511)

  const int hw = blockIdx.x;
  const int item = (hw & 7) * a.items_per_xcd + (hw >> 3);
  if (item >= a.total_items) return;
  const int split = item % a.n_split;
  const int rest = item / a.n_split;
  // SH: item = (group of 4 tokens, 16-head block, split); otherwise (token, head group, split)
  const int head0 = SH ? 16 * (rest % a.n_hg) : a.head_begin + (rest % a.n_hg) * 16 * NH;
  const int grp = rest / a.n_hg;                         // SH: group index
  const int tok = SH ? 0 : rest / a.n_hg;
  const int b = SH ? grp / a.groups_per_req : tok / a.q_len;
  const int t = SH ? 4 * (grp % a.groups_per_req) : tok % a.q_len;   // SH: the group's first token
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  // token, validity and global 16-head block of the workgroup's head block hb
  auto hb_tok = [&](int hb) -> int64_t { return SH ? (int64_t)b * a.q_len + t + hb : tok; };
  auto hb_valid = [&](int hb) -> bool { return !SH || t + hb < a.q_len; };
  auto hb_global = [&](int hb) -> int { return SH ? (head0 >> 4) : (head0 >> 4) + hb; };

  // ---- queries of head block w (math waves) -------------------------------------------------
  const bool qk_wave = math && w < NH && hb_valid(w);
  // QK lane block kg carries 8-dim group kdg of each 32-dim chunk (groups 0, 2, 1, 3): the
  // decoded-tile slots of odd groups are XOR-swizzled for the transposing V reads, and with this
  // order lanes 0-31 read unswizzled slots and lanes 32-63 swizzled ones, which keeps the QK
  // fragment reads free of LDS bank conflicts (with kdg = kg every such read was 2-way). The
  // queries follow the same order, so the contraction is unchanged.
  const int kdg = ((kg & 1) << 1) | (kg >> 1);
  const int64_t qrow = SH ? (hb_tok(qk_wave ? w : 0) * a.H + head0 + l16) * kQkDim + 8 * kdg
                          : ((int64_t)tok * a.H + head0 + 16 * (qk_wave ? w : 0) + l16) * kQkDim + 8 * kdg;
  half8v qf[kChunks];                         // queries as 18 FP16 fragments (math waves)
  // Loaded after the index compaction (their traffic would otherwise slow its dependent loads
  // down), while the producers' first gathers are in flight; converted to FP16 (softmax_scale *
  // log2(e) is applied to the scores).
  auto load_q = [&]() {
    if (!a.q_fp32) {
      uint4v qraw[kChunks];                   // bf16 queries: one 16-byte load per chunk
#pragma unroll
      for (int c = 0; c < kChunks; ++c) qraw[c] = uint4v{0u, 0u, 0u, 0u};
      if (qk_wave) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) qraw[c] = *(const uint4v*)((const uint16_t*)a.q + qrow + 32 * c);
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qf[c][2 * i] = (_Float16)__uint_as_float(qraw[c][i] << 16);
          qf[c][2 * i + 1] = (_Float16)__uint_as_float(qraw[c][i] & 0xFFFF0000u);
        }
    } else {                                  // fp32 queries (small launches)
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        float4v lo = float4v{0.f, 0.f, 0.f, 0.f}, hi = lo;
        if (qk_wave) {
          lo = *(const float4v*)((const float*)a.q + qrow + 32 * c);
          hi = *(const float4v*)((const float*)a.q + qrow + 32 * c + 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) { qf[c][i] = (_Float16)lo[i]; qf[c][4 + i] = (_Float16)hi[i]; }
      }
    }
  };

  // AP: the new rows' inputs, loaded by the math waves during the compaction
  constexpr int kApPasses = AP ? (kApMaxRows / 2 + 3) / 4 : 1;     // row pairs per math wave
  uint4v ap_xa[kApPasses], ap_xb[kApPasses];
  uint32_t ap_ra[kApPasses], ap_rb[kApPasses];
  int64_t ap_sl[kApPasses];

  // ---- rows of this split (producer waves) --------------------------------------------------
  int n_rows = 0;
  int p0 = 0;
  // Dense: every page of the split is mapped and lies wholly inside the cache, so no row needs a
  // validity mask beyond the split's row count (rows of other pages are empty slots: left out of
  // the softmax, as the sparse path's compaction leaves out its invalid entries).
  bool dense_ok = true;
  if constexpr (!DENSE) {
    // Compact the valid entries of [e0, e0 + cnt) into rowoff (16-byte units), in list order:
    // 4 rounds of 512 entries (all index loads first, then all block-table loads), ballot +
    // mbcnt inside a wave, per-wave counts through LDS.
    if (!math) {
      // SH: the group's union is the concatenation of its parts (pre[p] = entries before part
      // p); it is split evenly (whole tiles) across the splits
      int pre[kUnionParts + 1];
      int n_list = a.topk;
      if constexpr (SH) {
        pre[0] = 0;
#pragma unroll
        for (int p = 0; p < kUnionParts; ++p) pre[p + 1] = pre[p] + a.u_count[grp * kUnionParts + p];
        n_list = pre[kUnionParts];
      }
      const int chunk = SH ? (((n_list + a.n_split - 1) / a.n_split + kTileRows - 1) / kTileRows) * kTileRows
                           : a.split_rows;
      const int e0 = split * chunk;
      const int cnt = max(0, min(n_list, e0 + chunk) - e0);
      const int32_t* idx = a.topk_idx + (int64_t)tok * a.topk + e0;
      // SH: union entry e of the group -> its place in the parts' arrays
      auto u_at = [&](int e) -> int64_t {
        int p = 0;
#pragma unroll
        for (int k = 1; k < kUnionParts; ++k) p += (pre[k] <= e) ? 1 : 0;
        return ((int64_t)grp * kUnionParts + p) * a.u_stride + (e - pre[p]);
      };
      uint32_t mk[4] = {0u, 0u, 0u, 0u};      // SH: token masks of the entries
      // Branch-free loads (clamped addresses, results selected afterwards) so that all index
      // loads are in flight together, then all block-table loads.
      int jv[4] = {-1, -1, -1, -1}, pg[4] = {-1, -1, -1, -1};
      int64_t ap_slot = -1;
      bool ap_early = false;
      if (cnt > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = r * 512 + ptid;
          if constexpr (SH) {
            const int64_t ue = u_at(e0 + min(e, cnt - 1));
            jv[r] = (e < cnt) ? a.u_pos[ue] : -1;
            mk[r] = a.u_mask[ue];
          } else {
            const int v = idx[min(e, cnt - 1)];
            jv[r] = (e < cnt) ? v : -1;
          }
        }
        // AP: the slots of the request's new rows (lane k: row k), behind the index loads
        if constexpr (AP) ap_slot = a.ap_slots[(int64_t)b * a.q_len + min(lane, a.q_len - 1)];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool in = jv[r] >= 0 && jv[r] < a.max_pages * kPageRows;
          const int v = bt[in ? (jv[r] >> 6) : 0];
          pg[r] = in ? v : -1;
        }
      }
      // AP: lane k < q_len holds the cache row (16-byte units) of the request's new row k;
      // [ap_lo, ap_hi] spans them (an entry outside it reads none of them)
      uint32_t ap_o16 = kInvalid, ap_lo = kInvalid, ap_hi = 0u;
      if constexpr (AP) {
        const int64_t off = ap_slot < 0 ? -1 : (ap_slot / kPageRows) * a.page_stride + (ap_slot % kPageRows) * kRowBytes;
        if (lane < a.q_len && off >= 0 && off + kRowBytes <= a.cache_bytes) ap_o16 = (uint32_t)(off >> 4);
        for (int k = 0; k < a.q_len; ++k) {
          const uint32_t nk = __builtin_amdgcn_readlane(ap_o16, k);
          if (nk != kInvalid) { ap_lo = min(ap_lo, nk); ap_hi = max(ap_hi, nk); }
        }
      }
      uint32_t ap_hits = 0u;                  // AP: bit k: an entry of this wave reads new row k
      bool ap_hit_r[4] = {false, false, false, false};   // AP: entry r of this lane reads a new row
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok = false;
        uint32_t o16 = 0;
        if (pg[r] >= 0) {
          const int64_t off = (int64_t)pg[r] * a.page_stride + (int64_t)(jv[r] & 63) * RB;
          if (off + RB <= a.cache_bytes) { ok = true; o16 = (uint32_t)(off >> 4); }
        }
        if constexpr (AP) {
          // the full comparison only in a wave with an entry inside the new rows' span
          if (__ballot(ok && o16 >= ap_lo && o16 <= ap_hi) != 0ull) {
            for (int k = 0; k < a.q_len; ++k) {
              const bool h = ok && o16 == __builtin_amdgcn_readlane(ap_o16, k);
              ap_hit_r[r] = ap_hit_r[r] || h;
              if (__ballot(h) != 0ull) ap_hits |= 1u << k;
            }
          }
        }
        const uint64_t mask = __ballot(ok);
        if (lane == 0) cnt_s[r][pw] = __popcll(mask);
        jv[r] = ok ? (int)o16 : -1;               // keep the offset (or -1) for the write below
      }
      if constexpr (AP) {
        if (lane == 0) ap_hit_s[pw] = (int32_t)ap_hits;
      }
      lds_barrier();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int before = 0, total = 0;
#pragma unroll
        for (int v = 0; v < kProducers; ++v) {
          const int c = cnt_s[r][v];
          before += (v < pw) ? c : 0;
          total += c;
        }
        const bool ok = jv[r] != -1;
        const uint64_t mask = __ballot(ok);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (ok) {
          rowoff[n_rows + before + below] = (uint32_t)jv[r];
          if constexpr (SH) rowmask[n_rows + before + below] = (uint8_t)mk[r];
        }
        // AP: a new row among the first kRawSlots tiles, which the producers gather right after
        // the prologue barrier
        if constexpr (AP) ap_early = ap_early || (ok && ap_hit_r[r] && (int)(n_rows + before + below) < kRawSlots * kTileRows);
        n_rows += total;
      }
      if constexpr (AP) {
        const uint64_t early = __ballot(ap_early);
        if (lane == 0) ap_early_s[pw] = early != 0ull;
      }
    } else {
      if constexpr (AP) {
        // the new rows' inputs (pass i: rows 2p, 2p+1 with p = w + 4i), encoded after the
        // barrier, while the producers finish the compaction
#pragma unroll
        for (int i = 0; i < kApPasses; ++i) {
          const int p = w + 4 * i;
          if (2 * p < a.q_len) {
            const int64_t row = (int64_t)b * a.q_len + min(2 * p + (lane >> 5), a.q_len - 1);
            const uint16_t* lrow = a.ap_latent + row * a.ap_latent_stride + 16 * (lane & 31);
            ap_xa[i] = *(const uint4v*)lrow;
            ap_xb[i] = *(const uint4v*)(lrow + 8);
            ap_ra[i] = a.ap_rope[row * a.ap_rope_stride + (lane & 31)];
            ap_rb[i] = a.ap_rope[row * a.ap_rope_stride + 32 + (lane & 31)];
            ap_sl[i] = a.ap_slots[row];
          }
        }
      }
      lds_barrier();
    }
  } else {
    const int seq = min(a.seq_lens[b], a.max_pages * kPageRows);
    const int vis = seq - a.q_len + 1 + t;                 // positions 0 .. vis-1
    p0 = split * a.split_rows;
    n_rows = max(0, min(vis, p0 + a.split_rows) - p0);
    const int n_pages = (n_rows + 63) >> 6;
    int bad = 0;
    for (int i = tid; i < n_pages; i += kThreads) {
      // The page's byte offset is checked in 64 bits before it is narrowed to 16-byte units:
      // a page starting at or past cache_bytes (<= 2^36) is marked invalid, so a page id whose
      // offset exceeds 2^36 can never wrap onto a real page.
      const int pg = bt[(p0 >> 6) + i];
      const int64_t off = (int64_t)pg * a.page_stride;
      rowoff[i] = (pg < 0 || off >= a.cache_bytes) ? kInvalid : (uint32_t)(off >> 4);
      if (pg < 0 || off + (int64_t)kPageRows * RB > a.cache_bytes) bad = 1;
    }
    // one barrier, as on the sparse path; no gather is in flight yet
    dense_ok = __syncthreads_or(bad) == 0;
  }
  if (tid < 8) flag_s[tid >> 2][tid & 3] = 0;
  if constexpr (AP) {
    if (math) {
      // Encode the request's new rows (lanes 0-31 row 2p, lanes 32-63 row 2p+1) and write them
      // to their slots (as the append does: slots of -1 and slots outside the cache are not
      // written): the rows the list reads, and every row in the request's writer workgroup.
      // The stores complete before any gather of those rows: a math wave's vector-memory
      // operations complete in issue order, so its query loads after the next barrier wait for
      // them, and the gathers of tile 3 onwards come after the prologue barriers that follow;
      // when a new row is among the first tiles, which the producers gather right after the next
      // barrier, the workgroup waits for the stores and takes one barrier more (below).
      const int half = lane >> 5, g = lane & 31;
      const int4 h0 = *(const int4*)&ap_hit_s[0], h1 = *(const int4*)&ap_hit_s[4];
      const uint32_t hits = (uint32_t)(h0.x | h0.y | h0.z | h0.w | h1.x | h1.y | h1.z | h1.w);
      const bool writer = split == 0 && rest % a.n_hg == 0 && a.head_begin == 0 && t == 0;
      const uint32_t rows = writer ? 0xFFFFFFFFu : hits;       // rows this workgroup stores
#pragma unroll
      for (int i = 0; i < kApPasses; ++i) {
        const int k0 = 2 * (w + 4 * i), k = k0 + half;
        if (((rows >> k0) & 3u) != 0u && k0 < a.q_len) {
          const Nvfp4LaneOut e = nvfp4_encode_lane(ap_xa[i], ap_xb[i], ap_ra[i], ap_rb[i]);
          const int64_t slot = ap_sl[i];
          const int64_t off = slot < 0 ? -1 : (slot / kPageRows) * a.page_stride + (slot % kPageRows) * kRowBytes;
          if (((rows >> k) & 1u) != 0u && k < a.q_len && off >= 0 && off + kRowBytes <= a.cache_bytes) {
            uint8_t* dst = a.ap_cache + off;
            *(uint2v*)(dst + 8 * g) = uint2v{e.c0, e.c1};
            if (g < 24) ((uint32_t*)(dst + kScaleOff))[g] = e.tail;
          }
        }
      }
    }
  }
  if constexpr (!DENSE) {
    // the math waves learn the row count from the per-wave counts
    if (math) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int v = 0; v < kProducers; ++v) n_rows += cnt_s[r][v];
    }
  }
  lds_barrier();
  const int n_tiles = (n_rows + kTileRows - 1) / kTileRows;

  // No valid row (an empty list, or a split past the end of the list or of the visible
  // positions): every wave knows n_rows here, so the workgroup leaves together. The result is the
  // softmax over no rows, written by the producer waves in the epilogue's layout: zero outputs
  // and lse = -inf. No query load or gather has been issued yet.
  if constexpr (AP) {
    // a new row among the first tiles: its stores complete before the producers gather them
    const int4 e0 = *(const int4*)&ap_early_s[0], e1 = *(const int4*)&ap_early_s[4];
    if ((e0.x | e0.y | e0.z | e0.w | e1.x | e1.y | e1.z | e1.w) != 0) {
      if (math) wait_vmcnt<0>();
      lds_barrier();
    }
  }
  if (n_rows == 0) {
    if (!math) {
      const bool final_out = (a.n_split == 1);
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) {
        if (!hb_valid(hb)) continue;
        const int hbg = hb_global(hb);
        const int64_t otok = hb_tok(hb);
        if (final_out) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* dst = a.out + (otok * a.H + 16 * hbg + 4 * kg + e) * kLatent + 64 * pw + l16;
#pragma unroll
            for (int n = 0; n < 4; ++n) dst[16 * n] = 0.0f;
          }
        } else {
          _Float16* dst = a.ws_o + (((otok * a.n_split + split) * (a.H >> 4) + hbg) * 16 + 2 * pw) * 512 + 8 * lane;
#pragma unroll
          for (int m = 0; m < 2; ++m) *(uint4v*)(dst + 512 * m) = uint4v{0u, 0u, 0u, 0u};
        }
        if (pw == 0 && l16 == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int head = 16 * hbg + 4 * kg + e;
            if (final_out) {
              if (a.lse) a.lse[otok * a.H + head] = -INFINITY;
            } else {
              a.ws_lse[(otok * a.n_split + split) * a.H + head] = -INFINITY;
            }
          }
        }
      }
    }
    return;
  }

  float* fin_m = (float*)pbuf[0];               // epilogue: per-head running max and sum
  float* fin_l = fin_m + 64;

  // ---- gathers (issued by the math waves) ---------------------------------------------------
  // Piece p = k*256 + w*64 + lane (k = 0..2; math wave 3 has no k = 2 piece) of the tile's 704
  // 16-byte pieces (22 per row). Rows past the end and rows without a valid address read the
  // zero row, so the ring always holds finite data. The row offsets of a tile are read from LDS
  // one tile ahead of its gathers.
  const int nk = (w == 3) ? 2 : 3;
  uint32_t pk[3];                              // (row in tile << 16) | byte offset in the row
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int p = min(k * 256 + (w & 3) * 64 + lane, kRawPieces - 1);
    pk[k] = ((uint32_t)(p / 22) << 16) | (uint32_t)((p % 22) * 16);
  }
  // Offset (16-byte units) of row `row` of this split, kInvalid past the end or without a page.
  auto row_o16 = [&](int row) -> uint32_t {
    const bool ok = row < n_rows;
    if constexpr (!DENSE) {
      return ok ? rowoff[row] : kInvalid;
    } else {
      const int pos = p0 + (ok ? row : 0);
      const uint32_t pb = rowoff[(pos >> 6) - (p0 >> 6)];
      const int64_t o = (int64_t)pb + (pos & 63) * (RB / 16);     // 64-bit: no wrap
      return (ok && pb != kInvalid && o * 16 + RB <= a.cache_bytes) ? (uint32_t)o : kInvalid;
    }
  };
  // Source of byte pb of a row: the cache or the zero row. The two spellings give the same
  // address, but the compiler's register schedule follows them: with pb added to both operands
  // it hoists the zero-row pointer plus offset, and in the shared-rows instantiation the QK loop
  // then reads every LDS operand into one register quad and waits for each read before its
  // MFMA (34 serialized waits instead of 3; that kernel ran 40% slower). Selecting the base and
  // adding pb afterwards keeps those reads in flight; the fused-append instantiation is the one
  // measured faster with the other spelling.
  auto gather_src = [&](uint32_t o16, uint32_t pb) -> const uint8_t* {
    if constexpr (AP) return (o16 != kInvalid) ? a.cache + (int64_t)o16 * 16 + pb : g_zero_row + pb;
    return ((o16 != kInvalid) ? a.cache + (int64_t)o16 * 16 : g_zero_row) + pb;
  };
  auto tile_offsets = [&](int tile, uint32_t (&o16)[3]) {
#pragma unroll
    for (int k = 0; k < 3; ++k) o16[k] = row_o16(tile * kTileRows + (int)(pk[k] >> 16));
  };
  auto issue_tile = [&](int tile, const uint32_t (&o16)[3]) {
    uint8_t* dst = raw[tile % kRawSlots];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (k >= nk) break;
      const uint32_t pb = pk[k] & 0xFFFFu;
      gather16_to_lds(gather_src(o16[k], pb), dst + (k * 256 + w * 64) * 16);
    }
  };
  // Wait until the gathers issued before the last `after` tiles have landed in LDS.
  auto wait_tiles = [&](int after) {
    if (nk == 3) {
      if (after >= 2) wait_vmcnt<6>(); else if (after == 1) wait_vmcnt<3>(); else wait_vmcnt<0>();
    } else {
      if (after >= 2) wait_vmcnt<4>(); else if (after == 1) wait_vmcnt<2>(); else wait_vmcnt<0>();
    }
  };

  if (math) {
    // ================================ math waves ================================================
    // The first three tiles are gathered by the producer waves, so that no gather of this wave
    // is in flight while its query loads are waited for (they share the vector-memory counter).
    load_q();
#pragma unroll
    for (int c = 0; c < kChunks; ++c) asm volatile("" : "+v"(qf[c]));
    // AP: this wave's new-row stores are complete before any math wave gathers tile 3 (a wave
    // that loads queries has already waited for them: its operations complete in order)
    if constexpr (AP) wait_vmcnt<0>();
    lds_barrier();                            // prologue: tile 0 in LDS
    lds_barrier();                            // prologue: tile 0 decoded, tile 1 in LDS
    uint32_t next_o16[3] = {kInvalid, kInvalid, kInvalid};   // row offsets of the next tile to gather
    if constexpr (!FP8) tile_offsets(3, next_o16);
    float m_run = -INFINITY, l_run = 0.0f;     // running max (log2 units), partial sum
    const int kslot = ((kdg << 4) + (l16 ^ ((kdg & 1) << 2))) << 4;   // QK A-fragment slot
    // One loop per kind of math wave (head-block owners and, when a group has fewer than four
    // head blocks, gather-only waves), so that neither carries the other's registers.
    auto math_loop = [&](auto qkw_tag) {
      constexpr bool QKW = decltype(qkw_tag)::value;
      for (int i = 0; i <= n_tiles; ++i) {
        if (QKW && i < n_tiles) {
          const uint8_t* dt = dec[i % kDecSlots];
          float4v acc[2][2];
  #pragma unroll
          for (int rb = 0; rb < 2; ++rb) { acc[rb][0] = float4v{0.f, 0.f, 0.f, 0.f}; acc[rb][1] = acc[rb][0]; }
  #pragma unroll
          for (int c = 0; c < kChunks; ++c)
  #pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const half8v kf = *(const half8v*)(dt + (rb * kChunks + c) * kFragBytes + kslot);
              acc[rb][c & 1] = mfma16(kf, qf[c], acc[rb][c & 1]);
            }
          // Issue order: 8 fragment reads ahead of the MFMAs, then one read per MFMA, so LDS
          // latency stays hidden behind the matrix work.
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  #pragma unroll
          for (int k = 0; k < 2 * kChunks - 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          uint32_t cur_o16[3] = {next_o16[0], next_o16[1], next_o16[2]};
          if constexpr (!FP8) tile_offsets(i + 4, next_o16);   // LDS latency hides behind the softmax
          float sv[8];
          float mx = -INFINITY;
          const bool full = !SH && (i + 1) * kTileRows <= n_rows && dense_ok;
          if (full) {                                        // full tile: no row mask
  #pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const float4v sc = acc[rb][0] + acc[rb][1];
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                sv[4 * rb + e] = sc[e] * a.scale_log2;
                mx = fmaxf(mx, sv[4 * rb + e]);
              }
            }
          } else {
  #pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const float4v sc = acc[rb][0] + acc[rb][1];
              // SH: the token bits of rows 16*rb + 4*kg .. +3 (one byte each)
              const uint32_t mw = SH ? *(const uint32_t*)&rowmask[i * kTileRows + 16 * rb + 4 * kg] : 0u;
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int row = i * kTileRows + 16 * rb + 4 * kg + e;
                bool ok = row < n_rows;
                if constexpr (DENSE) ok = ok && (dense_ok || row_o16(row) != kInvalid);
                if constexpr (SH) ok = ok && ((mw >> (8 * e + w)) & 1u);
                sv[4 * rb + e] = ok ? sc[e] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, sv[4 * rb + e]);
              }
            }
          }
          mx = group4_max(mx);
          // The running max moves lazily: only when a tile's max exceeds it by more than 2^8, so
          // the probabilities stay <= 256 (exact range for FP16) and O is rescaled only then.
          const bool move = mx > m_run + 8.0f;        // also true on the first tile (m_run = -inf)
          const float m_new = move ? mx : m_run;
          const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
          half4v pf[2];
          if (full) {
  #pragma unroll
            for (int e = 0; e < 8; ++e) pf[e >> 2][e & 3] = (_Float16)__builtin_amdgcn_exp2f(sv[e] - m_new);
          } else {
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              // a masked row is 0 (also while no valid row has been seen: m_new = -inf)
              pf[e >> 2][e & 3] = (sv[e] == -INFINITY) ? (_Float16)0.0f
                                                       : (_Float16)__builtin_amdgcn_exp2f(sv[e] - m_new);
            }
          }
          // the row sum of the FP16 probabilities PV uses, in FP32: v_dot2_f32_f16 against (1, 1)
          // adds two of them per instruction (the products are exact)
          const half2v one2 = half2v{(_Float16)1.0f, (_Float16)1.0f};
          float psum = 0.0f;
  #pragma unroll
          for (int h = 0; h < 4; ++h)
            psum = __builtin_amdgcn_fdot2(half2v{pf[h >> 1][2 * (h & 1)], pf[h >> 1][2 * (h & 1) + 1]}, one2, psum, false);
          l_run = l_run * alpha + psum;
          m_run = m_new;
          const int ph = 16 * w + l16;
          uint8_t* prow_p = pbuf[i & 1] + ph * kPStride + 8 * (kg & 1);
          *(half4v*)(prow_p + p_col(ph, kg >> 1)) = pf[0];        // rows 4kg..4kg+3
          *(half4v*)(prow_p + p_col(ph, 2 + (kg >> 1))) = pf[1];  // rows 16+4kg..
          const uint64_t any = __ballot(move && i > 0);
          if (lane == 0) flag_s[i & 1][w] = any != 0ull;
          if (kg == 0) alpha_s[i & 1][16 * w + l16] = alpha;
          if constexpr (!FP8) issue_tile(i + 3, cur_o16);
        }
        if constexpr (!FP8) {
          if (!(QKW && i < n_tiles)) { issue_tile(i + 3, next_o16); tile_offsets(i + 4, next_o16); }
          wait_tiles(1);
        }
        lds_barrier();
      }
    };
    if (qk_wave) math_loop(std::true_type{});
    else math_loop(std::false_type{});
    wait_vmcnt<0>();                          // no gather may still target LDS at exit
    if (qk_wave) {
      const float lt = group4_sum(l_run);
      if (kg == 0) { fin_m[16 * w + l16] = m_run; fin_l[16 * w + l16] = lt; }
    }
    lds_barrier();
  } else {
    // ================================ producer waves ============================================
    // Decode: lane (pw, kg, l16) decodes code piece p = 4*(pw&3) + kg (32 latent dims =
    // K-chunk p) of row 16*(pw>>2) + l16; waves 0..3 also decode one rope group of 8 dims.
    const int dp = 4 * (pw & 3) + kg;
    const int drow = 16 * (pw >> 2) + l16;
    const int ru = (pw & 3) * 64 + lane;                  // rope unit (waves 0..3)
    const int rrow = ru & 31, rg = ru >> 5;
    struct DecodeIn { uint4v cw; uint32_t sc; uint2v rp; };
    auto decode_load = [&](int tile) {
      const uint8_t* src = raw[tile % kRawSlots];
      const uint8_t* row = src + drow * kRowBytes;
      DecodeIn d;
      d.cw = *(const uint4v*)(row + 16 * dp);
      d.sc = *(const uint16_t*)(row + kScaleOff + 2 * dp);
      d.rp = (pw < 4) ? *(const uint2v*)(src + rrow * kRowBytes + kRopeOff + 8 * rg) : uint2v{0u, 0u};
      return d;
    };
    auto decode_store = [&](int tile, const DecodeIn& d) {
      uint8_t* dst = dec[tile % kDecSlots];
      const half2v s01 = fp8x2_to_half2<false>(d.sc);
      const half2v s0 = half2v{s01[0], s01[0]}, s1 = half2v{s01[1], s01[1]};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *(half8v*)(dst + frag_off(drow, dp, k)) = decode_fp4x8(d.cw[k], k < 2 ? s0 : s1);
      if (pw < 4) *(half8v*)(dst + frag_off(rrow, 16 + (rg >> 2), rg & 3)) = decode_fp8x8(d.rp[0], d.rp[1]);
    };
    auto decode_tile = [&](int tile) { decode_store(tile, decode_load(tile)); };

    // FP8 rows: lane (pw, kg, l16) loads bytes 32*dp..32*dp+31 of row drow (K-chunk dp) and rope
    // bytes 4*rq..4*rq+3 of row ptid & 31 (rq = ptid >> 5), straight into registers.
    const int rq = ptid >> 5, rqrow = ptid & 31;
    struct Fp8In { uint4v a, b; uint32_t r; };
    auto row_src = [&](int row) -> const uint8_t* {
      uint32_t o16;
      if constexpr (!DENSE) {
        o16 = row < n_rows ? rowoff[row] : kInvalid;
      } else {
        const bool ok = row < n_rows;
        const int pos = p0 + (ok ? row : 0);
        const uint32_t pb = rowoff[(pos >> 6) - (p0 >> 6)];
        const int64_t o = (int64_t)pb + (pos & 63) * (RB / 16);   // 64-bit: no wrap
        o16 = (ok && pb != kInvalid && o * 16 + RB <= a.cache_bytes) ? (uint32_t)o : kInvalid;
      }
      return o16 != kInvalid ? a.cache + (int64_t)o16 * 16 : g_zero_row;
    };
    auto fp8_load = [&](int tile) {
      Fp8In d;
      const uint8_t* p = row_src(tile * kTileRows + drow) + 32 * dp;
      d.a = *(const uint4v*)p;
      d.b = *(const uint4v*)(p + 16);
      d.r = *(const uint32_t*)(row_src(tile * kTileRows + rqrow) + kLatent + 4 * rq);
      return d;
    };
    auto fp8_store = [&](int tile, const Fp8In& d) {
      uint8_t* dst = dec[tile % kDecSlots];
      *(half8v*)(dst + frag_off(drow, dp, 0)) = decode_fp8x8(d.a[0], d.a[1]);
      *(half8v*)(dst + frag_off(drow, dp, 1)) = decode_fp8x8(d.a[2], d.a[3]);
      *(half8v*)(dst + frag_off(drow, dp, 2)) = decode_fp8x8(d.b[0], d.b[1]);
      *(half8v*)(dst + frag_off(drow, dp, 3)) = decode_fp8x8(d.b[2], d.b[3]);
      const half2v r0 = fp8x2_to_half2<false>(d.r), r1 = fp8x2_to_half2<true>(d.r);
      *(half4v*)(dst + frag_off(rqrow, 16 + (rq >> 3), (rq >> 1) & 3) + 8 * (rq & 1)) =
          half4v{r0[0], r0[1], r1[0], r1[1]};
    };

    // Output accumulators of dims 64*pw + 16*n + l16, heads 16*hb + 4*kg + e.
    float4v o[NH][4];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb)
#pragma unroll
      for (int n = 0; n < 4; ++n) o[hb][n] = float4v{0.f, 0.f, 0.f, 0.f};
    Fp8In f1{};                               // FP8: registers of the next tile to convert
    if constexpr (FP8) {
      const Fp8In f0 = fp8_load(0);
      f1 = fp8_load(1);
      lds_barrier();                          // prologue (same barrier count as the gathers)
      if (n_tiles > 0) fp8_store(0, f0);
    } else {
      // Tiles 0..2: piece q = k*512 + ptid (k = 0, 1; only waves 0..2 have a k = 1 piece, as a
      // tile has 704 pieces), issued right after the compaction.
      const int np = (pw < 3) ? 2 : 1;
      auto prod_issue = [&](int tile) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (k == 1 && np == 1) break;
          const int q = k * 512 + ptid;
          const uint32_t pb = (uint32_t)((q % 22) * 16);
          const uint32_t o16 = row_o16(tile * kTileRows + q / 22);
          gather16_to_lds(gather_src(o16, pb), raw[tile % kRawSlots] + (k * 512 + pw * 64) * 16);
        }
      };
      prod_issue(0);
      prod_issue(1);
      prod_issue(2);
      if (np == 2) wait_vmcnt<4>(); else wait_vmcnt<2>();      // tile 0 landed
      lds_barrier();                          // prologue: tile 0 in LDS
      if (n_tiles > 0) decode_tile(0);
      if (np == 2) wait_vmcnt<2>(); else wait_vmcnt<1>();      // tile 1 landed
    }
    lds_barrier();                            // prologue: tile 0 decoded, tile 1 in LDS
    // Transposing-read offsets (V operand of PV): the lane supplies 4 dims
    // (16*n + 4*(l16&3) ..) of row 8*kg + (l16>>2) (+4 for the second read).
    const int vq = l16 >> 2, va = l16 & 3;
    const int vrow0 = 8 * kg + vq;
    for (int i = 0; i <= n_tiles; ++i) {
      // raw bytes of tile i+1 first: their LDS latency hides behind PV(i-1)
      const bool dec_next = i + 1 < n_tiles;
      DecodeIn din;
      Fp8In f2;
      if constexpr (FP8) f2 = fp8_load(i + 2);         // lands while PV(i-1) runs
      else if (dec_next) din = decode_load(i + 1);
      if (i >= 1) {
        // PV(i-1): rescale by alpha(i-1) where the running max moved, then O += P V.
        const int j = i - 1;
        const uint8_t* dt = dec[j % kDecSlots];
        const int4 fl = *(const int4*)flag_s[j & 1];
        if ((fl.x | fl.y | fl.z | fl.w) != 0) {
#pragma unroll
          for (int hb = 0; hb < NH; ++hb) {
            const int f = (hb == 0) ? fl.x : (hb == 1) ? fl.y : (hb == 2) ? fl.z : fl.w;
            if (f) {
              const float4v al = *(const float4v*)&alpha_s[j & 1][16 * hb + 4 * kg];
#pragma unroll
              for (int n = 0; n < 4; ++n) o[hb][n] *= al;
            }
          }
        }
        half8v pa[NH];
#pragma unroll
        for (int hb = 0; hb < NH; ++hb)
          pa[hb] = *(const half8v*)(pbuf[j & 1] + (16 * hb + l16) * kPStride + p_col(16 * hb + l16, kg));
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int ng = 4 * pw + n;
          const int dg = 2 * (ng & 1) + (va >> 1);
          const int off0 = frag_off(vrow0, ng >> 1, dg) + 8 * (va & 1);
          const int off1 = frag_off(vrow0 + 4, ng >> 1, dg) + 8 * (va & 1);
          const half4v v0 = lds_tr16(dt + off0);
          const half4v v1 = lds_tr16(dt + off1);
          const half8v vb = half8v{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int hb = 0; hb < NH; ++hb) o[hb][n] = mfma16(pa[hb], vb, o[hb][n]);
        }
      }
      if constexpr (FP8) {
        if (dec_next) fp8_store(i + 1, f1);
        f1 = f2;
      } else {
        if (dec_next) decode_store(i + 1, din);
        if (i == 0) wait_vmcnt<0>();          // tile 2 (gathered in the prologue) landed
      }
      lds_barrier();
    }
    lds_barrier();                              // fin_m / fin_l written by the math waves

    // ---- normalise and write ----------------------------------------------------------------
    const bool final_out = (a.n_split == 1);
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      if (!hb_valid(hb)) continue;
      const float4v mm = *(const float4v*)&fin_m[16 * hb + 4 * kg];
      const float4v ll = *(const float4v*)&fin_l[16 * hb + 4 * kg];
      float4v inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) inv[e] = ll[e] > 0.0f ? 1.0f / ll[e] : 0.0f;
      const int hbg = hb_global(hb);                      // global 16-head block
      const int64_t otok = hb_tok(hb);
      if (final_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float* dst = a.out + (otok * a.H + 16 * hbg + 4 * kg + e) * kLatent + 64 * pw + l16;
#pragma unroll
          for (int n = 0; n < 4; ++n) dst[16 * n] = o[hb][n][e] * inv[e];
        }
      } else {
        // FP16 partial in register order: [token][split][16-head block][pair of 16-dim blocks]
        // [lane][2 dim blocks][4 heads], so that each lane stores 16 bytes at a time (dim blocks
        // 4pw + 2m and 4pw + 2m + 1 of its 4 heads). With at most kStreamPartialSplits splits the
        // partials are written with streaming (non-temporal) stores: they then leave no dirty
        // lines for the end-of-kernel L2 write-back, which shortens this kernel by more than the
        // combine, whose single round of loads then reads them from the memory-side cache, loses.
        // With more splits the combine reads in several rounds and the partials are better kept
        // in the L2.
        _Float16* dst = a.ws_o + (((otok * a.n_split + split) * (a.H >> 4) + hbg) * 16 + 2 * pw) * 512 + 8 * lane;
        const bool stream = a.n_split <= kStreamPartialSplits;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float4v v0 = o[hb][2 * m] * inv, v1 = o[hb][2 * m + 1] * inv;
          const half8v hv = half8v{(_Float16)v0[0], (_Float16)v0[1], (_Float16)v0[2], (_Float16)v0[3],
                                   (_Float16)v1[0], (_Float16)v1[1], (_Float16)v1[2], (_Float16)v1[3]};
          if (stream)
            __builtin_nontemporal_store(__builtin_bit_cast(uint4v, hv), (uint4v*)(dst + 512 * m));
          else
            *(half8v*)(dst + 512 * m) = hv;
        }
      }
      if (pw == 0 && l16 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int head = 16 * hbg + 4 * kg + e;
          // log2 units (the max is kept in them); the split merge weighs in log2 units too, so
          // only the final value is scaled to the natural log
          const float lse2 = ll[e] > 0.0f ? mm[e] + __builtin_amdgcn_logf(ll[e]) : -INFINITY;
          if (final_out) {
            if (a.lse) a.lse[otok * a.H + head] = lse2 * 0.69314718055994530942f;
          } else {
            a.ws_lse[(otok * a.n_split + split) * a.H + head] = lse2;
          }
        }
      }
    }
  }
}

// Merge the n_split partial (o_s, lse_s) of each (token, head), with lse_s in log2 units as the
// decode writes them: M = max lse_s, w_s = 2^(lse_s - M), o = sum w_s o_s / sum w_s, and the
// natural-log lse = (M + log2(sum w_s)) ln 2.
// A unit position is (token, 16-head block, pair of 16-dim blocks; a lane: two dims 16 apart of
// 4 heads, the 16-byte FP16 unit the decode kernel stored). A workgroup has four waves: with
// G = 1 they own four unit positions and merge all splits in split order; with G = 4 they own
// one and take contiguous quarters of the splits, each merged in split order, then merged in
// wave order (a fixed tree, so the result is deterministic) with wave g finalizing head e = g.
// SCW > 0 handles up to SCW splits per wave with every load issued in one round; SCW == 0 any
// count, 8 splits at a time.
constexpr int kCombineChunk = 8;

template <int SCW, int G>
__global__ __launch_bounds__(256) void combine_kernel(int32_t T, int32_t H, int32_t S,
                                                         const _Float16* __restrict__ ws_o,
                                                         const float* __restrict__ ws_lse,
                                                         float* __restrict__ out,
                                                         float* __restrict__ lse,
                                                         int32_t per_xcd, int32_t total) {
  __shared__ float4v xs[G > 1 ? G : 1][4][64];   // per wave: max, weight sum, acc0, acc1 (4 heads)
  const int hw = blockIdx.x;
  const int L = (hw & 7) * per_xcd + (hw >> 3);
  if (L >= total) return;
  static_assert(G == 1 || G == 4, "one wave per unit position, or four sharing one");
  const int nhb = H >> 4;
  // the wave index through a scalar register: the split share and the per-split bases below are
  // then wave-uniform (scalar base plus a 32-bit lane offset per load)
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, kg = lane >> 4,
            l16 = lane & 15;
  // token, 16-head block, pair of dim blocks 2q, 2q + 1, share of the splits
  const int tok = G == 1 ? L / (nhb * 4) : L / (nhb * 16);
  const int r = G == 1 ? L % (nhb * 4) : L % (nhb * 16);
  const int hb = G == 1 ? r >> 2 : r >> 4;
  const int q = G == 1 ? (r & 3) * 4 + wv : r & 15;
  const int g = G == 1 ? 0 : wv;
  const int head = 16 * hb + 4 * kg;        // heads head..head+3
  const int64_t split_stride = (int64_t)H * kLatent;
  const _Float16* tok_o = ws_o + (int64_t)tok * S * split_stride;   // the token's partials
  const int o_lane = ((hb * 16 + q) * 64 + lane) * 8;                  // within one split's H x 512
  const float* lp = ws_lse + (int64_t)tok * S * H + head;
  auto o_at = [&](int s) { return *(const half8v*)(tok_o + (int64_t)s * split_stride + o_lane); };
  const int per = (S + G - 1) / G;
  const int s0 = min(g * per, S), s1 = min(s0 + per, S);   // this wave's splits
  const float4v ninf = float4v{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float4v M = ninf;
  float4v acc0 = float4v{0.f, 0.f, 0.f, 0.f}, acc1 = acc0, wsum = acc0;
  // Weights against the running max; a head with no valid row in any split (max -inf) takes 0
  // as its reference, so that every weight is exp2(-inf) = 0 without a test per split.
  float4v Mb;
  auto set_ref = [&]() {
#pragma unroll
    for (int e = 0; e < 4; ++e) Mb[e] = (M[e] == -INFINITY) ? 0.0f : M[e];
  };
  auto merge = [&](const float4v& ls, const half8v& hv) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float wgt = __builtin_amdgcn_exp2f(ls[e] - Mb[e]);
      acc0[e] += wgt * (float)hv[e];
      acc1[e] += wgt * (float)hv[4 + e];
      wsum[e] += wgt;
    }
  };
  if constexpr (SCW > 0) {
    float4v ls[SCW];
    half8v ov[SCW];
#pragma unroll
    for (int j = 0; j < SCW; ++j) {
      const int s = min(s0 + j, S - 1);                   // splits past the share: weight 0
      ls[j] = (s0 + j < s1) ? *(const float4v*)(lp + (int64_t)s * H) : ninf;
      ov[j] = o_at(s);
    }
#pragma unroll
    for (int j = 0; j < SCW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], ls[j][e]);
    set_ref();
#pragma unroll
    for (int j = 0; j < SCW; ++j) merge(ls[j], ov[j]);
  } else {
    for (int c0 = s0; c0 < s1; c0 += kCombineChunk) {
      float4v v[kCombineChunk];
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j)
        v[j] = (c0 + j < s1) ? *(const float4v*)(lp + (int64_t)(c0 + j) * H) : ninf;
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) M[e] = fmaxf(M[e], v[j][e]);
    }
    set_ref();
    for (int c0 = s0; c0 < s1; c0 += kCombineChunk) {
      float4v ls[kCombineChunk];
      half8v ov[kCombineChunk];
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        const int s = min(c0 + j, s1 - 1);
        ls[j] = (c0 + j < s1) ? *(const float4v*)(lp + (int64_t)s * H) : ninf;
        ov[j] = o_at(s);
      }
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) merge(ls[j], ov[j]);
    }
  }
  if constexpr (G == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // v_rcp_f32 (1 ulp): the weight sum is >= 1 when it is not 0 (the max split weighs 1)
      const float inv = wsum[e] > 0.0f ? __builtin_amdgcn_rcpf(wsum[e]) : 0.0f;
      float* o = out + ((int64_t)tok * H + head + e) * kLatent + 32 * q + l16;
      o[0] = acc0[e] * inv;
      o[16] = acc1[e] * inv;
    }
    if (lse && q == 0 && l16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lse[(int64_t)tok * H + head + e] =
            (M[e] == -INFINITY) ? -INFINITY : (M[e] + __builtin_amdgcn_logf(wsum[e])) * 0.69314718055994530942f;
    }
  } else {
    xs[g][0][lane] = M;
    xs[g][1][lane] = wsum;
    xs[g][2][lane] = acc0;
    xs[g][3][lane] = acc1;
    __syncthreads();
    // wave g finalizes head e = g over the four shares, in wave order
    const int e = g;
    float m = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) m = fmaxf(m, xs[h][0][lane][e]);
    float ws = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mh = xs[h][0][lane][e];
      const float f = (mh == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mh - m);
      ws += f * xs[h][1][lane][e];
      a0 += f * xs[h][2][lane][e];
      a1 += f * xs[h][3][lane][e];
    }
    const float inv = ws > 0.0f ? __builtin_amdgcn_rcpf(ws) : 0.0f;           // as above: ws >= 1
    float* o = out + ((int64_t)tok * H + head + e) * kLatent + 32 * q + l16;
    o[0] = a0 * inv;
    o[16] = a1 * inv;
    if (lse && q == 0 && l16 == 0)
      lse[(int64_t)tok * H + head + e] =
          (m == -INFINITY) ? -INFINITY : (m + __builtin_amdgcn_logf(ws)) * 0.69314718055994530942f;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int nh, bool dense, bool fp8, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid((unsigned)a.items_per_xcd * 8), block(kThreads);
  if (a.ap_slots) {                           // fused append: NVFP4 sparse only
    if (dense || fp8) return hipErrorInvalidValue;
#define MLA_LAUNCH_AP(NHV) \
  hipExtLaunchKernelGGL((decode_kernel<NHV, false, false, false, true>), grid, block, 0, stream, ev_start, ev_stop, 0, a)
    switch (nh) {
      case 1: MLA_LAUNCH_AP(1); break;
      case 2: MLA_LAUNCH_AP(2); break;
      case 3: MLA_LAUNCH_AP(3); break;
      case 4: MLA_LAUNCH_AP(4); break;
      default: return hipErrorInvalidValue;
    }
#undef MLA_LAUNCH_AP
    return hipGetLastError();
  }
#define MLA_LAUNCH(NHV, DV, FV) \
  hipExtLaunchKernelGGL((decode_kernel<NHV, DV, FV>), grid, block, 0, stream, ev_start, ev_stop, 0, a)
#define MLA_CASES(FV)                           \
  switch (nh * 2 + (dense ? 1 : 0)) {           \
    case 2: MLA_LAUNCH(1, false, FV); break;    \
    case 3: MLA_LAUNCH(1, true, FV); break;     \
    case 4: MLA_LAUNCH(2, false, FV); break;    \
    case 5: MLA_LAUNCH(2, true, FV); break;     \
    case 6: MLA_LAUNCH(3, false, FV); break;    \
    case 7: MLA_LAUNCH(3, true, FV); break;     \
    case 8: MLA_LAUNCH(4, false, FV); break;    \
    case 9: MLA_LAUNCH(4, true, FV); break;     \
    default: return hipErrorInvalidValue;       \
  }
  if (fp8) {
    MLA_CASES(true)
  } else {
    MLA_CASES(false)
  }
#undef MLA_CASES
#undef MLA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_shared(const DecodeArgs& a, hipStream_t stream, hipEvent_t ev_start,
                                hipEvent_t ev_stop) {
  hipExtLaunchKernelGGL((decode_kernel<4, false, false, true>), dim3((unsigned)a.items_per_xcd * 8),
                        dim3(kThreads), 0, stream, ev_start, ev_stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_combine(int32_t T, int32_t H, int32_t n_split, const _Float16* ws_o,
                          const float* ws_lse, float* out, float* lse, hipStream_t stream) {
  // whole tokens per XCD, as the decode deals its splits, so that a token's partials are read
  // from the L2 they were written to
#define MLA_COMBINE(SCW, G)                                                                       \
  do {                                                                                            \
    const int32_t total = T * (H / 16) * 16 / (4 / (G));                                          \
    const int32_t per_xcd = ((T + 7) / 8) * (H / 16) * 16 / (4 / (G));                            \
    hipLaunchKernelGGL((combine_kernel<SCW, G>), dim3((unsigned)per_xcd * 8), dim3(256), 0, stream, \
                       T, H, n_split, ws_o, ws_lse, out, lse, per_xcd, total);                    \
  } while (0)
  // up to 8 splits: one wave per unit position reads them all in one round (sharing them
  // across waves measured slower there); more splits: four waves share them
  if (n_split <= 8) MLA_COMBINE(8, 1);
  else if (n_split <= 16) MLA_COMBINE(4, 4);
  else MLA_COMBINE(0, 4);
#undef MLA_COMBINE
  return hipGetLastError();
}

}  // namespace mla
