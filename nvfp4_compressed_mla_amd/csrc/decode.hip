// Fused NVFP4 sparse / dense MLA decode for gfx950, plus the split log-sum-exp combine.
//
// Source of the computation: page "Prime Inference: Fast, Reliable Serving for Frontier Open
// Models", section "Native NVFP4 sparse MLA decode kernel": the kernel takes the positions the
// sparse indexer selected, loads the compressed 352-byte rows, unpacks them on chip right before
// use (no intermediate buffer in device memory) and computes attention with FP16 operands and
// FP32 accumulation; a query token's rows are split across cooperating blocks whose partial
// results are merged; -1 entries of the index list are skipped instead of being loaded.
//
// MI355X design (not the page's Blackwell design):
//  * One workgroup = 4 wavefronts = one (query token, head group of 16 or 32 heads, row split);
//    two workgroups share a compute unit (<= 256 registers per lane, <= 80 KB LDS each), so the
//    hardware interleaves one group's MFMA work with the other's decode and softmax.
//    The 576 QK dimensions and the 512 output dimensions are partitioned across the 4 waves:
//    wave w owns latent dims [128w, 128w+128) and rope dims [16w, 16w+16). Every row is therefore
//    decoded exactly once per workgroup, and each wave keeps only its slice of the queries
//    (FP16, 5 MFMA k-chunks x NH head blocks) and of the output accumulators in registers.
//  * Rows are gathered 32 at a time into a 3-slot LDS ring with gfx950 direct-to-LDS 16-byte
//    loads (global_load_lds_dwordx4), two tiles ahead of the math (the page's three-slot buffer,
//    as an LDS ring). Empty and out-of-range slots never reach the ring: sparse index lists are
//    compacted up front, and padding rows read a zero row.
//  * QK: v_mfma_f32_16x16x32_f16 with the decoded rows as the A operand (lane = token, 8 dims =
//    one packed dword + its group scale) and the query slice as B, giving S^T blocks whose lanes
//    hold 4 tokens of one head. The four per-wave partial score blocks are summed through LDS
//    (reduce-scatter: wave h owns head block h).
//  * Online softmax in FP32 (base-2, log2(e) folded into the scale) on the owning wave; the
//    probabilities are rounded to FP16 and, thanks to the S^T layout, each lane already holds the
//    8 token-slots of one head that form an MFMA A fragment, so P goes to LDS as 16-byte
//    fragments with no transpose.
//  * PV: each wave multiplies P by its 128-dim slice of the latent. The B operand needs 8 tokens
//    of one dim per lane: a lane reads one code dword (8 dims) from each of 8 rows, interleaves
//    the nibbles of token pairs, converts with v_cvt_scalef32_pk_f16_fp4 and applies the two
//    tokens' scales with one packed FP16 multiply; the 8 nibble positions feed 8 MFMAs whose
//    output columns are dims 8n+c.
//  * Splits write normalised partial outputs and their log-sum-exp; combine_kernel merges them
//    in split order (deterministic). With a single split the kernel writes the final output.
//  * Workgroup i is placed on XCD i % 8 by the hardware; items are remapped so that the splits
//    of one token are consecutive on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "nvfp4_device.h"

#define LDS_AS __attribute__((address_space(3)))

namespace mla {

constexpr int kTileRows = 32;
constexpr int kPiecesPerTile = kTileRows * kRowBytes / 16;   // 704 16-byte pieces
constexpr int kLoadsPerWave = 3;                              // 3 x 4 waves x 64 lanes = 768
constexpr int kStageBytes = kLoadsPerWave * 4 * 64 * 16;      // 12 KiB per ring slot
constexpr int kNBuf = 3;
constexpr uint32_t kInvalid = 0xFFFFFFFFu;

// Source of every load that has no row behind it (padding rows, padding pieces, bad pages).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[512] = {0};

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

__device__ __forceinline__ half8v q_to_half8(const void* q, int64_t off, bool fp32) {
  half8v h;
  if (fp32) {
    const float4v a = *(const float4v*)((const float*)q + off);
    const float4v b = *(const float4v*)((const float*)q + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = (_Float16)a[i]; h[4 + i] = (_Float16)b[i]; }
  } else {
    const uint4v u = *(const uint4v*)((const uint16_t*)q + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (_Float16)__uint_as_float(u[i] << 16);
      h[2 * i + 1] = (_Float16)__uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
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

template <int NH, bool DENSE>
__global__ __launch_bounds__(256, (NH <= 2) ? 2 : 1) void decode_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[kNBuf][kStageBytes];
  __shared__ __attribute__((aligned(16))) float4v sred[4][NH][2][64];
  __shared__ __attribute__((aligned(16))) half8v pbuf[NH][64];
  __shared__ __attribute__((aligned(16))) float alpha_s[64];
  __shared__ int32_t rescale_s[4];
  __shared__ __attribute__((aligned(16))) float mfin[64];
  __shared__ __attribute__((aligned(16))) float lfin[64];
  __shared__ uint32_t rowoff[DENSE ? kMaxDensePages : kMaxSplitRows];
  __shared__ int32_t wave_cnt[4];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;

  const int hw = blockIdx.x;
  const int item = (hw & 7) * a.items_per_xcd + (hw >> 3);
  if (item >= a.total_items) return;
  const int split = item % a.n_split;
  const int rest = item / a.n_split;
  const int hg = a.hg_begin + rest % a.n_hg;
  const int tok = rest / a.n_hg;
  const int b = tok / a.q_len, t = tok % a.q_len;
  const int head0 = hg * 16 * NH;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // ---- rows of this split -------------------------------------------------------------------
  int n_rows;
  int p0 = 0;
  if constexpr (!DENSE) {
    // Compact the valid entries of [e0, e1) into rowoff (16-byte units), in list order.
    const int e0 = split * a.split_rows;
    const int cnt = max(0, min(a.topk, e0 + a.split_rows) - e0);
    const int per_w = ((cnt + 3) / 4 + 63) & ~63;          // <= 512 entries, 8 rounds of 64
    const int32_t* idx = a.topk_idx + (int64_t)tok * a.topk + e0;
    uint32_t offs[8];
    uint64_t masks[8];
    int mine = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int e = w * per_w + r * 64 + lane;
      bool ok = false;
      uint32_t o16 = 0;
      if (r * 64 < per_w && e < cnt) {
        const int j = idx[e];
        if (j >= 0 && j < a.max_pages * kPageRows) {
          const int pg = bt[j >> 6];
          if (pg >= 0) {
            const int64_t off = (int64_t)pg * a.page_stride + (int64_t)(j & 63) * kRowBytes;
            if (off + kRowBytes <= a.cache_bytes) { ok = true; o16 = (uint32_t)(off >> 4); }
          }
        }
      }
      masks[r] = __ballot(ok);
      offs[r] = o16;
      mine += __popcll(masks[r]);
    }
    if (lane == 0) wave_cnt[w] = mine;
    lds_barrier();
    int base = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) base += (v < w) ? wave_cnt[v] : 0;
    n_rows = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(masks[r] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)masks[r], 0u));
      if ((masks[r] >> lane) & 1ull) rowoff[base + below] = offs[r];
      base += __popcll(masks[r]);
    }
  } else {
    const int seq = min(a.seq_lens[b], a.max_pages * kPageRows);
    const int vis = seq - a.q_len + 1 + t;                 // positions 0 .. vis-1
    p0 = split * a.split_rows;
    n_rows = max(0, min(vis, p0 + a.split_rows) - p0);
    const int n_pages = (n_rows + 63) >> 6;
    for (int i = tid; i < n_pages; i += 256) {
      const int pg = bt[(p0 >> 6) + i];
      const int64_t off = (int64_t)pg * a.page_stride;
      rowoff[i] = (pg < 0) ? kInvalid : (uint32_t)(off >> 4);
    }
  }
  lds_barrier();

  // ---- query slice (FP16) ---------------------------------------------------------------------
  half8v qa[NH][5];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    const int64_t qrow = ((int64_t)tok * a.H + head0 + 16 * hb + l16) * kQkDim;
#pragma unroll
    for (int c = 0; c < 4; ++c) qa[hb][c] = q_to_half8(a.q, qrow + 128 * w + 32 * kg + 8 * c, a.q_fp32);
    const half8v r = q_to_half8(a.q, qrow + kLatent + 16 * w + 8 * (kg & 1), a.q_fp32);
    qa[hb][4] = (kg < 2) ? r : half8v{};
  }
  // Make the query fragments opaque so the compiler keeps them in registers instead of
  // re-loading and re-converting them from memory inside the tile loop.
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int c = 0; c < 5; ++c) asm volatile("" : "+v"(qa[hb][c]));

  // ---- tile loader --------------------------------------------------------------------------
  // Each lane moves 16-byte pieces p = (j*4 + w)*64 + lane of the tile (22 pieces per row): the
  // row offsets are read from LDS together, then every lane issues its loads, with padding
  // pieces and rows past the end reading the zero row (no divergent branches).
  auto issue_tile = [&](int tile) {
    uint8_t* dst = stage[tile % kNBuf];
    uint32_t o16[kLoadsPerWave];
    int ri[kLoadsPerWave], piece[kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int p = min((j * 4 + w) * 64 + lane, kPiecesPerTile - 1);
      const int r = p / 22;
      piece[j] = p - r * 22;
      ri[j] = tile * kTileRows + r;
      const int rc = min(ri[j], n_rows - 1);
      if constexpr (!DENSE) {
        o16[j] = rowoff[rc];
      } else {
        const int pos = p0 + rc;
        const uint32_t pb = rowoff[(pos >> 6) - (p0 >> 6)];
        o16[j] = (pb == kInvalid) ? kInvalid : pb + (uint32_t)(pos & 63) * (kRowBytes / 16);
      }
    }
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int p = (j * 4 + w) * 64 + lane;
      bool ok = p < kPiecesPerTile && ri[j] < n_rows && o16[j] != kInvalid;
      if constexpr (DENSE) ok = ok && (int64_t)o16[j] * 16 + kRowBytes <= a.cache_bytes;
      const uint8_t* src = ok ? a.cache + (int64_t)o16[j] * 16 + piece[j] * 16
                              : g_zero_row + piece[j] * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (LDS_AS void*)(dst + (j * 4 + w) * 1024), 16, 0, 0);
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;       // owner waves: running max (log2 units) and sum
  float4v o[NH][8];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[hb][c] = float4v{0.f, 0.f, 0.f, 0.f};

  if (w >= NH && lane == 0) rescale_s[w] = 0;       // these waves own no head block
  const int n_tiles = (n_rows + kTileRows - 1) / kTileRows;
  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  for (int i = 0; i < n_tiles; ++i) {
    if (i + 1 < n_tiles) wait_vmcnt<kLoadsPerWave>(); else wait_vmcnt<0>();
    lds_barrier();                                   // tile i visible; slot (i-1)%3 free
    if (i + 2 < n_tiles) issue_tile(i + 2);
    const uint8_t* tb = stage[i % kNBuf];

    // -- QK: partial S^T over this wave's 144 dims, all heads -----------------------------------
    half8v kf[2][5];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint8_t* row = tb + (16 * h + l16) * kRowBytes;
      const uint4v cw = *(const uint4v*)(row + 64 * w + 16 * kg);
      const uint32_t sc = *(const uint16_t*)(row + kScaleOff + 8 * w + 2 * kg);
      const uint2v rp = *(const uint2v*)(row + kRopeOff + 16 * w + 8 * (kg & 1));
      const half2v s0 = scale_pair(sc & 0xFFu), s1 = scale_pair(sc >> 8);
      kf[h][0] = decode_fp4x8(cw[0], s0);
      kf[h][1] = decode_fp4x8(cw[1], s0);
      kf[h][2] = decode_fp4x8(cw[2], s1);
      kf[h][3] = decode_fp4x8(cw[3], s1);
      kf[h][4] = (kg < 2) ? decode_fp8x8(rp[0], rp[1]) : half8v{};
    }
    // chunk-major: consecutive MFMAs feed different accumulators (a dependent MFMA would wait
    // for its predecessor to drain)
    float4v acc[NH][2];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) { acc[hb][0] = float4v{0.f, 0.f, 0.f, 0.f}; acc[hb][1] = acc[hb][0]; }
#pragma unroll
    for (int c = 0; c < 5; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) acc[hb][h] = mfma16(kf[h][c], qa[hb][c], acc[hb][h]);
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {       // every block, the owner's too: no branch
      sred[w][hb][0][lane] = acc[hb][0];
      sred[w][hb][1][lane] = acc[hb][1];
    }
    lds_barrier();

    // -- online softmax on the owning wave ------------------------------------------------------
    if (w < NH) {
      float4v s0 = sred[0][w][0][lane], s1 = sred[0][w][1][lane];
#pragma unroll
      for (int src = 1; src < 4; ++src) { s0 += sred[src][w][0][lane]; s1 += sred[src][w][1][lane]; }
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ra = i * kTileRows + 4 * kg + r, rb = ra + 16;
        sv[r] = (ra < n_rows) ? s0[r] * a.scale_log2 : -INFINITY;
        sv[4 + r] = (rb < n_rows) ? s1[r] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(sv[r], sv[4 + r]));
      }
      mx = group4_max(mx);
      // The running max moves lazily: only when a tile's max exceeds it by more than 2^8, so the
      // probabilities stay <= 256 (exact range for FP16) and O is rescaled only on those tiles.
      const bool move = mx > m_run + 8.0f;        // also true on the first tile (m_run = -inf)
      const float m_new = move ? mx : m_run;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      half8v pf;
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(sv[e] - m_new);
        pf[e] = p;
        psum += (float)p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const uint64_t any = __ballot(move && i > 0);
      if (lane == 0) rescale_s[w] = any != 0ull;
      pbuf[w][lane] = pf;
      if (kg == 0) alpha_s[16 * w + l16] = alpha;
    }
    lds_barrier();

    // -- PV: this wave's 128 output dims, all heads ----------------------------------------------
    half8v pfr[NH];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) pfr[hb] = pbuf[hb][lane];
    const bool rescale = (rescale_s[0] | rescale_s[1] | rescale_s[2] | rescale_s[3]) != 0;
    // V fragments: 8 tokens of one dim per lane (the P fragment's token slots), decoded while the
    // P fragments are in flight.
    uint32_t D[8], SB[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int te = (e < 4) ? 4 * kg + e : 16 + 4 * kg + (e - 4);
      const uint8_t* row = tb + te * kRowBytes;
      D[e] = *(const uint32_t*)(row + 64 * w + 4 * l16);
      SB[e] = row[kScaleOff + 8 * w + (l16 >> 1)];
    }
    half8v v[8];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const uint32_t da = D[2 * pr], db = D[2 * pr + 1];
      const uint32_t ze = (da & 0x0F0F0F0Fu) | ((db & 0x0F0F0F0Fu) << 4);
      const uint32_t zo = ((da >> 4) & 0x0F0F0F0Fu) | (db & 0xF0F0F0F0u);
      const half2v sab = fp8x2_to_half2<false>(SB[2 * pr] | (SB[2 * pr + 1] << 8));
      half2v x;
      x = fp4x2_to_half2<0>(ze) * sab; v[0][2 * pr] = x[0]; v[0][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<0>(zo) * sab; v[1][2 * pr] = x[0]; v[1][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<1>(ze) * sab; v[2][2 * pr] = x[0]; v[2][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<1>(zo) * sab; v[3][2 * pr] = x[0]; v[3][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<2>(ze) * sab; v[4][2 * pr] = x[0]; v[4][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<2>(zo) * sab; v[5][2 * pr] = x[0]; v[5][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<3>(ze) * sab; v[6][2 * pr] = x[0]; v[6][2 * pr + 1] = x[1];
      x = fp4x2_to_half2<3>(zo) * sab; v[7][2 * pr] = x[0]; v[7][2 * pr + 1] = x[1];
    }
    if (rescale) {
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) {
        const float4v al = *(const float4v*)&alpha_s[16 * hb + 4 * kg];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[hb][c] *= al;
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) o[hb][c] = mfma16(pfr[hb], v[c], o[hb][c]);
  }

  // ---- normalise and write ------------------------------------------------------------------
  if (w < NH) {
    const float lt = group4_sum(l_run);
    if (kg == 0) { mfin[16 * w + l16] = m_run; lfin[16 * w + l16] = lt; }
  }
  lds_barrier();
  const bool final_out = (a.n_split == 1);
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    const float4v mm = *(const float4v*)&mfin[16 * hb + 4 * kg];
    const float4v ll = *(const float4v*)&lfin[16 * hb + 4 * kg];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = ll[r] > 0.0f ? 1.0f / ll[r] : 0.0f;
      const int head = head0 + 16 * hb + 4 * kg + r;
      float* dst = final_out
          ? a.out + ((int64_t)tok * a.H + head) * kLatent
          : a.ws_o + (((int64_t)tok * a.n_split + split) * a.H + head) * kLatent;
      dst += 128 * w + 8 * l16;
      const float4v lo = float4v{o[hb][0][r], o[hb][1][r], o[hb][2][r], o[hb][3][r]} * inv;
      const float4v hi = float4v{o[hb][4][r], o[hb][5][r], o[hb][6][r], o[hb][7][r]} * inv;
      *(float4v*)dst = lo;
      *(float4v*)(dst + 4) = hi;
      if (w == 0 && l16 == 0) {
        const float lse_v = ll[r] > 0.0f
            ? (mm[r] + __builtin_amdgcn_logf(ll[r])) * 0.69314718055994530942f : -INFINITY;
        if (final_out) {
          if (a.lse) a.lse[(int64_t)tok * a.H + head] = lse_v;
        } else {
          a.ws_lse[((int64_t)tok * a.n_split + split) * a.H + head] = lse_v;
        }
      }
    }
  }
}

// Merge the n_split partial (o_s, lse_s) of each (token, head) in split order:
// M = max lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s, lse = M + log(sum w_s).
__global__ __launch_bounds__(256) void combine_kernel(int32_t T, int32_t H, int32_t S,
                                                      const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_lse,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse,
                                                      int32_t per_xcd, int32_t total) {
  const int hw = blockIdx.x;
  const int L = (hw & 7) * per_xcd + (hw >> 3);
  if (L >= total) return;
  const int quads = H / 4;
  const int tok = L / quads;
  const int head = (L % quads) * 4 + (threadIdx.x >> 6);
  const int d = (threadIdx.x & 63) * 8;
  const float* lp = ws_lse + (int64_t)tok * S * H + head;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[(int64_t)s * H]);
  float4v acc0 = float4v{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  float wsum = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = lp[(int64_t)s * H];
      const float wgt = (ls == -INFINITY) ? 0.0f
                                          : __builtin_amdgcn_exp2f((ls - M) * 1.4426950408889634f);
      const float* op = ws_o + (((int64_t)tok * S + s) * H + head) * kLatent + d;
      acc0 += wgt * *(const float4v*)op;
      acc1 += wgt * *(const float4v*)(op + 4);
      wsum += wgt;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  float* dst = out + ((int64_t)tok * H + head) * kLatent + d;
  *(float4v*)dst = acc0 * inv;
  *(float4v*)(dst + 4) = acc1 * inv;
  if (lse && (threadIdx.x & 63) == 0)
    lse[(int64_t)tok * H + head] =
        (M == -INFINITY) ? -INFINITY : M + __builtin_amdgcn_logf(wsum) * 0.69314718055994530942f;
}

hipError_t launch_decode(const DecodeArgs& a, int nh, bool dense, hipStream_t stream) {
  const dim3 grid((unsigned)a.items_per_xcd * 8), block(256);
#define MLA_LAUNCH(NHV, DV) \
  hipLaunchKernelGGL((decode_kernel<NHV, DV>), grid, block, 0, stream, a)
  switch (nh * 2 + (dense ? 1 : 0)) {
    case 2: MLA_LAUNCH(1, false); break;
    case 3: MLA_LAUNCH(1, true); break;
    case 4: MLA_LAUNCH(2, false); break;
    case 5: MLA_LAUNCH(2, true); break;
    case 6: MLA_LAUNCH(3, false); break;
    case 7: MLA_LAUNCH(3, true); break;
    case 8: MLA_LAUNCH(4, false); break;
    case 9: MLA_LAUNCH(4, true); break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_combine(int32_t T, int32_t H, int32_t n_split, const float* ws_o,
                          const float* ws_lse, float* out, float* lse, hipStream_t stream) {
  const int32_t total = T * (H / 4);
  const int32_t per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)per_xcd * 8), dim3(256), 0, stream, T, H,
                     n_split, ws_o, ws_lse, out, lse, per_xcd, total);
  return hipGetLastError();
}

}  // namespace mla
