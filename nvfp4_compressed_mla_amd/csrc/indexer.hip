// Indexer scores: the FP8 scoring pass that feeds top-k position selection.
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Native NVFP4
// sparse MLA decode kernel": the decode reads the positions a sparse indexer selected, 2048 per
// query token (section "Decode: NVFP4 KV compression"); section "Making room for low-latency
// decode" keeps the indexer's own cache state unchanged beside the compressed MLA rows. The page
// does not define the indexer's scoring function. The reading implemented here (synthetic, no
// trained weights): every position s holds a 128-dim E4M3 indexer key k_s with a positive fp32
// scale c_s; query token t has 64 E4M3 indexer heads q_{t,j} (128 dims) and fp32 head weights
// w_{t,j}; the score is
//     score[t, s] = c_s * sum_j w_{t,j} * max(0, q_{t,j} . k_s).
// Token t of a request with seq_len positions and q_len query tokens scores positions
// 0 .. seq_len - q_len + t (the causal window the top-k step selects from).
//
// Indexer cache page (64 positions, MLA_INDEXER_PAGE_BYTES = 8448): 64 keys of 128 bytes, then 64
// fp32 scales. Pages are found through the request's block table, as the MLA rows are.
//
// MI355X design. One workgroup (8 waves) per (request, block of at most 512 positions, sized
// so that one launch fills two workgroups per CU); two workgroups per CU. The block's keys are staged once in LDS (64 KB, 16-byte pieces XOR-swizzled by row so
// that the operand reads are free of bank conflicts) and reused by every query token of the
// request: wave w scores tokens w, w+8, ... Per token the wave holds the queries of the 64 heads
// as four A operands (32 VGPRs) and runs v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit
// block scales, FP32 accumulation: the whole 128-dim dot product in one instruction) over
// 16-position tiles, four tiles at a time: a lane holds 4 heads of one position per MFMA and
// applies the ReLU and the head weights; lane swaps then sum the four lane groups so that lane
// group g ends with the whole score of tile g, and every lane stores one position. Products of two E4M3 values
// are exact in FP32, so the only rounding is the FP32 accumulation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"
#include "nvfp4_device.h"

namespace mla {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxThreads = 512;
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kIdxBlockRows = 512;                      // positions per workgroup, at most
constexpr int kIdxScaleOff = kPageRows * kIndexerDim;   // 8192: scales after the keys

// ReLU on the bits: a negative float (-0.0 included) has the sign bit set and so is a negative
// int, which the max replaces by 0 (= +0.0f); a positive float is a positive int and passes
// unchanged. One v_max_i32 with an inline 0 (a float max would add a NaN-canonicalising max, and a
// v_med3_f32 needs FLT_MAX in a register); exact here because the dot products are sums of exact
// products of finite E4M3 values, never NaN.
__device__ __forceinline__ float idx_relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__global__ __launch_bounds__(kIdxThreads, 2) void indexer_kernel(const IndexerArgs a) {
  // key r, 16-byte piece c (dims 16c..16c+15) at r*128 + 16*(c ^ (r & 7))
  __shared__ __attribute__((aligned(16))) uint8_t keys[kIdxBlockRows * kIndexerDim];
  __shared__ float kscale[kIdxBlockRows];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int b = blockIdx.y;
  const int p0 = blockIdx.x * a.block_rows;
  const int64_t n_cols = min((int64_t)a.n_max, (int64_t)a.max_pages * kPageRows);
  const int n_pos = (int)min((int64_t)a.seq_lens[b], n_cols);     // positions any token may see
  if (p0 >= n_pos) return;
  const int rows = min(a.block_rows, n_pos - p0);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // ---- stage the block's keys and scales (an unmapped or out-of-cache page reads as zeros) ----
  {
    const int c = tid & 7;
#pragma unroll 4
    for (int i = 0; i < kIdxBlockRows * 8 / kIdxThreads; ++i) {
      const int r = (tid >> 3) + (kIdxThreads / 8) * i;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows) {
        const int pos = p0 + r;
        const int pg = bt[pos >> 6];
        const int64_t off = (int64_t)pg * a.page_stride;
        if (pg >= 0 && off + kIndexerPageBytes <= a.cache_bytes)
          v = *(const uint4*)(a.cache + off + (int64_t)(pos & 63) * kIndexerDim + 16 * c);
      }
      *(uint4*)(keys + r * kIndexerDim + ((c ^ (r & 7)) << 4)) = v;
    }
    for (int r = tid; r < kIdxBlockRows; r += kIdxThreads) {
      float s = 0.0f;
      if (r < rows) {
        const int pos = p0 + r;
        const int pg = bt[pos >> 6];
        const int64_t off = (int64_t)pg * a.page_stride;
        if (pg >= 0 && off + kIndexerPageBytes <= a.cache_bytes)
          s = *(const float*)(a.cache + off + kIdxScaleOff + 4 * (pos & 63));
      }
      kscale[r] = s;
    }
  }
  __syncthreads();

  // ---- score: wave w takes query tokens w, w+8, ... ------------------------------------------
  // The wave index goes through a scalar register, so that everything per token is known to be
  // wave-uniform: the output's buffer resource then lives in scalar registers (a resource in
  // vector registers costs a compare-and-branch loop around every store).
  const int wu = __builtin_amdgcn_readfirstlane(w);
  for (int t = wu; t < a.q_len; t += kIdxWaves) {
    const int64_t tok = (int64_t)b * a.q_len + t;
    const int vis = min(a.seq_lens[b] - a.q_len + 1 + t, n_pos);   // positions 0 .. vis-1
    const int nr = min(vis - p0, a.block_rows);
    if (nr <= 0) continue;
    // A operands: lane (l16, kg) holds dims 32*kg .. 32*kg+31 of head 16*hb + l16; the B
    // operands (keys) below use the same lane -> dims map, so the MFMA sums all 128 dims.
    i32x8 qa[4];
    f32x4 wv[4];                               // weights of heads 16*hb + 4*kg + e (output rows)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const uint4* src = (const uint4*)(a.q + (tok * kIndexerHeads + 16 * hb + l16) * kIndexerDim + 32 * kg);
      const uint4 lo = src[0], hi = src[1];
      qa[hb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      wv[hb] = *(const f32x4*)(a.weights + tok * kIndexerHeads + 16 * hb + 4 * kg);
    }
    // The row's visible part as a buffer resource (0x00020000: raw 32-bit dwords on gfx9): the
    // hardware drops stores at offsets past nr positions, so the epilogue needs no branch.
    const __amdgpu_buffer_rsrc_t out_rs =
        __builtin_amdgcn_make_buffer_rsrc(a.scores + tok * a.n_max + p0, (short)0, nr * 4, 0x00020000);
    const int n_kt = (nr + 15) >> 4;
    // Lane l16 reads row l16 of every tile; rows step by 16, so the swizzle (row & 7 = l16 & 7)
    // is fixed.
    const uint8_t* kr0 = keys + l16 * kIndexerDim;
    const int koff0 = ((2 * kg) ^ (l16 & 7)) << 4, koff1 = ((2 * kg + 1) ^ (l16 & 7)) << 4;
    // Four 16-position tiles per step. n_kt <= 32, so tiles kt0 .. kt0 + 3 (kt0 < n_kt, a
    // multiple of 4) stay inside the 512 staged rows; rows past the block's end hold zeros and
    // their sums are not stored.
    auto kfrag = [&](int tile) -> i32x8 {
      const uint8_t* kr = kr0 + tile * 16 * kIndexerDim;
      const uint4 k0 = *(const uint4*)(kr + koff0);
      const uint4 k1 = *(const uint4*)(kr + koff1);
      return i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
    };
    i32x8 kn = kfrag(0);
    for (int kt0 = 0; kt0 < n_kt; kt0 += 4) {
      float part[4];                           // this lane group's 16 heads, tile kt0 + u
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x8 kb = kn;
        kn = kfrag(min(kt0 + u + 1, 31));      // the next tile's keys, read under this tile's work
        f32x4 d[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          // E4M3 x E4M3 (format 0 for both operands), E8M0 block scales 127 = 1.0
          d[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[hb], kb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        // ReLU and head weights: one weighted chain over the lane's 16 heads
        float s = wv[0][0] * idx_relu(d[0][0]);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int e = (hb == 0 ? 1 : 0); e < 4; ++e) s = __builtin_fmaf(wv[hb][e], idx_relu(d[hb][e]), s);
        part[u] = s;
      }
      // Reduce-scatter over the four lane groups: the 32-lane swaps pair groups g and g + 2
      // (the lower half keeps tiles 0 and 1, the upper half tiles 2 and 3), the 16-lane swap
      // pairs g and g + 1, so lane group kg ends with the whole sum of tile kt0 + kg.
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float r0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      const float r1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(r0), __float_as_uint(r1), false, false);
      const int r = (kt0 + kg) * 16 + l16;
      const float s = (__uint_as_float(z[0]) + __uint_as_float(z[1])) * kscale[r];
      // every lane stores its own position; offsets past the row are dropped
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), out_rs, 4 * r, 0, 0);
    }
  }
}

hipError_t launch_indexer(const IndexerArgs& a_in, hipStream_t stream) {
  IndexerArgs a = a_in;
  const int64_t n_cols = std::min<int64_t>(a.n_max, (int64_t)a.max_pages * kPageRows);
  // positions per workgroup: a multiple of 64, at most 512, and small enough that the launch
  // fills the two workgroup slots of every CU when it can (512 workgroups)
  const int64_t per = ((int64_t)a.B * n_cols + 511) / 512;
  a.block_rows = (int32_t)std::min<int64_t>(kIdxBlockRows, std::max<int64_t>(64, (per + 63) / 64 * 64));
  const dim3 grid((unsigned)((n_cols + a.block_rows - 1) / a.block_rows), (unsigned)a.B);
  hipLaunchKernelGGL(indexer_kernel, grid, dim3(kIdxThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
