// Union of the index lists of groups of consecutive query tokens (the shared-row decode's input).
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Native NVFP4
// sparse MLA decode kernel": each query token attends to the rows its indexer selected, and the
// decode launch carries several query tokens of a request at once (15 per launch in the page's
// figure). When those tokens select overlapping rows, a row gathered and decoded once can serve
// every token that selected it. This kernel lists, for each group of up to 4 consecutive query
// tokens of one request, the distinct positions their lists hold, in ascending order, with a
// 4-bit mask per position (bit u: token 4g+u selected it). Entries outside [0, n_pos) (-1 padding
// included) are left out, as the decode leaves them out; a position that one token's list holds
// twice is listed once.
//
// The positions [0, n_pos) of a group are cut into kUnionParts equal ranges, one workgroup each
// (256 threads): it reads the group's lists (the same 32 KB for every part, from the L2), marks
// the entries of its range in a bitmap of 4-bit cells in LDS with atomic ORs, counts the occupied
// cells of a contiguous run of words per thread, and after a workgroup scan writes its part of the
// union in position order, with its size. The union of a group is the concatenation of its parts
// in part order (the decode kernel reads it that way, from the part sizes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

constexpr int kUnionThreads = 256;
constexpr int kUnionPartWords = kUnionMaxPos / kUnionParts / 8;   // LDS words of one part

// Bit 4k of the result is set when 4-bit cell k of x is not zero.
__device__ __forceinline__ uint32_t occupied_cells(uint32_t x) {
  return (x | (x >> 1) | (x >> 2) | (x >> 3)) & 0x11111111u;
}

__global__ __launch_bounds__(kUnionThreads) void union_kernel(
    const int32_t* __restrict__ topk_idx, int32_t topk, int32_t q_len, int32_t groups_per_req,
    int32_t n_pos, int32_t part_pos, int32_t* __restrict__ u_pos, uint8_t* __restrict__ u_mask,
    int32_t* __restrict__ u_count, int32_t u_stride) {
  __shared__ uint32_t cell[kUnionPartWords];             // 8 positions (4 bits each) per word
  __shared__ int32_t wave_total[kUnionThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = blockIdx.x / kUnionParts, part = blockIdx.x % kUnionParts;
  const int b = grp / groups_per_req, t0 = 4 * (grp % groups_per_req);
  const int nt = min(4, q_len - t0);
  const int lo = part * part_pos;                         // this part: positions [lo, hi)
  const int hi = min(n_pos, lo + part_pos);
  const int words = max(0, (hi - lo + 7) >> 3);
  // every list entry of the group is loaded before the bitmap is cleared and set, so that the
  // loads are in flight together
  constexpr int kPer = 4 * kUnionMaxTopk / kUnionThreads;   // entries per thread
  int jv[kPer];
  const int n_ent = nt * topk;
  const int32_t* idx = topk_idx + ((int64_t)b * q_len + t0) * topk;   // the group's lists, contiguous
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kUnionThreads + tid;
    jv[k] = (e < n_ent) ? idx[e] : -1;
  }
  for (int i = tid; i < words; i += kUnionThreads) cell[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kUnionThreads + tid;
    const int j = jv[k];
    if (j >= lo && j < hi) atomicOr(&cell[(j - lo) >> 3], 1u << (4 * ((j - lo) & 7) + e / topk));
  }
  __syncthreads();
  const int per = (words + kUnionThreads - 1) / kUnionThreads;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  int cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(occupied_cells(cell[i]));
  // exclusive scan of the counts over the workgroup (thread order = position order)
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_total[wv] = incl;
  __syncthreads();
  int base = incl - cnt, total = 0;
#pragma unroll
  for (int v = 0; v < kUnionThreads / 64; ++v) {
    const int c = wave_total[v];
    base += (v < wv) ? c : 0;
    total += c;
  }
  int32_t* op = u_pos + ((int64_t)grp * kUnionParts + part) * u_stride;
  uint8_t* om = u_mask + ((int64_t)grp * kUnionParts + part) * u_stride;
  for (int i = w0; i < w1; ++i) {
    const uint32_t x = cell[i];
    uint32_t occ = occupied_cells(x);
    while (occ) {
      const int k = __ffs(occ) - 1;                     // bit 4*cell
      op[base] = lo + 8 * i + (k >> 2);
      om[base] = (uint8_t)((x >> k) & 0xFu);
      ++base;
      occ &= occ - 1;
    }
  }
  if (tid == 0) u_count[grp * kUnionParts + part] = total;
}

hipError_t launch_union(const int32_t* topk_idx, int32_t topk, int32_t B, int32_t q_len,
                        int32_t n_pos, int32_t* u_pos, uint8_t* u_mask, int32_t* u_count,
                        int32_t u_stride, hipStream_t stream) {
  if (n_pos < 1 || n_pos > kUnionMaxPos || topk < 1 || topk > kUnionMaxTopk) return hipErrorInvalidValue;
  const int32_t gpr = (q_len + 3) / 4;
  const int32_t part_pos = ((n_pos + kUnionParts - 1) / kUnionParts + 7) / 8 * 8;
  hipLaunchKernelGGL(union_kernel, dim3((unsigned)(B * gpr * kUnionParts)), dim3(kUnionThreads), 0,
                     stream, topk_idx, topk, q_len, gpr, n_pos, part_pos, u_pos, u_mask, u_count,
                     u_stride);
  return hipGetLastError();
}

}  // namespace mla
