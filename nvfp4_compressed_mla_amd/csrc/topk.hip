// Top-k position selection from per-position scores: the indexer step before the decode path.
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Native NVFP4
// sparse MLA decode kernel": the sparse indexer picks, for every query token, the positions that
// attention reads (2048 per token), and unused list slots hold -1. Query token t of request b may
// pick among positions 0 .. seq_len - q_len + t; the k positions with the largest scores are
// kept, scores ordered by the IEEE-754 total order of their float32 value (-0 below +0) and equal
// scores by position (smaller first); the list holds them in ascending position order, then -1.
//
// Two launches, both exact:
//  1. topk_chunk_kernel: one workgroup per (token, 16384-position chunk) loads the chunk's keys
//     (order-preserving uint32 images of the scores) into LDS, finds the chunk's k-th largest key
//     by a 4 x 8-bit radix select (LDS histograms), and writes the chunk's top k (key, position)
//     in position order. The token's top k is contained in the union of its chunks' top k.
//  2. topk_merge_kernel: one workgroup per token selects the top k of that union the same way
//     and writes the positions in ascending order, padded with -1.
// Both emit in position order with a block-wide scan of (greater, equal-to-threshold) counts, so
// the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

constexpr int kTopkThreads = 512;
constexpr int kTopkPerThread = 8;                          // positions per thread per emit round
constexpr int kTopkRound = kTopkThreads * kTopkPerThread;  // 4096

// Order-preserving image of a float: a > b (IEEE total order) <=> key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of two counters (512 threads = 8 waves); also returns the totals.
__device__ __forceinline__ void block_scan2(int a, int b, int& a_ex, int& b_ex, int& a_tot, int& b_tot,
                                            int* wsum /* LDS [2][8] */) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ta = __shfl_up(ia, d), tb = __shfl_up(ib, d);
    if (lane >= d) { ia += ta; ib += tb; }
  }
  if (lane == 63) { wsum[wv] = ia; wsum[8 + wv] = ib; }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int v = 0; v < kTopkThreads / 64; ++v) {
    const int sa = wsum[v], sb = wsum[8 + v];
    pa += (v < wv) ? sa : 0;
    pb += (v < wv) ? sb : 0;
    ta += sa;
    tb += sb;
  }
  a_ex = pa + ia - a;
  b_ex = pb + ib - b;
  a_tot = ta;
  b_tot = tb;
  __syncthreads();                                         // wsum is reused by the next call
}

constexpr int kHistStride = 257;                          // padded: lanes hit different banks

// k-th largest of keys[0:m) (1 <= k <= m): returns the threshold key and, through `need`, how many
// keys equal to it belong to the top k (all keys above it do). Scores cluster in few values of
// the leading digit and LDS atomics on one address serialize, so lane l of every wave counts into
// histogram l % NSUB (rows padded to 257 words, so that one bin of different histograms falls in
// different banks); the NSUB histograms are summed before the digit is chosen.
template <int NSUB>
__device__ uint32_t radix_select(const uint32_t* keys, int m, int k, uint32_t* hist /* LDS NSUB x 257 */,
                                 int* state /* LDS 2 */, int& need) {
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* my_hist = hist + (lane % NSUB) * kHistStride;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NSUB * kHistStride; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int p0 = tid; p0 < m; p0 += 8 * kTopkThreads) {   // 8 LDS reads in flight per lane
      uint32_t kk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = p0 + j * kTopkThreads;
        kk[j] = (p < m) ? keys[p] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (p0 + j * kTopkThreads < m && (kk[j] & mask) == prefix)
          atomicAdd(&my_hist[(kk[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t tot = 0;
    if (tid < 256) {
#pragma unroll 16
      for (int h = 0; h < NSUB; ++h) tot += hist[h * kHistStride + tid];
    }
    __syncthreads();
    if (tid < 256) hist[tid] = tot;                        // histogram 0 now holds the sums
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255-4l .. 252-4l (descending); counts above a lane's bins by a scan
      int c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = (int)hist[255 - 4 * lane - j]; s += c[j]; }
      int inc = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(inc, d);
        if (lane >= d) inc += t;
      }
      int run = inc - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < rem && run + c[j] >= rem) { state[0] = 255 - 4 * lane - j; state[1] = rem - run; }
        run += c[j];
      }
    }
    __syncthreads();
    const int d = state[0];
    rem = state[1];
    prefix |= (uint32_t)d << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  need = rem;
  return prefix;
}

// Emit, in list order, the entries of keys[0:m) above thr plus the first `need` equal to it:
// payload(i) is fetched for every entry of a thread's round up front (so that its loads overlap),
// then emit(slot, payload) is called for the selected ones.
template <typename Payload, typename Emit>
__device__ void ordered_emit(const uint32_t* keys, int m, uint32_t thr, int need, int* wsum,
                             Payload payload, Emit emit) {
  int gc = 0, ec = 0;                                     // carried over rounds
  for (int r0 = 0; r0 < m; r0 += kTopkRound) {
    const int p0 = r0 + threadIdx.x * kTopkPerThread;
    uint32_t kk[kTopkPerThread];
    int32_t pl[kTopkPerThread];
    int g = 0, e = 0;
#pragma unroll
    for (int j = 0; j < kTopkPerThread; ++j) {
      const int p = p0 + j;
      kk[j] = (p < m) ? keys[p] : 0u;
      pl[j] = (p < m) ? payload(p) : 0;
      g += (p < m && kk[j] > thr);
      e += (p < m && kk[j] == thr);
    }
    int g_ex, e_ex, g_tot, e_tot;
    block_scan2(g, e, g_ex, e_ex, g_tot, e_tot, wsum);
    int gb = gc + g_ex, eb = ec + e_ex;
#pragma unroll
    for (int j = 0; j < kTopkPerThread; ++j) {
      const int p = p0 + j;
      if (p >= m) break;
      if (kk[j] > thr) {
        emit(gb + min(eb, need), p, pl[j]);
        ++gb;
      } else if (kk[j] == thr) {
        if (eb < need) emit(gb + eb, p, pl[j]);
        ++eb;
      }
    }
    gc += g_tot;
    ec += e_tot;
  }
}

__device__ __forceinline__ int visible(const int32_t* seq_lens, int tok, int q_len, int64_t n_max) {
  const int b = tok / q_len, t = tok - b * q_len;
  const int64_t v = (int64_t)seq_lens[b] - q_len + 1 + t;
  return (int)(v < 0 ? 0 : (v > n_max ? n_max : v));
}

__global__ __launch_bounds__(kTopkThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t n_max, const int32_t* __restrict__ seq_lens,
    int32_t q_len, int32_t k, int32_t n_chunks, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_pos, int32_t* __restrict__ cand_cnt) {
  __shared__ uint32_t keys[kTopkChunk];
  __shared__ uint32_t hist[64 * kHistStride];
  __shared__ int state[2];
  __shared__ int wsum[16];
  const int tok = blockIdx.x / n_chunks, c = blockIdx.x - tok * n_chunks;
  const int n = visible(seq_lens, tok, q_len, n_max);
  const int c0 = c * kTopkChunk;
  const int m = max(0, min(n - c0, kTopkChunk));
  const int64_t cbase = ((int64_t)tok * n_chunks + c) * k;
  if (threadIdx.x == 0) cand_cnt[(int64_t)tok * n_chunks + c] = min(m, k);
  if (m == 0) return;                                      // workgroup-uniform
  const float* row = scores + (int64_t)tok * n_max + c0;
  {
    // every load of the chunk in flight at once (32 per thread), then the keys to LDS
    constexpr int kPer = kTopkChunk / kTopkThreads;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = threadIdx.x + j * kTopkThreads;
      v[j] = (p < m) ? row[p] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = threadIdx.x + j * kTopkThreads;
      if (p < m) keys[p] = score_key(v[j]);
    }
  }
  __syncthreads();
  int need = k;                                            // m <= k: keep everything
  const uint32_t thr = (m > k) ? radix_select<64>(keys, m, k, hist, state, need) : 0u;   // 0: below every finite key
  ordered_emit(keys, m, thr, need, wsum, [&](int p) { return c0 + p; },
               [&](int slot, int p, int32_t pos) {
                 cand_key[cbase + slot] = keys[p];
                 cand_pos[cbase + slot] = pos;
               });
}

__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    int64_t n_max, const int32_t* __restrict__ seq_lens, int32_t q_len, int32_t k,
    int32_t n_chunks, const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
    const int32_t* __restrict__ cand_cnt, int32_t* __restrict__ out) {
  __shared__ uint32_t keys[kTopkMaxChunks * kTopkMaxK];
  __shared__ uint32_t hist[16 * kHistStride];
  __shared__ int state[2];
  __shared__ int wsum[16];
  __shared__ int coff[kTopkMaxChunks + 1];
  const int tok = blockIdx.x;
  const int64_t tbase = (int64_t)tok * n_chunks;
  if (threadIdx.x == 0) {
    int o = 0;
    for (int c = 0; c < n_chunks; ++c) { coff[c] = o; o += cand_cnt[tbase + c]; }
    coff[n_chunks] = o;
  }
  __syncthreads();
  const int total = coff[n_chunks];
  {
    // all candidate loads in flight at once (at most 13 chunks x 4 per thread), then to LDS
    constexpr int kPerChunk = kTopkMaxK / kTopkThreads;
    uint32_t v[kTopkMaxChunks][kPerChunk];
#pragma unroll
    for (int c = 0; c < kTopkMaxChunks; ++c)
#pragma unroll
      for (int j = 0; j < kPerChunk; ++j) {
        const int i = threadIdx.x + j * kTopkThreads;
        const bool ok = c < n_chunks && i < coff[min(c + 1, n_chunks)] - coff[min(c, n_chunks)];
        v[c][j] = ok ? cand_key[(tbase + c) * k + i] : 0u;
      }
#pragma unroll
    for (int c = 0; c < kTopkMaxChunks; ++c)
#pragma unroll
      for (int j = 0; j < kPerChunk; ++j) {
        const int i = threadIdx.x + j * kTopkThreads;
        if (c < n_chunks && i < coff[c + 1] - coff[c]) keys[coff[c] + i] = v[c][j];
      }
  }
  __syncthreads();
  int need = k;
  const uint32_t thr = (total > k) ? radix_select<16>(keys, total, k, hist, state, need) : 0u;
  int32_t* orow = out + (int64_t)tok * k;
  int c = 0;                                               // chunk of the last candidate seen
  ordered_emit(keys, total, thr, need, wsum,
               [&](int i) {
                 while (c + 1 < n_chunks && coff[c + 1] <= i) ++c;   // i increases within a thread
                 return cand_pos[(tbase + c) * k + (i - coff[c])];
               },
               [&](int slot, int, int32_t pos) { orow[slot] = pos; });
  for (int s = min(total, k) + threadIdx.x; s < k; s += kTopkThreads) orow[s] = -1;
}

hipError_t launch_topk(const float* scores, int64_t n_max, const int32_t* seq_lens, int32_t T,
                       int32_t q_len, int32_t k, void* workspace, int32_t* out, hipStream_t stream) {
  const int32_t n_chunks = (int32_t)((n_max + kTopkChunk - 1) / kTopkChunk);
  uint32_t* cand_key = (uint32_t*)workspace;
  int32_t* cand_pos = (int32_t*)(cand_key + (int64_t)T * n_chunks * k);
  int32_t* cand_cnt = cand_pos + (int64_t)T * n_chunks * k;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)(T * n_chunks)), dim3(kTopkThreads), 0, stream,
                     scores, n_max, seq_lens, q_len, k, n_chunks, cand_key, cand_pos, cand_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)T), dim3(kTopkThreads), 0, stream, n_max,
                     seq_lens, q_len, k, n_chunks, cand_key, cand_pos, cand_cnt, out);
  return hipGetLastError();
}

}  // namespace mla
