// Top-k position selection from per-position scores: the indexer step before the decode path.
//
// Page "Prime Inference: Fast, Reliable Serving for Frontier Open Models", section "Native NVFP4
// sparse MLA decode kernel": the sparse indexer picks, for every query token, the positions that
// attention reads (2048 per token), and unused list slots hold -1. Query token t of request b may
// pick among positions 0 .. seq_len - q_len + t; the k positions with the largest scores are
// kept, scores ordered by the IEEE-754 total order of their float32 value (-0 below +0) and equal
// scores by position (smaller first); the list holds them in ascending position order, then -1.
//
// Two launches, both exact (every score is compared as an order-preserving uint32 key):
//  1. topk_filter_kernel, one workgroup per (token, slice of positions). Every workgroup of a
//     token draws the same sample of 2048 scores (256 evenly spaced runs of 8) and takes the
//     sample's r-th largest key, low 8 bits cleared, as a cut L, r chosen so that the number of
//     positions with a key >= L lies between k and the merge's capacity with overwhelming
//     probability. Each wave then streams its contiguous segment of the slice and appends the
//     positions with key >= L, in position order, to the segment's list (ballot + mbcnt; no
//     atomics, no histogram over the whole row).
//  2. topk_merge_kernel, one workgroup per token. If every list fitted and the lists hold between
//     k and 8192 entries, they contain the exact top k (every other key is below L, and L is at
//     most the k-th largest candidate), so the k-th largest candidate is found by a radix select
//     in LDS (12-bit digits of the key's offset from the smallest candidate) and the positions
//     are written in ascending order. Otherwise (a sample that missed, heavy ties) the workgroup selects from the
//     token's full row itself: the same radix select and ordered emission, reading the scores
//     from memory; slow, but exact. Tokens with at most 8192 visible positions are selected
//     directly from their row in LDS.
// The emission ranks every entry by wave ballots and a scan of the per-wave counts of (greater,
// equal-to-threshold) entries, so the result is deterministic. Wave-level scans and reductions use
// DPP row shifts and row broadcasts (no LDS round trip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {

constexpr int kFilterThreads = 512;
constexpr int kSegsPerSlice = kFilterThreads / 64;         // one list segment per filter wave
constexpr int kMergeThreads = 1024;
constexpr int kTopkRound = 8192;                           // emit round: one round for LDS lists
constexpr int kTopkSampleRuns = kTopkSample / 8;           // runs of 8 consecutive positions
constexpr int kFilterUnroll = 32;                          // loads in flight per lane
constexpr int kBins = 4096;                                // 12-bit digits

// Order-preserving image of a float: a > b (IEEE total order) <=> key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// x moved by a DPP pattern; lanes without a source (or in rows outside ROW_MASK) get `fill`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t fill, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive scan of the 64 lanes of a wave under `op`, `id` its identity: shifts by 1, 2, 4 and
// 8 lanes inside each row of 16, then the last lane of row 0 (2) into row 1 (3), and of row 1
// into rows 2 and 3.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_move<0x111, 0xF>(id, x));                // row_shr:1
  x = op(x, dpp_move<0x112, 0xF>(id, x));                // row_shr:2
  x = op(x, dpp_move<0x114, 0xF>(id, x));                // row_shr:4
  x = op(x, dpp_move<0x118, 0xF>(id, x));                // row_shr:8
  x = op(x, dpp_move<0x142, 0xA>(id, x));                // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_move<0x143, 0xC>(id, x));                // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ int wave_incl_sum(int x) {
  return (int)wave_scan((uint32_t)x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Block-wide exclusive sum over the NT threads (also the total). No barrier at the end: the
// caller passes one before wsum is written again.
template <int NT>
__device__ __forceinline__ int block_excl_sum(int a, int& tot, int* wsum /* LDS NT / 64 */) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ia = wave_incl_sum(a);
  if (lane == 63) wsum[wv] = ia;
  __syncthreads();
  int pa = 0, ta = 0;
#pragma unroll
  for (int v = 0; v < NT / 64; ++v) {
    const int sa = wsum[v];
    pa += (v < wv) ? sa : 0;
    ta += sa;
  }
  tot = ta;
  return pa + ia - a;
}

// Smallest and largest of key_at(0 .. m-1) (m >= 1), the same in every thread.
template <int NT, typename KeyAt>
__device__ void block_minmax(KeyAt key_at, int m, uint32_t& mn, uint32_t& mx, uint32_t* red /* LDS NT / 32 */) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t a = 0xFFFFFFFFu, b = 0u;
  for (int p = threadIdx.x; p < m; p += NT) {
    const uint32_t v = key_at(p);
    a = min(a, v);
    b = max(b, v);
  }
  a = wave_scan(a, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return min(x, y); });
  b = wave_scan(b, 0u, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 63) { red[wv] = a; red[W + wv] = b; }
  __syncthreads();
  mn = red[0];
  mx = red[W];
#pragma unroll
  for (int v = 1; v < W; ++v) { mn = min(mn, red[v]); mx = max(mx, red[W + v]); }
}

// k-th largest of key_at(0 .. m-1) (1 <= k <= m), all keys >= base and key - base < 2^(hi+1).
// The offsets d = key - base (same order as the keys) are resolved as radix digits of up to 12
// bits from bit hi down, at most `max_passes` of them (fewer passes leave the unresolved low bits
// zero: a lower bound of the k-th largest). Returns the threshold and, through `need`, how many
// keys equal to it belong to the top k (all keys above it do). Each pass counts the offsets that
// match the resolved prefix into a 4096-bin LDS histogram (two buffers: the next one is cleared
// while this one fills); thread t owns the B = 4096 / NT bins 4095 - B t - j (j < B), so a block
// scan of their sums gives the number of keys above them.
// REFINE: once the resolved bin holds at most 64 keys, they are gathered into LDS and one wave
// ranks them exactly (each lane counts the keys above and equal to its own), which ends the
// selection with the same threshold and count as further passes would. CLEARED: the caller
// has zeroed the first histogram buffer and state[3] (and synchronized).
template <int NT, bool REFINE = false, bool CLEARED = false, typename KeyAt>
__device__ uint32_t select_kth(KeyAt key_at, int m, int k, uint32_t base, int hi, int max_passes,
                               uint32_t* hist /* LDS 2 x 4096 */, int* wsum, int* state /* LDS 4 */,
                               int& need) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = (hi >= 31) ? 0u : ~((2u << hi) - 1u);
  int rem = k;
  constexpr int B = kBins / NT;
  if constexpr (!CLEARED) {
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    if (tid == 0) state[3] = 0;
    __syncthreads();
  }
  for (int pass = 0; hi >= 0 && pass < max_passes; ++pass) {
    const int shift = max(hi - 11, 0);
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
    uint32_t* h = hist + (pass & 1) * kBins;
    uint32_t* h_next = hist + ((pass + 1) & 1) * kBins;
    for (int p0 = tid; p0 < m; p0 += 8 * NT) {             // 8 reads in flight per lane
      uint32_t dd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = p0 + j * NT;
        dd[j] = (p < m) ? key_at(p) - base : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (p0 + j * NT < m && (dd[j] & mask) == prefix) atomicAdd(&h[(dd[j] >> shift) & dmask], 1u);
    }
    for (int i = tid; i < kBins; i += NT) h_next[i] = 0;
    __syncthreads();
    int c[B], sum = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) { c[j] = (int)h[kBins - 1 - B * tid - j]; sum += c[j]; }
    int tot;
    int run = block_excl_sum<NT>(sum, tot, wsum);
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (run < rem && run + c[j] >= rem) {
        state[0] = kBins - 1 - B * tid - j;
        state[1] = rem - run;
        state[2] = c[j];                                   // keys in the chosen bin
      }
      run += c[j];
    }
    __syncthreads();
    prefix |= (uint32_t)state[0] << shift;
    mask |= dmask << shift;
    rem = state[1];
    hi = shift - 1;
    if constexpr (REFINE) {
      if (hi >= 0 && state[2] <= 64) {                     // workgroup-uniform
        uint32_t* small = h_next;                          // cleared above, free until the next pass
        for (int p0 = tid; p0 < m; p0 += 8 * NT) {
          uint32_t dd[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int p = p0 + j * NT;
            dd[j] = (p < m) ? key_at(p) - base : 0u;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (p0 + j * NT < m && (dd[j] & mask) == prefix) small[atomicAdd(&state[3], 1)] = dd[j];
        }
        __syncthreads();
        if (tid < 64) {
          const int cnt = state[2];                        // == the entries gathered
          const uint32_t x = (tid < cnt) ? small[tid] : 0u;
          int gt = 0, eq = 0;
          for (int j = 0; j < cnt; ++j) {
            const uint32_t y = small[j];
            gt += (y > x);
            eq += (y == x);
          }
          if (tid < cnt && gt < rem && rem <= gt + eq) { state[0] = (int)x; state[1] = rem - gt; }
        }
        __syncthreads();
        need = state[1];
        return base + (uint32_t)state[0];
      }
    }
  }
  need = rem;
  return base + prefix;
}

// k-th largest of keys that sit in LDS (1 <= k <= m), on offsets from the smallest key.
template <int NT, typename KeyAt>
__device__ uint32_t select_kth_lds(KeyAt key_at, int m, int k, uint32_t* hist, int* wsum, int* state,
                                   uint32_t* red, int& need) {
  uint32_t mn, mx;
  block_minmax<NT>(key_at, m, mn, mx, red);
  if (mn == mx) { need = k; return mx; }
  return select_kth<NT, true>(key_at, m, k, mn, 31 - __builtin_clz(mx - mn), 3, hist, wsum, state, need);
}

// Emit, in list order, the entries of key_at(0 .. m-1) above thr plus the first `need` equal to
// it, as emit(slot, payload(i)). Rounds of 8192 entries: entry r0 + NT j + tid is thread tid's
// j-th, so an entry's rank is (counts of the waves' ballots of earlier (j, wave) pairs, scanned by
// wave 0) + (its rank in its own ballot).
template <int NT, typename KeyAt, typename Payload, typename Emit>
__device__ void ordered_emit(KeyAt key_at, int m, uint32_t thr, int need, int* cnt /* LDS 258 */,
                             Payload payload, Emit emit) {
  constexpr int kPer = kTopkRound / NT, kW = NT / 64;
  constexpr int kQ = kPer * kW;          // 128 (j, wave) pairs
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int gc = 0, ec = 0;                                     // carried over rounds
  for (int r0 = 0; r0 < m; r0 += kTopkRound) {
    const int jn = min(kPer, (m - r0 + NT - 1) / NT);   // rows present
    uint32_t kk[kPer];
    int32_t pl[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = r0 + j * NT + tid;
      kk[j] = (p < m) ? key_at(p) : 0u;
      pl[j] = (p < m) ? payload(p) : 0;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j >= jn) {                                       // workgroup-uniform
        if (lane == 0) { cnt[j * kW + w] = 0; cnt[kQ + j * kW + w] = 0; }
        continue;
      }
      const bool in = r0 + j * NT + tid < m;
      const uint64_t bg = __ballot(in && kk[j] > thr), be = __ballot(in && kk[j] == thr);
      if (lane == 0) { cnt[j * kW + w] = __popcll(bg); cnt[kQ + j * kW + w] = __popcll(be); }
    }
    __syncthreads();
    if (w == 0) {
      // lane l: pairs 2l and 2l + 1, for both counters; exclusive offsets replace the counts
      const int g0 = cnt[2 * lane], g1 = cnt[2 * lane + 1];
      const int e0 = cnt[kQ + 2 * lane], e1 = cnt[kQ + 2 * lane + 1];
      const int gi = wave_incl_sum(g0 + g1), ei = wave_incl_sum(e0 + e1);
      cnt[2 * lane] = gi - g0 - g1;
      cnt[2 * lane + 1] = gi - g1;
      cnt[kQ + 2 * lane] = ei - e0 - e1;
      cnt[kQ + 2 * lane + 1] = ei - e1;
      if (lane == 63) { cnt[2 * kQ] = gi; cnt[2 * kQ + 1] = ei; }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j >= jn) break;                                  // workgroup-uniform
      const bool in = r0 + j * NT + tid < m;
      const bool gt = in && kk[j] > thr, eq = in && kk[j] == thr;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      const int gb = gc + cnt[j * kW + w] +
                     (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bg, 0u));
      const int eb = ec + cnt[kQ + j * kW + w] +
                     (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
      if (gt) emit(gb + min(eb, need), pl[j]);
      else if (eq && eb < need) emit(gb + eb, pl[j]);
    }
    gc += cnt[2 * kQ];
    ec += cnt[2 * kQ + 1];
    __syncthreads();                                       // cnt is written again next round
  }
}

__device__ __forceinline__ int visible(const int32_t* seq_lens, int tok, int q_len, int64_t n_max) {
  const int b = tok / q_len, t = tok - b * q_len;
  const int64_t v = (int64_t)seq_lens[b] - q_len + 1 + t;
  return (int)(v < 0 ? 0 : (v > n_max ? n_max : v));
}

// Rank r of the cut in the sample (n > kTopkTakeAll). With e = k * 2048 / n sample entries
// expected among the top k, r = 1.5 e + 3 sqrt(e) + 2 puts the number of positions at or above
// the cut near 1.5 k + 3 sqrt(k n / 2048): above k, and below 8192 for k <= 2048, unless the
// sample is more than about five standard deviations off.
__device__ __forceinline__ int sample_rank(int k, int n) {
  const float e = (float)k * (float)kTopkSample / (float)n;
  const int r = (int)__builtin_ceilf(1.5f * e + 3.0f * __builtin_sqrtf(e)) + 2;
  return min(max(r, 1), kTopkSample);
}

// Position of sample entry i: run i / 8 of 256 evenly spaced runs of 8 positions.
__device__ __forceinline__ int sample_pos(int i, int n) {
  return (int)(((int64_t)(i >> 3) * n) / kTopkSampleRuns) + (i & 7);
}

// A wave-uniform pointer, rebuilt from scalar reads of its halves: a buffer resource made from
// it stays in scalar registers even where the compiler cannot prove the pointer uniform (a
// resource in vector registers costs a compare-and-branch loop around every access).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(kFilterThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t n_max, const int32_t* __restrict__ seq_lens,
    int32_t q_len, int32_t k, int64_t slice, int32_t n_slices, int32_t cap_seg,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_pos, int32_t* __restrict__ seg_cnt) {
  __shared__ uint32_t skeys[kTopkSample];
  __shared__ uint32_t hist[2 * kBins];
  __shared__ int wsum[kFilterThreads / 64];
  __shared__ int state[4];
  const int tok = blockIdx.x / n_slices, g = blockIdx.x - tok * n_slices;
  // the wave index through a scalar register: the segment, its positions and its buffer
  // resources are then known to be wave-uniform (a resource in vector registers costs a
  // compare-and-branch loop around every access)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t seg = ((int64_t)tok * n_slices + g) * kSegsPerSlice + w;
  const float* row = scores + (int64_t)tok * n_max;
  // this wave's segment of the slice, in batches of kFilterUnroll rows of 64 positions; the
  // first batch is loaded before the row length is known (bounded by the row's n_max entries)
  // and stays in flight while the cut is found
  const int64_t seg_len = slice / kSegsPerSlice;
  const int64_t p_begin = (int64_t)g * slice + w * seg_len;
  // A batch wholly before `lim` is read through a buffer resource over exactly its 64 x
  // kFilterUnroll entries (one load per entry with a constant lane offset, no address arithmetic;
  // every access is inside the resource); a batch that crosses `lim` re-reads entry lim - 1
  // (lim >= 1) for its positions at or past it, whose values are never selected (the selection
  // tests the position against the row's end).
  constexpr int64_t kBatch = 64 * kFilterUnroll;
  auto load_batch = [&](int64_t b0, int64_t lim, float (&v)[kFilterUnroll]) {
    if (b0 + kBatch <= lim) {                              // wave-uniform
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(row + b0), (short)0, (int)(4 * kBatch), 0x00020000);
#pragma unroll
      for (int j = 0; j < kFilterUnroll; ++j)
        v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, 256 * j, 0));
    } else {
#pragma unroll
      for (int j = 0; j < kFilterUnroll; ++j) v[j] = row[min(b0 + j * 64 + lane, lim - 1)];
    }
  };
  float cur[kFilterUnroll];
  load_batch(p_begin, min(p_begin + seg_len, n_max), cur);
  const int n = visible(seq_lens, tok, q_len, n_max);
  if (n <= kTopkTakeAll || (int64_t)g * slice >= n) {     // workgroup-uniform
    if (lane == 0) seg_cnt[seg] = 0;
    return;
  }
  const int64_t p_end = min(p_begin + seg_len, (int64_t)n);
  // the sample (identical in every workgroup of the token) and its cut: the top 24 bits of its
  // r-th largest key
#pragma unroll
  for (int j = 0; j < kTopkSample / kFilterThreads; ++j) {
    const int i = threadIdx.x * (kTopkSample / kFilterThreads) + j;
    skeys[i] = score_key(row[sample_pos(i, n)]);
  }
  __syncthreads();
  int unused;
  const uint32_t cut = select_kth<kFilterThreads>([&](int i) { return skeys[i]; }, kTopkSample, sample_rank(k, n),
                                  0u, 31, 2, hist, wsum, state, unused);
  // The segment's list through buffer resources of cap_seg entries (stores past the capacity are
  // skipped, while cnt keeps the true count).
  const __amdgpu_buffer_rsrc_t ck_rs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(cand_key + seg * cap_seg), (short)0, 4 * cap_seg, 0x00020000);
  const __amdgpu_buffer_rsrc_t cp_rs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(cand_pos + seg * cap_seg), (short)0, 4 * cap_seg, 0x00020000);
  int cnt = 0;
  // A cut at or above +0 (key >= 2^31): key(u) >= cut exactly when the score's bits, read as a
  // signed int, are >= cut - 2^31 (a negative score, -0 included, is a negative int and never
  // reaches it; a non-negative score's key is its bits plus 2^31). One compare per entry then,
  // and the key is formed only for the entries stored.
  const bool cut_nonneg = cut >= 0x80000000u;
  const int cut_bits = (int)(cut & 0x7FFFFFFFu);
  auto take_batch = [&](auto fast_tag, int64_t b0, const float (&v)[kFilterUnroll]) {
    constexpr bool FAST = decltype(fast_tag)::value;     // whole batch in range, cut >= +0
    const int rem = (int)min<int64_t>(p_end - b0, kBatch);
#pragma unroll
    for (int j = 0; j < kFilterUnroll; ++j) {
      const bool sel = FAST ? __float_as_int(v[j]) >= cut_bits : (j * 64 + lane < rem && score_key(v[j]) >= cut);
      const uint64_t mask = __ballot(sel);
      if (sel) {
        const int at = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (at < cap_seg) {
          __builtin_amdgcn_raw_buffer_store_b32(score_key(v[j]), ck_rs, 4 * at, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(b0 + j * 64 + lane), cp_rs, 4 * at, 0, 0);
        }
      }
      cnt += __popcll(mask);
    }
  };
  auto take = [&](int64_t b0, const float (&v)[kFilterUnroll]) {
    if (cut_nonneg && b0 + kBatch <= p_end) take_batch(std::true_type{}, b0, v);    // workgroup-uniform
    else take_batch(std::false_type{}, b0, v);
  };
  // Two register buffers used in turn (no copy between them, which would wait for the batch
  // just issued): while one batch is taken, the next one is in flight.
  float nxt[kFilterUnroll];
  for (int64_t b0 = p_begin; b0 < p_end; b0 += 2 * kBatch) {
    if (b0 + kBatch < p_end) load_batch(b0 + kBatch, p_end, nxt);
    take(b0, cur);
    if (b0 + kBatch >= p_end) break;
    if (b0 + 2 * kBatch < p_end) load_batch(b0 + 2 * kBatch, p_end, cur);
    take(b0 + kBatch, nxt);
  }
  if (lane == 0) seg_cnt[seg] = cnt;                       // the true count, even past cap_seg
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    const float* __restrict__ scores, int64_t n_max, const int32_t* __restrict__ seq_lens,
    int32_t q_len, int32_t k, int32_t n_slices, int32_t cap_seg,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
    const int32_t* __restrict__ seg_cnt, int32_t* __restrict__ out) {
  __shared__ uint32_t keys[kTopkCandCap];
  __shared__ int32_t pos[kTopkCandCap];
  __shared__ uint32_t hist[2 * kBins];
  __shared__ int state[4];
  constexpr int NT = kMergeThreads, W = NT / 64;
  __shared__ int wsum[W];
  __shared__ uint32_t red[2 * W];
  __shared__ int cnt[2 * 128 + 2];
  __shared__ int soff[kTopkMaxSlices * kSegsPerSlice + 1];
  __shared__ int fallback_s;
  const int tok = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  // The segment counts (wave 0) and the first 64 entries of every segment (wave w: segments
  // w, w + 8, ...) are loaded up front, together with the row length: their addresses do not
  // depend on it. Entries past a count are read but never used (the workspace holds
  // cap_seg >= 256 entries per segment); short rows do not use any of it.
  const int n_seg = n_slices * kSegsPerSlice;               // <= 128: two per lane of wave 0
  const int64_t sbase = (int64_t)tok * n_seg;
  int c0 = 0, c1 = 0;
  if (w == 0) {
    c0 = (2 * lane < n_seg) ? seg_cnt[sbase + 2 * lane] : 0;
    c1 = (2 * lane + 1 < n_seg) ? seg_cnt[sbase + 2 * lane + 1] : 0;
  }
  constexpr int kSegPerWave = kTopkMaxSlices * kSegsPerSlice / W;
  uint32_t kv[kSegPerWave];
  int32_t pv[kSegPerWave];
#pragma unroll
  for (int u = 0; u < kSegPerWave; ++u) {
    const int sg = w + W * u;
    const int64_t at = (sbase + sg) * cap_seg + lane;
    kv[u] = (sg < n_seg) ? cand_key[at] : 0u;
    pv[u] = (sg < n_seg) ? cand_pos[at] : 0;
  }
  const int n = visible(seq_lens, tok, q_len, n_max);
  const float* row = scores + (int64_t)tok * n_max;
  int32_t* orow = out + (int64_t)tok * k;
  auto lds_key = [&](int i) { return keys[i]; };
  auto to_out = [&](int slot, int32_t p) { if (slot < k) orow[slot] = p; };   // slot < k always; kept as a bound
  int need = k;
  if (n <= kTopkTakeAll) {
    // short row: all of it in LDS
    if (n > 0) {
      constexpr int kPer = kTopkTakeAll / NT;
      float v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * NT;
        v[j] = (i < n) ? row[i] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * NT;
        if (i < n) keys[i] = score_key(v[j]);
      }
      __syncthreads();
      // thr 0 (n <= k): below every finite key, so every entry is emitted
      const uint32_t thr = (n > k) ? select_kth_lds<NT>(lds_key, n, k, hist, wsum, state, red, need) : 0u;
      ordered_emit<NT>(lds_key, n, thr, need, cnt, [](int i) { return i; }, to_out);
    }
  } else {
    if (w == 0) {
      const int inc = wave_incl_sum(c0 + c1);
      const int ex = inc - c0 - c1;
      if (lane == 0) soff[0] = 0;
      if (2 * lane < n_seg) soff[2 * lane + 1] = ex + c0;
      if (2 * lane + 1 < n_seg) soff[2 * lane + 2] = ex + c0 + c1;
      const bool over = __ballot(c0 > cap_seg || c1 > cap_seg) != 0ull;
      const int o = __builtin_amdgcn_readlane(inc, 63);
      if (lane == 0) fallback_s = over || o > kTopkCandCap || o < k;
    }
    __syncthreads();
    const int total = soff[n_seg];
    if (!fallback_s) {
      // the lists into LDS in position order (segment by segment), with the smallest and
      // largest key and the selection's first histogram cleared in the same phase
      int longest = 0;
      uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
#pragma unroll
      for (int u = 0; u < kSegPerWave; ++u) {
        const int sg = min(w + W * u, n_seg);
        const int o = soff[sg], c = soff[min(sg + 1, n_seg)] - o;
        longest = max(longest, c);
        if (lane < c && o + lane < kTopkCandCap) {
          keys[o + lane] = kv[u];
          pos[o + lane] = pv[u];
          lmn = min(lmn, kv[u]);
          lmx = max(lmx, kv[u]);
        }
      }
      if (longest > 64) {                                    // entries 64.. of longer segments (rare)
        for (int sg = w; sg < n_seg; sg += W) {
          const int o = soff[sg], c = soff[sg + 1] - o;
          for (int e = 64 + lane; e < c && o + e < kTopkCandCap; e += 64) {
            const int64_t at = (sbase + sg) * cap_seg + e;
            const uint32_t kk = cand_key[at];
            keys[o + e] = kk;
            pos[o + e] = cand_pos[at];
            lmn = min(lmn, kk);
            lmx = max(lmx, kk);
          }
        }
      }
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      if (tid == 0) state[3] = 0;
      lmn = wave_scan(lmn, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return min(x, y); });
      lmx = wave_scan(lmx, 0u, [](uint32_t x, uint32_t y) { return max(x, y); });
      if (lane == 63) { red[w] = lmn; red[W + w] = lmx; }
      __syncthreads();
      uint32_t mn = red[0], mx = red[W];
#pragma unroll
      for (int v = 1; v < W; ++v) { mn = min(mn, red[v]); mx = max(mx, red[W + v]); }
      uint32_t thr = 0u;                                     // 0 (total <= k): every entry
      if (total > k) {
        if (mn == mx) { need = k; thr = mx; }
        else thr = select_kth<NT, true, true>(lds_key, total, k, mn, 31 - __builtin_clz(mx - mn), 3, hist, wsum, state, need);
      }
      ordered_emit<NT>(lds_key, total, thr, need, cnt, [&](int i) { return pos[i]; }, to_out);
    } else {
      // the whole row from memory (exact whatever the sample did)
      auto mem_key = [&](int i) { return score_key(row[i]); };
      const uint32_t thr = select_kth<NT>(mem_key, n, k, 0u, 31, 3, hist, wsum, state, need);
      ordered_emit<NT>(mem_key, n, thr, need, cnt, [](int i) { return i; }, to_out);
    }
  }
  for (int s = min(n, k) + tid; s < k; s += NT) orow[s] = -1;
}

hipError_t launch_topk(const float* scores, int64_t n_max, const int32_t* seq_lens, int32_t T,
                       int32_t q_len, int32_t k, void* workspace, int32_t* out, hipStream_t stream) {
  const TopkPlan pl = topk_plan(T, n_max);
  const int64_t n_entries = (int64_t)T * pl.n_slices * kSegsPerSlice * pl.cap_seg;
  uint32_t* cand_key = (uint32_t*)workspace;
  int32_t* cand_pos = (int32_t*)(cand_key + n_entries);
  int32_t* seg_cnt = cand_pos + n_entries;
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)(T * pl.n_slices)), dim3(kFilterThreads), 0,
                     stream, scores, n_max, seq_lens, q_len, k, pl.slice, pl.n_slices, pl.cap_seg,
                     cand_key, cand_pos, seg_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)T), dim3(kMergeThreads), 0, stream, scores,
                     n_max, seq_lens, q_len, k, pl.n_slices, pl.cap_seg, cand_key, cand_pos,
                     seg_cnt, out);
  return hipGetLastError();
}

}  // namespace mla
