// Block-level selection helpers (exact radix select over unique 64-bit keys,
// the bucketed position sort, row emission with the page map) shared by the
// kernels of the fused, dense, tiled and decode paths.
#pragma once

#include "mqa_device.h"

namespace mqa {

// ---------------------------------------------------------------------------
// Block-level exact radix select (256 or 1024 threads) over unique 64-bit keys
// produced by a source functor: src(i, &key) -> bool (valid), i in [0, n).
// Digits of DBITS bits, starting at the highest bit where the valid keys differ.
// Returns T with exactly k valid keys >= T (k <= number of valid keys), or
// sets *ok = false if the keys break the invariants.
// ---------------------------------------------------------------------------
template <int NT>
struct BlockScratch {
  uint64_t red64[2][NT / 64];
  uint32_t digit[4];   // the select's chosen digit: bin, keys at or above it, keys in it
  int32_t redi[NT / 64];
  uint32_t wtot[NT / 64];
};

template <int NT>
__device__ __forceinline__ void block_or_and(uint64_t& vor, uint64_t& vand, BlockScratch<NT>& s) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  vor = wave_all_or64(vor);
  vand = wave_all_and64(vand);
  if (lane == 0) {
    s.red64[0][w] = vor;
    s.red64[1][w] = vand;
  }
  __syncthreads();
  vor = 0;
  vand = ~0ull;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    vor |= s.red64[0][i];
    vand &= s.red64[1][i];
  }
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ int block_max_i32(int v, BlockScratch<NT>& s) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = wave_all_max_i32(v);
  if (lane == 0) s.redi[w] = v;
  __syncthreads();
  int r = INT_MIN;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = max(r, s.redi[i]);
  __syncthreads();
  return r;
}

// Inclusive suffix sum over the NT threads (thread order).
template <int NT>
__device__ __forceinline__ uint32_t block_suffix_sum(uint32_t v, BlockScratch<NT>& s) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t pre = wave_prefix_sum_dpp(v);
  v = lane63(pre) - pre + v;
  if (lane == 0) s.wtot[w] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i)
    if (i > w) add += s.wtot[i];
  __syncthreads();
  return v + add;
}

// Core of the selection: visit(f) calls f(key) for every valid key the calling
// thread holds. Each digit pass takes three barriers: the histogram is complete;
// the wave totals of the bin counts are posted; the one bin where the count of
// keys at or above it first reaches the remaining rank is posted (its thread
// finds it alone, since that count falls by bin), and every thread clears the
// bins it read for the next pass. The wave-level sums and reductions go through
// DPP. hist holds 2^DBITS counters.
template <int NT, int DBITS, class Visit>
__device__ uint64_t block_radix_select_core(const Visit& visit, int k, uint32_t* hist, BlockScratch<NT>& s,
                                            bool* ok) {
  constexpr int BINS = 1 << DBITS;
  constexpr int BPT = BINS / NT;  // bins per thread: [tid BPT, tid BPT + BPT)
  constexpr int NW = NT / 64;
  static_assert(BPT >= 1 && BINS % NT == 0, "bins must be a multiple of threads");
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  uint64_t vor = 0, vand = ~0ull;
  visit([&](uint64_t x) {
    vor |= x;
    vand &= x;
  });
  vor = wave_all_or64(vor);
  vand = wave_all_and64(vand);
  if (lane == 0) {
    s.red64[0][w] = vor;
    s.red64[1][w] = vand;
  }
#pragma unroll
  for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0u;
  __syncthreads();
  vor = 0;
  vand = ~0ull;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    vor |= s.red64[0][i];
    vand &= s.red64[1][i];
  }
  if (vor == vand) {   // at most one distinct valid key
    __syncthreads();   // red64 is read before anyone returns
    *ok = (k == 1);
    return vand;
  }
  int hb = 63 - __clzll(static_cast<long long>(vor ^ vand));
  uint64_t pmask = ~((2ull << hb) - 1ull);
  uint64_t prefix = vand & pmask;
  uint32_t krem = static_cast<uint32_t>(k);
  for (;;) {
    const int shift = hb >= DBITS - 1 ? hb - (DBITS - 1) : 0;
    visit([&](uint64_t x) {
      if ((x & pmask) == prefix) atomicAdd(&hist[static_cast<uint32_t>(x >> shift) & (BINS - 1)], 1u);
    });
    __syncthreads();
    uint32_t c[BPT];
    uint32_t tsum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[tid * BPT + j];
      tsum += c[j];
    }
    const uint32_t pre = wave_prefix_sum_dpp(tsum);
    const uint32_t wave_total = lane63(pre);
    if (lane == 0) s.wtot[w] = wave_total;
    if (tid == 0) s.digit[0] = ~0u;   // no bin reaches krem unless a thread posts one
    __syncthreads();
    uint32_t suf = wave_total - pre;   // keys in the bins of the wave's later lanes
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (i > w) suf += s.wtot[i];
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      const uint32_t above = suf;   // keys in bins after bin tid BPT + j
      suf += c[j];
      if (suf >= krem && above < krem) {
        s.digit[0] = static_cast<uint32_t>(tid * BPT + j);
        s.digit[1] = suf;
        s.digit[2] = c[j];
      }
      hist[tid * BPT + j] = 0u;
    }
    __syncthreads();
    const uint32_t dstar = s.digit[0];
    if (dstar == ~0u) {
      *ok = false;
      return prefix;
    }
    const uint32_t suffix_d = s.digit[1], cnt_d = s.digit[2];
    krem -= suffix_d - cnt_d;
    prefix |= static_cast<uint64_t>(dstar) << shift;
    pmask |= static_cast<uint64_t>(BINS - 1) << shift;
    if (cnt_d == krem || shift == 0) break;
    hb = shift - 1;
  }
  *ok = true;
  return prefix;
}

// Keys read through src(i, &key) -> valid, i in [0, n), thread t taking
// i = t, t + NT, ... (each pass reads them again).
template <int NT, int DBITS, class Src>
__device__ uint64_t block_radix_select(const Src& src, int64_t n, int k, uint32_t* hist, BlockScratch<NT>& s,
                                       bool* ok) {
  const int tid = threadIdx.x;
  auto visit = [&](auto&& f) {
    for (int64_t i = tid; i < n; i += NT) {
      uint64_t x;
      if (src(i, x)) f(x);
    }
  };
  return block_radix_select_core<NT, DBITS>(visit, k, hist, s, ok);
}

// Keys held in registers: x[j] is valid iff bit j of `valid` is set.
template <int NT, int DBITS, int E>
__device__ uint64_t block_radix_select_regs(const uint64_t (&x)[E], uint32_t valid, int k, uint32_t* hist,
                                            BlockScratch<NT>& s, bool* ok) {
  static_assert(E >= 1 && E <= 32, "validity mask width");
  auto visit = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((valid >> j) & 1u) f(x[j]);
  };
  return block_radix_select_core<NT, DBITS>(visit, k, hist, s, ok);
}

// Loads keys[i] for i = t + j NT < n into x[j]; returns the validity mask.
template <int NT, int E>
__device__ __forceinline__ uint32_t load_keys_regs(const uint64_t* __restrict__ keys, int n, uint64_t (&x)[E]) {
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = static_cast<int>(threadIdx.x) + j * NT;
    x[j] = i < n ? keys[i] : 0ull;
    if (i < n) valid |= 1u << j;
  }
  return valid;
}

// Appends the keys >= T of x (valid ones) to sel[*n_sel] (LDS, at most K).
template <int K, int E>
__device__ __forceinline__ void gather_at_least(const uint64_t (&x)[E], uint32_t valid, uint64_t T, uint64_t* sel,
                                                int32_t* n_sel) {
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (((valid >> j) & 1u) && x[j] >= T) {
      const int at = atomicAdd(n_sel, 1);
      if (at < K) sel[at] = x[j];
    }
  }
}

// Sorts the K values v[] (LDS) ascending by their high 32 bits, which are
// distinct non-negative positions: K position buckets between the smallest and
// largest position (a monotone bucket function, so bucket order is position
// order), a prefix sum of the bucket counts, a scatter into the buckets, and
// inside each bucket a rank by counting the smaller positions. Six barriers
// (the extremes and the cleared buckets share one, the prefix sum takes one
// through DPP wave sums) where a bitonic network takes fifty-five (K = 1024).
template <int K, int NT>
__device__ __forceinline__ void block_position_sort(uint64_t* v) {
  constexpr int NW = NT / 64;
  __shared__ uint64_t s_tmp[K];
  __shared__ uint32_t s_start[K];
  __shared__ uint32_t s_fill[K];
  __shared__ int32_t s_hi[NW], s_nlo[NW];
  __shared__ uint32_t s_wsum[NW];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  int hi = INT_MIN, nlo = INT_MIN;
  for (int i = tid; i < K; i += NT) {
    const int p = static_cast<int>(v[i] >> 32);
    hi = max(hi, p);
    nlo = max(nlo, -p);
  }
  hi = wave_all_max_i32(hi);
  nlo = wave_all_max_i32(nlo);
  if (lane == 0) {
    s_hi[w] = hi;
    s_nlo[w] = nlo;
  }
  for (int b = tid; b < K; b += NT) {
    s_start[b] = 0u;
    s_fill[b] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    hi = max(hi, s_hi[i]);
    nlo = max(nlo, s_nlo[i]);
  }
  const int lo = -nlo;
  const float scale = static_cast<float>(K) / (static_cast<float>(hi - lo) + 1.0f);
  auto bucket = [&](uint64_t x) -> int {
    return min(K - 1, static_cast<int>(static_cast<float>(static_cast<int>(x >> 32) - lo) * scale));
  };
  for (int i = tid; i < K; i += NT) atomicAdd(&s_start[bucket(v[i])], 1u);
  __syncthreads();
  constexpr int B = (K + NT - 1) / NT;   // buckets per thread: [tid B, tid B + B)
  uint32_t c[B];
  uint32_t tsum = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int b = tid * B + j;
    c[j] = b < K ? s_start[b] : 0u;
    tsum += c[j];
  }
  const uint32_t pre = wave_prefix_sum_dpp(tsum);   // inclusive, over the wave's lanes
  if (lane == 63) s_wsum[w] = pre;
  __syncthreads();
  uint32_t run = pre - tsum;   // keys in earlier buckets
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < w) run += s_wsum[i];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const int b = tid * B + j;
    if (b < K) s_start[b] = run;
    run += c[j];
  }
  __syncthreads();
  for (int i = tid; i < K; i += NT) {
    const uint64_t x = v[i];
    const int b = bucket(x);
    s_tmp[s_start[b] + atomicAdd(&s_fill[b], 1u)] = x;
  }
  __syncthreads();
  for (int k = tid; k < K; k += NT) {
    const uint64_t x = s_tmp[k];
    const int b = bucket(x);
    const uint32_t s0 = s_start[b], n = s_fill[b], p = static_cast<uint32_t>(x >> 32);
    uint32_t r = 0;
    for (uint32_t j = s0; j < s0 + n; ++j) r += static_cast<uint32_t>(s_tmp[j] >> 32) < p ? 1u : 0u;
    v[s0 + r] = x;
  }
  __syncthreads();
}

// Writes one long row's K selected keys (in s_sel) in ascending position order
// with their physical slots. s_sel is overwritten.
template <int K, int NT>
__device__ __forceinline__ void emit_row(uint64_t* s_sel, int64_t row, const int32_t* __restrict__ page_table,
                                         int64_t P_log, int32_t* __restrict__ out_raw,
                                         int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count,
                                         float* __restrict__ out_score) {
  for (int i = threadIdx.x; i < K; i += NT) {
    const uint64_t key = s_sel[i];
    s_sel[i] = (static_cast<uint64_t>(key_pos(key)) << 32) | static_cast<uint32_t>(key >> 32);
  }
  __syncthreads();
  // keys gathered in buffer order from one wave's appends are already in
  // ascending position order: one compare per element instead of the sort
  int unsorted = 0;
  for (int i = threadIdx.x; i + 1 < K; i += NT) unsorted |= s_sel[i] > s_sel[i + 1];
  if (__syncthreads_or(unsorted)) block_position_sort<K, NT>(s_sel);
  const size_t base = static_cast<size_t>(row) * K;
  for (int i = threadIdx.x; i < K; i += NT) {
    const uint64_t v = s_sel[i];
    const uint32_t pos = static_cast<uint32_t>(v >> 32);
    const int64_t lp = pos / kPage;   // always < P_log for keys of validated windows
    out_raw[base + i] = static_cast<int32_t>(pos);
    out_slot[base + i] = lp < P_log ? static_cast<int32_t>(static_cast<int64_t>(page_table[lp]) * kPage + pos % kPage)
                                    : -1;
    if (out_score) out_score[base + i] = key_score(static_cast<uint64_t>(static_cast<uint32_t>(v)) << 32);
  }
  if (threadIdx.x == 0) out_count[row] = K;
}

template <int K, int NT>
__device__ __forceinline__ void fail_row(int64_t row, int code, int32_t* __restrict__ out_raw,
                                         int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count,
                                         float* __restrict__ out_score, int32_t* status) {
  const size_t base = static_cast<size_t>(row) * K;
  for (int i = threadIdx.x; i < K; i += NT) {
    out_raw[base + i] = -1;
    out_slot[base + i] = -1;
    if (out_score) out_score[base + i] = __uint_as_float(0x7FC00000u);
  }
  if (threadIdx.x == 0) {
    out_count[row] = code;
    atomicOr(status, code == kCodeUnderfill ? kStUnderfill : kStSelector);
  }
}


// Candidates the sample must keep: x + 4 sqrt(x) + 8 where x = K m / n is the
// expected number of the row's true top-K positions among m sampled ones.
__device__ __forceinline__ int sample_keep(int K, int m, int n) {
  const float x = static_cast<float>(K) * static_cast<float>(m) / static_cast<float>(n);
  return static_cast<int>(ceilf(x + 4.0f * sqrtf(x) + 8.0f));
}

}  // namespace mqa
