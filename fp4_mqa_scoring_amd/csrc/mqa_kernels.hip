// HIP kernels of the FP4 paged-MQA prefill indexer with exact TopK (gfx950).
//
// Pipeline of the fused path (all on the caller's stream):
//   row_prep        validate windows and pages, answer short rows (length <= K)
//   fused_topk      per (8-row tile, context split): stream 256-position score
//                   blocks through LDS, MXFP4 MFMA scoring, ReLU + head-weighted
//                   sum in registers, exact streaming selection in a bounded LDS
//                   pool per row; emit <= K keys per (row, split)
//   merge_emit      per row: exact TopK over the split candidates, ascending
//                   order, raw -> physical page mapping
// The dense comparator replaces fused_topk + merge_emit by dense_score (fp32
// logits [Q, S]) + logits_topk.
//
// Sources: "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR 5309),
// Implementation; "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK" (ROCm/aiter
// PR 5282), Changes and Scope.
#include "mqa_device.h"
#include "mqa_launch.h"

#include <climits>

namespace mqa {

// Sticky per-device status word (MQA_STATUS_* bits).
__device__ int32_t g_status;

// ---------------------------------------------------------------------------
// Row preparation. Window rules and short-row contract of PR 5282 (Changes);
// fail closed on invalid metadata/pages (PR 5309, Implementation).
// mode 0 (TopK): invalid rows -> -1 outputs and a negative count; short rows ->
//   positions start..end-1 then -1, count = length; long rows -> kRowLong.
// mode 1 (logits only): every valid non-empty row -> kRowLong, no outputs.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) row_prep_kernel(
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ row_end,
    const int32_t* __restrict__ page_table, int64_t P_log, int64_t P_phys, int32_t K, int mode,
    int32_t* __restrict__ out_raw, int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count,
    float* __restrict__ out_score, int32_t* __restrict__ row_state) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t start = row_start[row], end = row_end[row];
  int code = 0;
  if (start < 0 || end < start || end > kPage * P_log) {
    code = kCodeBadWindow;
  } else if (end > start) {
    const int64_t p0 = start / kPage, p1 = (end - 1) / kPage;
    int bad = 0;
    for (int64_t p = p0 + tid; p <= p1; p += blockDim.x) {
      const int64_t e = page_table[p];
      bad |= (e < 0 || e >= P_phys);
    }
    if (__syncthreads_or(bad)) code = kCodeBadPage;
  }
  const int64_t len = end - start;
  if (mode == 1) {
    if (tid == 0) row_state[row] = (code == 0 && len > 0) ? kRowLong : kRowDone;
    return;
  }
  if (code == 0 && len > K) {
    if (tid == 0) row_state[row] = kRowLong;
    return;
  }
  const size_t base = static_cast<size_t>(row) * K;
  for (int i = tid; i < K; i += blockDim.x) {
    int32_t raw = -1, slot = -1;
    if (code == 0 && i < len) {
      const int64_t s = start + i;
      raw = static_cast<int32_t>(s);
      slot = static_cast<int32_t>(static_cast<int64_t>(page_table[s / kPage]) * kPage + s % kPage);
    }
    out_raw[base + i] = raw;
    out_slot[base + i] = slot;
    if (out_score) out_score[base + i] = __uint_as_float(0x7FC00000u);
  }
  if (tid == 0) {
    out_count[row] = code ? code : static_cast<int32_t>(len);
    row_state[row] = kRowDone;
    if (code) atomicOr(&g_status, code == kCodeBadWindow ? kStBadWindow : kStBadPage);
  }
}

// ---------------------------------------------------------------------------
// Score-block streaming shared by the fused and the dense scorer.
// One CTA = 8 query rows (one per wave) x one contiguous range of 256-position
// score blocks. Each block (4 pages = 16 KiB codes + 1 KiB scales) is gathered
// through the page table with coalesced 32-byte-per-thread loads into registers
// one block ahead, then written to a double-buffered LDS image.
// ---------------------------------------------------------------------------
struct TileLoader {
  v4i c0, c1, sc;
  int32_t code_entry, scale_entry;   // raw page-table entries fetched ahead
  int64_t code_page, scale_page;     // validated physical pages of the tile to load next

  __device__ __forceinline__ static int64_t valid_or_neg(int32_t e, int64_t P_phys) {
    return (e >= 0 && e < P_phys) ? e : -1;
  }

  // Page-table entries of score block t for this thread's code chunk and (first
  // wave) scale chunk; -1 beyond the table. Issued two blocks ahead of use.
  __device__ __forceinline__ void fetch_entries(const int32_t* pt, int64_t P_log, int t) {
    const int tid = threadIdx.x;
    const int64_t lp = static_cast<int64_t>(t) * kTilePages + (tid >> 7);
    code_entry = lp < P_log ? pt[lp] : -1;
    const int64_t slp = static_cast<int64_t>(t) * kTilePages + ((tid & 63) >> 4);
    scale_entry = slp < P_log ? pt[slp] : -1;
  }

  __device__ __forceinline__ void resolve(int64_t P_phys) {
    code_page = valid_or_neg(code_entry, P_phys);
    scale_page = valid_or_neg(scale_entry, P_phys);
  }

  // Global -> registers for the resolved score block. Pages with an
  // out-of-range entry are not read (their rows were rejected by row_prep).
  __device__ __forceinline__ void load(const uint8_t* k_pages, const uint8_t* k_scale) {
    const int tid = threadIdx.x;
    const int within = tid & 127;
    if (code_page >= 0) {
      const v4i* src = reinterpret_cast<const v4i*>(k_pages + static_cast<size_t>(code_page) * kPage * kVecBytes +
                                                    static_cast<size_t>(within) * 32);
      c0 = src[0];
      c1 = src[1];
    } else {
      c0 = v4i{0, 0, 0, 0};
      c1 = v4i{0, 0, 0, 0};
    }
    if (tid < 64) {
      const int off = (tid & 15) * 16;
      sc = scale_page >= 0
               ? *reinterpret_cast<const v4i*>(k_scale + static_cast<size_t>(scale_page) * kPage * kVecScales + off)
               : v4i{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(uint8_t* s_codes, uint8_t* s_scales) const {
    const int tid = threadIdx.x;
    const int pi = tid >> 7, within = tid & 127;
    const int p = pi * kPage + (within >> 1), half = within & 1;
    const int sw = chunk_swizzle(p);
    uint8_t* dst = s_codes + p * kVecBytes;
    *reinterpret_cast<v4i*>(dst + 16 * ((2 * half) ^ sw)) = c0;
    *reinterpret_cast<v4i*>(dst + 16 * ((2 * half + 1) ^ sw)) = c1;
    if (tid < 64) *reinterpret_cast<v4i*>(s_scales + (tid >> 4) * (kPage * kVecScales) + (tid & 15) * 16) = sc;
  }

  // Prologue: block t_begin into LDS buffer t_begin & 1, entries of the next
  // block in flight.
  __device__ __forceinline__ void prologue(const uint8_t* k_pages, const uint8_t* k_scale, const int32_t* pt,
                                           int64_t P_log, int64_t P_phys, int t_begin, int t_end,
                                           uint8_t* s_codes, uint8_t* s_scales) {
    fetch_entries(pt, P_log, t_begin);
    resolve(P_phys);
    load(k_pages, k_scale);
    if (t_begin + 1 < t_end) fetch_entries(pt, P_log, t_begin + 1);
    store(s_codes, s_scales);
  }

  // Start of block t: data loads of block t+1 (entries fetched one block ago)
  // and page-table loads of block t+2.
  __device__ __forceinline__ void advance(const uint8_t* k_pages, const uint8_t* k_scale, const int32_t* pt,
                                          int64_t P_log, int64_t P_phys, int t, int t_end) {
    resolve(P_phys);
    load(k_pages, k_scale);
    if (t + 2 < t_end) fetch_entries(pt, P_log, t + 2);
  }
};

struct ScanArgs {
  const uint8_t* q;
  const uint8_t* q_scale;
  const float* weights;
  const uint8_t* k_pages;
  const uint8_t* k_scale;
  int64_t P_phys;
  const int32_t* page_table;
  int64_t P_log;
  const int32_t* row_start;
  const int32_t* row_end;
  const int32_t* row_state;
  int32_t Q;
  int32_t splits;
};

// CTA-uniform score-block range [t_begin, t_end) of this split over the union
// of the CTA's active row windows; returns false when the CTA has no active row.
__device__ __forceinline__ bool cta_tile_range(const ScanArgs& a, int32_t* s_lo, int32_t* s_hi,
                                               bool active, int start, int end, int wave, int lane,
                                               int* t_begin, int* t_end) {
  if (lane == 0) {
    s_lo[wave] = active ? start : INT_MAX;
    s_hi[wave] = active ? end : INT_MIN;
  }
  __syncthreads();
  int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
  for (int i = 0; i < kRowsPerCta; ++i) {
    lo = min(lo, s_lo[i]);
    hi = max(hi, s_hi[i]);
  }
  if (lo >= hi) return false;
  const int u0 = lo / kTile, u1 = (hi + kTile - 1) / kTile;
  const int64_t nt = u1 - u0;
  *t_begin = u0 + static_cast<int>(nt * blockIdx.y / a.splits);
  *t_end = u0 + static_cast<int>(nt * (blockIdx.y + 1) / a.splits);
  return true;
}

// ---------------------------------------------------------------------------
// Fused scorer + streaming exact TopK ("[FlyDSL][DSv4] Prototype FP4 MQA
// streaming TopK", Changes: scores stream through a bounded LDS pool; each CTA
// emits only candidate values, indices and a valid count).
//
// Each wave owns one query row and its LDS pool of CAP unique keys. A key enters
// the pool only if it beats the row's gate T (the smallest key that can still be
// in the row's TopK of this split). When a batch would overflow the pool, the
// wave radix-selects the K largest keys, drops the rest and raises T.
// ---------------------------------------------------------------------------
template <int K, int CAP>
__global__ void __launch_bounds__(kCtaThreads, 1) fused_topk_kernel(ScanArgs a, uint64_t* __restrict__ cand_keys,
                                                                    int32_t* __restrict__ cand_count) {
  static_assert(CAP >= K + 64, "pool must hold K keys plus one batch");
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][kTile * kVecBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[2][kTile * kVecScales];
  __shared__ uint64_t s_pool[kRowsPerCta][CAP];
  __shared__ uint32_t s_hist[kRowsPerCta][256];
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerCta + wave;
  const bool active = row < a.Q && a.row_state[row] == kRowLong;
  int start = 0, end = 0;
  if (active) {
    start = a.row_start[row];
    end = a.row_end[row];
  }
  int t_begin = 0, t_end = 0;
  if (!cta_tile_range(a, s_lo, s_hi, active, start, end, wave, lane, &t_begin, &t_end)) return;

  QRow qr;
  if (active)
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);

  uint64_t* pool = s_pool[wave];
  uint32_t* hist = s_hist[wave];
  int fill = 0;          // wave-uniform
  uint64_t gate = 0;     // keys > gate may still be in this split's TopK
  bool failed = false;

  // query operands and weights must be in registers before the scan loop
  __builtin_amdgcn_s_waitcnt(0);
  TileLoader ld;
  if (t_begin < t_end) {
    ld.prologue(a.k_pages, a.k_scale, a.page_table, a.P_log, a.P_phys, t_begin, t_end, s_codes[t_begin & 1],
                s_scales[t_begin & 1]);
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < t_end;
    if (more) ld.advance(a.k_pages, a.k_scale, a.page_table, a.P_log, a.P_phys, t, t_end);
    const int tb = t * kTile;
    if (active && tb < end && tb + kTile > start) {
#pragma unroll 1
      for (int blk = 0; blk < kTile / 64; ++blk) {
        const int p0 = tb + 64 * blk;
        if (p0 >= end || p0 + 64 <= start) continue;
        const float sc = score64(qr, s_codes[buf], s_scales[buf], blk, lane);
        const int pos = p0 + lane;
        const uint64_t key = make_key(sc, static_cast<uint32_t>(pos));
        bool pass = pos >= start && pos < end && key > gate;
        uint64_t m = __ballot(pass);
        if (m == 0) continue;
        int cnt = __popcll(m);
        if (fill + cnt > CAP) {
          const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
          if (sel.kept != K) failed = true;
          fill = K;
          gate = sel.T - 1;
          pass = pass && key > gate;
          m = __ballot(pass);
          cnt = __popcll(m);
        }
        if (pass) pool[fill + mbcnt64(m)] = key;
        fill += cnt;
      }
    }
    if (more) ld.store(s_codes[buf ^ 1], s_scales[buf ^ 1]);
    __syncthreads();
  }

  if (!active) return;
  wave_lds_sync();
  if (fill > K) {
    const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
    if (sel.kept != K) failed = true;
    fill = K;
  }
  const size_t slot = static_cast<size_t>(row) * a.splits + blockIdx.y;
  uint64_t* dst = cand_keys + slot * K;
  for (int i = lane; i < fill; i += 64) dst[i] = pool[i];
  if (lane == 0) cand_count[slot] = failed ? kCodeSelector : fill;
}

// ---------------------------------------------------------------------------
// Dense scorer (comparator): same streaming and the same score64() as the fused
// kernel, but every score inside an active row's window goes to logits[row, s].
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kCtaThreads, 1) dense_score_kernel(ScanArgs a, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][kTile * kVecBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[2][kTile * kVecScales];
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerCta + wave;
  const bool active = row < a.Q && a.row_state[row] == kRowLong;
  int start = 0, end = 0;
  if (active) {
    start = a.row_start[row];
    end = a.row_end[row];
  }
  int t_begin = 0, t_end = 0;
  if (!cta_tile_range(a, s_lo, s_hi, active, start, end, wave, lane, &t_begin, &t_end)) return;
  QRow qr;
  if (active)
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);
  float* out = logits + static_cast<size_t>(row) * (a.P_log * kPage);

  // query operands and weights must be in registers before the scan loop
  __builtin_amdgcn_s_waitcnt(0);
  TileLoader ld;
  if (t_begin < t_end) {
    ld.prologue(a.k_pages, a.k_scale, a.page_table, a.P_log, a.P_phys, t_begin, t_end, s_codes[t_begin & 1],
                s_scales[t_begin & 1]);
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < t_end;
    if (more) ld.advance(a.k_pages, a.k_scale, a.page_table, a.P_log, a.P_phys, t, t_end);
    const int tb = t * kTile;
    if (active && tb < end && tb + kTile > start) {
#pragma unroll 1
      for (int blk = 0; blk < kTile / 64; ++blk) {
        const int p0 = tb + 64 * blk;
        if (p0 >= end || p0 + 64 <= start) continue;
        const float sc = score64(qr, s_codes[buf], s_scales[buf], blk, lane);
        const int pos = p0 + lane;
        if (pos >= start && pos < end) __builtin_nontemporal_store(sc, out + pos);
      }
    }
    if (more) ld.store(s_codes[buf ^ 1], s_scales[buf ^ 1]);
    __syncthreads();
  }
}

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
  uint32_t red32[NT / 64];
  int32_t redi[NT / 64];
  uint32_t wtot[NT / 64];
};

template <int NT>
__device__ __forceinline__ void block_or_and(uint64_t& vor, uint64_t& vand, BlockScratch<NT>& s) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  vor = wave_or64(vor);
  vand = wave_and64(vand);
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
  v = wave_max_i32(v);
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
  v = wave_suffix_sum(v, lane);
  if (lane == 0) s.wtot[w] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i)
    if (i > w) add += s.wtot[i];
  __syncthreads();
  return v + add;
}

template <int NT, int DBITS, class Src>
__device__ uint64_t block_radix_select(const Src& src, int64_t n, int k, uint32_t* hist,
                                       BlockScratch<NT>& s, bool* ok) {
  constexpr int BINS = 1 << DBITS;
  constexpr int BPT = BINS / NT;  // bins per thread
  static_assert(BPT >= 1 && BINS % NT == 0, "bins must be a multiple of threads");
  const int tid = threadIdx.x;
  uint64_t vor = 0, vand = ~0ull;
  for (int64_t i = tid; i < n; i += NT) {
    uint64_t x;
    if (src(i, x)) {
      vor |= x;
      vand &= x;
    }
  }
  block_or_and<NT>(vor, vand, s);
  if (vor == vand) {   // at most one distinct valid key
    *ok = (k == 1);
    return vand;
  }
  int hb = 63 - __clzll(static_cast<long long>(vor ^ vand));
  uint64_t pmask = ~((2ull << hb) - 1ull);
  uint64_t prefix = vand & pmask;
  uint32_t krem = static_cast<uint32_t>(k);
  for (;;) {
    const int shift = hb >= DBITS - 1 ? hb - (DBITS - 1) : 0;
    for (int b = tid; b < BINS; b += NT) hist[b] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += NT) {
      uint64_t x;
      if (src(i, x) && (x & pmask) == prefix)
        atomicAdd(&hist[static_cast<uint32_t>(x >> shift) & (BINS - 1)], 1u);
    }
    __syncthreads();
    uint32_t c[BPT];
    uint32_t tsum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[tid * BPT + j];
      tsum += c[j];
    }
    const uint32_t incl = block_suffix_sum<NT>(tsum, s);
    uint32_t suf = incl - tsum;   // suffix strictly after this thread's bins
    int local = -1;
    uint32_t local_suffix = 0;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      suf += c[j];
      if (suf >= krem && local < 0) {
        local = tid * BPT + j;
        local_suffix = suf;
      }
    }
    const int dstar = block_max_i32<NT>(local, s);
    if (dstar < 0) {
      *ok = false;
      return prefix;
    }
    if (local == dstar) s.red32[0] = local_suffix;
    __syncthreads();
    const uint32_t suffix_d = s.red32[0];
    const uint32_t cnt_d = hist[dstar];
    __syncthreads();
    krem -= suffix_d - cnt_d;
    prefix |= static_cast<uint64_t>(dstar) << shift;
    pmask |= static_cast<uint64_t>(BINS - 1) << shift;
    if (cnt_d == krem || shift == 0) break;
    hb = shift - 1;
  }
  *ok = true;
  return prefix;
}

// Sorts N (power of two) 64-bit values ascending in LDS with NT threads.
template <int N, int NT>
__device__ __forceinline__ void block_bitonic_sort(uint64_t* v) {
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < N / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = v[lo], y = v[hi];
        if ((x > y) == up) {
          v[lo] = y;
          v[hi] = x;
        }
      }
      __syncthreads();
    }
  }
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
  block_bitonic_sort<K, NT>(s_sel);
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
                                         float* __restrict__ out_score) {
  const size_t base = static_cast<size_t>(row) * K;
  for (int i = threadIdx.x; i < K; i += NT) {
    out_raw[base + i] = -1;
    out_slot[base + i] = -1;
    if (out_score) out_score[base + i] = __uint_as_float(0x7FC00000u);
  }
  if (threadIdx.x == 0) {
    out_count[row] = code;
    atomicOr(&g_status, code == kCodeUnderfill ? kStUnderfill : kStSelector);
  }
}

// ---------------------------------------------------------------------------
// Exact merge of the split candidates ("exact candidate union", PR 5282) +
// page mapping + emission. One 256-thread CTA per long row.
// ---------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(256) merge_emit_kernel(
    const int32_t* __restrict__ row_state, const uint64_t* __restrict__ cand_keys,
    const int32_t* __restrict__ cand_count, int32_t splits, const int32_t* __restrict__ page_table,
    int64_t P_log, int32_t* __restrict__ out_raw, int32_t* __restrict__ out_slot,
    int32_t* __restrict__ out_count, float* __restrict__ out_score) {
  constexpr int NT = 256;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[256];
  __shared__ int32_t s_cnt[256];
  __shared__ int32_t s_off[257];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const uint64_t* keys = cand_keys + static_cast<size_t>(row) * splits * K;
  for (int i = threadIdx.x; i < splits; i += NT) s_cnt[i] = cand_count[static_cast<size_t>(row) * splits + i];
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0, bad = 0;
    for (int i = 0; i < splits; ++i) {
      s_off[i] = acc;
      if (s_cnt[i] < 0 || s_cnt[i] > K) bad = 1;
      else acc += s_cnt[i];
    }
    s_off[splits] = bad ? -1 : acc;
  }
  __syncthreads();
  const int total = s_off[splits];
  if (total < K) {   // a long row always has >= K candidates
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score);
    return;
  }
  if (total == K) {
    for (int e = threadIdx.x; e < splits * K; e += NT) {
      const int sp = e / K, j = e % K;
      if (j < s_cnt[sp]) s_sel[s_off[sp] + j] = keys[e];
    }
    __syncthreads();
  } else {
    auto src = [&](int64_t e, uint64_t& x) -> bool {
      const int sp = static_cast<int>(e / K), j = static_cast<int>(e % K);
      if (j >= s_cnt[sp]) return false;
      x = keys[e];
      return true;
    };
    bool ok = false;
    const uint64_t T = block_radix_select<NT, 8>(src, static_cast<int64_t>(splits) * K, K, s_hist, s_red, &ok);
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    if (ok) {
      for (int e = threadIdx.x; e < splits * K; e += NT) {
        uint64_t x;
        if (src(e, x) && x >= T) {
          const int at = atomicAdd(&s_n, 1);
          if (at < K) s_sel[at] = x;
        }
      }
    }
    __syncthreads();
    if (!ok || s_n != K) {
      fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score);
      return;
    }
  }
  emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
}

// ---------------------------------------------------------------------------
// Dense selector: exact TopK over fp32 logits of one long row's window.
// One 1024-thread CTA per row, 11-bit digits.
// ---------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(1024) logits_topk_kernel(
    const float* __restrict__ logits, int64_t S, int64_t P_log, const int32_t* __restrict__ row_state,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ row_end,
    const int32_t* __restrict__ page_table, int32_t* __restrict__ out_raw,
    int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count, float* __restrict__ out_score) {
  constexpr int NT = 1024;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[2048];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const int64_t start = row_start[row], n = row_end[row] - start;
  const float* lg = logits + static_cast<size_t>(row) * S + start;
  auto src = [&](int64_t i, uint64_t& x) -> bool {
    x = make_key(lg[i], static_cast<uint32_t>(start + i));
    return true;
  };
  bool ok = false;
  const uint64_t T = block_radix_select<NT, 11>(src, n, K, s_hist, s_red, &ok);
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  if (ok) {
    for (int64_t i = threadIdx.x; i < n; i += NT) {
      uint64_t x;
      src(i, x);
      if (x >= T) {
        const int at = atomicAdd(&s_n, 1);
        if (at < K) s_sel[at] = x;
      }
    }
  }
  __syncthreads();
  if (!ok || s_n != K) {
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score);
    return;
  }
  emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
}

// Pool capacity per row: all LDS left after the two score-block buffers and the
// per-wave histograms (160 KiB per CTA on gfx950).
constexpr int kPoolCap = 1856;

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static ScanArgs scan_args(const PathArgs& p, const int32_t* row_state, int32_t splits) {
  ScanArgs a;
  a.q = p.q;
  a.q_scale = p.q_scale;
  a.weights = p.weights;
  a.k_pages = p.k_pages;
  a.k_scale = p.k_scale;
  a.P_phys = p.P_phys;
  a.page_table = p.page_table;
  a.P_log = p.P_log;
  a.row_start = p.row_start;
  a.row_end = p.row_end;
  a.row_state = row_state;
  a.Q = static_cast<int32_t>(p.Q);
  a.splits = splits;
  return a;
}

hipError_t launch_row_prep(const PathArgs& p, int mode, int32_t* row_state, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  row_prep_kernel<<<dim3(static_cast<unsigned>(p.Q)), dim3(256), 0, st>>>(
      p.row_start, p.row_end, p.page_table, p.P_log, p.P_phys, p.K, mode, p.out_raw, p.out_slot,
      p.out_count, p.out_score, row_state);
  return hipGetLastError();
}

hipError_t launch_fused(const PathArgs& p, const int32_t* row_state, int32_t splits, uint64_t* cand_keys,
                        int32_t* cand_count, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.Q + kRowsPerCta - 1) / kRowsPerCta), static_cast<unsigned>(splits));
  const ScanArgs a = scan_args(p, row_state, splits);
  if (p.K == 512)
    fused_topk_kernel<512, kPoolCap><<<grid, dim3(kCtaThreads), 0, st>>>(a, cand_keys, cand_count);
  else
    fused_topk_kernel<1024, kPoolCap><<<grid, dim3(kCtaThreads), 0, st>>>(a, cand_keys, cand_count);
  return hipGetLastError();
}

hipError_t launch_merge(const PathArgs& p, const int32_t* row_state, int32_t splits, const uint64_t* cand_keys,
                        const int32_t* cand_count, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.Q));
  if (p.K == 512)
    merge_emit_kernel<512><<<grid, dim3(256), 0, st>>>(row_state, cand_keys, cand_count, splits, p.page_table,
                                                        p.P_log, p.out_raw, p.out_slot, p.out_count, p.out_score);
  else
    merge_emit_kernel<1024><<<grid, dim3(256), 0, st>>>(row_state, cand_keys, cand_count, splits, p.page_table,
                                                         p.P_log, p.out_raw, p.out_slot, p.out_count, p.out_score);
  return hipGetLastError();
}

hipError_t launch_dense_score(const PathArgs& p, const int32_t* row_state, int32_t splits, float* logits,
                              hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.Q + kRowsPerCta - 1) / kRowsPerCta), static_cast<unsigned>(splits));
  dense_score_kernel<<<grid, dim3(kCtaThreads), 0, st>>>(scan_args(p, row_state, splits), logits);
  return hipGetLastError();
}

hipError_t launch_logits_topk(const PathArgs& p, const float* logits, const int32_t* row_state,
                              hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.Q));
  const int64_t S = p.P_log * kPage;
  if (p.K == 512)
    logits_topk_kernel<512><<<grid, dim3(1024), 0, st>>>(logits, S, p.P_log, row_state, p.row_start, p.row_end,
                                                          p.page_table, p.out_raw, p.out_slot, p.out_count,
                                                          p.out_score);
  else
    logits_topk_kernel<1024><<<grid, dim3(1024), 0, st>>>(logits, S, p.P_log, row_state, p.row_start, p.row_end,
                                                           p.page_table, p.out_raw, p.out_slot, p.out_count,
                                                           p.out_score);
  return hipGetLastError();
}

hipError_t status_take(hipStream_t st, int32_t* host_out) {
  int32_t zero = 0;
  hipError_t e = hipMemcpyFromSymbolAsync(host_out, HIP_SYMBOL(g_status), sizeof(int32_t), 0,
                                          hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_status), &zero, sizeof(int32_t), 0, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

int pool_capacity() { return kPoolCap; }

}  // namespace mqa
