// Decode / multi-sequence variant of the FP4 paged-MQA indexer with exact TopK
// (gfx950). Every row has its own page table (block table row seq_of_row[r]),
// so rows share no key tiles: each wave streams one (row, context split) item's
// pages by itself, the way the pages' first fused design works per CTA
// ("[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK", Changes: running
// candidates held in a fixed-size LDS pool, an exact radix selection on the
// total-order key, only candidates and their number handed on, an exact merge
// of the splits, then the page-table mapping). Decode workloads are the adjacent shape the pages
// leave on the older path ("[AMD][DSv4] Add experimental AITER FP4 streaming
// TopK", Changes / Scope) and whose graph-capture support they defer ([P2]
// Scope); this entry point takes its scratch from the caller, never allocates
// or synchronises, and reports row failures only on the device, so it can be
// captured into a HIP graph and replayed.
//
// Pipeline (all on the caller's stream):
//   row_prep   windows, per-row pages, sequences, short rows
//   gate       per row (one block): score the row's sampled pages (every 32nd
//              page) and keep their keys in registers; the k'-th largest (k' as
//              in the prefill path's calibration) is the row's gate; the
//              candidate count is reset
//   scan       per (row, split) wave: every page of the split; keys above the
//              gate are staged in LDS and appended to the row's bounded buffer
//   merge      per row: exact top-K of the candidates (if K <= count <= cap),
//              emitted through the row's page table; other rows are listed
//   fallback   listed rows only: per-wave exact streaming TopK in a bounded LDS
//              pool (radix compaction), then the splits merged exactly
// Roof: with one row per sequence every key byte is read once per row, 68 bytes
// per scored pair from HBM (against 8 TB/s), plus the MXFP4 MFMA and fp32
// epilogue work of the prefill scan.
#include "mqa_device.h"
#include "mqa_launch.h"
#include "mqa_select.h"

namespace mqa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kPageBytes = kPage * kVecBytes;
constexpr int kPageScaleBytes = kPage * kVecScales;
constexpr int kDecSampleStride = 32;   // the calibration scores every 32nd page (a 1/16
                                       // sample measured 5% slower per call: twice the gate's
                                       // page chain, for a gate the scan did not need)
constexpr int kDecStage = 128;         // staged candidate keys per wave (keeps a 4-wave scan block
                                       // at 38,912 B of LDS: four blocks per CU)
constexpr int kDecFallbackBlocks = 512;

template <int K>
struct DecGeom;
template <>
struct DecGeom<512> {
  static constexpr int kCap = 640;    // fallback pool keys per wave: K plus two 64-key batches
};
template <>
struct DecGeom<1024> {
  static constexpr int kCap = 1152;
};

struct DecArgs {
  const uint8_t* q;
  const uint8_t* q_scale;
  const float* weights;
  const uint8_t* k_pages;
  const uint8_t* k_scale;
  int64_t P_phys;
  const int32_t* block_table;
  int64_t max_pages;
  const int32_t* seq_of_row;
  const int32_t* row_start;
  const int32_t* row_end;
  const int32_t* row_state;
  int32_t Q;
  int32_t splits;
  DecodeScratch w;
  int32_t cap;        // candidate keys per row
  int32_t no_fallback;   // fail closed instead of listing rows for the fallback
};

__device__ __forceinline__ void vm_wait_all() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ const int32_t* row_table(const DecArgs& a, int row) {
  return a.block_table + static_cast<size_t>(a.seq_of_row[row]) * a.max_pages;
}

// One page (64 positions) of the paged cache into the wave's LDS slot, in the
// score-block image (position p at p * 64, chunk c at slot c ^ chunk_swizzle(p));
// the swizzle is applied on the source side because a lane's LDS destination is
// fixed by its lane id. Out-of-range entries are not copied (row_prep failed
// every row whose window touches them).
__device__ __forceinline__ void page_dma(const DecArgs& a, int32_t e, uint8_t* codes, uint8_t* scales, int lane) {
  if (e < 0 || e >= a.P_phys) return;
  const uint8_t* page = a.k_pages + static_cast<size_t>(e) * kPageBytes;
  const int pq = lane >> 2, slot = lane & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 16 * j + pq;
    __builtin_amdgcn_global_load_lds(page + p * kVecBytes + 16 * (slot ^ chunk_swizzle(p)), codes + 16 * j * kVecBytes,
                                     16, 0, 0);
  }
  __builtin_amdgcn_global_load_lds(a.k_scale + static_cast<size_t>(e) * kPageScaleBytes + lane * kVecScales, scales, 4,
                                   0, 0);
}

// fp32 scores of the 64 positions of one LDS page image: lane l, position l.
__device__ __forceinline__ float score_page(const QRow& qr, const uint8_t* codes, const uint8_t* scales,
                                            const LaneOffsets& lo) {
  const GroupAcc g0 = mfma_group<0>(qr, codes, scales, lo);
  const float h0 = head_partial(qr, g0.d0, g0.d1);
  const GroupAcc g1 = mfma_group<1>(qr, codes, scales, lo);
  const float h1 = head_partial(qr, g1.d0, g1.d1);
  return combine_halves(h0, h1);
}

// The wave's LDS: two page buffers as separate variables (read and written
// under static names, the loop below is unrolled by two), so that the copy of
// the next page is not waited for before the current page's reads.
struct WavePages {
  uint8_t* c0;
  uint8_t* s0;
  uint8_t* c1;
  uint8_t* s1;
};

// Streams pages first, first + stride, ... (< end_pg) of `table` through the
// wave's two buffers and calls body(page, codes, scales) for each. Table entries
// come 64 pages per vector load, the next chunk prefetched.
template <class Body>
__device__ __forceinline__ void stream_pages(const DecArgs& a, const int32_t* table, int first, int end_pg,
                                             int stride, const WavePages& b, int lane, Body&& body) {
  if (first >= end_pg) return;
  const int n = (end_pg - first + stride - 1) / stride;
  auto chunk = [&](int c) -> int32_t {
    const int i = 64 * c + lane;
    return i < n ? table[first + stride * i] : -1;
  };
  int32_t cur = chunk(0), nxt = chunk(1);
  int base = 0;   // first stream index of chunk `cur`
  auto entry = [&](int j) -> int32_t {   // stream index base + j, j < 128
    return (j >> 6) == 0 ? __builtin_amdgcn_readlane(cur, j & 63) : __builtin_amdgcn_readlane(nxt, j & 63);
  };
  auto step = [&](int i, const uint8_t* codes, const uint8_t* scales, uint8_t* nc, uint8_t* ns) {
    if (i + 1 < n) {
      page_dma(a, entry(i + 1 - base), nc, ns, lane);
      if (((i + 1 - base) >> 6) != 0) {   // page i + 1 opened the next chunk
        cur = nxt;
        base += 64;
        nxt = chunk(base / 64 + 1);
      }
    }
    body(first + stride * i, codes, scales);
    vm_wait_all();
  };
  vm_wait_all();
  page_dma(a, entry(0), b.c0, b.s0, lane);
  vm_wait_all();
  for (int i = 0; i < n; i += 2) {
    step(i, b.c0, b.s0, b.c1, b.s1);
    if (i + 1 < n) step(i + 1, b.c1, b.s1, b.c0, b.s0);
  }
}

// Pages [pa, pb) of split `split` of the row's window pages.
__device__ __forceinline__ void split_pages(int start, int end, int split, int splits, int* pa, int* pb) {
  const int pg0 = start / kPage, n_pages = (end - 1) / kPage + 1 - pg0;
  *pa = pg0 + static_cast<int>(static_cast<int64_t>(n_pages) * split / splits);
  *pb = pg0 + static_cast<int>(static_cast<int64_t>(n_pages) * (split + 1) / splits);
}

// Sampled positions of a window: those in pages whose index is a multiple of
// `stride`.
__device__ __forceinline__ int sampled_positions(int start, int end, int stride) {
  int m = 0;
  for (int pg = (start / kPage + stride - 1) / stride * stride; pg * kPage < end; pg += stride)
    m += min(end, (pg + 1) * kPage) - max(start, pg * kPage);
  return m;
}

#define MQA_WAVE_PAGES                                                               \
  __shared__ __attribute__((aligned(16))) uint8_t s_c0[kDecWaves][kPageBytes];       \
  __shared__ __attribute__((aligned(16))) uint8_t s_c1[kDecWaves][kPageBytes];       \
  __shared__ __attribute__((aligned(16))) uint8_t s_s0[kDecWaves][kPageScaleBytes];  \
  __shared__ __attribute__((aligned(16))) uint8_t s_s1[kDecWaves][kPageScaleBytes]

// ---- calibration and gate per row ---------------------------------------------------
// One 1024-thread block per long row. Its 16 waves score the row's sampled pages
// (index a multiple of the sample stride), wave w taking sampled pages w, w + 16,
// ..., each streamed through the wave's two LDS page buffers; every lane keeps
// the key of its position of each page in a register (0 = no key: a real key's
// low word is ~position, never 0). The block's exact radix select over those
// registers gives the k'-th largest sampled key, and the gate just below it.
// The stride is kDecSampleStride pages, or on windows of more than
// kDecSampleStride * 16 * kDecGateRegs pages (262,144 positions) the multiple
// of it that keeps the sample within 16 * kDecGateRegs pages; any gate keeps the
// result exact, a coarser one only lets more candidates through.
// mode 0: gate from the sample; 1: every long row to the exact fallback (no
// prefilter); 2: gate above every key (forced underfill, then the fallback).
constexpr int kDecGateWaves = 16;
constexpr int kDecGateRegs = 8;   // sampled pages per wave

template <int K>
__global__ void __launch_bounds__(kDecGateWaves * 64) decode_gate_kernel(DecArgs a, int mode) {
  constexpr int NT = kDecGateWaves * 64;
  __shared__ __attribute__((aligned(16))) uint8_t s_c0[kDecGateWaves][kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_c1[kDecGateWaves][kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_s0[kDecGateWaves][kPageScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_s1[kDecGateWaves][kPageScaleBytes];
  __shared__ uint32_t s_hist[2048];
  __shared__ BlockScratch<NT> s_red;
  const int row = blockIdx.x;
  if (a.row_state[row] != kRowLong) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int start = a.row_start[row], end = a.row_end[row];
  const int pg0 = start / kPage, pg1 = (end - 1) / kPage + 1;   // the window's pages [pg0, pg1)
  // L pages hold at most ceil(L / s) multiples of s: this stride leaves at most
  // B = 16 * kDecGateRegs sampled pages (kDecSampleStride up to that many times B pages).
  constexpr int kBudget = kDecGateWaves * kDecGateRegs;
  const int L = pg1 - pg0;
  const int stride = kDecSampleStride * max(1, (L + kDecSampleStride * kBudget - 1) / (kDecSampleStride * kBudget));
  const int m = sampled_positions(start, end, stride);
  const int kp = sample_keep(K, m, end - start);
  uint64_t gate = 0;
  uint32_t count = 0;
  if (mode == 1) {
    gate = ~0ull;
    count = static_cast<uint32_t>(a.cap) + 1;   // overflow marker: exact fallback
  } else if (mode == 2) {
    gate = ~0ull;                                // nothing passes: underfill, then the fallback
  } else if (m > kp) {
    QRow qr;
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);
    const LaneOffsets lo = lane_offsets(lane);
    uint64_t x[kDecGateRegs];
#pragma unroll
    for (int j = 0; j < kDecGateRegs; ++j) x[j] = 0ull;
    const int first = (pg0 + stride - 1) / stride * stride + stride * wave;
    stream_pages(a, row_table(a, row), first, pg1, stride * kDecGateWaves,
                 WavePages{s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]}, lane,
                 [&](int pg, const uint8_t* codes, const uint8_t* scales) {
      const float sc = score_page(qr, codes, scales, lo);
      const int pos = pg * kPage + lane;
      // shift register: the newest key enters at the top (static register names)
#pragma unroll
      for (int j = 0; j + 1 < kDecGateRegs; ++j) x[j] = x[j + 1];
      x[kDecGateRegs - 1] = (pos >= start && pos < end) ? make_key(sc, static_cast<uint32_t>(pos)) : 0ull;
    });
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < kDecGateRegs; ++j)
      if (x[j] != 0ull) valid |= 1u << j;
    bool ok = false;
    const uint64_t T = block_radix_select_regs<NT, 11, kDecGateRegs>(x, valid, kp, s_hist, s_red, &ok);
    if (ok) {
      gate = T - 1;
    } else {
      gate = ~0ull;
      count = static_cast<uint32_t>(a.cap) + 1;
    }
  }
  if (threadIdx.x == 0) {
    a.w.gate[row] = gate;
    a.w.cand_n[row] = count;
  }
}

// ---- gated scan ---------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(kDecThreads, 2) decode_gscan_kernel(DecArgs a) {
  MQA_WAVE_PAGES;
  __shared__ uint64_t s_stage[kDecWaves][kDecStage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kDecWaves + wave;
  if (item >= static_cast<int64_t>(a.Q) * a.splits) return;
  const int row = static_cast<int>(item / a.splits), split = static_cast<int>(item % a.splits);
  if (a.row_state[row] != kRowLong) return;
  if (a.w.cand_n[row] > static_cast<uint32_t>(a.cap)) return;   // already sent to the fallback
  const int start = a.row_start[row], end = a.row_end[row];
  const uint64_t gate = a.w.gate[row];
  const float gate_f = gate_floor(gate);
  int pa, pb;
  split_pages(start, end, split, a.splits, &pa, &pb);
  QRow qr;
  load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
            a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
            a.weights + static_cast<size_t>(row) * kHeads, lane);
  const LaneOffsets lo = lane_offsets(lane);
  uint64_t* stage = s_stage[wave];
  uint64_t* dst = a.w.cand + static_cast<size_t>(row) * a.cap;
  int sf = 0;
  auto flush = [&]() {
    wave_lds_sync();
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&a.w.cand_n[row], static_cast<uint32_t>(sf));
    base = __shfl(base, 0, 64);
    for (int i = lane; i < sf; i += 64) {
      const uint32_t at = base + static_cast<uint32_t>(i);
      if (at < static_cast<uint32_t>(a.cap)) dst[at] = stage[i];
    }
    wave_lds_sync();
    sf = 0;
  };
  stream_pages(a, row_table(a, row), pa, pb, 1, WavePages{s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]}, lane,
               [&](int pg, const uint8_t* codes, const uint8_t* scales) {
    const float sc = score_page(qr, codes, scales, lo);
    const int p0 = pg * kPage;
    const uint64_t win = (p0 >= start && p0 + kPage <= end) ? ~0ull : window_lanes(p0, start, end);
    uint64_t msk = __ballot(!(sc < gate_f)) & win;   // superset of key > gate
    if (msk == 0) return;
    const uint64_t key = make_key(sc, static_cast<uint32_t>(p0 + lane));
    msk &= __ballot(key > gate);
    if (msk == 0) return;
    const int cnt = __popcll(msk);
    if (sf + cnt > kDecStage) flush();
    if ((msk >> lane) & 1ull) stage[sf + mbcnt64(msk)] = key;
    sf += cnt;
  });
  if (sf > 0) flush();
}

// ---- exact merge of the candidates ------------------------------------------------
template <int K>
__global__ void __launch_bounds__(1024) decode_gmerge_kernel(DecArgs a, int32_t* __restrict__ out_raw,
                                                             int32_t* __restrict__ out_slot,
                                                             int32_t* __restrict__ out_count,
                                                             float* __restrict__ out_score, int32_t* status) {
  constexpr int NT = 1024;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[2048];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  const int64_t row = blockIdx.x;
  if (a.row_state[row] != kRowLong) return;
  const uint32_t n = a.w.cand_n[row];
  if (n > static_cast<uint32_t>(a.cap) || n < static_cast<uint32_t>(K)) {
    if (a.no_fallback) {   // fail closed: underfill (fewer than K above the gate) or overflow
      fail_row<K, NT>(row, n < static_cast<uint32_t>(K) ? kCodeUnderfill : kCodeSelector, out_raw, out_slot,
                      out_count, out_score, status);
      return;
    }
    if (threadIdx.x == 0) a.w.fb_list[atomicAdd(a.w.fb_count, 1)] = static_cast<int32_t>(row);
    return;
  }
  const uint64_t* keys = a.w.cand + static_cast<size_t>(row) * a.cap;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  constexpr int E = (decode_candidate_cap(K) + NT - 1) / NT;   // every candidate in registers (n <= cap)
  uint64_t x[E];
  const uint32_t valid = load_keys_regs<NT, E>(keys, static_cast<int>(n), x);
  bool ok = true;
  uint64_t T = 0;
  if (n > static_cast<uint32_t>(K)) T = block_radix_select_regs<NT, 11, E>(x, valid, K, s_hist, s_red, &ok);
  if (ok) gather_at_least<K, E>(x, valid, T, s_sel, &s_n);
  __syncthreads();
  if (!ok || s_n != K) {
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, status);
    return;
  }
  emit_row<K, NT>(s_sel, row, row_table(a, static_cast<int>(row)), a.max_pages, out_raw, out_slot, out_count,
                  out_score);
}

// ---- fallback: exact streaming TopK of the listed rows ----------------------------
// Persistent over (listed row, split) items, one per wave; each wave keeps an
// exact LDS pool (a key enters only above the pool's gate; when a batch would
// overflow it the wave radix-selects the K largest and raises the gate).
template <int K>
__global__ void __launch_bounds__(kDecThreads, 2) decode_fb_scan_kernel(DecArgs a) {
  constexpr int CAP = DecGeom<K>::kCap;
  static_assert(CAP >= K + 128, "pool holds K keys and two batches");
  MQA_WAVE_PAGES;
  __shared__ uint64_t s_pool[kDecWaves][CAP];
  __shared__ uint32_t s_hist[kDecWaves][256];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t items = static_cast<int64_t>(*a.w.fb_count) * a.splits;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kDecWaves;
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * kDecWaves + wave; item < items; item += waves) {
    const int row = a.w.fb_list[item / a.splits], split = static_cast<int>(item % a.splits);
    const int start = a.row_start[row], end = a.row_end[row];
    int pa, pb;
    split_pages(start, end, split, a.splits, &pa, &pb);
    QRow qr;
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);
    const LaneOffsets lo = lane_offsets(lane);
    uint64_t* pool = s_pool[wave];
    uint32_t* hist = s_hist[wave];
    int fill = 0;
    uint64_t gate = 0;
    bool failed = false;
    stream_pages(a, row_table(a, row), pa, pb, 1, WavePages{s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]}, lane,
                 [&](int pg, const uint8_t* codes, const uint8_t* scales) {
      const float sc = score_page(qr, codes, scales, lo);
      const int p0 = pg * kPage;
      const uint64_t win = (p0 >= start && p0 + kPage <= end) ? ~0ull : window_lanes(p0, start, end);
      const uint64_t key = make_key(sc, static_cast<uint32_t>(p0 + lane));
      bool pass = ((win >> lane) & 1ull) && key > gate;
      uint64_t msk = __ballot(pass);
      if (msk == 0) return;
      int cnt = __popcll(msk);
      if (fill + cnt > CAP) {
        const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
        if (sel.kept != K) failed = true;
        fill = K;
        gate = sel.T - 1;
        pass = pass && key > gate;
        msk = __ballot(pass);
        cnt = __popcll(msk);
      }
      if (pass) pool[fill + mbcnt64(msk)] = key;
      fill += cnt;
    });
    wave_lds_sync();
    if (fill > K) {
      const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
      if (sel.kept != K) failed = true;
      fill = K;
    }
    uint64_t* dst = a.w.keys + (static_cast<size_t>(row) * a.splits + split) * K;
    for (int i = lane; i < fill; i += 64) dst[i] = pool[i];
    if (lane == 0) a.w.counts[static_cast<size_t>(row) * a.splits + split] = failed ? kCodeSelector : fill;
    wave_lds_sync();   // the pool is reused by the wave's next item
  }
}

// One 1024-thread block per listed row (persistent); 11-bit radix digits (the
// splits hold up to 64 K keys per row, so wide digits save passes over them).
template <int K>
__global__ void __launch_bounds__(1024) decode_fb_merge_kernel(DecArgs a, int32_t* __restrict__ out_raw,
                                                               int32_t* __restrict__ out_slot,
                                                               int32_t* __restrict__ out_count,
                                                               float* __restrict__ out_score, int32_t* status) {
  constexpr int NT = 1024;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[2048];
  __shared__ int32_t s_cnt[kMaxDecodeSplits];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n, s_total;
  const int listed = *a.w.fb_count;
  const int splits = a.splits;
  for (int li = blockIdx.x; li < listed; li += gridDim.x) {
    const int64_t row = a.w.fb_list[li];
    const uint64_t* keys = a.w.keys + static_cast<size_t>(row) * splits * K;
    if (threadIdx.x == 0) {
      int total = 0;
      bool bad = false;
      for (int i = 0; i < splits; ++i) {
        s_cnt[i] = a.w.counts[static_cast<size_t>(row) * splits + i];
        bad |= s_cnt[i] < 0 || s_cnt[i] > K;
        total += s_cnt[i];
      }
      s_total = bad ? -1 : total;
      s_n = 0;
    }
    __syncthreads();
    if (s_total < K) {   // a split's selector failed (-1), or fewer than K keys survived: fail closed
      fail_row<K, NT>(row, s_total < 0 ? kCodeSelector : kCodeUnderfill, out_raw, out_slot, out_count, out_score,
                      status);
      __syncthreads();
      continue;
    }
    auto src = [&](int64_t e, uint64_t& x) -> bool {
      const int sp = static_cast<int>(e / K), j = static_cast<int>(e % K);
      if (j >= s_cnt[sp]) return false;
      x = keys[e];
      return true;
    };
    bool ok = true;
    uint64_t T = 0;
    if (s_total > K) T = block_radix_select<NT, 11>(src, static_cast<int64_t>(splits) * K, K, s_hist, s_red, &ok);
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
      fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, status);
    } else {
      emit_row<K, NT>(s_sel, row, row_table(a, static_cast<int>(row)), a.max_pages, out_raw, out_slot, out_count,
                      out_score);
    }
    __syncthreads();
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <int K>
void launch_decode_k(const DecArgs& a, const PathArgs& p, int mode, int32_t* status, hipStream_t st,
                     StageMark mark) {
  const int64_t items = p.Q * a.splits;
  const dim3 sgrid(static_cast<unsigned>((items + kDecWaves - 1) / kDecWaves));
  const dim3 rgrid(static_cast<unsigned>(p.Q));
  const int64_t fb_cap = (items + kDecWaves - 1) / kDecWaves;
  const dim3 fgrid(static_cast<unsigned>(fb_cap < kDecFallbackBlocks ? fb_cap : kDecFallbackBlocks));
  decode_gate_kernel<K><<<rgrid, dim3(kDecGateWaves * 64), 0, st>>>(a, mode);
  if (mark) mark(2, st);   // before the gated scan
  decode_gscan_kernel<K><<<sgrid, dim3(kDecThreads), 0, st>>>(a);
  if (mark) mark(3, st);   // after it
  decode_gmerge_kernel<K><<<rgrid, dim3(1024), 0, st>>>(a, p.out_raw, p.out_slot, p.out_count, p.out_score, status);
  decode_fb_scan_kernel<K><<<fgrid, dim3(kDecThreads), 0, st>>>(a);
  const unsigned mblocks = static_cast<unsigned>(p.Q < kDecFallbackBlocks ? p.Q : kDecFallbackBlocks);
  decode_fb_merge_kernel<K><<<dim3(mblocks), dim3(1024), 0, st>>>(a, p.out_raw, p.out_slot, p.out_count,
                                                                  p.out_score, status);
}

}  // namespace

size_t decode_scratch_bytes(int64_t Q, int32_t K, int32_t splits) {
  const size_t q = static_cast<size_t>(Q), s = static_cast<size_t>(splits);
  const size_t cap = static_cast<size_t>(decode_candidate_cap(K));
  return align256(q * sizeof(int32_t)) + align256(q * s * sizeof(int32_t)) +
         align256(q * s * static_cast<size_t>(K) * sizeof(uint64_t)) + align256(q * sizeof(uint64_t)) +
         align256(q * sizeof(uint32_t)) + align256(q * cap * sizeof(uint64_t)) + align256(q * sizeof(int32_t)) +
         align256(sizeof(int32_t));
}

DecodeScratch decode_scratch_layout(void* base, int64_t Q, int32_t K, int32_t splits) {
  const size_t q = static_cast<size_t>(Q), s = static_cast<size_t>(splits);
  const size_t cap = static_cast<size_t>(decode_candidate_cap(K));
  char* b = static_cast<char*>(base);
  DecodeScratch w;
  auto take = [&](size_t bytes) {
    char* at = b;
    b += align256(bytes);
    return at;
  };
  w.row_state = reinterpret_cast<int32_t*>(take(q * sizeof(int32_t)));
  w.counts = reinterpret_cast<int32_t*>(take(q * s * sizeof(int32_t)));
  w.keys = reinterpret_cast<uint64_t*>(take(q * s * static_cast<size_t>(K) * sizeof(uint64_t)));
  w.gate = reinterpret_cast<uint64_t*>(take(q * sizeof(uint64_t)));
  w.cand_n = reinterpret_cast<uint32_t*>(take(q * sizeof(uint32_t)));
  w.cand = reinterpret_cast<uint64_t*>(take(q * cap * sizeof(uint64_t)));
  w.fb_list = reinterpret_cast<int32_t*>(take(q * sizeof(int32_t)));
  w.fb_count = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  return w;
}

hipError_t launch_decode(const PathArgs& p, const DecodeScratch& w, int32_t splits, int mode, bool no_fallback,
                         hipStream_t st, StageMark mark) {
  if (p.Q == 0) return hipSuccess;
  int32_t* status = status_word();
  if (status == nullptr) return hipErrorInvalidSymbol;
  DecArgs a;
  a.q = p.q;
  a.q_scale = p.q_scale;
  a.weights = p.weights;
  a.k_pages = p.k_pages;
  a.k_scale = p.k_scale;
  a.P_phys = p.P_phys;
  a.block_table = p.page_table;
  a.max_pages = p.P_log;
  a.seq_of_row = p.seq_of_row;
  a.row_start = p.row_start;
  a.row_end = p.row_end;
  a.row_state = w.row_state;
  a.Q = static_cast<int32_t>(p.Q);
  a.splits = splits;
  a.w = w;
  a.cap = decode_candidate_cap(p.K);
  a.no_fallback = no_fallback ? 1 : 0;
  if (p.K == 512) launch_decode_k<512>(a, p, mode, status, st, mark);
  else launch_decode_k<1024>(a, p, mode, status, st, mark);
  return hipGetLastError();
}

}  // namespace mqa
