// Decode / multi-sequence variant of the FP4 paged-MQA indexer with exact TopK
// (gfx950). Every row has its own page table (block table row seq_of_row[r]),
// so rows share no key tiles: each wave streams its own pages, the way the
// pages' first fused design works per CTA ("[FlyDSL][DSv4] Prototype FP4 MQA
// streaming TopK", Changes: running candidates held in a fixed-size LDS pool,
// an exact radix selection on the total-order key, only candidates and their
// number handed on, an exact merge of the splits, then the page-table
// mapping). Decode workloads are the adjacent shape the pages leave on the
// older path ("[AMD][DSv4] Add experimental AITER FP4 streaming TopK", Changes
// / Scope) and whose graph-capture support they defer ("[FlyDSL][DSv4]
// Prototype FP4 MQA streaming TopK", Scope); this entry point takes its
// scratch from the caller, never allocates or synchronises,
// and reports row failures only on the device, so it can be captured into a
// HIP graph and replayed.
//
// Pipeline (all on the caller's stream):
//   row_prep   windows, per-row pages, sequences, short rows
//   gate       per row (one block): score the row's sampled pages (every 32nd
//              page) and keep their keys in registers; the k'-th largest (k' as
//              in the prefill path's calibration) is the row's gate; the
//              row's shared candidate count is reset. Block 0 writes the plan:
//              which pages of which row each scan wave reads
//   scan       one resident round of waves, each streaming its planned pages
//              (three LDS buffers, two pages in flight); keys above the row's
//              gate are held in registers and written to the wave's own region
//   merge      per row: gather the row's candidates from its waves' regions
//              (and the shared buffer), exact top-K if K <= count <= cap,
//              emitted through the row's page table; other rows are listed
//   fallback   listed rows only: per-wave exact streaming TopK in a bounded LDS
//              pool (radix compaction), then the splits merged exactly
// Roof: with one row per sequence every key byte is read once per row, 68 bytes
// per scored pair from HBM (against 8 TB/s), plus the MXFP4 MFMA and fp32
// epilogue work of the prefill scan.
#include <atomic>

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
constexpr int kLaneSlots = 4;          // candidate keys a lane of the gated scan holds before writing
constexpr int kDecFallbackBlocks = 512;
constexpr int kDecScanBlocksPerCu = 3;   // three 4-wave scan blocks (52,224 B of LDS each) fit one CU,
                                         // unless the occupancy query says otherwise
constexpr int kDecMinPages = 2;          // pages per scan wave at least (small batches use fewer waves)

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
  int32_t P_phys;   // fits int32 (the host checks 64 P_phys against INT32_MAX): a scalar page check
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
  int32_t scan_waves;    // waves of the gated scan's grid
};

__device__ __forceinline__ void vm_wait_all() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

// The lane index from an instruction the compiler cannot move out of a loop:
// per-lane addresses derived from it are recomputed where they are used rather
// than hoisted and held in registers across the loop.
__device__ __forceinline__ int fresh_lane() {
  int lane;
  __asm__ __volatile__("v_and_b32 %0, 63, %1" : "=v"(lane) : "v"(static_cast<int>(threadIdx.x)));
  return lane;
}

__device__ __forceinline__ const int32_t* row_table(const DecArgs& a, int row) {
  return a.block_table + static_cast<size_t>(a.seq_of_row[row]) * a.max_pages;
}

// One page (64 positions) of the paged cache into a wave's LDS buffer, in the
// score-block image (position p at p * 64, chunk c at slot c ^ chunk_swizzle(p));
// the swizzle is applied on the source side because a lane's LDS destination is
// fixed by its lane id. Five vector memory operations, whatever the entry: an
// entry outside the cache is replaced by page 0 (row_prep has already failed
// every row whose window touches one; this only keeps the copy in bounds). The
// key cache is read once per row, so its lines are fetched with the
// non-temporal policy (kNonTemporal).
constexpr int kNonTemporal = 2;   // NT bit of the gfx950 cache-policy operand

__device__ __forceinline__ void copy_page(const DecArgs& a, int32_t e, uint8_t* codes, uint8_t* scales, int lane) {
  e = (e >= 0 && e < a.P_phys) ? e : 0;
  const uint8_t* page = a.k_pages + static_cast<size_t>(e) * kPageBytes;
  const int pq = lane >> 2, slot = lane & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 16 * j + pq;
    __builtin_amdgcn_global_load_lds(page + p * kVecBytes + 16 * (slot ^ chunk_swizzle(p)), codes + 16 * j * kVecBytes,
                                     16, 0, kNonTemporal);
  }
  __builtin_amdgcn_global_load_lds(a.k_scale + static_cast<size_t>(e) * kPageScaleBytes + lane * kVecScales, scales, 4,
                                   0, kNonTemporal);
}

// fp32 scores of the 64 positions of one LDS page image (lane l, position l),
// its LDS reads in inline asm; used by the gate, the gated scan and the
// fallback. The compiler inserts a wait for every outstanding LDS copy before
// an LDS read it cannot prove independent of them, and across the page loops
// it cannot, which would serialise the page streams; the streams order the
// reads after the copies with their own waits instead (stream_pages2,
// stream_pages3). Each asm block waits for its reads before it ends, and its
// memory clobber keeps it between the copies around it. The MFMA groups and
// head sums are the prefill scan's (mfma_group, head_partial, combine_halves),
// in the same order, so a position's score is the same bit for bit.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <int GRP>
__device__ __forceinline__ GroupAcc mfma_group_asm(const QRow& r, uint32_t codes, uint32_t scales,
                                                   const LaneOffsets& o) {
  v4i b0, b1;
  int ks;
  __asm__ __volatile__(
      "ds_read_b128 %0, %3 offset:%6\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_u16 %2, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(b0), "=v"(b1), "=v"(ks)
      : "v"(codes + o.code0), "v"(codes + o.code1), "v"(scales + o.scale), "i"(GRP * 32 * kVecBytes),
        "i"(GRP * 32 * kVecScales)
      : "memory");
  const v16f z = {};
  GroupAcc acc;
  __builtin_amdgcn_s_setprio(1);
  acc.d0 = mfma_fp4<0, 0>(r.a[0][0], b0, z, r.scale, ks);
  acc.d0 = mfma_fp4<1, 1>(r.a[0][1], b1, acc.d0, r.scale, ks);
  acc.d1 = mfma_fp4<2, 0>(r.a[1][0], b0, z, r.scale, ks);
  acc.d1 = mfma_fp4<3, 1>(r.a[1][1], b1, acc.d1, r.scale, ks);
  __builtin_amdgcn_s_setprio(0);
  return acc;
}

__device__ __forceinline__ float score_page_asm(const QRow& qr, const uint8_t* codes, const uint8_t* scales,
                                                const LaneOffsets& lo) {
  const uint32_t c = lds_addr(codes), sc = lds_addr(scales);
  const GroupAcc g0 = mfma_group_asm<0>(qr, c, sc, lo);
  const float h0 = head_partial(qr, g0.d0, g0.d1);
  const GroupAcc g1 = mfma_group_asm<1>(qr, c, sc, lo);
  const float h1 = head_partial(qr, g1.d0, g1.d1);
  return combine_halves(h0, h1);
}

// The gate and fallback kernels' LDS: two page buffers per wave.
struct WavePages {
  uint8_t* c0;
  uint8_t* s0;
  uint8_t* c1;
  uint8_t* s1;
};

// Pages first .. end_pg - 1 of `table` through the wave's three buffers: while
// one page is scored the next two are in flight. The table entries of each run
// of up to 64 pages come in one vector load, complete before the run starts
// (a load result still in flight across the loop would make the compiler wait
// for every outstanding copy). The scan reads its pages with inline-asm LDS
// reads (score_page_asm) that the compiler does not see, so the waits here,
// not the compiler's, order the reads after the copies: a step that issued a
// copy ends with a wait that leaves that copy in flight (five vector memory
// operations: s_waitcnt counts them in issue order, so the copy of the next
// page, issued one step earlier, is complete); the last two steps of a run
// issue none and wait for everything. The scoring issues no vector memory
// operation except, rarely, stores of candidates (the wait after those waits
// for more than it needs to; it stays correct). An entry outside the cache is
// replaced by page 0: row_prep has already failed every row whose window
// touches one; this only keeps the copy in bounds.
struct WavePages3 {
  uint8_t* c0;
  uint8_t* s0;
  uint8_t* c1;
  uint8_t* s1;
  uint8_t* c2;
  uint8_t* s2;
};

// s_waitcnt through the builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima), which the compiler's own
// wait insertion takes into account, unlike a wait written in inline asm.
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0)
constexpr int kWaitVm5 = 0x0F75;   // vmcnt(5): all but the last page copy issued
// (The non-temporal policy on the page copies: on a 64-row decode batch the gated
// scan 69 -> 63 us with identical outputs; the SC0 bit alone changed nothing.)

__device__ __forceinline__ void vm_wait_but_one_page() {
  __builtin_amdgcn_s_waitcnt(kWaitVm5);
  __asm__ __volatile__("" ::: "memory");
}

__device__ __forceinline__ void vm_wait_all_known() {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __asm__ __volatile__("" ::: "memory");
}

template <class Body>
__device__ __forceinline__ void stream_pages3(const DecArgs& a, const int32_t* table, int first, int end_pg,
                                              const WavePages3& b, int lane, Body&& body) {
  for (int run = first; run < end_pg; run += 64) {
    const int n = min(64, end_pg - run);
    const int32_t ent = lane < n ? table[run + lane] : -1;
    vm_wait_all_known();   // the entries
    auto issue = [&](int i, uint8_t* c, uint8_t* sc) { copy_page(a, __builtin_amdgcn_readlane(ent, i), c, sc, lane); };
    // page i in buffer (c, s), page i + 2 to buffer (fc, fs) if there is one
    auto step = [&](int i, const uint8_t* c, const uint8_t* sc, uint8_t* fc, uint8_t* fs) {
      const bool more = i + 2 < n;
      if (more) issue(i + 2, fc, fs);
      body(run + i, c, sc);
      if (more) vm_wait_but_one_page();
      else vm_wait_all_known();
    };
    issue(0, b.c0, b.s0);
    if (n > 1) {
      issue(1, b.c1, b.s1);
      vm_wait_but_one_page();
    } else {
      vm_wait_all_known();
    }
    for (int i = 0; i < n; i += 3) {   // page i in c0, i + 1 in c1, i + 2 in c2
      step(i, b.c0, b.s0, b.c2, b.s2);
      if (i + 1 < n) step(i + 1, b.c1, b.s1, b.c0, b.s0);
      if (i + 2 < n) step(i + 2, b.c2, b.s2, b.c1, b.s1);
    }
  }
}

// Pages first, first + stride, ... (< end_pg) of `table` through the wave's two
// buffers, the gate's and the fallback's stream: while page i is scored the
// copy of page i + 1 is in flight. Entries, reads and waits as in
// stream_pages3: body reads its page with inline-asm LDS reads (which complete
// before it returns, so the next copy may overwrite the buffer), and the waits
// here order the reads after the copies.
template <class Body>
__device__ __forceinline__ void stream_pages2(const DecArgs& a, const int32_t* table, int first, int end_pg, int stride,
                                              const WavePages& b, int lane, Body&& body) {
  if (first >= end_pg) return;
  const int total = (end_pg - first + stride - 1) / stride;
  for (int run = 0; run < total; run += 64) {
    const int n = min(64, total - run);
    const int32_t ent = lane < n ? table[first + stride * (run + lane)] : -1;
    vm_wait_all_known();   // the entries
    auto issue = [&](int i, uint8_t* c, uint8_t* sc) { copy_page(a, __builtin_amdgcn_readlane(ent, i), c, sc, lane); };
    // page i in buffer (c, s), then its buffer takes page i + 2 if there is one
    auto step = [&](int i, uint8_t* c, uint8_t* sc) {
      body(first + stride * (run + i), c, sc);
      if (i + 2 < n) {
        issue(i + 2, c, sc);
        vm_wait_but_one_page();   // page i + 1 is in
      } else {
        vm_wait_all_known();
      }
    };
    issue(0, b.c0, b.s0);
    if (n > 1) {
      issue(1, b.c1, b.s1);
      vm_wait_but_one_page();
    } else {
      vm_wait_all_known();
    }
    for (int i = 0; i < n; i += 2) {
      step(i, b.c0, b.s0);
      if (i + 1 < n) step(i + 1, b.c1, b.s1);
    }
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

// Equal shares of the plan's T pages among the scan's used waves (at least
// kDecMinPages each): wave w takes pages [begin(w), begin(w + 1)), the first
// `extra` waves one page more than the others.
struct Shares {
  int64_t total, used, share, extra;
  __device__ int64_t begin(int64_t w) const { return w * share + min(w, extra); }
  __device__ int64_t wave_of(int64_t g) const {   // the wave whose share holds page g < total
    const int64_t big = extra * (share + 1);
    return g < big ? g / (share + 1) : extra + (g - big) / share;
  }
};

__device__ __forceinline__ Shares scan_shares(int64_t total, int64_t waves) {
  Shares s;
  s.total = total;
  s.used = min(waves, max(static_cast<int64_t>(1), total / kDecMinPages));
  s.share = total / s.used;
  s.extra = total % s.used;
  return s;
}

// ---- plan of the gated scan -------------------------------------------------------
// Block 0 of the gate kernel (the other blocks are the rows' gates, concurrent
// with it). plan[r] = the pages the gated scan reads for rows 0 .. r-1, plan[Q]
// = all of them (T): a long row contributes its window's pages, other rows
// nothing (a long row that its gate sends to the fallback keeps its pages in
// the plan; the scan skips them). Then the scan's waves get their pages,
// written as wave_desc[w] = {g0, g1, first row} over the plan's concatenated
// list, and each row the waves over its pages (row_w0, row_nw):
//  - rows at most half as many as the waves (and at most kPlanLdsRows): every
//    row gets its own waves, ceil(pages / C) of them, C = ceil(T / (W - rows)),
//    its pages split evenly among them; no wave crosses a row, and no wave has
//    more than C pages;
//  - more rows: equal shares of the list (Shares), a wave may cover several
//    rows one after another.
// A wave's start then costs one descriptor load, and the merge finds a row's
// candidates without searching.
constexpr int kPlanLdsRows = 4096;
constexpr int kPlanThreads = 1024;   // the gate kernel's block

__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int off) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __shfl_up(static_cast<uint32_t>(u), off, 64);
  const uint32_t hi = __shfl_up(static_cast<uint32_t>(u >> 32), off, 64);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int32_t scanned_pages(const DecArgs& a, int64_t r) {
  const int32_t state = a.row_state[r], start = a.row_start[r], end = a.row_end[r];
  return state == kRowLong ? (end - 1) / kPage + 1 - start / kPage : 0;
}

// Exclusive prefix of one value per thread (thread order) and the block's total.
__device__ __forceinline__ int64_t block_exclusive_i64(int64_t v, int64_t* s_wave, int64_t* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = shfl_up_i64(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) s_wave[wv] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    if (i < wv) before += s_wave[i];
    all += s_wave[i];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ void put_desc(const DecArgs& a, int64_t w, int64_t g0, int64_t g1, int64_t row) {
  int64_t* d = a.w.wave_desc + 3 * w;
  d[0] = g0;
  d[1] = g1;
  d[2] = row;
}

// s_wave: kPlanThreads / 64 words; s_gpre: kPlanLdsRows + 1; s_wpre, s_pg: kPlanLdsRows + 1.
__device__ void plan_block(const DecArgs& a, int64_t* s_wave, int64_t* s_gpre, int32_t* s_wpre, int32_t* s_pg) {
  const int t = threadIdx.x;
  const int64_t Q = a.Q, W = a.scan_waves;
  const bool in_lds = Q <= kPlanLdsRows;
  const int64_t per = (Q + kPlanThreads - 1) / kPlanThreads;   // a run of consecutive rows per thread
  const int64_t r0 = min(Q, per * t), r1 = min(Q, r0 + per);
  auto pages = [&](int64_t r) -> int64_t { return in_lds ? s_pg[r] : scanned_pages(a, r); };
  int64_t own = 0, own_rows = 0;
  for (int64_t r = r0; r < r1; ++r) {
    const int32_t p = scanned_pages(a, r);
    if (in_lds) s_pg[r] = p;
    own += p;
    own_rows += p > 0;
  }
  int64_t T = 0, rows = 0;
  const int64_t first = block_exclusive_i64(own, s_wave, &T);
  block_exclusive_i64(own_rows, s_wave, &rows);
  int64_t at = first;
  for (int64_t r = r0; r < r1; ++r) {
    a.w.plan[r] = at;
    at += pages(r);
  }
  if (t == 0) a.w.plan[Q] = T;
  if (in_lds && 2 * rows <= W && T > 0) {
    const int64_t C = (T + (W - rows) - 1) / (W - rows);
    int64_t own_w = 0;
    for (int64_t r = r0; r < r1; ++r) own_w += (pages(r) + C - 1) / C;
    int64_t used = 0;
    int64_t wat = block_exclusive_i64(own_w, s_wave, &used);
    int64_t gat = first;
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t p = pages(r), nw = (p + C - 1) / C;
      s_wpre[r] = static_cast<int32_t>(wat);
      s_gpre[r] = gat;
      a.w.row_w0[r] = static_cast<uint32_t>(wat);
      a.w.row_nw[r] = static_cast<uint32_t>(nw);
      wat += nw;
      gat += p;
    }
    if (t == 0) {
      s_wpre[Q] = static_cast<int32_t>(used);
      s_gpre[Q] = T;
    }
    __syncthreads();
    for (int64_t w = t; w < W; w += kPlanThreads) {
      if (w >= used) {
        put_desc(a, w, 0, 0, 0);
        continue;
      }
      int lo = 0, hi = static_cast<int>(Q) - 1;   // the last row r with s_wpre[r] <= w: its waves hold w
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_wpre[mid] <= w) lo = mid;
        else hi = mid - 1;
      }
      const int64_t k = w - s_wpre[lo], nw = s_wpre[lo + 1] - s_wpre[lo], p = s_gpre[lo + 1] - s_gpre[lo];
      put_desc(a, w, s_gpre[lo] + p * k / nw, s_gpre[lo] + p * (k + 1) / nw, lo);
    }
  } else {
    const Shares sh = scan_shares(T, W);
    int64_t g = first;
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t p = pages(r);
      if (p > 0) {
        const int64_t w0 = sh.wave_of(g);
        a.w.row_w0[r] = static_cast<uint32_t>(w0);
        a.w.row_nw[r] = static_cast<uint32_t>(sh.wave_of(g + p - 1) - w0 + 1);
        // the waves whose share starts in this row
        for (int64_t w = sh.begin(w0) == g ? w0 : w0 + 1; w < sh.used && sh.begin(w) < g + p; ++w)
          put_desc(a, w, sh.begin(w), sh.begin(w + 1), r);
      }
      g += p;
    }
    for (int64_t w = (T > 0 ? sh.used : 0) + t; w < W; w += kPlanThreads) put_desc(a, w, 0, 0, 0);
  }
}

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
  static_assert(NT == kPlanThreads, "the plan runs in a gate block");
  static_assert(sizeof(s_c0) >= (kPlanLdsRows + 1) * sizeof(int64_t) &&
                    sizeof(s_c1) >= 2 * (kPlanLdsRows + 1) * sizeof(int32_t),
                "the plan's LDS fits the page buffers");
  if (blockIdx.x == 0) {
    plan_block(a, reinterpret_cast<int64_t*>(s_red.red64[0]), reinterpret_cast<int64_t*>(&s_c0[0][0]),
               reinterpret_cast<int32_t*>(&s_c1[0][0]), reinterpret_cast<int32_t*>(&s_c1[0][0]) + kPlanLdsRows + 1);
    return;
  }
  const int row = blockIdx.x - 1;
  // the window is read beside the row's state rather than after it: one memory
  // round trip less ahead of the page-table entries
  const int state = a.row_state[row], start = a.row_start[row], end = a.row_end[row];
  if (state != kRowLong) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
    stream_pages2(a, row_table(a, row), first, pg1, stride * kDecGateWaves,
                 WavePages{s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]}, lane,
                 [&](int pg, const uint8_t* codes, const uint8_t* scales) {
      const float sc = score_page_asm(qr, codes, scales, lo);
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

// The row r >= from with plan[r] <= g < plan[r + 1], given plan[from] <= g <
// plan[Q] (plan is non-decreasing). The wave's lanes read 64 entries at a time:
// the 64 rows after `from` first (the usual case: the next row), then coarse
// steps over the rest.
__device__ __forceinline__ int find_row(const int64_t* plan, int from, int Q, int64_t g, int lane) {
  {
    const int64_t i = static_cast<int64_t>(from) + lane;
    const uint64_t m = __ballot(i <= Q && plan[i] <= g);
    if (~m != 0ull) return from + 63 - __clzll(static_cast<long long>(m));
  }
  int64_t a0 = from + 63, n = static_cast<int64_t>(Q) + 1 - a0;   // plan[a0] <= g
  while (n > 64) {
    const int64_t step = (n + 63) / 64;
    const int64_t i = a0 + lane * step;
    const uint64_t m = __ballot(i < a0 + n && plan[i] <= g);
    const int l = 63 - __clzll(static_cast<long long>(m));
    a0 += l * step;
    n = min(step, n - l * step);
  }
  const uint64_t m = __ballot(lane < n && plan[a0 + lane] <= g);
  return static_cast<int>(a0) + 63 - __clzll(static_cast<long long>(m));
}

// ---- gated scan ---------------------------------------------------------------------
// Wave w of the grid's W (used) waves scans pages [T w / W, T (w + 1) / W) of the
// plan's concatenated list (T = plan[Q]); within a row, pages run in window order.
template <int K>
__global__ void __launch_bounds__(kDecThreads, 3) decode_gscan_kernel(DecArgs a) {
  // each buffer one LDS object (codes, then scales): three copy destinations
  // for the compiler to tell apart
  __shared__ __attribute__((aligned(16))) uint8_t s_p0[kDecWaves][kPageBytes + kPageScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p1[kDecWaves][kPageBytes + kPageScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p2[kDecWaves][kPageBytes + kPageScaleBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kDecWaves + wave;
  const int64_t* desc = a.w.wave_desc + 3 * w;
  int64_t g = desc[0];
  const int64_t g_end = desc[1];
  if (g >= g_end) return;
  int row = static_cast<int>(desc[2]);
  const LaneOffsets lofs = lane_offsets(lane);
  const WavePages3 bufs{s_p0[wave], s_p0[wave] + kPageBytes, s_p1[wave], s_p1[wave] + kPageBytes,
                        s_p2[wave], s_p2[wave] + kPageBytes};
  // The wave's candidates go to its own region of the workspace, in page order
  // (segment after segment), and the scan records per row where they are.
  // Each lane holds up to kLaneSlots keys of its own positions in registers;
  // they are written out with plain stores when a lane's slots are full (rare)
  // and at the end of each segment, so a step of the page stream issues no
  // memory operation besides its page copy and needs no atomic: a wait in the
  // stream would also wait for the copies in flight (vector memory operations
  // retire in issue order). Keys beyond the region's kDecWaveKeys go to the
  // row's shared buffer under an atomic reservation.
  uint64_t* wkeys = a.w.wave_keys + static_cast<size_t>(w) * kDecWaveStride;
  uint32_t woff = 0;   // keys in the region
  for (;;) {
    const int64_t row_base = a.w.plan[row];
    const int64_t seg_end = min(g_end, a.w.plan[row + 1]);
    const int start = a.row_start[row], end = a.row_end[row];
    const int pa = start / kPage + static_cast<int>(g - row_base);
    const int pb = start / kPage + static_cast<int>(seg_end - row_base);
    const uint64_t gate = a.w.gate[row];
    const float gate_f = gate_floor(gate);
    // (the query addresses of a row, hoisted out of this loop, would stay live
    // across the page stream)
    QRow qr;
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, fresh_lane());
    const uint32_t seg_off = woff;
    const bool to_fallback = a.w.cand_n[row] > static_cast<uint32_t>(a.cap);   // nothing to scan
    uint64_t held[kLaneSlots];
    int nh = 0;   // keys this lane holds, in held[0 .. nh-1] (newest first)
    auto flush = [&]() {
      uint64_t m[kLaneSlots];
      uint32_t total = 0;
#pragma unroll
      for (int j = 0; j < kLaneSlots; ++j) {
        m[j] = __ballot(nh > j);
        total += static_cast<uint32_t>(__popcll(m[j]));
      }
      uint32_t at = woff, spill_n = 0;
      if (woff + total > static_cast<uint32_t>(kDecWaveKeys)) {   // (rare) beyond the region
        spill_n = woff + total - static_cast<uint32_t>(kDecWaveKeys);
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.w.cand_n[row], spill_n);
        base = __builtin_amdgcn_readfirstlane(base);
        spill_n = base;   // reuse: first shared slot
      }
#pragma unroll
      for (int j = 0; j < kLaneSlots; ++j) {
        const uint32_t k = at + static_cast<uint32_t>(mbcnt64(m[j]));
        if (nh > j) {
          if (k < static_cast<uint32_t>(kDecWaveKeys)) {
            wkeys[k] = held[j];
          } else {
            const uint32_t sh = spill_n + (k - static_cast<uint32_t>(kDecWaveKeys));
            if (sh < static_cast<uint32_t>(a.cap)) a.w.cand[static_cast<size_t>(row) * a.cap + sh] = held[j];
          }
        }
        at += static_cast<uint32_t>(__popcll(m[j]));
      }
      woff = min(at, static_cast<uint32_t>(kDecWaveKeys));
      nh = 0;
    };
    stream_pages3(a, row_table(a, row), pa, to_fallback ? pa : pb, bufs, lane,
                  [&](int pg, const uint8_t* codes, const uint8_t* scales) {
      const float sc = score_page_asm(qr, codes, scales, lofs);
      const int p0 = pg * kPage;
      const uint64_t win = (p0 >= start && p0 + kPage <= end) ? ~0ull : window_lanes(p0, start, end);
      uint64_t msk = __ballot(!(sc < gate_f)) & win;   // superset of key > gate
      if (msk == 0) return;
      // as in the prefill scan: lanes strictly above the gate's score are above
      // the gate and not NaN; otherwise the exact 64-bit key test decides
      uint32_t hi = order_bits_finite(sc);
      const uint32_t lo32 = ~static_cast<uint32_t>(p0) - static_cast<uint32_t>(lane);   // ~(p0 + lane)
      if ((__ballot(sc > gate_f) & win) != msk) {
        if (__builtin_isnan(sc)) hi = 0u;
        msk &= __ballot(((static_cast<uint64_t>(hi) << 32) | lo32) > gate);
        if (msk == 0) return;
      }
      const uint64_t key = (static_cast<uint64_t>(hi) << 32) | lo32;   // make_key(sc, p0 + lane)
      // the wave-uniform mask as the lanes' predicate
      if ((__ballot(nh == kLaneSlots) & msk) != 0ull) flush();
      if (__builtin_amdgcn_inverse_ballot_w64(msk)) {
        // shift register (static register names): held[0 .. nh-1] are the lane's keys
#pragma unroll
        for (int j = kLaneSlots - 1; j > 0; --j) held[j] = held[j - 1];
        held[0] = key;
        ++nh;
      }
    });
    if (__ballot(nh > 0) != 0ull) flush();
    if (lane == 0) {
      const uint32_t cnt = woff - seg_off;
      if (g == row_base) {   // this wave holds the row's first page
        a.w.row_off[row] = seg_off;
        a.w.row_first[row] = cnt;
      } else {               // only a wave's first segment starts inside a row
        a.w.wave_first[w] = cnt;
      }
    }
    g = seg_end;
    if (g >= g_end) break;
    row = find_row(a.w.plan, row + 1, a.Q, g, lane);
  }
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
  __shared__ uint32_t s_pre[kDecScanWaves + 2];
  const int64_t row = blockIdx.x;
  if (a.row_state[row] != kRowLong) return;
  // The row's candidates: the region parts of the scan waves that covered its
  // pages (wave w0's from row_off, the later waves' from the start of their
  // regions), then the row's shared buffer (keys that did not fit a region).
  // A row the gate sent to the fallback has a shared count above the cap.
  const uint32_t shared_n = a.w.cand_n[row];
  int S = 0;   // region sources
  int64_t w0 = 0;
  if (shared_n <= static_cast<uint32_t>(a.cap)) {
    w0 = a.w.row_w0[row];
    S = static_cast<int>(a.w.row_nw[row]);
  }
  auto src_n = [&](int s) -> uint32_t {
    return s == 0 ? a.w.row_first[row] : s < S ? a.w.wave_first[w0 + s] : shared_n;
  };
  if (threadIdx.x == 0) s_pre[0] = 0;
  uint32_t carry = 0;
  for (int b0 = 0; b0 <= S; b0 += NT) {   // s_pre[s + 1] = keys of sources 0 .. s
    const int s = b0 + static_cast<int>(threadIdx.x);
    const uint32_t v = s <= S ? src_n(s) : 0u;
    const uint32_t suffix = block_suffix_sum<NT>(v, s_red);   // sum over threads >= this one
    if (threadIdx.x == 0) s_red.wtot[0] = suffix;              // thread 0's: the round's total
    __syncthreads();
    const uint32_t block_total = s_red.wtot[0];
    if (s <= S) s_pre[s + 1] = carry + block_total - suffix + v;
    carry += block_total;
    __syncthreads();
  }
  const uint32_t n = shared_n > static_cast<uint32_t>(a.cap) ? shared_n : carry;
  if (n > static_cast<uint32_t>(a.cap) || n < static_cast<uint32_t>(K)) {
    if (a.no_fallback) {   // fail closed: underfill (fewer than K above the gate) or overflow
      fail_row<K, NT>(row, n < static_cast<uint32_t>(K) ? kCodeUnderfill : kCodeSelector, out_raw, out_slot,
                      out_count, out_score, status);
      return;
    }
    if (threadIdx.x == 0) a.w.fb_list[atomicAdd(a.w.fb_count, 1)] = static_cast<int32_t>(row);
    return;
  }
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  constexpr int E = (decode_candidate_cap(K) + NT - 1) / NT;   // every candidate in registers (n <= cap)
  uint64_t x[E];
  uint32_t valid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t j = threadIdx.x + NT * e;
    x[e] = 0ull;
    if (j < n) {
      int lo = 0, hi = S;   // the source s with s_pre[s] <= j < s_pre[s + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= j) lo = mid;
        else hi = mid - 1;
      }
      const uint32_t k = j - s_pre[lo];
      x[e] = lo < S ? a.w.wave_keys[static_cast<size_t>(w0 + lo) * kDecWaveStride + (lo == 0 ? a.w.row_off[row] : 0u) + k]
                    : a.w.cand[static_cast<size_t>(row) * a.cap + k];
      valid |= 1u << e;
    }
  }
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
    stream_pages2(a, row_table(a, row), pa, pb, 1, WavePages{s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]}, lane,
                 [&](int pg, const uint8_t* codes, const uint8_t* scales) {
      const float sc = score_page_asm(qr, codes, scales, lo);
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
void launch_decode_k(const DecArgs& a0, const PathArgs& p, int mode, int cus, int32_t* status, hipStream_t st,
                     StageMark mark) {
  const int64_t items = p.Q * a0.splits;
  // one resident round of scan blocks: the waves split the pages among themselves
  static std::atomic<int> per_cu{0};
  int occ = per_cu.load(std::memory_order_relaxed);
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_gscan_kernel<K>, kDecThreads, 0) != hipSuccess ||
        occ < 1) {
      (void)hipGetLastError();   // a failed query is not the launch's error
      occ = kDecScanBlocksPerCu;
    }
    per_cu.store(occ, std::memory_order_relaxed);
  }
  const int64_t blocks = min(static_cast<int64_t>(occ) * cus, static_cast<int64_t>(kDecScanWaves / kDecWaves));
  const dim3 sgrid(static_cast<unsigned>(blocks));
  DecArgs a = a0;
  a.scan_waves = static_cast<int32_t>(blocks * kDecWaves);
  const dim3 rgrid(static_cast<unsigned>(p.Q));
  const int64_t fb_cap = (items + kDecWaves - 1) / kDecWaves;
  const dim3 fgrid(static_cast<unsigned>(fb_cap < kDecFallbackBlocks ? fb_cap : kDecFallbackBlocks));
  decode_gate_kernel<K><<<dim3(static_cast<unsigned>(p.Q + 1)), dim3(kDecGateWaves * 64), 0, st>>>(a, mode);
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
         align256(sizeof(int32_t)) + align256((q + 1) * sizeof(int64_t)) +
         align256(static_cast<size_t>(kDecScanWaves) * kDecWaveStride * sizeof(uint64_t)) +
         align256(static_cast<size_t>(kDecScanWaves) * sizeof(uint32_t)) + 4 * align256(q * sizeof(uint32_t)) +
         align256(static_cast<size_t>(kDecScanWaves) * 3 * sizeof(int64_t));
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
  w.plan = reinterpret_cast<int64_t*>(take((q + 1) * sizeof(int64_t)));
  w.wave_keys = reinterpret_cast<uint64_t*>(take(static_cast<size_t>(kDecScanWaves) * kDecWaveStride * sizeof(uint64_t)));
  w.wave_first = reinterpret_cast<uint32_t*>(take(static_cast<size_t>(kDecScanWaves) * sizeof(uint32_t)));
  w.row_off = reinterpret_cast<uint32_t*>(take(q * sizeof(uint32_t)));
  w.row_first = reinterpret_cast<uint32_t*>(take(q * sizeof(uint32_t)));
  w.row_w0 = reinterpret_cast<uint32_t*>(take(q * sizeof(uint32_t)));
  w.row_nw = reinterpret_cast<uint32_t*>(take(q * sizeof(uint32_t)));
  w.wave_desc = reinterpret_cast<int64_t*>(take(static_cast<size_t>(kDecScanWaves) * 3 * sizeof(int64_t)));
  return w;
}

hipError_t launch_decode(const PathArgs& p, const DecodeScratch& w, int32_t splits, int mode, bool no_fallback,
                         int cus, hipStream_t st, StageMark mark) {
  if (p.Q == 0) return hipSuccess;
  int32_t* status = status_word();
  if (status == nullptr) return hipErrorInvalidSymbol;
  DecArgs a;
  a.q = p.q;
  a.q_scale = p.q_scale;
  a.weights = p.weights;
  a.k_pages = p.k_pages;
  a.k_scale = p.k_scale;
  a.P_phys = static_cast<int32_t>(p.P_phys);
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
  if (cus < 1) cus = 1;
  if (p.K == 512) launch_decode_k<512>(a, p, mode, cus, status, st, mark);
  else launch_decode_k<1024>(a, p, mode, cus, status, st, mark);
  return hipGetLastError();
}

}  // namespace mqa
