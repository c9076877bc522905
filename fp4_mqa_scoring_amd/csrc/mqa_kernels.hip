// HIP kernels of the FP4 paged-MQA prefill indexer with exact TopK (gfx950).
//
// Fused path (all on the caller's stream, no host synchronisation):
//   row_prep     validate windows and pages, answer short rows (length <= K)
//   calib        per row: score a sample (every 32nd position of the row tile's
//                range), keep the sample's exact top-k' and derive the gate T0 =
//                its k'-th key (split over the context when the row tiles alone
//                leave CUs idle; calib_combine then takes the k'-th key of the
//                splits' lists)
//   scan         per (8-row tile, context split): score every 256-position block
//                with MXFP4 MFMA, ReLU + head-weighted sum in registers; keys >= T0
//                are staged per wave in LDS and appended to the row's bounded
//                global candidate buffer
//   merge        per row: the candidates are exactly the window's keys >= T0; if
//                there are at least K of them their top-K is the row's top-K:
//                exact radix select, ascending order, raw -> physical mapping.
//                Rows with fewer than K (gate too high) or more than the buffer
//                holds go to a device-side list
//   fallback     listed rows only: exact streaming TopK without a gate in bounded
//                LDS pools, then the same exact merge; costs one empty launch pair
//                when the list is empty
// The dense comparator replaces everything after row_prep by dense_score (fp32
// logits [Q, S]) + logits_topk.
//
// Sources: "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR 5309),
// Implementation (a calibrated filter of candidates, exact and stable selection,
// the page map, failing closed); "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK"
// (ROCm/aiter PR 5282), Changes and Scope.
#include <atomic>

#include "mqa_device.h"
#include "mqa_launch.h"
#include "mqa_select.h"

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
// Block 0 also clears the fallback list counter of this call (if any).
// ---------------------------------------------------------------------------
// With seq_of_row (multi-sequence form) row r reads the page table
// page_table + seq_of_row[r] * P_log; a sequence index outside [0, n_seq) is
// invalid metadata (code -1).
__global__ void __launch_bounds__(256) row_prep_kernel(
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ row_end,
    const int32_t* __restrict__ page_table_base, int64_t P_log, int64_t P_phys, int32_t K, int mode,
    int32_t* __restrict__ out_raw, int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count,
    float* __restrict__ out_score, int32_t* __restrict__ row_state, int32_t* __restrict__ fb_count,
    const int32_t* __restrict__ seq_of_row, int64_t n_seq) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  if (row == 0 && tid == 0 && fb_count) *fb_count = 0;
  const int64_t start = row_start[row], end = row_end[row];
  const int64_t seq = seq_of_row ? seq_of_row[row] : 0;
  const int32_t* page_table = page_table_base + (seq_of_row && seq >= 0 && seq < n_seq ? seq * P_log : 0);
  int code = 0;
  if (start < 0 || end < start || end > kPage * P_log || (seq_of_row && (seq < 0 || seq >= n_seq))) {
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


struct ScanArgs {
  const uint8_t* q;
  const uint8_t* q_scale;
  const float* weights;
  const uint8_t* k_pages;
  const uint8_t* k_scale;
  int32_t P_phys;   // page counts fit int32: the host checks 64 P_phys and 64 P_log against INT32_MAX,
  const int32_t* page_table;
  int32_t P_log;    // so the kernels' page tests are 32-bit scalar compares
  const int32_t* row_start;
  const int32_t* row_end;
  const int32_t* row_state;
  int32_t Q;
  int32_t splits;
};

// Candidate buffers of the gated path (scratch of one call).
struct CandArgs {
  uint64_t* gate;        // [Q] keys > gate are candidates
  uint32_t* count;       // [Q] candidates appended (may exceed cap: overflow)
  uint64_t* cand;        // [Q, cap]
  int32_t* fb_list;      // [Q] rows sent to the exact fallback
  int32_t* fb_count;     // [1]
  int32_t* fb_cnt;       // [Q, 4] per (row, fallback split) key counts
  int32_t* work;         // [1] next (split, tile) item of the gated scan; zeroed by the calibration
  int32_t cap;
  int32_t no_fallback;   // fail closed instead of listing rows for the fallback
};

template <int K>
struct Geometry;
template <>
struct Geometry<512> {
  static constexpr int kCap = candidate_cap(512);
  static constexpr int kFbSplits = 4;      // fallback splits per listed row: at most
  static constexpr int kFbSplitsMin = 4;   // ... and when the list is long
};
template <>
struct Geometry<1024> {
  static constexpr int kCap = candidate_cap(1024);
  static constexpr int kFbSplits = 4;
  static constexpr int kFbSplitsMin = 2;
};
// Fallback pool per row: all LDS left after the block buffers and histograms.
constexpr int kPoolCap = 1856;
constexpr int kFallbackGrid = 256;

// The calibration samples every 64th position: a quarter of a 1/16 sample's
// scoring work. The looser gate (about 64 k' keys pass it) needs the larger
// candidate buffer (candidate_cap). Measured at Q = 8192, C4 = 196,608, K = 1024
// (same session, outputs identical): 1/32 sample with a 4,096-key buffer,
// calibration 0.33 ms, call 8.24 ms; 1/64 with 5,120 keys, 0.185 ms, scan +0.06
// and merge +0.02 ms, call 8.17 ms; 1/64 with 4,096 keys overflowed rows into the
// exact fallback (call 9.28 ms).
constexpr int kCalStride = 64;
constexpr int kCalPerPage = kPage / kCalStride;   // sampled positions per page
static_assert(kCalStride >= 16 && kCalStride <= kPage && kPage % kCalStride == 0, "stride divides the page");
constexpr int kCalCap = 512;         // calibration pool per row
// Context splits of the calibration (rows with few row tiles): each split keeps
// the exact top-k' of its sample blocks in a list of at most kCalListCap keys in
// the row's candidate buffer (unused until the scan), followed by one header
// word per split; a combine kernel takes the k'-th key of the lists' union.
constexpr int kCalMaxSplits = 8;
constexpr int kCalMinSplitBlocks = 4;   // fewer sample blocks per split: the combine launch costs more than it saves
constexpr int kCalListCap = 128;
constexpr int kCalHeaders = kCalMaxSplits * kCalListCap;   // header words start here
static_assert(kCalHeaders + kCalMaxSplits <= candidate_cap(512), "split lists fit the smallest candidate buffer");

// Score blocks [a, a+n) visited by a CTA.
struct BlockSeq {
  int a, n;
  __device__ __forceinline__ int tile(int i) const { return a + i; }
};

// CTA-uniform block range [u0, u1) covering the union of the CTA's active row
// windows; false when no row of the CTA is active.
__device__ __forceinline__ bool row_tile_range(int32_t* s_lo, int32_t* s_hi, bool active, int start, int end,
                                               int wave, int lane, int* u0, int* u1) {
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
  __syncthreads();   // s_lo / s_hi may be reused right after
  if (lo >= hi) return false;
  *u0 = lo / kTile;
  *u1 = (hi + kTile - 1) / kTile;
  return true;
}

__device__ __forceinline__ BlockSeq split_range(int u0, int u1, int split, int splits) {
  const int64_t nt = u1 - u0;
  const int a = u0 + static_cast<int>(nt * split / splits);
  const int b = u0 + static_cast<int>(nt * (split + 1) / splits);
  return BlockSeq{a, b - a};
}

// ---------------------------------------------------------------------------
// Score-block streaming by direct global -> LDS loads (gfx950 LDS DMA), used by
// every kernel that scores whole blocks. Wave w copies positions 32w .. 32w+31
// of a block, which all lie in page w/2 of it: two 16-byte-per-lane loads for
// the codes and one 4-byte-per-lane load (lanes 0-31) for the scales. A lane's
// LDS destination is fixed by its lane id, so the chunk swizzle is applied on
// the source side: the lane that fills chunk slot s of position p reads chunk
// s ^ chunk_swizzle(p). Blocks are double-buffered (the copy of block i+1 runs
// while block i is scored); page-table entries are read one block ahead.
// Pages whose entry is out of range are not copied: row_prep rejected every row
// whose window touches them, so no active row uses those positions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void vm_wait_all() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

struct BlockDma {
  int src0, src1, src_sc;   // per-lane byte offsets inside a page
  int wave;                 // wave-uniform
  int run;                  // first block position of the wave's 32

  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
    const int pin = 32 * (w & 1), pq = lane >> 2, slot = lane & 3;
    const int pb = 64 * (w >> 1) + pin + pq;   // block position of run 0 of this lane
    src0 = (pin + pq) * kVecBytes + 16 * (slot ^ chunk_swizzle(pb));
    src1 = (pin + 16 + pq) * kVecBytes + 16 * (slot ^ chunk_swizzle(pb + 16));
    src_sc = (pin + (lane & 31)) * kVecScales;
    run = 32 * w;
  }

  // Lane l holds the page-table entry of page l % 4 of block t (-1 beyond the table).
  // (Logical page indices fit in int32: the host checks 64 * P_log <= INT32_MAX.)
  // Addresses are a uniform base plus a 32-bit unsigned lane offset, so the loads
  // take a scalar base and no 64-bit address arithmetic per lane.
  using Ent = int32_t;
  __device__ __forceinline__ Ent entries(const ScanArgs& a, int t, int lane) const {
    const int lp = t * kTilePages + (lane & 3);
    const uint32_t off = static_cast<uint32_t>(lp) * 4u;
    return lp < a.P_log ? *reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(a.page_table) + off) : -1;
  }

  __device__ __forceinline__ void issue(const ScanArgs& a, const Ent& ent, uint8_t* codes, uint8_t* scales,
                                        int lane) const {
    const int32_t e = __builtin_amdgcn_readlane(ent, wave >> 1);
    if (e < 0 || e >= a.P_phys) return;
    const uint8_t* page = a.k_pages + static_cast<size_t>(e) * (kPage * kVecBytes);
    __builtin_amdgcn_global_load_lds(page + static_cast<uint32_t>(src0), codes + run * kVecBytes, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(page + static_cast<uint32_t>(src1), codes + (run + 16) * kVecBytes, 16, 0, 0);
    if (lane < 32)
      __builtin_amdgcn_global_load_lds(a.k_scale + static_cast<size_t>(e) * (kPage * kVecScales) +
                                           static_cast<uint32_t>(src_sc),
                                       scales + run * kVecScales, 4, 0, 0);
  }
};

// "Sample blocks" of the calibration. The calibration samples every
// kCalStride-th position of the row tile's range: J = (u1 - u0) * kTile /
// kCalStride samples, sample j at position base + kCalStride * j (base = first
// position of the range, a multiple of 256). Sample block v (0 <= v < nb =
// ceil(J / 256)) holds samples j = v + nb * p, p = 0..255: each block is spread
// over the whole range, so the samples a row has seen after a few blocks are an
// even subset of its whole sample, which the calibration's early compaction
// relies on (and which keeps rows whose order is decided by index away from the
// fallback). Same LDS image as a score block (sample p at slot p, same chunk
// swizzle), so the block scorer applies unchanged. Every lane copies from its
// own page.
struct SampleDma {
  int base_pg;   // first logical page of the sampled range
  int nb;        // sample blocks of the range
  int run;       // first block slot of the wave's 32

  __device__ __forceinline__ void init(int u0, int blocks, int w) {
    base_pg = u0 * kTilePages;
    nb = blocks;
    run = 32 * w;
  }

  // Per-lane source layout of block v, recomputed at every use from a lane index
  // the compiler cannot hoist (an opaque copy): loop-invariant 64-bit per-lane
  // addresses kept for the whole calibration do not fit the 128-VGPR budget of
  // four waves per SIMD.
  struct Lane {
    int j0, j1, js;           // sample indices of the lane's two code chunks and its scale
    int off0, off1, off_sc;   // byte offsets inside their source pages
  };
  __device__ __forceinline__ Lane lane_layout(int v) const {
    int lane;
    __asm__ __volatile__("v_and_b32 %0, 63, %1" : "=v"(lane) : "v"(static_cast<int>(threadIdx.x)));
    const int pq = lane >> 2, slot = lane & 3;
    const int p0 = run + pq, p1 = p0 + 16, ps = run + (lane & 31);
    const int j0 = v + nb * p0, j1 = v + nb * p1, js = v + nb * ps;
    return Lane{j0, j1, js,
                kCalStride * (j0 % kCalPerPage) * kVecBytes + 16 * (slot ^ chunk_swizzle(p0)),
                kCalStride * (j1 % kCalPerPage) * kVecBytes + 16 * (slot ^ chunk_swizzle(p1)),
                kCalStride * (js % kCalPerPage) * kVecScales};
  }

  struct Ent {
    int32_t e0, e1, es;
    int v;   // the block (wave-uniform)
  };
  // Uniform base + 32-bit unsigned byte offset (lp < 2^25), so the load uses a
  // scalar base and one offset VGPR per entry. Entries beyond the table (samples
  // past the range's end) are -1: nothing is copied for them.
  __device__ __forceinline__ static int32_t entry(const ScanArgs& a, int lp) {
    const uint32_t off = static_cast<uint32_t>(lp) * 4u;
    return lp < a.P_log ? *reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(a.page_table) + off) : -1;
  }
  __device__ __forceinline__ Ent entries(const ScanArgs& a, int v, int) const {
    const Lane l = lane_layout(v);
    return Ent{entry(a, base_pg + l.j0 / kCalPerPage), entry(a, base_pg + l.j1 / kCalPerPage),
               entry(a, base_pg + l.js / kCalPerPage), v};
  }

  __device__ __forceinline__ void issue(const ScanArgs& a, const Ent& e, uint8_t* codes, uint8_t* scales,
                                        int lane) const {
    const Lane l = lane_layout(e.v);
    if (e.e0 >= 0 && e.e0 < a.P_phys)
      __builtin_amdgcn_global_load_lds(a.k_pages + static_cast<size_t>(e.e0) * (kPage * kVecBytes) + l.off0,
                                       codes + run * kVecBytes, 16, 0, 0);
    if (e.e1 >= 0 && e.e1 < a.P_phys)
      __builtin_amdgcn_global_load_lds(a.k_pages + static_cast<size_t>(e.e1) * (kPage * kVecBytes) + l.off1,
                                       codes + (run + 16) * kVecBytes, 16, 0, 0);
    if (lane < 32 && e.es >= 0 && e.es < a.P_phys)
      __builtin_amdgcn_global_load_lds(a.k_scale + static_cast<size_t>(e.es) * (kPage * kVecScales) + l.off_sc,
                                       scales + run * kVecScales, 4, 0, 0);
  }
};

// Samples j in [lo, hi) with va <= j mod nb < vb: the samples of blocks [va, vb)
// inside a row's sample range.
__device__ __forceinline__ int samples_in_blocks(int lo, int hi, int nb, int va, int vb) {
  auto f = [&](int x) { return (x / nb) * (vb - va) + min(max(x % nb - va, 0), vb - va); };
  return hi > lo ? f(hi) - f(lo) : 0;
}

// Keys the calibration pool keeps when it fills before the end of the row's
// sample: having seen `seen` of its m samples (an even subset, see SampleDma),
// the number of the sample's final top-k' among them is about Binomial(seen,
// k'/m) with mean mu; keeping the top mu + 6 sqrt(mu) + 6 (at most k') of what
// was seen loses none of the final top-k' except with probability below 1e-8,
// and the gate raised to the kept ones' smallest key lets few later keys in, so
// the pool rarely fills again. (Should it lose one, the row's final gate is a
// smaller key: a superset of candidates, still exact.)
__device__ __forceinline__ int provisional_keep(int kp, int seen, int m) {
  const float mu = static_cast<float>(kp) * static_cast<float>(seen) / static_cast<float>(max(m, 1));
  return min(kp, static_cast<int>(ceilf(mu + 6.0f * sqrtf(mu) + 6.0f)));
}

// One step of the stream: start the copy of block i+1 into the other buffer,
// score block i, then wait for the copy and for every wave.
template <class Dma, class Body>
__device__ __forceinline__ void stream_step(const ScanArgs& a, const BlockSeq& seq, const Dma& d,
                                            typename Dma::Ent& ent, int i, int lane, const uint8_t* codes,
                                            const uint8_t* scales, uint8_t* next_codes, uint8_t* next_scales,
                                            Body& body) {
  if (i + 1 < seq.n) {
    d.issue(a, ent, next_codes, next_scales, lane);
    if (i + 2 < seq.n) ent = d.entries(a, seq.tile(i + 2), lane);
  }
  body(seq.tile(i), codes, scales);
  vm_wait_all();
  __syncthreads();
}

// Streams the blocks of seq through LDS and calls body(block, codes, scales)
// for every block, in every wave (uniformly). The two buffers are separate LDS
// variables and the loop is unrolled by two, so that every access names its
// buffer statically: the compiler then knows that scoring one buffer does not
// read what the copy into the other writes, and does not wait for that copy
// before the scoring's LDS reads.
template <class Dma, class Body>
__device__ __forceinline__ void stream_dma(const ScanArgs& a, const Dma& d, const BlockSeq& seq, uint8_t* codes0,
                                           uint8_t* scales0, uint8_t* codes1, uint8_t* scales1, Body&& body) {
  if (seq.n <= 0) return;
  const int lane = threadIdx.x & 63;
  typename Dma::Ent ent = d.entries(a, seq.tile(0), lane);
  vm_wait_all();
  d.issue(a, ent, codes0, scales0, lane);
  if (seq.n > 1) ent = d.entries(a, seq.tile(1), lane);
  vm_wait_all();
  __syncthreads();
  for (int i = 0; i < seq.n; i += 2) {
    stream_step(a, seq, d, ent, i, lane, codes0, scales0, codes1, scales1, body);
    if (i + 1 < seq.n) stream_step(a, seq, d, ent, i + 1, lane, codes1, scales1, codes0, scales0, body);
  }
}

// One step of the paired stream: start the copies of blocks i+2 and i+3 into
// the other pair of buffers, score blocks i and i+1, then wait for the copies
// and for every wave (one barrier per two blocks).
template <class Dma, class Body>
__device__ __forceinline__ void stream_pair_step(const ScanArgs& a, const BlockSeq& seq, const Dma& d,
                                                 typename Dma::Ent& ent0, typename Dma::Ent& ent1, int i, int lane,
                                                 const uint8_t* c0, const uint8_t* s0, const uint8_t* c1,
                                                 const uint8_t* s1, uint8_t* nc0, uint8_t* ns0, uint8_t* nc1,
                                                 uint8_t* ns1, Body& body) {
  if (i + 2 < seq.n) {
    d.issue(a, ent0, nc0, ns0, lane);
    if (i + 4 < seq.n) ent0 = d.entries(a, seq.tile(i + 4), lane);
  }
  if (i + 3 < seq.n) {
    d.issue(a, ent1, nc1, ns1, lane);
    if (i + 5 < seq.n) ent1 = d.entries(a, seq.tile(i + 5), lane);
  }
  body(seq.tile(i), c0, s0);
  if (i + 1 < seq.n) body(seq.tile(i + 1), c1, s1);
  vm_wait_all();
  __syncthreads();
}

// Streams the blocks of seq two at a time through four LDS buffers (pairs A
// and B, every access named statically as in stream_dma): half the barriers
// of the single-block stream.
template <class Body>
__device__ __forceinline__ void stream_block_pairs(const ScanArgs& a, const BlockSeq& seq, uint8_t* ca0, uint8_t* sa0,
                                                   uint8_t* ca1, uint8_t* sa1, uint8_t* cb0, uint8_t* sb0,
                                                   uint8_t* cb1, uint8_t* sb1, Body&& body) {
  if (seq.n <= 0) return;
  BlockDma d;
  d.init(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
  const int lane = threadIdx.x & 63;
  BlockDma::Ent ent0 = d.entries(a, seq.tile(0), lane);
  BlockDma::Ent ent1 = seq.n > 1 ? d.entries(a, seq.tile(1), lane) : ent0;
  vm_wait_all();
  d.issue(a, ent0, ca0, sa0, lane);
  if (seq.n > 1) d.issue(a, ent1, ca1, sa1, lane);
  if (seq.n > 2) ent0 = d.entries(a, seq.tile(2), lane);
  if (seq.n > 3) ent1 = d.entries(a, seq.tile(3), lane);
  vm_wait_all();
  __syncthreads();
  for (int i = 0; i < seq.n; i += 4) {
    stream_pair_step(a, seq, d, ent0, ent1, i, lane, ca0, sa0, ca1, sa1, cb0, sb0, cb1, sb1, body);
    if (i + 2 < seq.n)
      stream_pair_step(a, seq, d, ent0, ent1, i + 2, lane, cb0, sb0, cb1, sb1, ca0, sa0, ca1, sa1, body);
  }
}

template <class Body>
__device__ __forceinline__ void stream_blocks(const ScanArgs& a, const BlockSeq& seq, uint8_t* codes0, uint8_t* scales0,
                                              uint8_t* codes1, uint8_t* scales1, Body&& body) {
  BlockDma d;
  d.init(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
  stream_dma(a, d, seq, codes0, scales0, codes1, scales1, static_cast<Body&&>(body));
}

// LDS of the block stream: two buffers of one score block each.
#define MQA_BLOCK_BUFFERS                                                        \
  __shared__ __attribute__((aligned(16))) uint8_t s_codes0[kTile * kVecBytes];   \
  __shared__ __attribute__((aligned(16))) uint8_t s_codes1[kTile * kVecBytes];   \
  __shared__ __attribute__((aligned(16))) uint8_t s_scales0[kTile * kVecScales]; \
  __shared__ __attribute__((aligned(16))) uint8_t s_scales1[kTile * kVecScales]

// Calls f(p0, blk) for each 64-position block of score block t that intersects
// [start, end).
template <class F>
__device__ __forceinline__ void for_blocks_in_window(int t, int start, int end, F&& f) {
  const int tb = t * kTile;
  if (tb >= end || tb + kTile <= start) return;
#pragma unroll 1
  for (int blk = 0; blk < kTile / 64; ++blk) {
    const int p0 = tb + 64 * blk;
    if (p0 >= end || p0 + 64 <= start) continue;
    f(p0, blk);
  }
}

// Smallest key of pool[0..n) (n >= 1).
__device__ __forceinline__ uint64_t wave_min_key(const uint64_t* pool, int n, int lane) {
  uint64_t m = ~0ull;
  for (int i = lane; i < n; i += 64) m = min(m, pool[i]);
  return wave_all_min64(m);
}


// ---------------------------------------------------------------------------
// Calibration of the candidate gate ("calibrated candidate filtering", PR 5309
// Implementation). Per row: exact top-k' of the keys of a sample of its window
// (every kCalStride-th position); the gate is set just below the sample's k'-th
// key, so that about kCalStride k' of the window's keys pass it. k' = x + 4 sqrt(x) + 8, where
// x = K m / n is the expected number of the row's top-K among the m sampled
// positions, makes "fewer than K keys pass" (underfill) a > 4-sigma event; an
// underfilled row is still exact, it just takes the fallback. Rows whose sample
// is not larger than k' get no gate. mode 1 sends every long row to the exact
// fallback (no prefilter), mode 2 forces an underfill (gate above every key);
// both exist for testing. With gridDim.y > 1 (mode 0 only) split y streams its
// share of the sample blocks and leaves its exact top-k' list and a header word
// in the row's candidate buffer for calib_combine_kernel, which sets the gate.
// ---------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(kCtaThreads, 4) calib_kernel(ScanArgs a, CandArgs c, int mode) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *c.work = 0;   // the scan's item counter
  MQA_BLOCK_BUFFERS;
  __shared__ uint64_t s_pool[kRowsPerCta][kCalCap];
  __shared__ uint32_t s_hist[kRowsPerCta][256];
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerCta + wave;
  const bool active = row < a.Q && a.row_state[row] == kRowLong;
  int start = 0, end = 0;
  if (active) {
    start = a.row_start[row];
    end = a.row_end[row];
  }
  int u0 = 0, u1 = 0;
  if (!row_tile_range(s_lo, s_hi, active, start, end, wave, lane, &u0, &u1)) return;
  const int base = u0 * kTile;
  // sampled positions base + kCalStride j inside this row's window
  const int j_lo = (start - base + kCalStride - 1) / kCalStride;
  const int j_hi = (end - base + kCalStride - 1) / kCalStride;
  const int m = active ? max(0, j_hi - j_lo) : 0;
  const int kp = active ? sample_keep(K, m, end - start) : 0;
  const bool gated = mode == 0 && active && kp < m;

  QRow qr;
  if (gated)
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);
  __builtin_amdgcn_s_waitcnt(0);

  uint64_t* pool = s_pool[wave];
  int fill = 0;
  uint64_t gate = 0;
  bool bad = false;
  if (mode == 0) {
    const int nb = ((u1 - u0) * (kTile / kCalStride) + kTile - 1) / kTile;   // sample blocks
    const BlockSeq seq = split_range(0, nb, static_cast<int>(blockIdx.y), static_cast<int>(gridDim.y));
    // this split's samples inside the row's window (all of them when unsplit)
    const int m_here = gated ? samples_in_blocks(j_lo, j_hi, nb, seq.a, seq.a + seq.n) : 0;
    SampleDma d;
    d.init(u0, nb, wave);
    const LaneOffsets lo = lane_offsets(lane);
    int seen = 0;   // samples of the row's window scored so far (wave-uniform)
    stream_dma(a, d, seq, s_codes0, s_scales0, s_codes1, s_scales1,
               [&](int v, const uint8_t* codes, const uint8_t* scales) {
      if (!gated) return;
      score_block(qr, codes, scales, lo, [&](int blk, float sc) {
        // from a lane index the compiler cannot hoist: a per-lane multiple of nb kept
        // for the whole calibration would push it past 128 VGPRs
        int ln;
        __asm__ __volatile__("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"(static_cast<int>(threadIdx.x)));
        const int pos = base + kCalStride * (v + nb * (64 * blk + ln));
        const bool in_win = pos >= start && pos < end;
        seen += __popcll(__ballot(in_win));
        const uint64_t key = make_key(sc, static_cast<uint32_t>(pos));
        bool pass = in_win && key > gate;
        uint64_t msk = __ballot(pass);
        if (msk == 0) return;
        int cnt = __popcll(msk);
        if (fill + cnt > kCalCap) {
          const int keep = min(provisional_keep(kp, seen, m_here), fill - 1);
          const Selected sel = wave_select_compact(pool, fill, keep, s_hist[wave], lane);
          if (sel.kept != keep) bad = true;
          fill = keep;
          gate = sel.T - 1;
          pass = pass && key > gate;
          msk = __ballot(pass);
          cnt = __popcll(msk);
        }
        if (pass) pool[fill + mbcnt64(msk)] = key;
        fill += cnt;
      });
    });
  }
  if (!active) return;
  wave_lds_sync();
  if (gridDim.y > 1) {
    // split: this split's exact top-min(k', fill) keys and a header word
    // (bit 63 selector failure, bit 62 gated, bits 32..47 k', bits 0..31 keys)
    uint64_t* list = c.cand + static_cast<size_t>(row) * c.cap;
    int n = 0;
    if (gated) {
      if (fill > kp) {
        const Selected sel = wave_select_compact(pool, fill, kp, s_hist[wave], lane);
        if (sel.kept != kp) bad = true;
        fill = kp;
      }
      if (kp > kCalListCap) bad = true;
      n = bad ? 0 : fill;
      uint64_t* dst = list + static_cast<size_t>(blockIdx.y) * kCalListCap;
      for (int i = lane; i < n; i += 64) dst[i] = pool[i];
    }
    if (lane == 0)
      list[kCalHeaders + blockIdx.y] = (bad ? 1ull << 63 : 0ull) | (gated ? 1ull << 62 : 0ull) |
                                       (static_cast<uint64_t>(kp & 0xFFFF) << 32) | static_cast<uint32_t>(n);
    return;
  }
  uint32_t start_count = 0;
  uint64_t row_gate = 0;
  if (mode == 1) {
    start_count = static_cast<uint32_t>(c.cap) + 1;   // overflow marker: exact fallback
    row_gate = ~0ull;
  } else if (mode == 2) {
    row_gate = ~0ull;                                 // nothing passes: underfill
  } else if (gated) {
    uint64_t T = 0;
    if (fill > kp) {
      const Selected sel = wave_select_compact(pool, fill, kp, s_hist[wave], lane);
      if (sel.kept != kp) bad = true;
      T = sel.T;
    } else if (fill == kp) {
      T = wave_min_key(pool, fill, lane);
    } else {
      bad = true;   // an early compaction kept too few keys (probability < 1e-8): exact fallback
    }
    row_gate = T - 1;
    if (bad) {                                        // selector failure: exact fallback
      start_count = static_cast<uint32_t>(c.cap) + 1;
      row_gate = ~0ull;
    }
  }
  if (lane == 0) {
    c.count[row] = start_count;
    c.gate[row] = row_gate;
  }
}

// Combine of a split calibration (mode 0 only): per long row, the k'-th key of
// the union of the splits' top-k' lists is the k'-th key of the whole sample,
// so the gate equals the one an unsplit calibration sets.
constexpr int kCombineRows = 4;
__global__ void __launch_bounds__(64 * kCombineRows) calib_combine_kernel(ScanArgs a, CandArgs c, int splits) {
  __shared__ uint64_t s_pool[kCombineRows][kCalMaxSplits * kCalListCap];
  __shared__ uint32_t s_hist[kCombineRows][256];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = blockIdx.x * kCombineRows + wave;
  if (row >= a.Q || a.row_state[row] != kRowLong) return;
  const uint64_t* list = c.cand + static_cast<size_t>(row) * c.cap;
  uint64_t* pool = s_pool[wave];
  bool bad = false, gated = false;
  int kp = 0, n = 0;
  for (int s = 0; s < splits; ++s) {
    const uint64_t h = list[kCalHeaders + s];
    bad |= (h >> 63) != 0;
    gated = ((h >> 62) & 1ull) != 0;
    kp = static_cast<int>((h >> 32) & 0xFFFF);
    const int ns = static_cast<int>(static_cast<uint32_t>(h));
    for (int i = lane; i < ns; i += 64) pool[n + i] = list[static_cast<size_t>(s) * kCalListCap + i];
    n += ns;
  }
  uint32_t start_count = 0;
  uint64_t row_gate = 0;
  if (gated) {
    wave_lds_sync();
    uint64_t T = 0;
    if (!bad && n > kp) {
      const Selected sel = wave_select_compact(pool, n, kp, s_hist[wave], lane);
      if (sel.kept != kp) bad = true;
      T = sel.T;
    } else if (!bad && n == kp && n > 0) {
      T = wave_min_key(pool, n, lane);
    } else {
      bad = true;
    }
    row_gate = T - 1;
    if (bad) {                                        // selector failure: exact fallback
      start_count = static_cast<uint32_t>(c.cap) + 1;
      row_gate = ~0ull;
    }
  }
  if (lane == 0) {
    c.count[row] = start_count;
    c.gate[row] = row_gate;
  }
}

// Split `split` of [u0, u1) when earlier splits take larger shares: split s of
// S gets (S - s) / (S (S + 1) / 2) of the blocks, so the items the gated scan
// hands out last are the shortest.
__device__ __forceinline__ BlockSeq split_range_tapered(int u0, int u1, int split, int splits) {
  const int64_t nt = u1 - u0, S = splits;
  auto at = [&](int64_t s) { return u0 + static_cast<int>(nt * (s * (2 * S - s + 1)) / (S * (S + 1))); };
  const int a = at(split), b = at(split + 1);
  return BlockSeq{a, b - a};
}

// ---------------------------------------------------------------------------
// Gated scan: every score block of the split; keys above the row's gate are
// staged per wave in LDS and appended to the row's candidate buffer (one global
// atomic per flush). Appends beyond the buffer are dropped but still counted,
// which the merge detects as an overflow.
// Items are (split, tile) pairs in split-major order. With at least four items
// per resident CTA the launch is persistent: a resident grid takes items from
// one counter, and the splits are tapered so the shortest items go last.
// Workgroups are bound to XCDs round-robin and the XCDs run the same work at
// speeds up to ~5% apart, so one CTA per item left the fast XCDs idle for the
// last ~0.4 ms at the headline shape; from a common counter the fast XCDs take
// more items. With fewer items per CTA there is little to rebalance, and one
// CTA per item (equal splits) measured faster.
// ---------------------------------------------------------------------------
template <int K>
// Four waves per SIMD (the second launch bound is a minimum of waves per SIMD):
// two CTAs per CU, at most 128 VGPRs.
__global__ void __launch_bounds__(kCtaThreads, 4) scan_kernel(ScanArgs a, CandArgs c, int tiles, int persistent) {
  // Four block buffers (two pairs) and 128 staged keys per wave: 77,824 B, so
  // two CTAs still fit per CU.
  constexpr int kScanStage = 128;
  MQA_BLOCK_BUFFERS;
  __shared__ __attribute__((aligned(16))) uint8_t s_codes2[kTile * kVecBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes3[kTile * kVecBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales2[kTile * kVecScales];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales3[kTile * kVecScales];
  __shared__ uint64_t s_stage[kRowsPerCta][kScanStage];
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];
  __shared__ int32_t s_item;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int items = tiles * a.splits;
  int next = static_cast<int>(blockIdx.x);   // one item per CTA, unless persistent
  if (persistent && threadIdx.x == 0) next = atomicAdd(c.work, 1);
  for (;;) {
    if (threadIdx.x == 0) s_item = next;
    __syncthreads();
    const int item = s_item;
    __syncthreads();
    if (item >= items) break;
    const int split = item / tiles, tile = item - split * tiles;
    const int row = tile * kRowsPerCta + wave;
    bool active = row < a.Q && a.row_state[row] == kRowLong;
    int start = 0, end = 0;
    if (active) {
      start = a.row_start[row];
      end = a.row_end[row];
    }
    int u0 = 0, u1 = 0;
    if (!row_tile_range(s_lo, s_hi, active, start, end, wave, lane, &u0, &u1)) {
      if (threadIdx.x == 0) next = persistent ? atomicAdd(c.work, 1) : items;
      continue;
    }
    const BlockSeq seq =
        persistent ? split_range_tapered(u0, u1, split, a.splits) : split_range(u0, u1, split, a.splits);
    uint64_t gate = 0;
    if (active) {
      gate = c.gate[row];
      if (c.count[row] > static_cast<uint32_t>(c.cap)) active = false;   // already sent to the fallback
    }
    QRow qr;
    if (active)
      load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
                a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
                a.weights + static_cast<size_t>(row) * kHeads, lane);
    __builtin_amdgcn_s_waitcnt(0);

    const float gate_f = gate_floor(gate);
    uint64_t* stage = s_stage[wave];
    uint64_t* dst = c.cand + static_cast<size_t>(active ? row : 0) * c.cap;
    int sf = 0;   // staged keys (wave-uniform)
    auto flush = [&]() {
      wave_lds_sync();
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&c.count[row], static_cast<uint32_t>(sf));
      base = __shfl(base, 0, 64);
      for (int i = lane; i < sf; i += 64) {
        const uint32_t at = base + static_cast<uint32_t>(i);
        if (at < static_cast<uint32_t>(c.cap)) dst[at] = stage[i];
      }
      wave_lds_sync();
      sf = 0;
    };
    const LaneOffsets lo = lane_offsets(lane);
    stream_block_pairs(a, seq, s_codes0, s_scales0, s_codes1, s_scales1, s_codes2, s_scales2, s_codes3, s_scales3,
                       [&](int t, const uint8_t* codes, const uint8_t* scales) {
      if (!active) return;
      const int tb = t * kTile;
      if (tb >= end || tb + kTile <= start) return;
      const bool inside = tb >= start && tb + kTile <= end;   // no window mask needed
      score_block(qr, codes, scales, lo, [&](int blk, float sc) {
        const int p0 = tb + 64 * blk;
        // wave-uniform window mask; one float compare rejects almost every lane
        const uint64_t win = inside ? ~0ull : window_lanes(p0, start, end);
        uint64_t msk = __ballot(!(sc < gate_f)) & win;
        if (msk == 0) return;
        // A score strictly above the gate's score (as floats) has a key above the
        // gate whatever its position, and is not NaN: when every lane the prefilter
        // passed is such a score, those lanes are the candidates and their keys need
        // no NaN class. Otherwise (a lane at the gate's score, a NaN, a gate in the
        // NaN class) the exact 64-bit key test decides.
        uint32_t hi = order_bits_finite(sc);
        const uint32_t lo32 = ~static_cast<uint32_t>(p0) - static_cast<uint32_t>(lane);   // ~(p0 + lane)
        if ((__ballot(sc > gate_f) & win) != msk) {
          if (__builtin_isnan(sc)) hi = 0u;   // NaN class: as order_bits
          msk &= __ballot(((static_cast<uint64_t>(hi) << 32) | lo32) > gate);
          if (msk == 0) return;
        }
        const uint64_t key = (static_cast<uint64_t>(hi) << 32) | lo32;   // make_key(sc, p0 + lane)
        const int cnt = __popcll(msk);
        if (sf + cnt > kScanStage) flush();
        // the wave-uniform mask as the lanes' predicate (no per-lane bit test)
        if (__builtin_amdgcn_inverse_ballot_w64(msk)) stage[sf + mbcnt64(msk)] = key;
        sf += cnt;
      });
    });
    // the following item is taken as this one ends, so items go to the CTAs that
    // finish first (its latency overlaps the last flush)
    if (threadIdx.x == 0) next = persistent ? atomicAdd(c.work, 1) : items;
    if (active && sf > 0) flush();
  }
}

// ---------------------------------------------------------------------------
// Exact streaming TopK without a gate (the fallback of listed rows). Each wave
// owns one listed row and an LDS pool of CAP unique keys; a key enters only if
// it beats the pool's gate, and when a batch would overflow the pool the wave
// radix-selects the K largest, drops the rest and raises the gate. Per (row,
// fallback split) the top-K keys go to the row's candidate buffer at split * K.
// Persistent: a fixed grid loops over (8-row chunk of the list, split) items.
// A short list takes FBS splits per row (more of the grid on each row: a lone
// fallback row is what adds latency to a call); a long one FBS_MIN, which is
// less merge work for the same scan work.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int fallback_splits(int listed, int fbs, int fbs_min) {
  const int chunks = (listed + kRowsPerCta - 1) / kRowsPerCta;
  return chunks * fbs <= kFallbackGrid ? fbs : fbs_min;
}

template <int K, int CAP, int FBS, int FBS_MIN>
__global__ void __launch_bounds__(kCtaThreads, 1) fallback_scan_kernel(ScanArgs a, CandArgs c) {
  static_assert(CAP >= K + 64, "pool must hold K keys plus one batch");
  MQA_BLOCK_BUFFERS;
  __shared__ uint64_t s_pool[kRowsPerCta][CAP];
  __shared__ uint32_t s_hist[kRowsPerCta][256];
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int listed = *c.fb_count;
  const int chunks = (listed + kRowsPerCta - 1) / kRowsPerCta;
  const int fbs = fallback_splits(listed, FBS, FBS_MIN);
  for (int item = blockIdx.x; item < chunks * fbs; item += gridDim.x) {
    const int chunk = item / fbs, split = item % fbs;
    const int li = chunk * kRowsPerCta + wave;
    const bool active = li < listed;
    const int row = active ? c.fb_list[li] : 0;
    int start = 0, end = 0;
    if (active) {
      start = a.row_start[row];
      end = a.row_end[row];
    }
    int u0 = 0, u1 = 0;
    if (!row_tile_range(s_lo, s_hi, active, start, end, wave, lane, &u0, &u1)) continue;
    const BlockSeq seq = split_range(u0, u1, split, fbs);
    QRow qr;
    if (active)
      load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
                a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
                a.weights + static_cast<size_t>(row) * kHeads, lane);
    __builtin_amdgcn_s_waitcnt(0);
    uint64_t* pool = s_pool[wave];
    uint32_t* hist = s_hist[wave];
    int fill = 0;
    uint64_t gate = 0;
    bool failed = false;
    stream_blocks(a, seq, s_codes0, s_scales0, s_codes1, s_scales1, [&](int t, const uint8_t* codes, const uint8_t* scales) {
      if (!active) return;
      for_blocks_in_window(t, start, end, [&](int p0, int blk) {
        const float sc = score64(qr, codes, scales, blk, lane);
        const int pos = p0 + lane;
        const uint64_t key = make_key(sc, static_cast<uint32_t>(pos));
        bool pass = pos >= start && pos < end && key > gate;
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
    });
    if (active) {
      wave_lds_sync();
      if (fill > K) {
        const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
        if (sel.kept != K) failed = true;
        fill = K;
      }
      uint64_t* dst = c.cand + static_cast<size_t>(row) * c.cap + static_cast<size_t>(split) * K;
      for (int i = lane; i < fill; i += 64) dst[i] = pool[i];
      if (lane == 0) c.fb_cnt[static_cast<size_t>(row) * 4 + split] = failed ? kCodeSelector : fill;
    }
    __syncthreads();   // LDS pools and block buffers are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// Exact merge of the gated candidates + page mapping + emission. One 256-thread
// CTA per long row. The candidates are all of the window's keys above the gate;
// with at least K of them the row's top-K is among them ("exact candidate
// union", PR 5282). Otherwise (or on overflow) the row is listed for the exact
// fallback and its outputs are written there.
// ---------------------------------------------------------------------------
template <int K>
__global__ void __launch_bounds__(256) merge_kernel(const int32_t* __restrict__ row_state, CandArgs c,
                                                    const int32_t* __restrict__ page_table, int64_t P_log,
                                                    int32_t* __restrict__ out_raw, int32_t* __restrict__ out_slot,
                                                    int32_t* __restrict__ out_count, float* __restrict__ out_score) {
  constexpr int NT = 256;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[256];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const uint32_t n = c.count[row];
  if (n > static_cast<uint32_t>(c.cap) || n < static_cast<uint32_t>(K)) {
    if (c.no_fallback) {   // fail closed: underfill (fewer than K above the gate) or overflow
      fail_row<K, NT>(row, n < static_cast<uint32_t>(K) ? kCodeUnderfill : kCodeSelector, out_raw, out_slot,
                      out_count, out_score, &g_status);
      return;
    }
    if (threadIdx.x == 0) c.fb_list[atomicAdd(c.fb_count, 1)] = static_cast<int32_t>(row);
    return;
  }
  const uint64_t* keys = c.cand + static_cast<size_t>(row) * c.cap;
  if (n == static_cast<uint32_t>(K)) {
    for (int i = threadIdx.x; i < K; i += NT) s_sel[i] = keys[i];
    __syncthreads();
  } else {
    // Thread t holds the contiguous chunk [t C, t C + C) of the candidates in
    // registers (C <= E: n <= cap) for the radix passes and the gather.
    constexpr int E = (candidate_cap(K) + NT - 1) / NT;
    const int C = (static_cast<int>(n) + NT - 1) / NT;
    const int i0 = min(static_cast<int>(n), static_cast<int>(threadIdx.x) * C);
    const int m = min(static_cast<int>(n), i0 + C) - i0;   // keys in this thread's chunk
    uint64_t x[E];
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      x[j] = j < m ? keys[i0 + j] : 0ull;
      if (j < m) valid |= 1u << j;
    }
    bool ok = false;
    const uint64_t T = block_radix_select_regs<NT, 8, E>(x, valid, K, s_hist, s_red, &ok);
    if (ok) {
      // Stable gather: a suffix count over the chunks places thread t's kept
      // keys; they stay in buffer order. A row whose candidates came from one
      // wave (one split) is then already in ascending position order and the
      // emit skips its sort.
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) cnt += (((valid >> j) & 1u) && x[j] >= T) ? 1u : 0u;
      const uint32_t incl = block_suffix_sum<NT>(cnt, s_red);   // kept keys in chunks t .. NT-1
      int at = K - static_cast<int>(incl);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if (((valid >> j) & 1u) && x[j] >= T) {
          if (at >= 0 && at < K) s_sel[at] = x[j];
          ++at;
        }
      }
      if (threadIdx.x == 0) s_n = static_cast<int>(incl);   // all kept keys
    } else if (threadIdx.x == 0) {
      s_n = 0;
    }
    __syncthreads();
    if (!ok || s_n != K) {
      fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, &g_status);
      return;
    }
  }
  emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
}

// Exact merge of the fallback's per-split top-K keys of each listed row.
// Persistent over the list. A listed row always has >= K candidates (it is
// longer than K); fewer means a selector failure and fails the row closed.
template <int K, int FBS, int FBS_MIN>
__global__ void __launch_bounds__(256) fallback_merge_kernel(CandArgs c, const int32_t* __restrict__ page_table,
                                                             int64_t P_log, int32_t* __restrict__ out_raw,
                                                             int32_t* __restrict__ out_slot,
                                                             int32_t* __restrict__ out_count,
                                                             float* __restrict__ out_score) {
  constexpr int NT = 256;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[256];
  __shared__ int32_t s_cnt[FBS];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n, s_total;
  const int listed = *c.fb_count;
  const int fbs = fallback_splits(listed, FBS, FBS_MIN);   // as the scan chose
  for (int li = blockIdx.x; li < listed; li += gridDim.x) {
    const int64_t row = c.fb_list[li];
    const uint64_t* keys = c.cand + static_cast<size_t>(row) * c.cap;
    if (threadIdx.x == 0) {
      int total = 0;
      bool bad = false;
      for (int i = 0; i < fbs; ++i) {
        s_cnt[i] = c.fb_cnt[static_cast<size_t>(row) * 4 + i];
        bad |= s_cnt[i] < 0 || s_cnt[i] > K;
        total += s_cnt[i];
      }
      s_total = bad ? -1 : total;
      s_n = 0;
    }
    __syncthreads();
    if (s_total < K) {   // a split's selector failed (-1), or fewer than K keys survived: fail closed
      fail_row<K, NT>(row, s_total < 0 ? kCodeSelector : kCodeUnderfill, out_raw, out_slot, out_count, out_score,
                      &g_status);
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
    if (s_total > K) T = block_radix_select<NT, 8>(src, static_cast<int64_t>(fbs) * K, K, s_hist, s_red, &ok);
    if (ok) {
      for (int e = threadIdx.x; e < fbs * K; e += NT) {
        uint64_t x;
        if (src(e, x) && x >= T) {
          const int at = atomicAdd(&s_n, 1);
          if (at < K) s_sel[at] = x;
        }
      }
    }
    __syncthreads();
    if (!ok || s_n != K) {
      fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, &g_status);
    } else {
      emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Dense scorer (comparator): same streaming and the same score64() as the
// fused path, but every score inside an active row's window goes to
// logits[row, s].
// ---------------------------------------------------------------------------
// Scores of the positions in [lo, hi) of every active row's window go to
// logits[row * ld + (pos - lo)]: the dense comparator uses [0, S) with ld = S,
// the context-tiled path one tile [lo, lo + ld) at a time.
__global__ void __launch_bounds__(kCtaThreads, 4) dense_score_kernel(ScanArgs a, float* __restrict__ logits,
                                                                     int64_t ld, int32_t lo, int32_t hi) {
  MQA_BLOCK_BUFFERS;
  __shared__ int32_t s_lo[kRowsPerCta], s_hi[kRowsPerCta];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerCta + wave;
  bool active = row < a.Q && a.row_state[row] == kRowLong;
  int start = 0, end = 0;
  if (active) {
    start = max(a.row_start[row], lo);
    end = min(a.row_end[row], hi);
    active = start < end;
  }
  int u0 = 0, u1 = 0;
  if (!row_tile_range(s_lo, s_hi, active, start, end, wave, lane, &u0, &u1)) return;
  QRow qr;
  if (active)
    load_qrow(qr, a.q + static_cast<size_t>(row) * kHeads * kVecBytes,
              a.q_scale + static_cast<size_t>(row) * kHeads * kVecScales,
              a.weights + static_cast<size_t>(row) * kHeads, lane);
  __builtin_amdgcn_s_waitcnt(0);
  float* out = logits + static_cast<size_t>(active ? row : 0) * ld;   // column pos - lo
  stream_blocks(a, split_range(u0, u1, blockIdx.y, a.splits), s_codes0, s_scales0, s_codes1, s_scales1,
                [&](int t, const uint8_t* codes, const uint8_t* scales) {
                  if (!active) return;
                  for_blocks_in_window(t, start, end, [&](int p0, int blk) {
                    const float sc = score64(qr, codes, scales, blk, lane);
                    const int pos = p0 + lane;
                    if (pos >= start && pos < end) __builtin_nontemporal_store(sc, out + (pos - lo));
                  });
                });
}

// ---------------------------------------------------------------------------
// Dense selector: exact TopK over fp32 logits of one long row's window.
// One 1024-thread CTA per row, 11-bit digits. A gate first: the k'-th largest
// key of a sample of the window (up to 128 chunks of 64 consecutive logits, so
// that whole cache lines are read; k' as in the fused path's calibration), then
// one pass over the window keeps the keys above the gate in LDS, and the exact
// select runs there. The row's top-K is among those candidates whenever there
// are at least K of them (every other key is at or below the gate); a row with
// fewer, or more than the LDS buffer holds, or a window too short to sample,
// takes the exact select over all its logits (one read per radix digit).
// ---------------------------------------------------------------------------
constexpr int kSelChunks = 128;      // sample chunks per row
constexpr int kSelChunk = 64;        // consecutive logits per chunk
constexpr int kSelMinChunks = 4;
constexpr int kSelPassUnroll = 4;    // logits per thread per step of the candidate pass

// Two rows per CU (eight waves per SIMD: at most 64 VGPRs, a few values spill):
// the selector's phases are chains of barriers and memory round trips, so two
// rows in flight nearly halve its time (4.3 -> 2.5 ms at Q=8192, C4=196,608).
template <int K>
__global__ void __launch_bounds__(1024, 8) logits_topk_kernel(
    const float* __restrict__ logits, int64_t S, int64_t P_log, const int32_t* __restrict__ row_state,
    const int32_t* __restrict__ row_start, const int32_t* __restrict__ row_end,
    const int32_t* __restrict__ page_table, int32_t* __restrict__ out_raw,
    int32_t* __restrict__ out_slot, int32_t* __restrict__ out_count, float* __restrict__ out_score) {
  constexpr int NT = 1024;
  constexpr int E = kSelChunks * kSelChunk / NT;   // sample keys per thread
  constexpr int CAP = selector_candidate_cap(K);
  __shared__ uint64_t s_cand[CAP];
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[2048];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  __shared__ uint32_t s_nc;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const int64_t start = row_start[row], n = row_end[row] - start;
  const float* lg = logits + static_cast<size_t>(row) * S + start;
  const int t = threadIdx.x, lane = t & 63;
  auto key_at = [&](int64_t i) -> uint64_t { return make_key(lg[i], static_cast<uint32_t>(start + i)); };
  if (t == 0) s_n = 0;
  bool ok = false;
  bool done = false;
  // chunk c of the sample starts at floor(c n / nch) rounded down to 64, which
  // keeps it inside the window (n >= 2048 nch)
  const int nch = static_cast<int>(min<int64_t>(kSelChunks, n / 2048));
  if (nch >= kSelMinChunks) {
    uint64_t x[E];
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = t + j * NT, c = e / kSelChunk;
      x[j] = 0ull;
      if (c < nch) {
        const int64_t i = ((static_cast<int64_t>(c) * n / nch) & ~static_cast<int64_t>(kSelChunk - 1)) + e % kSelChunk;
        x[j] = key_at(i);
        valid |= 1u << j;
      }
    }
    const int m = nch * kSelChunk;
    const int kp = sample_keep(K, m, static_cast<int>(min<int64_t>(n, 0x7FFFFFFF)));
    if (m > kp) {
      bool sok = false;
      const uint64_t Tg = block_radix_select_regs<NT, 11, E>(x, valid, kp, s_hist, s_red, &sok);
      if (sok) {
        const uint64_t gate = Tg - 1;
        if (t == 0) s_nc = 0u;
        __syncthreads();
        // software-pipelined: the next step's logits are loaded before this
        // step's keys are tested (2.5 -> 1.6 ms for the selector)
        constexpr int64_t kStep = static_cast<int64_t>(NT) * kSelPassUnroll;
        float nxt[kSelPassUnroll];
#pragma unroll
        for (int u = 0; u < kSelPassUnroll; ++u) {
          const int64_t i = static_cast<int64_t>(u) * NT + t;
          nxt[u] = i < n ? lg[i] : 0.0f;
        }
        for (int64_t i0 = 0; i0 < n; i0 += kStep) {
          uint64_t k[kSelPassUnroll];
#pragma unroll
          for (int u = 0; u < kSelPassUnroll; ++u) {
            const int64_t i = i0 + static_cast<int64_t>(u) * NT + t;
            k[u] = i < n ? make_key(nxt[u], static_cast<uint32_t>(start + i)) : 0ull;
          }
#pragma unroll
          for (int u = 0; u < kSelPassUnroll; ++u) {
            const int64_t i = i0 + kStep + static_cast<int64_t>(u) * NT + t;
            nxt[u] = i < n ? lg[i] : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < kSelPassUnroll; ++u) {
            const bool pass = k[u] > gate;
            const uint64_t msk = __ballot(pass);
            if (msk == 0) continue;
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_nc, static_cast<uint32_t>(__popcll(msk)));
            base = __shfl(base, 0, 64);
            const uint32_t at = base + static_cast<uint32_t>(mbcnt64(msk));
            if (pass && at < static_cast<uint32_t>(CAP)) s_cand[at] = k[u];
          }
        }
        __syncthreads();
        const uint32_t nc = s_nc;
        if (nc >= static_cast<uint32_t>(K) && nc <= static_cast<uint32_t>(CAP)) {
          auto lsrc = [&](int64_t i, uint64_t& y) -> bool {
            y = s_cand[i];
            return true;
          };
          const uint64_t T = block_radix_select<NT, 11>(lsrc, static_cast<int64_t>(nc), K, s_hist, s_red, &ok);
          if (ok) {
            for (int i = t; i < static_cast<int>(nc); i += NT) {
              const uint64_t y = s_cand[i];
              if (y >= T) {
                const int at = atomicAdd(&s_n, 1);
                if (at < K) s_sel[at] = y;
              }
            }
          }
          done = true;
        }
      }
    }
  }
  if (!done) {   // the exact select over every logit of the window
    auto src = [&](int64_t i, uint64_t& y) -> bool {
      y = key_at(i);
      return true;
    };
    const uint64_t T = block_radix_select<NT, 11>(src, n, K, s_hist, s_red, &ok);
    if (ok) {
      for (int64_t i = t; i < n; i += NT) {
        const uint64_t y = key_at(i);
        if (y >= T) {
          const int at = atomicAdd(&s_n, 1);
          if (at < K) s_sel[at] = y;
        }
      }
    }
  }
  __syncthreads();
  if (!ok || s_n != K) {
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, &g_status);
    return;
  }
  emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
}

// ---------------------------------------------------------------------------
// Bounded context-tiled exact TopK ("[FlyDSL][DSv4] Prototype FP4 MQA streaming
// TopK", Changes: besides the fused operator the pages keep an exact path whose
// memory is bounded by tiling the context, for correctness checks and as a
// reference). The context is visited in tiles of `tile` positions; the
// dense scorer writes one tile's fp32 scores of every row into a [Q, tile]
// buffer, then each row merges the tile into its pool. A row's pool holds at
// most tile_pool_cap(K) keys and a floor: no key at or below the floor can be
// among the row's top K (K pool keys are above it). The tile's keys above the
// floor are appended to the pool; when the pool would overflow, pool and tile
// keys are compacted to their top K by an exact radix select and the floor
// rises to the K-th key. Every position of a window is seen in exactly one
// tile, so after the last tile the pool's top K is the window's. The K-th key
// of the first t tiles leaves about K / t keys of the next tile above it, so a
// row compacts about K ln(tiles) / K times and most tiles cost one read of
// their logits. No gate, no calibration; scratch
// Q (4 tile + 8 tile_pool_cap(K) + 16) bytes, independent of the context length.
// ---------------------------------------------------------------------------
constexpr int kTileNewCap = 1024;   // tile keys above the floor gathered in LDS

__global__ void __launch_bounds__(256) tile_reset_kernel(int32_t* __restrict__ run_count,
                                                         uint64_t* __restrict__ run_floor, int64_t Q) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < Q) {
    run_count[i] = 0;
    run_floor[i] = 0ull;   // every key is above 0 (its low word is ~position)
  }
}

template <int K>
__global__ void __launch_bounds__(256) tile_merge_kernel(const int32_t* __restrict__ row_state,
                                                         const int32_t* __restrict__ row_start,
                                                         const int32_t* __restrict__ row_end,
                                                         const float* __restrict__ tile_logits, int32_t tile,
                                                         int32_t lo, int32_t hi, uint64_t* __restrict__ pool,
                                                         int32_t* __restrict__ run_count,
                                                         uint64_t* __restrict__ run_floor) {
  constexpr int NT = 256;
  constexpr int CAP = tile_pool_cap(K);
  __shared__ uint64_t s_pool[CAP];
  __shared__ uint64_t s_new[kTileNewCap];
  __shared__ uint32_t s_hist[256];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n, s_m;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const int32_t a = max(row_start[row], lo), b = min(row_end[row], hi);
  if (a >= b) return;
  const int c = run_count[row];
  if (c < 0) return;   // an earlier compaction failed: the emit fails the row closed
  const uint64_t floor_key = run_floor[row];
  const int n_tile = b - a;
  uint64_t* run = pool + static_cast<size_t>(row) * CAP;
  const float* lg = tile_logits + static_cast<size_t>(row) * tile + (a - lo);   // position a at lg[0]
  auto key_at = [&](int i) -> uint64_t { return make_key(lg[i], static_cast<uint32_t>(a + i)); };
  if (threadIdx.x == 0) {
    s_m = 0;
    s_n = 0;
  }
  __syncthreads();
  // eight logits per thread in flight before any is tested (the atomic append
  // would otherwise serialise the loads into one round trip per step)
  constexpr int U = 8;
  for (int i0 = 0; i0 < n_tile; i0 += NT * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + static_cast<int>(threadIdx.x);
      v[u] = i < n_tile ? lg[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + static_cast<int>(threadIdx.x);
      if (i >= n_tile) continue;
      const uint64_t x = make_key(v[u], static_cast<uint32_t>(a + i));
      if (x > floor_key) {
        const int at = atomicAdd(&s_m, 1);
        if (at < kTileNewCap) s_new[at] = x;
      }
    }
  }
  __syncthreads();
  const int m = s_m;   // tile keys above the floor (all counted, at most kTileNewCap kept)
  if (m == 0) return;
  const bool in_lds = m <= kTileNewCap;
  if (c + m <= CAP) {   // room in the pool: append
    if (in_lds) {
      for (int i = threadIdx.x; i < m; i += NT) run[c + i] = s_new[i];
    } else {
      for (int i = threadIdx.x; i < n_tile; i += NT) {
        const uint64_t x = key_at(i);
        if (x > floor_key) run[c + atomicAdd(&s_n, 1)] = x;
      }
    }
    if (threadIdx.x == 0) run_count[row] = c + m;
    return;
  }
  // compact: top K of the pool and the tile's keys above the floor
  for (int i = threadIdx.x; i < c; i += NT) s_pool[i] = run[i];
  __syncthreads();
  auto src = [&](int64_t i, uint64_t& x) -> bool {
    if (i < c) {
      x = s_pool[i];
      return true;
    }
    if (in_lds) {
      x = s_new[i - c];
      return true;
    }
    x = key_at(static_cast<int>(i - c));
    return x > floor_key;
  };
  const int64_t n = static_cast<int64_t>(c) + (in_lds ? m : n_tile);
  bool ok = false;
  const uint64_t T = block_radix_select<NT, 8>(src, n, K, s_hist, s_red, &ok);
  if (ok) {
    for (int64_t i = threadIdx.x; i < n; i += NT) {
      uint64_t x;
      if (src(i, x) && x >= T) {
        const int at = atomicAdd(&s_n, 1);
        if (at < K) run[at] = x;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool good = ok && s_n == K;
    run_count[row] = good ? K : -1;   // -1: the emit fails the row closed
    run_floor[row] = good ? T : ~0ull;
  }
}

// Per long row: the top K of its pool (exact select when it holds more), then
// the ascending position order and the page map.
template <int K>
__global__ void __launch_bounds__(256) tile_emit_kernel(const int32_t* __restrict__ row_state,
                                                        const uint64_t* __restrict__ pool,
                                                        const int32_t* __restrict__ run_count,
                                                        const int32_t* __restrict__ page_table, int64_t P_log,
                                                        int32_t* __restrict__ out_raw, int32_t* __restrict__ out_slot,
                                                        int32_t* __restrict__ out_count, float* __restrict__ out_score) {
  constexpr int NT = 256;
  constexpr int CAP = tile_pool_cap(K);
  __shared__ uint64_t s_pool[CAP];
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[256];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n;
  const int64_t row = blockIdx.x;
  if (row_state[row] != kRowLong) return;
  const int c = run_count[row];
  if (c < K || c > CAP) {   // -1: a compaction failed; fewer than K keys: underfill; both fail closed
    fail_row<K, NT>(row, c >= 0 && c < K ? kCodeUnderfill : kCodeSelector, out_raw, out_slot, out_count, out_score,
                    &g_status);
    return;
  }
  const uint64_t* run = pool + static_cast<size_t>(row) * CAP;
  for (int i = threadIdx.x; i < c; i += NT) s_pool[i] = run[i];
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  bool ok = true;
  uint64_t T = 0;
  if (c > K) {
    auto src = [&](int64_t i, uint64_t& x) -> bool {
      x = s_pool[i];
      return true;
    };
    T = block_radix_select<NT, 8>(src, c, K, s_hist, s_red, &ok);
  }
  if (ok) {
    for (int i = threadIdx.x; i < c; i += NT) {
      const uint64_t x = s_pool[i];
      if (x >= T) {
        const int at = atomicAdd(&s_n, 1);
        if (at < K) s_sel[at] = x;
      }
    }
  }
  __syncthreads();
  if (!ok || s_n != K) {
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, &g_status);
    return;
  }
  emit_row<K, NT>(s_sel, row, page_table, P_log, out_raw, out_slot, out_count, out_score);
}

static_assert(Geometry<512>::kFbSplits * 512 <= Geometry<512>::kCap, "fallback keys fit the candidate buffer");
static_assert(Geometry<1024>::kFbSplits * 1024 <= Geometry<1024>::kCap, "fallback keys fit the candidate buffer");
static_assert(Geometry<512>::kFbSplits <= 4 && Geometry<1024>::kFbSplits <= 4, "fb_cnt holds 4 counts per row");

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
  a.P_phys = static_cast<int32_t>(p.P_phys);
  a.page_table = p.page_table;
  a.P_log = static_cast<int32_t>(p.P_log);
  a.row_start = p.row_start;
  a.row_end = p.row_end;
  a.row_state = row_state;
  a.Q = static_cast<int32_t>(p.Q);
  a.splits = splits;
  return a;
}

static CandArgs cand_args(const GatedScratch& g, int K, bool no_fallback) {
  CandArgs c;
  c.gate = g.gate;
  c.count = g.count;
  c.cand = g.cand;
  c.fb_list = g.fb_list;
  c.fb_count = g.fb_count;
  c.fb_cnt = g.fb_cnt;
  c.work = g.work;
  c.cap = candidate_cap(K);
  c.no_fallback = no_fallback ? 1 : 0;
  return c;
}

hipError_t launch_row_prep(const PathArgs& p, int mode, int32_t* row_state, int32_t* fb_count, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  row_prep_kernel<<<dim3(static_cast<unsigned>(p.Q)), dim3(256), 0, st>>>(
      p.row_start, p.row_end, p.page_table, p.P_log, p.P_phys, p.K, mode, p.out_raw, p.out_slot,
      p.out_count, p.out_score, row_state, fb_count, p.seq_of_row, p.n_seq);
  return hipGetLastError();
}

template <int K>
static hipError_t launch_gated_k(const PathArgs& p, const GatedScratch& g, int32_t splits, int32_t calib_splits,
                                 int calib_mode, bool no_fallback, int stage, int cus, hipStream_t st) {
  using G = Geometry<K>;
  const ScanArgs a = scan_args(p, g.row_state, splits);
  const CandArgs c = cand_args(g, K, no_fallback);
  const unsigned tiles = static_cast<unsigned>((p.Q + kRowsPerCta - 1) / kRowsPerCta);
  switch (stage) {
    case 0: {
      // split the calibration over the context when the row tiles alone leave CUs
      // idle and every split still gets kCalMinSplitBlocks sample blocks
      const int64_t sample_blocks = (p.P_log * kPage + kCalStride * kTile - 1) / (kCalStride * kTile);
      int64_t cs = calib_mode == 0 ? calib_splits : 1;
      if (cs > kCalMaxSplits) cs = kCalMaxSplits;
      if (cs > sample_blocks / kCalMinSplitBlocks) cs = sample_blocks / kCalMinSplitBlocks;
      if (cs < 1) cs = 1;
      calib_kernel<K><<<dim3(tiles, static_cast<unsigned>(cs)), dim3(kCtaThreads), 0, st>>>(a, c, calib_mode);
      if (cs > 1)
        calib_combine_kernel<<<dim3(static_cast<unsigned>((p.Q + kCombineRows - 1) / kCombineRows)),
                               dim3(64 * kCombineRows), 0, st>>>(a, c, static_cast<int>(cs));
      break;
    }
    case 1: {
      // a resident round of CTAs pulling (split, tile) items, or one CTA per item
      static std::atomic<int> per_cu{0};
      int occ = per_cu.load(std::memory_order_relaxed);
      if (occ == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, scan_kernel<K>, kCtaThreads, 0) != hipSuccess ||
            occ < 1) {
          (void)hipGetLastError();   // a failed query is not the launch's error
          occ = 2;
        }
        per_cu.store(occ, std::memory_order_relaxed);
      }
      const int64_t items = static_cast<int64_t>(tiles) * splits, resident = static_cast<int64_t>(occ) * cus;
      const int persistent = items >= 4 * resident ? 1 : 0;
      const int64_t grid = persistent ? resident : items;
      scan_kernel<K><<<dim3(static_cast<unsigned>(grid)), dim3(kCtaThreads), 0, st>>>(a, c, static_cast<int>(tiles),
                                                                                      persistent);
      break;
    }
    case 2:
      merge_kernel<K><<<dim3(static_cast<unsigned>(p.Q)), dim3(256), 0, st>>>(
          g.row_state, c, p.page_table, p.P_log, p.out_raw, p.out_slot, p.out_count, p.out_score);
      break;
    case 3:
      fallback_scan_kernel<K, kPoolCap, G::kFbSplits, G::kFbSplitsMin><<<dim3(kFallbackGrid), dim3(kCtaThreads), 0, st>>>(a, c);
      break;
    default:
      fallback_merge_kernel<K, G::kFbSplits, G::kFbSplitsMin><<<dim3(kFallbackGrid), dim3(256), 0, st>>>(
          c, p.page_table, p.P_log, p.out_raw, p.out_slot, p.out_count, p.out_score);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gated_stage(const PathArgs& p, const GatedScratch& g, int32_t splits, int32_t calib_splits,
                              int calib_mode, bool no_fallback, int stage, int cus, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  return p.K == 512 ? launch_gated_k<512>(p, g, splits, calib_splits, calib_mode, no_fallback, stage, cus, st)
                    : launch_gated_k<1024>(p, g, splits, calib_splits, calib_mode, no_fallback, stage, cus, st);
}

hipError_t launch_dense_score(const PathArgs& p, const int32_t* row_state, int32_t splits, float* logits,
                              hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.Q + kRowsPerCta - 1) / kRowsPerCta), static_cast<unsigned>(splits));
  const int64_t S = p.P_log * kPage;
  dense_score_kernel<<<grid, dim3(kCtaThreads), 0, st>>>(scan_args(p, row_state, splits), logits, S, 0,
                                                          static_cast<int32_t>(S));
  return hipGetLastError();
}

hipError_t launch_tiled(const PathArgs& p, const int32_t* row_state, int32_t splits, int32_t tile, float* tile_logits,
                        uint64_t* running, int32_t* run_count, uint64_t* run_floor, hipStream_t st) {
  if (p.Q == 0) return hipSuccess;
  const int64_t S = p.P_log * kPage;
  const dim3 sgrid(static_cast<unsigned>((p.Q + kRowsPerCta - 1) / kRowsPerCta), static_cast<unsigned>(splits));
  const dim3 rgrid(static_cast<unsigned>(p.Q));
  const ScanArgs a = scan_args(p, row_state, splits);
  tile_reset_kernel<<<dim3(static_cast<unsigned>((p.Q + 255) / 256)), dim3(256), 0, st>>>(run_count, run_floor,
                                                                                           p.Q);
  for (int64_t lo = 0; lo < S; lo += tile) {
    const int32_t hi = static_cast<int32_t>(lo + tile < S ? lo + tile : S);
    dense_score_kernel<<<sgrid, dim3(kCtaThreads), 0, st>>>(a, tile_logits, tile, static_cast<int32_t>(lo), hi);
    if (p.K == 512)
      tile_merge_kernel<512><<<rgrid, dim3(256), 0, st>>>(row_state, p.row_start, p.row_end, tile_logits, tile,
                                                          static_cast<int32_t>(lo), hi, running, run_count,
                                                          run_floor);
    else
      tile_merge_kernel<1024><<<rgrid, dim3(256), 0, st>>>(row_state, p.row_start, p.row_end, tile_logits, tile,
                                                           static_cast<int32_t>(lo), hi, running, run_count,
                                                           run_floor);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.K == 512)
    tile_emit_kernel<512><<<rgrid, dim3(256), 0, st>>>(row_state, running, run_count, p.page_table, p.P_log,
                                                       p.out_raw, p.out_slot, p.out_count, p.out_score);
  else
    tile_emit_kernel<1024><<<rgrid, dim3(256), 0, st>>>(row_state, running, run_count, p.page_table, p.P_log,
                                                        p.out_raw, p.out_slot, p.out_count, p.out_score);
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

// Cached per device after the first lookup (the address is fixed for the
// process), so that calls made while a stream is being captured do no lookups.
int32_t* status_word() {
  constexpr int kMaxDevices = 64;
  static int32_t* cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (dev < kMaxDevices && cache[dev] != nullptr) return cache[dev];
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_status)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (dev < kMaxDevices) cache[dev] = static_cast<int32_t*>(p);
  return static_cast<int32_t*>(p);
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

}  // namespace mqa
