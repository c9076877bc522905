// Decode / multi-sequence variant of the FP4 paged-MQA indexer with exact TopK
// (gfx950). Every row has its own page table (block table row seq_of_row[r]),
// so rows share no key tiles: each wave streams one (row, context split) item's
// pages by itself, the way the pages' first fused design keeps a bounded pool
// per CTA ("[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK", Changes: scores
// stream through a bounded LDS pool, exact total-order radix, each CTA emits
// only candidates and a count, splits merged exactly, raw positions mapped
// through the page table). Decode workloads are the adjacent shape the pages
// leave on the older path ("[AMD][DSv4] Add experimental AITER FP4 streaming
// TopK", Changes / Scope) and whose graph-capture support they defer ([P2]
// Scope); this entry point takes its scratch from the caller, never allocates
// or synchronises, and reports row failures only on the device, so it can be
// captured into a HIP graph and replayed.
//
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

template <int K>
struct DecGeom;
template <>
struct DecGeom<512> {
  static constexpr int kCap = 640;    // pool keys per wave: K plus two 64-key batches
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
  uint64_t* keys;     // [Q, splits, K]
  int32_t* counts;    // [Q, splits]
};

__device__ __forceinline__ void vm_wait_all() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

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

template <int K>
__global__ void __launch_bounds__(kDecThreads, 2) decode_scan_kernel(DecArgs a) {
  constexpr int CAP = DecGeom<K>::kCap;
  static_assert(CAP >= K + 128, "pool holds K keys and two batches");
  // two page buffers as separate LDS variables, read and written under static
  // names (the loop below is unrolled by two), so that the copy of the next page
  // is not waited for before the current page's reads
  __shared__ __attribute__((aligned(16))) uint8_t s_c0[kDecWaves][kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_c1[kDecWaves][kPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_s0[kDecWaves][kPageScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_s1[kDecWaves][kPageScaleBytes];
  __shared__ uint64_t s_pool[kDecWaves][CAP];
  __shared__ uint32_t s_hist[kDecWaves][256];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kDecWaves + wave;
  if (item >= static_cast<int64_t>(a.Q) * a.splits) return;   // waves are independent: no block barrier below
  const int row = static_cast<int>(item / a.splits), split = static_cast<int>(item % a.splits);
  if (a.row_state[row] != kRowLong) return;
  const int start = a.row_start[row], end = a.row_end[row];
  const int32_t* table = a.block_table + static_cast<size_t>(a.seq_of_row[row]) * a.max_pages;
  const int pg0 = start / kPage, n_pages = (end - 1) / kPage + 1 - pg0;
  const int pa = pg0 + static_cast<int>(static_cast<int64_t>(n_pages) * split / a.splits);
  const int pb = pg0 + static_cast<int>(static_cast<int64_t>(n_pages) * (split + 1) / a.splits);

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

  auto body = [&](int pg, const uint8_t* codes, const uint8_t* scales) {
    const int p0 = pg * kPage;
    const uint64_t win = (p0 >= start && p0 + kPage <= end) ? ~0ull : window_lanes(p0, start, end);
    const GroupAcc g0 = mfma_group<0>(qr, codes, scales, lo);
    const float h0 = head_partial(qr, g0.d0, g0.d1);
    const GroupAcc g1 = mfma_group<1>(qr, codes, scales, lo);
    const float h1 = head_partial(qr, g1.d0, g1.d1);
    const float sc = combine_halves(h0, h1);   // lane l: position p0 + l
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
  };

  // block-table entries, 64 pages per vector load, the next chunk prefetched
  auto chunk = [&](int c) -> int32_t {
    const int pg = pa + 64 * c + lane;
    return pg < pb ? table[pg] : -1;
  };
  int32_t cur = chunk(0), nxt = chunk(1);
  auto entry = [&](int i) -> int32_t {   // page pa + i, i within the current or the next chunk
    return (i >> 6) == 0 ? __builtin_amdgcn_readlane(cur, i & 63) : __builtin_amdgcn_readlane(nxt, i & 63);
  };
  // Step i: copy page i + 1 into the other buffer, score page i, wait. At a
  // chunk boundary the chunks rotate after the copy that used the next one.
  int base = 0;   // first page index (relative to pa) of chunk `cur`
  auto step = [&](int i, const uint8_t* codes, const uint8_t* scales, uint8_t* nc, uint8_t* ns) {
    if (pa + i + 1 < pb) {
      page_dma(a, entry(i + 1 - base), nc, ns, lane);
      if (((i + 1 - base) >> 6) != 0) {   // page i + 1 opened the next chunk
        cur = nxt;
        base += 64;
        nxt = chunk(base / 64 + 1);
      }
    }
    body(pa + i, codes, scales);
    vm_wait_all();
  };
  vm_wait_all();   // query row and the first chunks
  if (pa < pb) page_dma(a, entry(0), s_c0[wave], s_s0[wave], lane);
  vm_wait_all();
  for (int i = 0; pa + i < pb; i += 2) {
    step(i, s_c0[wave], s_s0[wave], s_c1[wave], s_s1[wave]);
    if (pa + i + 1 < pb) step(i + 1, s_c1[wave], s_s1[wave], s_c0[wave], s_s0[wave]);
  }

  wave_lds_sync();
  if (fill > K) {
    const Selected sel = wave_select_compact(pool, fill, K, hist, lane);
    if (sel.kept != K) failed = true;
    fill = K;
  }
  uint64_t* dst = a.keys + (static_cast<size_t>(row) * a.splits + split) * K;
  for (int i = lane; i < fill; i += 64) dst[i] = pool[i];
  if (lane == 0) a.counts[static_cast<size_t>(row) * a.splits + split] = failed ? kCodeSelector : fill;
}

// One 1024-thread block per long row; 11-bit radix digits (the splits hold up
// to 64 K keys per row, so wide digits save passes over them).
template <int K>
__global__ void __launch_bounds__(1024) decode_merge_kernel(DecArgs a, int32_t* __restrict__ out_raw,
                                                            int32_t* __restrict__ out_slot,
                                                            int32_t* __restrict__ out_count,
                                                            float* __restrict__ out_score, int32_t* status) {
  constexpr int NT = 1024;
  __shared__ uint64_t s_sel[K];
  __shared__ uint32_t s_hist[2048];
  __shared__ int32_t s_cnt[kMaxDecodeSplits];
  __shared__ BlockScratch<NT> s_red;
  __shared__ int32_t s_n, s_total;
  const int64_t row = blockIdx.x;
  if (a.row_state[row] != kRowLong) return;
  const int splits = a.splits;
  const int32_t* table = a.block_table + static_cast<size_t>(a.seq_of_row[row]) * a.max_pages;
  const uint64_t* keys = a.keys + static_cast<size_t>(row) * splits * K;
  if (threadIdx.x == 0) {
    int total = 0;
    for (int i = 0; i < splits; ++i) {
      s_cnt[i] = a.counts[static_cast<size_t>(row) * splits + i];
      if (s_cnt[i] < 0 || s_cnt[i] > K) total = -1000000;
      total += s_cnt[i];
    }
    s_total = total;
    s_n = 0;
  }
  __syncthreads();
  if (s_total < K) {   // a long row holds more than K positions: anything else is a selector failure
    fail_row<K, NT>(row, kCodeSelector, out_raw, out_slot, out_count, out_score, status);
    return;
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
    return;
  }
  emit_row<K, NT>(s_sel, row, table, a.max_pages, out_raw, out_slot, out_count, out_score);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t decode_scratch_bytes(int64_t Q, int32_t K, int32_t splits) {
  const size_t q = static_cast<size_t>(Q), s = static_cast<size_t>(splits);
  return align256(q * sizeof(int32_t)) + align256(q * s * sizeof(int32_t)) +
         align256(q * s * static_cast<size_t>(K) * sizeof(uint64_t));
}

DecodeScratch decode_scratch_layout(void* base, int64_t Q, int32_t K, int32_t splits) {
  const size_t q = static_cast<size_t>(Q), s = static_cast<size_t>(splits);
  char* b = static_cast<char*>(base);
  DecodeScratch w;
  w.row_state = reinterpret_cast<int32_t*>(b);
  w.counts = reinterpret_cast<int32_t*>(b + align256(q * sizeof(int32_t)));
  w.keys = reinterpret_cast<uint64_t*>(b + align256(q * sizeof(int32_t)) + align256(q * s * sizeof(int32_t)));
  (void)K;
  return w;
}

hipError_t launch_decode(const PathArgs& p, const DecodeScratch& w, int32_t splits, hipStream_t st) {
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
  a.keys = w.keys;
  a.counts = w.counts;
  const int64_t items = p.Q * splits;
  const dim3 sgrid(static_cast<unsigned>((items + kDecWaves - 1) / kDecWaves));
  const dim3 mgrid(static_cast<unsigned>(p.Q));
  if (p.K == 512) {
    decode_scan_kernel<512><<<sgrid, dim3(kDecThreads), 0, st>>>(a);
    decode_merge_kernel<512><<<mgrid, dim3(1024), 0, st>>>(a, p.out_raw, p.out_slot, p.out_count, p.out_score, status);
  } else {
    decode_scan_kernel<1024><<<sgrid, dim3(kDecThreads), 0, st>>>(a);
    decode_merge_kernel<1024><<<mgrid, dim3(1024), 0, st>>>(a, p.out_raw, p.out_slot, p.out_count, p.out_score, status);
  }
  return hipGetLastError();
}

}  // namespace mqa
