// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

// Everything one call of the operator needs. Device pointers; sizes in elements.
struct PathArgs {
  const uint8_t* q;
  const uint8_t* q_scale;
  int64_t Q;
  const uint8_t* k_pages;
  const uint8_t* k_scale;
  int64_t P_phys;
  const float* weights;
  const int32_t* page_table;
  int64_t P_log;
  const int32_t* row_start;
  const int32_t* row_end;
  int32_t K;
  int32_t* out_raw;
  int32_t* out_slot;
  int32_t* out_count;
  float* out_score;
  // Multi-sequence form (nullptr = one page table for every row): row r uses
  // the page table page_table + seq_of_row[r] * P_log of n_seq tables.
  const int32_t* seq_of_row = nullptr;
  int64_t n_seq = 0;
};

// Scratch of the gated fused path (one call).
struct GatedScratch {
  int32_t* row_state;   // [Q]
  uint64_t* gate;       // [Q]
  uint32_t* count;      // [Q]
  int32_t* fb_list;     // [Q]
  int32_t* fb_count;    // [1]
  int32_t* fb_cnt;      // [Q, 4]
  uint64_t* cand;       // [Q, candidate_cap(K)]
  int32_t* work;        // [1] the gated scan's item counter
};

// Candidate keys kept per row by the fused path's gated scan. The gate is the
// k'-th key of a 1/64 position sample (k' = x + 4 sqrt(x) + 8, x = K m / n: 40
// at K = 1024, 28 at K = 512); the keys above it number k' + NegBinomial(k',
// 1/64): 2,560 +- 405 and 1,792 +- 339. 5,120 and 4,096 keys make an overflow
// (the row then takes the exact fallback) rarer than 1e-6 per row.
constexpr int candidate_cap(int K) { return K == 512 ? 4096 : 5120; }
// The decode path's gate samples every 32nd page (about 2,016 +- 254 and 1,280
// +- 202 keys pass it), and the dense selector's samples 128 chunks of 64
// logits: both keep the smaller buffers.
constexpr int decode_candidate_cap(int K) { return K == 512 ? 3072 : 4096; }
constexpr int selector_candidate_cap(int K) { return K == 512 ? 3072 : 4096; }

// Keys a row's pool holds in the context-tiled path (K after each compaction,
// appended tile keys above its floor up to this many).
constexpr int tile_pool_cap(int K) { return 2 * K; }

// mode 0: TopK (answers short and invalid rows); mode 1: logits only.
// fb_count (nullable) is cleared for the gated path.
hipError_t launch_row_prep(const PathArgs& p, int mode, int32_t* row_state, int32_t* fb_count, hipStream_t st);
// Stages of the gated fused path: 0 calibration (calib_mode 0 normal, 1 no
// prefilter, 2 forced underfill; calib_splits context splits), 1 gated scan
// (splits context splits), 2 merge, 3 fallback scan, 4 fallback merge. With
// no_fallback the merge fails closed the rows it would list for the fallback
// (underfill -3, overflow -4) and the list stays empty.
hipError_t launch_gated_stage(const PathArgs& p, const GatedScratch& g, int32_t splits, int32_t calib_splits,
                              int calib_mode, bool no_fallback, int stage, int cus, hipStream_t st);
hipError_t launch_dense_score(const PathArgs& p, const int32_t* row_state, int32_t splits, float* logits,
                              hipStream_t st);
// Decode / multi-sequence path: per-wave streaming exact TopK over each row's
// own pages, then an exact merge of the splits. Scratch comes from the caller.
struct DecodeScratch {
  int32_t* row_state;   // [Q]
  int32_t* counts;      // [Q, splits]      fallback: keys per (row, split)
  uint64_t* keys;       // [Q, splits, K]   fallback: top-K per (row, split)
  uint64_t* gate;       // [Q]
  uint32_t* cand_n;     // [Q]              candidates appended (may exceed cap: overflow)
  uint64_t* cand;       // [Q, decode_candidate_cap(K)]
  int32_t* fb_list;     // [Q]              rows sent to the fallback
  int32_t* fb_count;    // [1]              (cleared by row_prep)
  int64_t* plan;        // [Q + 1]          gated scan: pages of the rows before each row
  uint64_t* wave_keys;  // [kDecScanWaves, kDecWaveStride] gated scan: each wave's candidates
  uint32_t* wave_first; // [kDecScanWaves]  candidates of the wave's first segment
  uint32_t* row_off;    // [Q]              where the row's first segment's candidates start
  uint32_t* row_first;  // [Q]              and how many there are
  uint32_t* row_w0;     // [Q]              first scan wave over the row's pages
  uint32_t* row_nw;     // [Q]              and the number of waves
  int64_t* wave_desc;   // [kDecScanWaves, 3] a scan wave's pages [g0, g1) and its first row
};
constexpr int kDecScanWaves = 3072;   // gated scan waves at most (three 4-wave blocks per CU on 256 CUs)
constexpr int kDecWaveKeys = 512;     // candidate keys a scan wave keeps before spilling to the row's buffer
constexpr int kDecWaveStride = kDecWaveKeys + 16;   // and a 128-byte line its lanes without a key write to
constexpr int kMaxDecodeSplits = 64;
size_t decode_scratch_bytes(int64_t Q, int32_t K, int32_t splits);
DecodeScratch decode_scratch_layout(void* base, int64_t Q, int32_t K, int32_t splits);
// Measurement marker called between launches (index, stream); may be null.
typedef void (*StageMark)(int, hipStream_t);
// mode 0 gated, 1 no prefilter (every long row takes the exact fallback), 2 forced underfill;
// no_fallback: rows the gated pass cannot finish fail closed instead (as for the prefill path).
// The gated scan runs on a fixed grid for `cus` compute units; `splits` is the
// fallback's context splits per row.
hipError_t launch_decode(const PathArgs& p, const DecodeScratch& w, int32_t splits, int mode, bool no_fallback,
                         int cus, hipStream_t st, StageMark mark = nullptr);

// Bounded context-tiled exact TopK over long rows (row_state from row_prep):
// tile_logits [Q, tile] fp32, running [Q, K] keys and run_count [Q] are scratch.
hipError_t launch_tiled(const PathArgs& p, const int32_t* row_state, int32_t splits, int32_t tile, float* tile_logits,
                        uint64_t* running, int32_t* run_count, uint64_t* run_floor, hipStream_t st);
hipError_t launch_logits_topk(const PathArgs& p, const float* logits, const int32_t* row_state,
                              hipStream_t st);
// Copies the sticky status word to *host_out and clears it (synchronises st).
hipError_t status_take(hipStream_t st, int32_t* host_out);
// Device address of the current device's sticky status word (nullptr on error).
int32_t* status_word();

// MXFP4 quantisation of n_vec 128-element fp32 vectors (OCP MX conversion). With
// positions == nullptr vector v goes to row v of codes / scales; otherwise to
// the physical slot of logical C4 position positions[v] (cache writer).
hipError_t launch_mx_quantize(const float* x, int64_t n_vec, uint8_t* codes, uint8_t* scales,
                              const int32_t* positions, const int32_t* page_table, int64_t P_log, int64_t P_phys,
                              int cus, hipStream_t st);

}  // namespace mqa
