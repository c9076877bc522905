/*
 * mqa_fp4_topk.h -- C ABI of the MI355X (gfx950) FP4 paged-MQA prefill indexer
 * fused with exact TopK.
 *
 * What the operator computes
 * --------------------------
 * Sources: "[FlyDSL] Add FP4 LiteTopK prefill operator" (ROCm/aiter PR 5309),
 * Summary and Implementation; "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK"
 * (ROCm/aiter PR 5282), Changes and Scope.
 *
 * For every query row q and every logical C4 position s of the row's window
 * [row_start[q], row_end[q]) the DeepSeek-V4 indexer score is
 *
 *     score[q, s] = sum_{h<64} weights[q, h] * ReLU(dot_h(q, s))
 *     dot_h(q, s) = sum_{b<4} 2^(qs[q,h,b]-127) * 2^(ks[s,b]-127)
 *                   * sum_{j<32} e2m1(q[q,h,32b+j]) * e2m1(k[s,32b+j])
 *
 * computed in fp32 (ReLU(x) = x if x > 0 else +0). Each row returns the K
 * positions first in the total order "score descending, then logical index
 * ascending; NaN below every number; +0 above -0" (PR 5282, Changes), written
 * in ascending position order, together with their physical cache slots
 * page_table[s / 64] * 64 + s % 64 and a valid count. A row whose window
 * length is <= K returns every position of the window in order, padded with
 * -1 (PR 5282, Changes: short-row contract). The [Q, S] score matrix is never
 * materialised by mqa_fp4_topk_prefill; its scratch does not depend on S.
 *
 * Data layout (all tensors C-contiguous, all pointers DEVICE pointers on one
 * gfx950 device, owned by the caller; the library never frees or keeps them):
 *   q          uint8  [Q, 64, 64]        E2M1 codes, element 2j = low nibble of byte j
 *   q_scale    uint8  [Q, 64, 4]         UE8M0 byte per 32 elements along D=128
 *   k_pages    uint8  [P_phys, 64, 64]   paged C4 key cache, page size 64
 *   k_scale    uint8  [P_phys, 64, 4]
 *   weights    float  [Q, 64]
 *   page_table int32  [P_log]            logical page -> physical page; S = 64 * P_log
 *   row_start, row_end int32 [Q]         window [start, end) in logical C4 positions
 *   out_raw, out_slot  int32 [Q, K]      filled in place by the library (sglang PR 38101,
 *                                        Changes: slots and, optionally, raw
 *                                        positions go straight into caller buffers)
 *   out_count  int32  [Q]                min(len, K), or a negative per-row code
 *   out_score  float  [Q, K] (optional)  fp32 score of each selected position;
 *                                        NaN for padding and for short rows
 * q, k_pages and k_scale must be 16-byte aligned, the others 4-byte aligned.
 *
 * Errors (fail closed, PR 5309 Implementation)
 * --------------------------------------------
 * A negative return value is a host-detected error: nothing was launched and no
 * output was written. A row that the device finds invalid gets out_raw and
 * out_slot all -1 and a negative out_count (MQA_ROW_*), and sets a sticky bit
 * in the per-device status word read by mqa_fp4_status().
 *
 * Streams and devices (PR 5309 Implementation: preserve caller device/stream
 * ownership, 64-bit addressing). Work is enqueued on `stream` (a hipStream_t;
 * NULL = the legacy default stream of the current device), which must belong to
 * the device the tensors live on; the caller's current device is restored
 * before returning. The success path never synchronises. A capturing stream is
 * refused with MQA_ERR_CAPTURING (PR 5282, Scope: no graph capture in the first
 * version). Calls on the same stream are ordered; calls on different streams
 * use separate stream-ordered scratch and may run concurrently.
 *
 * Scratch of the allocating entry points comes from the device's default
 * memory pool (hipMallocAsync on `stream`, hipFreeAsync when the call's work
 * is enqueued). On its first call on a device the library sets that pool's
 * release threshold to its maximum, so that freed scratch stays in the pool
 * for the next call instead of going back to the driver: a process-wide
 * setting of the default pool, which other users of that pool share.
 */
#ifndef MQA_FP4_TOPK_H
#define MQA_FP4_TOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------- */
#define MQA_OK 0
#define MQA_ERR_UNSUPPORTED_K (-1)   /* K not in {512, 1024} (PR 5309: explicit supported-K contract) */
#define MQA_ERR_NULL_POINTER (-2)    /* a required pointer is NULL while its tensor is non-empty */
#define MQA_ERR_MISALIGNED (-3)      /* a pointer breaks the alignment stated above */
#define MQA_ERR_BAD_SIZE (-4)        /* negative size, or Q / 64*P_log / 64*P_phys beyond int32 */
#define MQA_ERR_DEVICE (-5)          /* not device memory, tensors on different devices, stream on
                                        another device, or the device is not gfx950 */
#define MQA_ERR_CAPTURING (-6)       /* the stream is capturing a graph */
#define MQA_ERR_HIP (-7)             /* a HIP runtime call failed (allocation, launch) */
#define MQA_ERR_BAD_FLAGS (-8)       /* unknown bits in flags */

/* ---- per-row codes in out_count -------------------------------------------- */
#define MQA_ROW_BAD_WINDOW (-1)      /* start < 0, end < start or end > 64 * P_log */
#define MQA_ROW_BAD_PAGE (-2)        /* a page touched by the window maps outside [0, P_phys) */
#define MQA_ROW_UNDERFILL (-3)       /* fewer than K candidates survived the candidate gate and no exact
                                        recomputation supplied the rest (MQA_FLAG_NO_FALLBACK), or an
                                        exact recomputation itself ended with fewer than K keys */
#define MQA_ROW_SELECTOR (-4)        /* the row's candidates overflowed their bounded buffer and were
                                        not recomputed (MQA_FLAG_NO_FALLBACK), or an internal selection
                                        invariant was violated */

/* ---- sticky status bits ---------------------------------------------------- */
#define MQA_STATUS_BAD_WINDOW 1
#define MQA_STATUS_BAD_PAGE 2
#define MQA_STATUS_UNDERFILL 4
#define MQA_STATUS_SELECTOR 8

/* ---- flags of the _ex entry point -------------------------------------------- */
#define MQA_FLAG_SPLITS_MASK 0xFFu   /* context splits per row tile, 0 = automatic (1..255) */
#define MQA_FLAG_NO_PREFILTER 0x100u /* no calibrated candidate gate: every long row takes the
                                        exact ungated streaming path */
#define MQA_FLAG_FORCE_UNDERFILL 0x200u /* gate above every key, so every long row underfills
                                           and takes the fallback (for tests) */
#define MQA_FLAG_NO_FALLBACK 0x400u  /* no exact recomputation of rows the gated pass cannot finish:
                                        an underfilled row fails closed with MQA_ROW_UNDERFILL
                                        (status MQA_STATUS_UNDERFILL), an overflowed one with
                                        MQA_ROW_SELECTOR (status MQA_STATUS_SELECTOR); with
                                        MQA_FLAG_FORCE_UNDERFILL every long row fails closed (for
                                        tests of the fail-closed path, PR 5309 Implementation: fail
                                        closed on underfill); not combinable with
                                        MQA_FLAG_NO_PREFILTER */

/*
 * Fused FP4 scoring + exact TopK + page mapping (the hot path).
 *   num_rows          0 <= Q <= INT32_MAX
 *   num_phys_pages    P_phys >= 0, 64 * P_phys <= INT32_MAX
 *   num_logical_pages P_log >= 0, 64 * P_log <= INT32_MAX - 512
 *   K                 512 or 1024
 * Returns MQA_OK or a negative MQA_ERR_*.
 */
int32_t mqa_fp4_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                             const uint8_t* k_pages, const uint8_t* k_scale,
                             int64_t num_phys_pages, const float* weights,
                             const int32_t* page_table, int64_t num_logical_pages,
                             const int32_t* row_start, const int32_t* row_end, int32_t K,
                             int32_t* out_raw, int32_t* out_slot, int32_t* out_count,
                             void* stream);

/* As mqa_fp4_topk_prefill, plus an optional fp32 score output (NULL = none)
 * and flags (MQA_FLAG_*). Outputs do not depend on the splits chosen.
 * The flags expose for tests the properties the pages check: the exact merge
 * of split candidates ("[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK"
 * (PR 5282), Changes, and its Validation: exact candidate union) for any
 * number of context splits; the calibrated candidate filtering of "[FlyDSL]
 * Add FP4 LiteTopK prefill operator" (PR 5309), Implementation, as a pure
 * speed-up -- the same TopK sets with it switched off (MQA_FLAG_NO_PREFILTER)
 * or forced to underfill (MQA_FLAG_FORCE_UNDERFILL); and the same
 * Implementation's fail-closed rule on underfill (MQA_FLAG_NO_FALLBACK).
 * out_score holds the fp32 score of each selected position (the fp32 scores
 * of PR 5282, Motivation). */
int32_t mqa_fp4_topk_prefill_ex(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                const uint8_t* k_pages, const uint8_t* k_scale,
                                int64_t num_phys_pages, const float* weights,
                                const int32_t* page_table, int64_t num_logical_pages,
                                const int32_t* row_start, const int32_t* row_end, int32_t K,
                                int32_t* out_raw, int32_t* out_slot, int32_t* out_count,
                                float* out_score, uint32_t flags, void* stream);

/*
 * Allocation-free form of mqa_fp4_topk_prefill_ex, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, flags, outputs and fail-
 * closed rules as mqa_fp4_topk_prefill_ex (the same kernels run). The call's
 * scratch -- mqa_fp4_topk_scratch_bytes(num_rows, K, device) bytes -- comes
 * from a fixed array of MQA_STATIC_SCRATCH_BYTES bytes that the library keeps
 * on every device it runs on until the process ends, so num_rows is limited to
 * what fits: 1,636 rows at K = 1024 and 2,045 at K = 512; a larger batch
 * returns MQA_ERR_BAD_SIZE with nothing launched. The call allocates and frees
 * nothing, never synchronises, and accepts a capturing stream (the kernels
 * write every scratch word before reading it, so replays need no clearing).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap in time on one device (on streams not
 * ordered with each other, or from several host threads) race and give
 * undefined outputs -- order them on one stream.
 */
#define MQA_STATIC_SCRATCH_BYTES (64ll << 20)
int32_t mqa_fp4_topk_prefill_static(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                    const uint8_t* k_pages, const uint8_t* k_scale,
                                    int64_t num_phys_pages, const float* weights,
                                    const int32_t* page_table, int64_t num_logical_pages,
                                    const int32_t* row_start, const int32_t* row_end, int32_t K,
                                    int32_t* out_raw, int32_t* out_slot, int32_t* out_count,
                                    float* out_score, uint32_t flags, void* stream);

/*
 * Dense comparator (the legacy full-logits path the pages measure against:
 * PR 5282 Motivation, where the whole fp32 row-by-context score matrix is built
 * first and TopK runs on it afterwards). Writes the fp32 score of every position inside each
 * long row's window (length > K) into logits[q * 64 * P_log + s] (caller-owned
 * [Q, S] buffer; entries outside those windows are left untouched), then selects
 * exactly as mqa_fp4_topk_prefill. Scores are bit-identical to the fused path.
 */
int32_t mqa_fp4_dense_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                   const uint8_t* k_pages, const uint8_t* k_scale,
                                   int64_t num_phys_pages, const float* weights,
                                   const int32_t* page_table, int64_t num_logical_pages,
                                   const int32_t* row_start, const int32_t* row_end, int32_t K,
                                   float* logits, int32_t* out_raw, int32_t* out_slot,
                                   int32_t* out_count, float* out_score, void* stream);

/*
 * Bounded context-tiled exact TopK: the correctness / reference fallback of
 * "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK" (ROCm/aiter PR 5282),
 * Changes. Same inputs, outputs and contract as mqa_fp4_topk_prefill (K, short
 * rows, windows, pages, fail closed, page map), computed another way: the
 * context is visited in tiles of tile_positions logical positions (a multiple
 * of 256; 0 = 4096); per tile the fp32 scores of every row are written to a
 * [Q, tile_positions] scratch buffer by the dense scorer, and every long row
 * appends the tile's keys above its floor to a pool of at most 2K keys,
 * compacted to its exact top K by radix select when full. No
 * gate, no calibration. Outputs are identical to mqa_fp4_topk_prefill's
 * (scores bit-identical). Stream-ordered scratch:
 * mqa_fp4_tiled_scratch_bytes(Q, K, tile) = O(Q) + Q*2K*8 + Q*tile*4 bytes,
 * independent of the context length. Returns MQA_ERR_BAD_SIZE for a bad tile.
 */
int32_t mqa_fp4_tiled_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                   const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                                   const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                                   const int32_t* row_start, const int32_t* row_end, int32_t K,
                                   int32_t tile_positions, int32_t* out_raw, int32_t* out_slot,
                                   int32_t* out_count, float* out_score, void* stream);
int64_t mqa_fp4_tiled_scratch_bytes(int64_t num_rows, int32_t K, int32_t tile_positions);

/* The dense path's scorer alone: logits as above, for every row with a valid
 * window and valid pages (no length condition). */
int32_t mqa_fp4_dense_logits(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                             const uint8_t* k_pages, const uint8_t* k_scale,
                             int64_t num_phys_pages, const float* weights,
                             const int32_t* page_table, int64_t num_logical_pages,
                             const int32_t* row_start, const int32_t* row_end, float* logits,
                             void* stream);

/* The dense path's selector alone: exact TopK over caller-provided fp32 logits
 * [Q, 64 * P_log] under the same total order, windows, short-row rule, page
 * validation and page mapping. */
int32_t mqa_fp4_logits_topk(const float* logits, int64_t num_rows, const int32_t* page_table,
                            int64_t num_logical_pages, int64_t num_phys_pages,
                            const int32_t* row_start, const int32_t* row_end, int32_t K,
                            int32_t* out_raw, int32_t* out_slot, int32_t* out_count,
                            float* out_score, void* stream);

/* Capability probe (sglang PR 38101, Dependency: probe by exact symbol).
 * Writes up to `capacity` supported K values into ks and their number into *n. */
int32_t mqa_fp4_supported_k(int32_t* ks, int32_t capacity, int32_t* n);

/* Bytes of stream-ordered device scratch mqa_fp4_topk_prefill allocates for
 * num_rows rows on `device`: O(num_rows) bookkeeping plus a bounded candidate
 * buffer per row, independent of the context length (candidate and merge
 * scratch independent of the context: "[FlyDSL][DSv4] Prototype FP4 MQA
 * streaming TopK" (PR 5282), Changes, with its sizes in the MI355X runtime
 * update; "[AMD][DSv4] Add experimental AITER FP4 streaming TopK", Memory
 * geometry). Negative on error (MQA_ERR_UNSUPPORTED_K, MQA_ERR_BAD_SIZE,
 * MQA_ERR_DEVICE for a device that is not a gfx950). */
int64_t mqa_fp4_topk_scratch_bytes(int64_t num_rows, int32_t K, int32_t device);

/* Synchronises `stream`, then returns in *status the OR of the sticky status
 * bits (MQA_STATUS_*) set by calls on the stream's device since the last read,
 * and clears them: the device-side half of failing closed ("[FlyDSL] Add FP4
 * LiteTopK prefill operator" (PR 5309), Implementation), for rows the device
 * finds invalid or cannot finish. Returns MQA_ERR_NULL_POINTER for a NULL
 * status, MQA_ERR_DEVICE / MQA_ERR_HIP when the stream or the copy fails. */
int32_t mqa_fp4_status(void* stream, int32_t* status);

/* Measurement hook. After this call, every fused or dense TopK call made by
 * the calling host thread records the n == 5 caller-created hipEvent_t handles
 * in events[] on the call's stream: [0] before row preparation, [1] before the
 * gate calibration, [2] before the scoring kernel (fused and decode: the gated
 * scan; dense: the logits kernel; [1] and [2] coincide on the dense path), [3]
 * after it, [4] after the last kernel of the call. (The tiled path records them
 * too, around all of its tiles.) The array must stay valid until the hook
 * is replaced; n == 0 (or events == NULL) turns it off. Adds no
 * synchronisation. Returns MQA_ERR_BAD_SIZE for other n. */
int32_t mqa_fp4_set_stage_events(void* const* events, int32_t n);

/*
 * Decode / multi-sequence form, capturable into a HIP graph. Every row has its
 * own page table: row r belongs to sequence seq_of_row[r] and reads logical page
 * p through block_table[seq_of_row[r] * max_pages + p]; windows, K, the short-row
 * rule, the total order and the outputs are those of mqa_fp4_topk_prefill, with
 * slots block_table[seq][s / 64] * 64 + s % 64 ("[FlyDSL][DSv4] Prototype FP4 MQA
 * streaming TopK", Changes and Scope; decode is the adjacent shape that
 * "[AMD][DSv4] Add experimental AITER FP4 streaming TopK" keeps on the older
 * path, and graph capture the support PR 5282's Scope defers).
 *   block_table int32 [num_seqs, max_pages]   64 * max_pages <= INT32_MAX - 512,
 *                                             num_seqs * max_pages <= INT32_MAX
 *   seq_of_row  int32 [Q]                     a row whose sequence is outside
 *                                             [0, num_seqs) fails with code -1
 *   workspace   device memory of at least mqa_fp4_decode_workspace_bytes(Q, K,
 *               splits, device) bytes, 256-byte aligned, owned by the caller;
 *               its contents need no initialisation and are scratch only (the
 *               size is O(Q * splits * K) plus a fixed 12.5 MiB for the gated
 *               scan's per-wave candidate regions, independent of the context)
 *   splits      context splits per row of the exact fallback (1..64), 0 =
 *               automatic for the device
 * The call allocates nothing, never synchronises and accepts a capturing
 * stream; row failures are reported in out_count and the sticky status word
 * only (read mqa_fp4_status outside the graph). Each row is scanned
 * independently (no key sharing between rows): a calibrated gate per row from
 * every 32nd page (PR 5309's calibrated candidate filter; a coarser multiple of
 * 32 on windows beyond 262,144 positions), then a gated scan in which the
 * device's waves share all rows' pages evenly (each wave's share within one row
 * when rows are few), each keeping its candidates in a region of its own, and
 * an exact merge per row; rows that underfill or overflow are recomputed
 * exactly by per-wave bounded LDS pools (PR 5282's streaming design) with an
 * exact merge of the splits. flags: MQA_FLAG_NO_PREFILTER or
 * MQA_FLAG_FORCE_UNDERFILL (for tests), MQA_FLAG_NO_FALLBACK (fail closed
 * instead of the fallback, as for mqa_fp4_topk_prefill_ex; not with
 * MQA_FLAG_NO_PREFILTER); the split bits must be 0, splits are the separate
 * argument. Outputs do not depend on the splits or the flags (except rows that
 * MQA_FLAG_NO_FALLBACK fails closed). Two calls that share a workspace must be
 * ordered (same stream).
 */
int32_t mqa_fp4_topk_decode(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows, const uint8_t* k_pages,
                            const uint8_t* k_scale, int64_t num_phys_pages, const float* weights,
                            const int32_t* block_table, int64_t num_seqs, int64_t max_pages,
                            const int32_t* seq_of_row, const int32_t* row_start, const int32_t* row_end, int32_t K,
                            int32_t* out_raw, int32_t* out_slot, int32_t* out_count, float* out_score,
                            void* workspace, int64_t workspace_bytes, int32_t splits, uint32_t flags,
                            void* stream);
int64_t mqa_fp4_decode_workspace_bytes(int64_t num_rows, int32_t K, int32_t splits, int32_t device);

/*
 * MXFP4 quantisation: the producer of the FP4 inputs above. Source: the
 * payload named in "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK" (ROCm/aiter
 * PR 5282), Scope (FP4 E2M1 with UE8M0 scales); the conversion rule is the OCP
 * Microscaling Formats (MX) v1.0 conversion of a vector of scalars to an MX block,
 * for E2M1 elements: per 32-element block, shared exponent floor(log2 max|v|) - 2,
 * elements v / 2^shared rounded to the nearest E2M1 value with ties to the even
 * mantissa bit, saturating at +-6, sign kept (-0 is code 8). Scale byte = shared
 * + 127 clamped to [0, 254]; an all-zero block gets byte 0; a block holding a NaN
 * or an infinity gets byte 0xFF (UE8M0 NaN) and zero codes.
 *   x      float [n_vec, 128] (16-byte aligned)   e.g. q as [Q * 64, 128]
 *   codes  uint8 [n_vec, 64]  (2-byte aligned)    element 2j = low nibble of byte j
 *   scales uint8 [n_vec, 4]
 * All device pointers on one gfx950 device, owned by the caller. HBM-bound: 512
 * bytes read, 68 written per vector. Errors as for the operator (host-detected,
 * nothing launched).
 */
int32_t mqa_fp4_quantize(const float* x, int64_t n_vec, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * C4 paged key-cache writer: quantises n fp32 key vectors k [n, 128] as above and
 * stores vector i at logical C4 position positions[i], i.e. in row
 * page_table[p / 64] * 64 + p % 64 of k_pages [P_phys, 64, 64] / k_scale
 * [P_phys, 64, 4] (the operator's cache layout; "[FlyDSL][DSv4] Prototype FP4 MQA
 * streaming TopK", Changes: raw C4 positions map through the page table). A
 * vector whose position is outside [0, 64 * P_log) is not written and sets
 * MQA_STATUS_BAD_WINDOW; one whose page maps outside [0, P_phys) is not written
 * and sets MQA_STATUS_BAD_PAGE (read with mqa_fp4_status). Positions must be
 * distinct within a call (which of two vectors lands at one slot is unspecified).
 */
int32_t mqa_fp4_cache_write(const float* k, int64_t n, const int32_t* positions, const int32_t* page_table,
                            int64_t num_logical_pages, int64_t num_phys_pages, uint8_t* k_pages, uint8_t* k_scale,
                            void* stream);

/* Static description of a return code. */
const char* mqa_fp4_error_string(int32_t code);

/* ABI version of this header (incremented on incompatible change). */
int32_t mqa_fp4_abi_version(void);
#define MQA_FP4_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* MQA_FP4_TOPK_H */
