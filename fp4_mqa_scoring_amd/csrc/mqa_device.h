// Device-side building blocks of the FP4 paged-MQA indexer (gfx950 / CDNA4).
//
// Shared by the fused scorer+TopK kernel and the dense comparator so that the
// two paths produce bit-identical fp32 scores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kPage = 64;          // C4 positions per KV page
constexpr int kVecBytes = 64;      // 128 E2M1 codes
constexpr int kVecScales = 4;      // one UE8M0 byte per 32 elements
constexpr int kTile = 256;         // positions per score block = 4 pages
constexpr int kTilePages = kTile / kPage;
constexpr int kRowsPerCta = 8;     // one query row per wave
constexpr int kCtaThreads = 64 * kRowsPerCta;

enum : int32_t { kRowDone = 0, kRowLong = 1 };
enum : int32_t { kCodeBadWindow = -1, kCodeBadPage = -2, kCodeUnderfill = -3, kCodeSelector = -4 };
enum : int32_t { kStBadWindow = 1, kStBadPage = 2, kStUnderfill = 4, kStSelector = 8 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// 64-bit selection key. "[FlyDSL][DSv4] Prototype FP4 MQA streaming TopK",
// Changes: a four-byte score radix followed by a four-byte logical-index radix
// gives score descending, index ascending; NaN below numbers; +0 above -0.
// Larger key = ranks first. Keys of distinct positions are distinct.
// ---------------------------------------------------------------------------
// order_bits of a score that is not NaN (a NaN's bits land in a wrong class here).
__device__ __forceinline__ uint32_t order_bits_finite(float s) {
  const uint32_t b = __float_as_uint(s);
  // non-negative (sign 0): set the top bit; negative (and -0): flip all bits
  return b ^ (static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t order_bits(float s) {
  return __builtin_isnan(s) ? 0u : order_bits_finite(s);   // every NaN: lowest class
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t pos) {
  return (static_cast<uint64_t>(order_bits(s)) << 32) | static_cast<uint32_t>(~pos);
}

__device__ __forceinline__ uint32_t key_pos(uint64_t k) { return ~static_cast<uint32_t>(k); }

__device__ __forceinline__ float key_score(uint64_t k) {
  const uint32_t o = static_cast<uint32_t>(k >> 32);
  if (o == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Float prefilter for "key > gate": every key above the gate has upper 32 bits
// >= those of the gate, and every score with such upper bits satisfies
// !(score < gate_floor(gate)) (non-negative classes compare as floats, larger
// bit patterns of negative scores are smaller magnitudes, -0 >= any negative
// float, and a NaN gate class admits everything, NaN included). So the float
// test is a superset of the exact key test and never drops a candidate.
__device__ __forceinline__ float gate_floor(uint64_t gate) {
  const uint32_t o = static_cast<uint32_t>(gate >> 32);
  if (o == 0u) return -__builtin_inff();
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Lanes l of a 64-position run starting at p0 with start <= p0 + l < end.
__device__ __forceinline__ uint64_t window_lanes(int p0, int start, int end) {
  const int lo = min(max(start - p0, 0), 64), hi = min(max(end - p0, 0), 64);
  const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
  return below_hi & ~below_lo;
}

// ---------------------------------------------------------------------------
// Wave helpers (wave64).
// ---------------------------------------------------------------------------

__device__ __forceinline__ int mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// Orders this wave's LDS accesses across lanes: waits for outstanding LDS
// operations and stops the compiler from moving memory accesses across it.
__device__ __forceinline__ void wave_lds_sync() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Cross-lane steps through DPP (gfx9 encodings), for code that runs with all 64
// lanes active. dpp_take<CTRL, ROWS>(id, v) returns, in the rows set in ROWS, the
// v of the lane that CTRL names, and `id` where that lane does not exist or the
// row is not in ROWS: row_shr:n (0x110 + n) takes lane l - n of the same row of
// 16, row_bcast:15 (0x142) lane 15 of the row before, row_bcast:31 (0x143)
// lane 31.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_take(uint32_t id, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

// Inclusive scan over lanes 0 .. this lane of an associative, commutative op
// with identity id (Kogge-Stone inside each row of 16, then the row totals).
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_take<0x111, 0xF>(id, v));
  v = op(v, dpp_take<0x112, 0xF>(id, v));
  v = op(v, dpp_take<0x114, 0xF>(id, v));
  v = op(v, dpp_take<0x118, 0xF>(id, v));
  v = op(v, dpp_take<0x142, 0xA>(id, v));   // rows 1 and 3 take the row before
  v = op(v, dpp_take<0x143, 0xC>(id, v));   // rows 2 and 3 take lanes 0 .. 31
  return v;
}

// Inclusive prefix sum over lanes (all lanes active).
__device__ __forceinline__ uint32_t wave_prefix_sum_dpp(uint32_t v) {
  return wave_scan_dpp(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}

// Lane 63's value, zero-extended (readlane returns a signed int).
__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// OR, AND and signed max of all 64 lanes, as a wave-uniform value (all lanes active).
__device__ __forceinline__ uint64_t wave_all_or64(uint64_t v) {
  auto op = [](uint32_t x, uint32_t y) { return x | y; };
  const uint32_t lo = wave_scan_dpp(static_cast<uint32_t>(v), 0u, op);
  const uint32_t hi = wave_scan_dpp(static_cast<uint32_t>(v >> 32), 0u, op);
  return (static_cast<uint64_t>(lane63(hi)) << 32) | lane63(lo);
}

__device__ __forceinline__ uint64_t wave_all_and64(uint64_t v) {
  auto op = [](uint32_t x, uint32_t y) { return x & y; };
  const uint32_t lo = wave_scan_dpp(static_cast<uint32_t>(v), ~0u, op);
  const uint32_t hi = wave_scan_dpp(static_cast<uint32_t>(v >> 32), ~0u, op);
  return (static_cast<uint64_t>(lane63(hi)) << 32) | lane63(lo);
}

__device__ __forceinline__ int wave_all_max_i32(int v) {
  const uint32_t m = wave_scan_dpp(static_cast<uint32_t>(v), static_cast<uint32_t>(INT_MIN),
                                   [](uint32_t x, uint32_t y) {
                                     return static_cast<uint32_t>(max(static_cast<int>(x), static_cast<int>(y)));
                                   });
  return __builtin_amdgcn_readlane(static_cast<int>(m), 63);
}

// One step of a 64-bit min over lanes: both halves of the neighbour's value move.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t min64_step(uint64_t v) {
  const uint64_t y = (static_cast<uint64_t>(dpp_take<CTRL, ROWS>(~0u, static_cast<uint32_t>(v >> 32))) << 32) |
                     dpp_take<CTRL, ROWS>(~0u, static_cast<uint32_t>(v));
  return v < y ? v : y;
}

// Smallest 64-bit value over the 64 lanes, wave-uniform (all lanes active), in
// the steps of wave_scan_dpp.
__device__ __forceinline__ uint64_t wave_all_min64(uint64_t v) {
  v = min64_step<0x111, 0xF>(v);
  v = min64_step<0x112, 0xF>(v);
  v = min64_step<0x114, 0xF>(v);
  v = min64_step<0x118, 0xF>(v);
  v = min64_step<0x142, 0xA>(v);
  v = min64_step<0x143, 0xC>(v);
  return (static_cast<uint64_t>(lane63(static_cast<uint32_t>(v >> 32))) << 32) | lane63(static_cast<uint32_t>(v));
}

// ---------------------------------------------------------------------------
// MXFP4 scaled MFMA, 32x32x64, both operands FP4 (format code 4).
// Lane l of an operand holds 32 consecutive elements (one UE8M0 block) of
// row/column l % 32, k-group l / 32; the scale byte of that block sits in the
// lane's scale register at the byte selected by OA / OB. The accumulator lane l,
// register v holds D[8*(v/4) + 4*(l/32) + v%4][l % 32].
// ---------------------------------------------------------------------------
template <int OA, int OB>
__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
  const v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, OA, sa, OB, sb);
}

// Query row operand, loop-invariant over the context scan. Head block hb holds
// heads 32*hb .. 32*hb+31. The contraction over D=128 is split into two MFMAs
// (kh = 0, 1); lane l feeds D-chunk 2*(l/32)+kh (16 bytes = 32 codes), so every
// lane reads 32 contiguous bytes of a head and of a key.
struct QRow {
  v4i a[2][2];      // [hb][kh]
  int scale;        // byte 2*hb+kh: UE8M0 of head 32*hb + l%32, chunk 2*(l/32)+kh
  float w[2][16];   // [hb][v]: weight of head 32*hb + 8*(v/4) + 4*(l/32) + v%4
};

__device__ __forceinline__ void load_qrow(QRow& r, const uint8_t* q_row, const uint8_t* qs_row,
                                          const float* w_row, int lane) {
  const int hl = lane & 31, g = lane >> 5;
  int sc = 0;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hb + hl;
    const v4i* src = reinterpret_cast<const v4i*>(q_row + head * kVecBytes + 32 * g);
    r.a[hb][0] = src[0];
    r.a[hb][1] = src[1];
    const uint8_t* s = qs_row + head * kVecScales + 2 * g;
    sc |= static_cast<int>(s[0]) << (8 * (2 * hb));
    sc |= static_cast<int>(s[1]) << (8 * (2 * hb + 1));
#pragma unroll
    for (int v = 0; v < 16; ++v) r.w[hb][v] = w_row[32 * hb + 8 * (v >> 2) + 4 * g + (v & 3)];
  }
  r.scale = sc;
}

// LDS image of one score block: position p's 64 code bytes at p*64, with its
// 16-byte chunk c stored at chunk slot c ^ chunk_swizzle(p).
// On gfx950 a wave's ds_read_b128 is served 16 lanes per LDS cycle across 64
// four-byte banks, and each cycle's 16 lanes hold, for every x < 16, one of
// lanes x and x + 16 of the wave half (bank-conflict counter on a read-pattern
// probe: a linear pattern takes 0 extra cycles per read, the former swizzle
// ((p >> 1) ^ (p >> 3)) & 3 took 4, no swizzle 12). The lane reading chunk c of
// position r (r < 32) hits bank quad 4 (r & 3) + (c ^ chunk_swizzle(r)) mod 16;
// the four lanes of a cycle that share r & 3 differ in bits 2..3 of r, so with
// the swizzle taken from those bits all 16 quads are distinct.
__device__ __forceinline__ int chunk_swizzle(int p) { return (p >> 2) & 3; }

__device__ __forceinline__ void load_keys32(const uint8_t* s_codes, const uint8_t* s_scales, int grp,
                                            int lane, v4i& b0, v4i& b1, int& ks) {
  const int p = 32 * grp + (lane & 31), g = lane >> 5;
  const int sw = chunk_swizzle(p);
  const uint8_t* base = s_codes + p * kVecBytes;
  b0 = *reinterpret_cast<const v4i*>(base + 16 * ((2 * g) ^ sw));
  b1 = *reinterpret_cast<const v4i*>(base + 16 * ((2 * g + 1) ^ sw));
  ks = *reinterpret_cast<const uint16_t*>(s_scales + p * kVecScales + 2 * g);
}

// ReLU on the fp32 bit pattern: negative values and -0 become +0 (one integer
// max, exact for every non-NaN input).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Partial indexer score of the 32 heads this lane holds for its position:
// sum over (hb, v) in a fixed order, starting at +0. One dependent chain: with
// four waves per SIMD the FMA latency is hidden by the other waves, and extra
// accumulators only add instructions.
__device__ __forceinline__ float head_partial(const QRow& r, const v16f& d0, const v16f& d1) {
  float p = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) p = __builtin_fmaf(r.w[0][v], relu_bits(d0[v]), p);
#pragma unroll
  for (int v = 0; v < 16; ++v) p = __builtin_fmaf(r.w[1][v], relu_bits(d1[v]), p);
  return p;
}

// fp32 indexer scores of 64 consecutive positions (positions 64*blk .. 64*blk+63
// of the LDS score block) for one query row. Lane l returns the score of
// position 64*blk + l. The summation order is the same for every position.
__device__ __forceinline__ float score64(const QRow& r, const uint8_t* s_codes,
                                         const uint8_t* s_scales, int blk, int lane) {
  float part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v4i b0, b1;
    int ks;
    load_keys32(s_codes, s_scales, 2 * blk + h, lane, b0, b1, ks);
    const v16f z = {};
    v16f d0 = mfma_fp4<0, 0>(r.a[0][0], b0, z, r.scale, ks);
    d0 = mfma_fp4<1, 1>(r.a[0][1], b1, d0, r.scale, ks);
    v16f d1 = mfma_fp4<2, 0>(r.a[1][0], b0, z, r.scale, ks);
    d1 = mfma_fp4<3, 1>(r.a[1][1], b1, d1, r.scale, ks);
    part[h] = head_partial(r, d0, d1);
  }
  // lanes l and l+32 hold complementary heads of one position: swap halves so
  // that lane l < 32 sums position l of group 0 and lane l >= 32 position l of
  // group 1 (= position 64*blk + l).
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                   __float_as_uint(part[1]), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// ---------------------------------------------------------------------------
// Scoring of one 256-position score block for one row, as 8 groups of 32
// positions (4 MFMAs each, then the ReLU + head-weighted epilogue). On gfx950 a
// SIMD runs MFMA and VALU work largely one after the other (measured: one MFMA
// wave beside two fp32-FMA waves hides about 15% of the shorter work), so there
// is little to gain from keeping two groups in flight inside a wave; the
// register budget goes to occupancy instead (four waves per SIMD hide the MFMA
// and LDS latencies).
// The swizzled LDS chunk offsets depend only on lane % 32, so every B-operand
// address is a per-lane base plus a compile-time offset. Same arithmetic, in the
// same order, as score64(): the scores are bit-identical.
// emit(blk, score) is called for blk = 0..3 with lane l holding position
// 64*blk + l of the block.
// ---------------------------------------------------------------------------
struct LaneOffsets {
  int code0, code1, scale;
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  const int r = lane & 31, g = lane >> 5;
  const int sw = chunk_swizzle(r);   // equal to chunk_swizzle(32 * grp + r) for every grp
  return LaneOffsets{r * kVecBytes + 16 * ((2 * g) ^ sw), r * kVecBytes + 16 * ((2 * g + 1) ^ sw),
                     r * kVecScales + 2 * g};
}

struct GroupAcc {
  v16f d0, d1;
};

template <int GRP>
__device__ __forceinline__ GroupAcc mfma_group(const QRow& r, const uint8_t* s_codes, const uint8_t* s_scales,
                                               const LaneOffsets& o) {
  const v4i b0 = *reinterpret_cast<const v4i*>(s_codes + o.code0 + GRP * 32 * kVecBytes);
  const v4i b1 = *reinterpret_cast<const v4i*>(s_codes + o.code1 + GRP * 32 * kVecBytes);
  const int ks = *reinterpret_cast<const uint16_t*>(s_scales + o.scale + GRP * 32 * kVecScales);
  const v16f z = {};
  GroupAcc acc;
  // the wave issues its group's four MFMAs at raised priority, so the SIMD's
  // arbiter keeps them together rather than interleaving other waves' epilogue
  // instructions between them (measured: scan kernel about 1% shorter)
  __builtin_amdgcn_s_setprio(1);
  acc.d0 = mfma_fp4<0, 0>(r.a[0][0], b0, z, r.scale, ks);
  acc.d0 = mfma_fp4<1, 1>(r.a[0][1], b1, acc.d0, r.scale, ks);
  acc.d1 = mfma_fp4<2, 0>(r.a[1][0], b0, z, r.scale, ks);
  acc.d1 = mfma_fp4<3, 1>(r.a[1][1], b1, acc.d1, r.scale, ks);
  __builtin_amdgcn_s_setprio(0);
  return acc;
}

// Lanes l and l+32 hold complementary heads of one position; swapping halves
// gives lane l < 32 position l of group x and lane l >= 32 position l of group y.
__device__ __forceinline__ float combine_halves(float x, float y) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int G, class Emit>
__device__ __forceinline__ void score_groups(const QRow& r, const uint8_t* s_codes, const uint8_t* s_scales,
                                             const LaneOffsets& o, float& even, Emit& emit) {
  if constexpr (G < 8) {
    const GroupAcc a = mfma_group<G>(r, s_codes, s_scales, o);
    const float p = head_partial(r, a.d0, a.d1);
    if constexpr (G % 2 == 0) {
      even = p;
    } else {
      emit(G / 2, combine_halves(even, p));
    }
    score_groups<G + 1>(r, s_codes, s_scales, o, even, emit);
  }
}

template <class Emit>
__device__ __forceinline__ void score_block(const QRow& r, const uint8_t* s_codes, const uint8_t* s_scales,
                                            const LaneOffsets& o, Emit&& emit) {
  float even = 0.0f;
  score_groups<0>(r, s_codes, s_scales, o, even, emit);
}

// ---------------------------------------------------------------------------
// Wave-level exact selection over a pool of unique keys in LDS.
// Radix select on 8-bit digits starting at the highest bit where the keys
// differ, so that the first histogram already spreads the candidates.
// Returns T such that exactly k of the n keys are >= T, moves the keys >= T to
// the front of the pool and returns their number in .kept (== k unless the keys
// were not unique, which callers report as a selector failure). Needs 1 <= k < n.
// ---------------------------------------------------------------------------
struct Selected {
  uint64_t T;
  int kept;
};

__device__ __noinline__ Selected wave_select_compact(uint64_t* pool, int n, int k, uint32_t* hist,
                                                     int lane) {
  uint64_t vor = 0, vand = ~0ull;
  for (int i = lane; i < n; i += 64) {
    const uint64_t x = pool[i];
    vor |= x;
    vand &= x;
  }
  vor = wave_all_or64(vor);
  vand = wave_all_and64(vand);
  if (vor == vand) return Selected{vand, -1};   // all keys equal: they were not unique
  int hb = 63 - __clzll(static_cast<long long>(vor ^ vand));
  uint64_t pmask = ~((2ull << hb) - 1ull);       // bits above hb are common
  uint64_t prefix = vand & pmask;
  uint32_t krem = static_cast<uint32_t>(k);
  int shift;
  for (;;) {
    shift = hb >= 7 ? hb - 7 : 0;
    for (int b = lane; b < 256; b += 64) hist[b] = 0u;
    wave_lds_sync();
    for (int i = lane; i < n; i += 64) {
      const uint64_t x = pool[i];
      if ((x & pmask) == prefix) atomicAdd(&hist[static_cast<uint32_t>(x >> shift) & 255u], 1u);
    }
    wave_lds_sync();
    const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
    const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
    const uint32_t lsum = c0 + c1 + c2 + c3;
    const uint32_t pre = wave_prefix_sum_dpp(lsum);
    const uint32_t s3 = lane63(pre) - pre + c3, s2 = s3 + c2, s1 = s2 + c1, s0 = s1 + c0;
    const int local = s3 >= krem ? 4 * lane + 3
                    : s2 >= krem ? 4 * lane + 2
                    : s1 >= krem ? 4 * lane + 1
                    : s0 >= krem ? 4 * lane : -1;
    const int dstar = wave_all_max_i32(local);
    if (dstar < 0) return Selected{prefix, -1};  // fewer matching keys than krem
    const int sel = dstar & 3;
    const uint32_t my_suffix = sel == 0 ? s0 : sel == 1 ? s1 : sel == 2 ? s2 : s3;
    const uint32_t suffix_d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(my_suffix), dstar >> 2));
    const uint32_t cnt_d = hist[dstar];
    krem -= suffix_d - cnt_d;
    prefix |= static_cast<uint64_t>(dstar) << shift;
    pmask |= 255ull << shift;
    wave_lds_sync();
    if (cnt_d == krem || shift == 0) break;
    hb = shift - 1;
  }
  const uint64_t T = prefix;
  int out = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const uint64_t x = i < n ? pool[i] : 0ull;
    const bool keep = i < n && x >= T;
    const uint64_t m = __ballot(keep);
    wave_lds_sync();
    if (keep) pool[out + mbcnt64(m)] = x;
    out += __popcll(m);
  }
  wave_lds_sync();
  return Selected{T, out};
}

}  // namespace mqa
