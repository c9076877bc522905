// MXFP4 quantisation and the C4 paged key-cache writer: the producers of the
// indexer's FP4 inputs (gfx950).
//
// The pages name the payload only ("[FlyDSL][DSv4] Prototype FP4 MQA streaming
// TopK", Scope: FP4 E2M1 payload with UE8M0 scales, page size 64). The
// conversion follows the OCP Microscaling Formats (MX) v1.0 rule for turning a
// vector of scalars into an MX block, read for E2M1 elements and a UE8M0 scale:
// shared exponent floor(log2 max|v|) - 2 (2 = E2M1's largest exponent), every
// element v / 2^shared rounded to the nearest E2M1 value with ties to the even
// mantissa bit, saturating at 6, sign kept. Where the rule leaves the encoding
// open: the scale byte is clamped to [0, 254], an all-zero block gets byte 0,
// a block with a NaN or infinite element gets byte 0xFF and zero codes.
//
// HBM-bound: 512 bytes read and 68 written per 128-element vector. One wave
// converts two vectors per step with 16-byte loads (lane l: vector l / 32,
// elements 4 (l % 32) .. +3; eight lanes per 32-element block), a three-step
// lane butterfly for the block maximum, and 16-bit code stores.
#include "mqa_device.h"
#include "mqa_launch.h"

namespace mqa {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// E2M1 magnitude code (0..7) of a >= 0, already divided by the block scale:
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, above 6
// saturating. The midpoints 0.25, 1.25, 2.5 and 5 lie above an even code (they
// round down, hence ">"); 0.75, 1.75 and 3.5 lie below one (they round up, ">=").
__device__ __forceinline__ uint32_t e2m1_magnitude(float a) {
  return static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) + static_cast<uint32_t>(a > 1.25f) +
         static_cast<uint32_t>(a >= 1.75f) + static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
         static_cast<uint32_t>(a > 5.0f);
}

__device__ __forceinline__ uint32_t e2m1_code(float v, float inv_scale) {
  const float t = v * inv_scale;                 // exact: a power-of-two scaling
  return e2m1_magnitude(__builtin_fabsf(t)) | ((__float_as_uint(t) >> 31) << 3);
}

// Pairs of vectors per wave per step: four 16-byte loads in flight per lane
// (measured: 1, 2, 4, 8 give 5.02, 5.28, 5.29, 4.81 TB/s back to back, against
// 5.42 TB/s for a plain device copy of the same bytes).
constexpr int kQuantUnroll = 4;

// Converts one pair's lane data (vector v = 2 * pair + lane / 32) and stores it.
// Vector v goes to row v of codes [.., 64] / scales [.., 4], or (cache writer)
// to the physical slot of logical position positions[v]; vectors with an
// invalid position or page are not written and set a status bit.
__device__ __forceinline__ void quantize_store(float4 e, int64_t v, bool live, int q, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, const int32_t* __restrict__ positions,
                                               const int32_t* __restrict__ page_table, int64_t P_log,
                                               int64_t P_phys, int32_t* __restrict__ status) {
  // block maximum of |x| on the bit patterns: finite values keep their order,
  // infinities and NaNs sort above every finite value
  uint32_t m = max(max(abs_bits(e.x), abs_bits(e.y)), max(abs_bits(e.z), abs_bits(e.w)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1, 64)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 2, 64)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 4, 64)));
  const bool bad = m >= 0x7F800000u;
  // biased exponent field of the maximum = floor(log2 max) + 127 for normal
  // numbers; byte = floor(log2 max) - 2 + 127, below zero (tiny, subnormal or
  // zero blocks) clamped to 0; the largest finite float gives 252
  const int byte = bad ? 0xFF : max(0, static_cast<int>(m >> 23) - 2);
  const float inv = __uint_as_float(static_cast<uint32_t>(254 - (bad ? 0 : byte)) << 23);   // 2^(127 - byte)
  uint32_t packed = 0;
  if (!bad)
    packed = e2m1_code(e.x, inv) | (e2m1_code(e.y, inv) << 4) | (e2m1_code(e.z, inv) << 8) |
             (e2m1_code(e.w, inv) << 12);
  if (!live) return;
  int64_t row = v;
  if (positions != nullptr) {
    const int32_t p = positions[v];
    int code = 0;
    if (p < 0 || p >= kPage * P_log) {
      code = kStBadWindow;
    } else {
      const int32_t pg = page_table[p / kPage];
      if (pg < 0 || pg >= P_phys) code = kStBadPage;
      else row = static_cast<int64_t>(pg) * kPage + p % kPage;
    }
    if (code) {
      if (q == 0) atomicOr(status, code);
      return;
    }
  }
  reinterpret_cast<uint16_t*>(codes + row * kVecBytes)[q] = static_cast<uint16_t>(packed);
  if ((q & 7) == 0) scales[row * kVecScales + (q >> 3)] = static_cast<uint8_t>(byte);
}

__global__ void __launch_bounds__(kQuantThreads) mx_quantize_kernel(
    const float* __restrict__ x, int64_t n_vec, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ page_table, int64_t P_log, int64_t P_phys,
    int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63, half = lane >> 5, q = lane & 31;
  const int64_t n_pairs = (n_vec + 1) / 2;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kQuantThreads / 64);
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * (kQuantThreads / 64) + (threadIdx.x >> 6);
  // step s of a wave covers pairs w0 + (s * kQuantUnroll + u) * waves, u < kQuantUnroll
  for (int64_t base = w0; base < n_pairs; base += waves * kQuantUnroll) {
    float4 e[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t v = 2 * (base + u * waves) + half;
      e[u] = v < n_vec ? reinterpret_cast<const float4*>(x + v * kDim)[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t v = 2 * (base + u * waves) + half;
      quantize_store(e[u], v, v < n_vec, q, codes, scales, positions, page_table, P_log, P_phys, status);
    }
  }
}

}  // namespace

hipError_t launch_mx_quantize(const float* x, int64_t n_vec, uint8_t* codes, uint8_t* scales,
                              const int32_t* positions, const int32_t* page_table, int64_t P_log, int64_t P_phys,
                              int cus, hipStream_t st) {
  if (n_vec <= 0) return hipSuccess;
  int32_t* status = status_word();
  if (status == nullptr) return hipErrorInvalidSymbol;
  const int64_t waves_needed = ((n_vec + 1) / 2 + kQuantUnroll - 1) / kQuantUnroll;
  const int64_t per_block = kQuantThreads / 64;
  int64_t blocks = (waves_needed + per_block - 1) / per_block;
  const int64_t cap = static_cast<int64_t>(cus) * 8;   // grid-stride beyond 8 blocks per CU
  if (blocks > cap) blocks = cap;
  mx_quantize_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kQuantThreads), 0, st>>>(
      x, n_vec, codes, scales, positions, page_table, P_log, P_phys, status);
  return hipGetLastError();
}

}  // namespace mqa
