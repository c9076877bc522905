// Peak probes: a pure MXFP4 MFMA loop, a pure fp32 FMA loop and the two side by
// side on every SIMD, launched on the caller's stream so that the sustained
// rates, and whether a SIMD overlaps the two kinds of work, can be measured
// under the same clocks and power state the operator runs in (MI355X's
// published peaks are quoted at 2.4 GHz; the shader clock is lower under dense
// MFMA load). Three more kinds time LDS read patterns, so that the bank
// behaviour of the score-block image can be checked on the device.
#include "mqa_device.h"
#include "mqa_fp4_topk.h"

namespace mqa {
namespace {

constexpr int kProbeThreads = 512;

// Four independent accumulator chains per wave, one 32x32x64 FP4 MFMA each per
// iteration (2*32*32*64 FLOP). Codes and scales are arbitrary finite values.
__device__ __noinline__ float mfma_loop(int iters, int l) {
  const v4i a = {l * 0x01010101, l * 0x03030303, l * 0x05050505, l * 0x07070707};
  v4i b = a ^ v4i{0x55555555, 0x33333333, 0x0F0F0F0F, 0x11111111};
  const int sc = 0x7F7F7F7F;
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma_fp4<0, 0>(a, b, c0, sc, sc);
    c1 = mfma_fp4<0, 0>(a, b, c1, sc, sc);
    c2 = mfma_fp4<0, 0>(a, b, c2, sc, sc);
    c3 = mfma_fp4<0, 0>(a, b, c3, sc, sc);
  }
  return c0[0] + c1[1] + c2[2] + c3[3];
}

// Eight independent chains, 64 fp32 FMAs per lane per iteration.
__device__ __noinline__ float fma_loop(int iters, int l) {
  float w[16], x[16], p[8];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w[i] = 1.0f + 0x1p-20f * static_cast<float>(l + i);
    x[i] = 0.5f - 0x1p-21f * static_cast<float>(l * i);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) p[c] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i & 7] = __builtin_fmaf(w[i], x[(i + r) & 15], p[i & 7]);
    x[0] = __builtin_fmaf(p[0], 0x1p-100f, x[0]);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += p[c];
  return s;
}

// Two 16-byte LDS reads per lane per iteration from one of the eight 32-position
// groups of a score-block image (group it % 8, 2 KB apart); inlined so that the
// reads stay ds_read_b128 on the LDS pointer.
constexpr int kProbeImageBytes = 8 * 32 * kVecBytes;
__device__ __forceinline__ float lds_loop(const uint8_t* img, int o0, int o1, int iters) {
  v4i acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    const uint8_t* g = img + (it & 7) * (32 * kVecBytes);
    const v4i x = *reinterpret_cast<const v4i*>(g + o0);
    const v4i y = *reinterpret_cast<const v4i*>(g + o1);
    acc ^= x + y;
    __asm__ __volatile__("" ::: "memory");   // no reuse of the loads across iterations
  }
  return static_cast<float>(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// kind 0: every wave runs the MFMA loop; 1: every wave the FMA loop; 2: waves
// 0-3 of the block the MFMA loop and waves 4-7 the FMA loop. Wave w of a block
// runs on SIMD w % 4, so with kind 2 each SIMD holds one wave of each: its time
// against half of kind 0's plus half of kind 1's shows whether the SIMD runs
// MFMA and VALU work at the same time.
__global__ void __launch_bounds__(kProbeThreads) peak_probe_kernel(int kind, int iters, float* __restrict__ out) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool mfma = kind == 0 || (kind == 2 && w < 4);
  const float v = mfma ? mfma_loop(iters, l) : fma_loop(iters, l);
  out[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = v;
}

// kinds 3-5: LDS reads of a score-block image: 3 the scan's own operand reads
// (lane_offsets, i.e. with the chunk swizzle), 4 a linear pattern (lane l reads
// bytes 16 l .. 16 l + 15 of each 1 KB half of a group, free of bank conflicts
// under any lane grouping), 5 the image without a swizzle. Kind 3 taking the
// time of kind 4 means the image is read without bank conflicts.
// Offsets stay inside a group: 3: 31*64 + 48 + 16 = 2048; 4: 1024 + 63*16 + 16
// = 2048; 5: 31*64 + 32 + 16 + 16 = 2048.
__global__ void __launch_bounds__(kProbeThreads) lds_probe_kernel(int kind, int iters, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t s_img[kProbeImageBytes];
  const int l = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kProbeImageBytes / 4; i += kProbeThreads)
    reinterpret_cast<uint32_t*>(s_img)[i] = static_cast<uint32_t>(i) * 2654435761u;
  __syncthreads();
  int o0, o1;
  if (kind == 3) {
    const LaneOffsets lo = lane_offsets(l);
    o0 = lo.code0;
    o1 = lo.code1;
  } else if (kind == 4) {
    o0 = 16 * l;
    o1 = 1024 + 16 * l;
  } else {
    o0 = (l & 31) * kVecBytes + 32 * (l >> 5);
    o1 = o0 + 16;
  }
  out[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = lds_loop(s_img, o0, o1, iters);
}

}  // namespace
}  // namespace mqa

extern "C" int32_t mqa_fp4_peak_probe(int32_t kind, float* out, int32_t blocks, int32_t iters, void* stream) {
  if (kind < 0 || kind > 5 || blocks <= 0 || iters <= 0) return MQA_ERR_BAD_SIZE;
  if (out == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return MQA_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind <= 2)
    mqa::peak_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(mqa::kProbeThreads), 0, st>>>(kind, iters, out);
  else
    mqa::lds_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(mqa::kProbeThreads), 0, st>>>(kind, iters, out);
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}
