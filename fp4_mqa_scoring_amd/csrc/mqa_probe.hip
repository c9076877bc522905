// Peak probes: a pure MXFP4 MFMA loop, a pure fp32 FMA loop and the two side by
// side on every SIMD, launched on the caller's stream so that the sustained
// rates, and whether a SIMD overlaps the two kinds of work, can be measured
// under the same clocks and power state the operator runs in (MI355X's
// published peaks are quoted at 2.4 GHz; the shader clock is lower under dense
// MFMA load).
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

}  // namespace
}  // namespace mqa

extern "C" int32_t mqa_fp4_peak_probe(int32_t kind, float* out, int32_t blocks, int32_t iters, void* stream) {
  if (kind < 0 || kind > 2 || blocks <= 0 || iters <= 0) return MQA_ERR_BAD_SIZE;
  if (out == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return MQA_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  mqa::peak_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(mqa::kProbeThreads), 0, st>>>(kind, iters, out);
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}
