// Measurement library beside the operator (libmqa_fp4_probe.so, declared in
// include/mqa_fp4_probe.h): synthetic loops that measure, in shader cycles per
// SIMD, the issue rates the scan kernel is built from -- MXFP4 MFMAs, fp32 VALU
// operations, both side by side on one SIMD -- and the LDS read pattern of the
// score-block image. No operator work runs here.
#include "mqa_device.h"
#include "mqa_fp4_topk.h"
#include "mqa_fp4_probe.h"

#include <cstring>

namespace mqa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// One block per CU: the issue probe asks for more LDS than half a CU holds.
constexpr int kIssueLdsBytes = 96 * 1024;
constexpr int kLdsProbeThreads = 512;
// The valu-waves probe: a CU's LDS, and the most waves per SIMD it asks for
// (the FMA loop's register count lets six waves share a SIMD).
constexpr int kCuLdsBytes = 160 * 1024;
constexpr int kValuProbeMaxWaves = 6;

// Four independent accumulator chains per wave, one 32x32x64 FP4 MFMA each per
// iteration. Codes and scales are arbitrary finite values.
__device__ __noinline__ float mfma_loop(int iters, int l) {
  const v4i a = {l * 0x01010101, l * 0x03030303, l * 0x05050505, l * 0x07070707};
  const v4i b = a ^ v4i{0x55555555, 0x33333333, 0x0F0F0F0F, 0x11111111};
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

// The same FLOPs per iteration as eight 16x16x128 MXFP4 MFMAs (eight chains
// of four accumulator registers instead of four chains of sixteen).
__device__ __noinline__ float mfma16_loop(int iters, int l) {
  const v8i a = {l * 0x01010101, l * 0x03030303, l * 0x05050505, l * 0x07070707, 0, 0, 0, 0};
  const v8i b = a ^ v8i{0x55555555, 0x33333333, 0x0F0F0F0F, 0x11111111, 0, 0, 0, 0};
  const int sc = 0x7F7F7F7F;
  v4f c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 4, 4, 0, sc, 0, sc);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += c[i][i & 3];
  return s;
}

// Sixteen independent chains, 64 fp32 FMAs per lane per iteration.
__device__ __noinline__ float fma_loop(int iters, int l) {
  float w[16], x[16], p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w[i] = 1.0f + 0x1p-20f * static_cast<float>(l + i);
    x[i] = 0.5f - 0x1p-21f * static_cast<float>(l * i);
    p[i] = 0.0f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_fmaf(w[i], x[(i + r) & 15], p[i]);
    __asm__ __volatile__("" : "+v"(x[0]), "+v"(x[5]), "+v"(x[10]));   // no hoisting across iterations
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += p[i];
  return s;
}

__global__ void __launch_bounds__(1024) issue_probe_kernel(int n_mfma, int shape16, int iters,
                                                           uint64_t* __restrict__ rec, float* __restrict__ sink) {
  extern __shared__ char s_reserve[];   // only reserved: one block per CU
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  if (threadIdx.x == 0) s_reserve[0] = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const float v = (w >> 2) < n_mfma ? (shape16 ? mfma16_loop(iters, l) : mfma_loop(iters, l)) : fma_loop(iters, l);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = v;
  if (l == 0) {
    uint64_t* o = rec + (static_cast<size_t>(blockIdx.x) * nw + w) * 3;
    o[0] = t0;
    o[1] = t1;
    // HW_ID (wave slot, SIMD, CU, shader engine) and XCC_ID hardware registers
    o[2] = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 4))) |
           (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 20))) << 32);
  }
}

// Blocks of four waves (one per SIMD) that only run the FMA loop; the caller's
// LDS request caps how many blocks share a CU, and so the waves per SIMD.
__global__ void __launch_bounds__(256) valu_waves_probe_kernel(int iters, uint64_t* __restrict__ rec,
                                                               float* __restrict__ sink) {
  extern __shared__ char s_reserve[];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (threadIdx.x == 0) s_reserve[0] = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const float v = fma_loop(iters, l);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = v;
  if (l == 0) {
    uint64_t* o = rec + (static_cast<size_t>(blockIdx.x) * 4 + w) * 3;
    o[0] = t0;
    o[1] = t1;
    o[2] = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 4))) |
           (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 20))) << 32);
  }
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

// Offsets stay inside a group: 0: 31*64 + 48 + 16 = 2048; 1: 1024 + 63*16 + 16
// = 2048; 2: 31*64 + 32 + 16 + 16 = 2048.
__global__ void __launch_bounds__(kLdsProbeThreads) lds_probe_kernel(int pattern, int iters, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t s_img[kProbeImageBytes];
  const int l = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kProbeImageBytes / 4; i += kLdsProbeThreads)
    reinterpret_cast<uint32_t*>(s_img)[i] = static_cast<uint32_t>(i) * 2654435761u;
  __syncthreads();
  int o0, o1;
  if (pattern == 0) {
    const LaneOffsets lo = lane_offsets(l);
    o0 = lo.code0;
    o1 = lo.code1;
  } else if (pattern == 1) {
    o0 = 16 * l;
    o1 = 1024 + 16 * l;
  } else {
    o0 = (l & 31) * kVecBytes + 32 * (l >> 5);
    o1 = o0 + 16;
  }
  out[static_cast<size_t>(blockIdx.x) * kLdsProbeThreads + threadIdx.x] = lds_loop(s_img, o0, o1, iters);
}

// ---- host checks ---------------------------------------------------------------

// The stream's device, made current for the call; restored on scope exit.
struct Guard {
  int saved = -1, dev = -1;
  bool changed = false;
  int32_t enter(hipStream_t st) {
    if (hipGetDevice(&saved) != hipSuccess) return MQA_ERR_HIP;
    dev = saved;
    if (st != nullptr && hipStreamGetDevice(st, &dev) != hipSuccess) {
      (void)hipGetLastError();
      return MQA_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MQA_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MQA_ERR_DEVICE;
    cus = prop.multiProcessorCount;
    if (dev != saved) {
      if (hipSetDevice(dev) != hipSuccess) return MQA_ERR_HIP;
      changed = true;
    }
    return MQA_OK;
  }
  ~Guard() {
    if (changed) (void)hipSetDevice(saved);
  }
  int cus = 0;
};

// Device (or managed) memory of device `dev`, with the given alignment.
int32_t check_out(const void* p, uintptr_t align, int dev) {
  if (p == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(p) % align) return MQA_ERR_MISALIGNED;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return MQA_ERR_DEVICE;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return MQA_ERR_DEVICE;
  return attr.device == dev ? MQA_OK : MQA_ERR_DEVICE;
}

int32_t launched() { return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP; }

}  // namespace
}  // namespace mqa

extern "C" {

int32_t mqa_probe_blocks(void* stream) {
  mqa::Guard g;
  const int32_t rc = g.enter(static_cast<hipStream_t>(stream));
  return rc == MQA_OK ? g.cus : rc;
}

namespace {
int32_t issue_probe(int32_t n_mfma_waves, int32_t n_valu_waves, int shape16, int32_t iters, uint64_t* rec, float* sink,
                    void* stream) {
  if (n_mfma_waves < 0 || n_valu_waves < 0 || n_mfma_waves + n_valu_waves < 1 || n_mfma_waves + n_valu_waves > 4 ||
      iters < 1)
    return MQA_ERR_BAD_SIZE;
  if (rec == nullptr || sink == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(rec) % 8 || reinterpret_cast<uintptr_t>(sink) % 4) return MQA_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  mqa::Guard g;
  int32_t rc = g.enter(st);
  if (rc != MQA_OK) return rc;
  if ((rc = mqa::check_out(rec, 8, g.dev)) != MQA_OK || (rc = mqa::check_out(sink, 4, g.dev)) != MQA_OK) return rc;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(mqa::issue_probe_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, mqa::kIssueLdsBytes) != hipSuccess) {
    (void)hipGetLastError();
    return MQA_ERR_HIP;
  }
  const unsigned threads = 256u * static_cast<unsigned>(n_mfma_waves + n_valu_waves);
  mqa::issue_probe_kernel<<<dim3(static_cast<unsigned>(g.cus)), dim3(threads), mqa::kIssueLdsBytes, st>>>(
      n_mfma_waves, shape16, iters, rec, sink);
  return mqa::launched();
}
}  // namespace

int32_t mqa_probe_issue(int32_t n_mfma_waves, int32_t n_valu_waves, int32_t iters, uint64_t* rec, float* sink,
                        void* stream) {
  return issue_probe(n_mfma_waves, n_valu_waves, 0, iters, rec, sink, stream);
}

int32_t mqa_probe_issue16(int32_t n_mfma_waves, int32_t n_valu_waves, int32_t iters, uint64_t* rec, float* sink,
                          void* stream) {
  return issue_probe(n_mfma_waves, n_valu_waves, 1, iters, rec, sink, stream);
}

int32_t mqa_probe_valu_waves(int32_t waves_per_simd, int32_t iters, uint64_t* rec, float* sink, void* stream) {
  if (waves_per_simd < 1 || waves_per_simd > mqa::kValuProbeMaxWaves || iters < 1) return MQA_ERR_BAD_SIZE;
  if (rec == nullptr || sink == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(rec) % 8 || reinterpret_cast<uintptr_t>(sink) % 4) return MQA_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  mqa::Guard g;
  int32_t rc = g.enter(st);
  if (rc != MQA_OK) return rc;
  if ((rc = mqa::check_out(rec, 8, g.dev)) != MQA_OK || (rc = mqa::check_out(sink, 4, g.dev)) != MQA_OK) return rc;
  // k blocks of this size fit a CU's 160 KB of LDS, k + 1 do not
  const int lds = mqa::kCuLdsBytes / waves_per_simd - 1024;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(mqa::valu_waves_probe_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
    (void)hipGetLastError();
    return MQA_ERR_HIP;
  }
  mqa::valu_waves_probe_kernel<<<dim3(static_cast<unsigned>(g.cus * waves_per_simd)), dim3(256), lds, st>>>(
      iters, rec, sink);
  return mqa::launched();
}

int32_t mqa_probe_lds(int32_t pattern, float* out, int32_t blocks, int32_t iters, void* stream) {
  if (pattern < 0 || pattern > 2 || blocks <= 0 || iters <= 0) return MQA_ERR_BAD_SIZE;
  if (out == nullptr) return MQA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return MQA_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  mqa::Guard g;
  int32_t rc = g.enter(st);
  if (rc != MQA_OK) return rc;
  if ((rc = mqa::check_out(out, 4, g.dev)) != MQA_OK) return rc;
  mqa::lds_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(mqa::kLdsProbeThreads), 0, st>>>(pattern, iters,
                                                                                                      out);
  return mqa::launched();
}

}  // extern "C"
