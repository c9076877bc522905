// Host side of the C ABI declared in include/mqa_fp4_topk.h.
//
// Fail-closed host checks (PR 5309 "[FlyDSL] Add FP4 LiteTopK prefill
// operator", Implementation: explicit supported-K contract, fail closed,
// preserve caller device/stream ownership, 64-bit addressing), graph-capture
// rejection (PR 5282, Scope), launch planning and stream-ordered scratch.
#include "mqa_fp4_topk.h"
#include "mqa_launch.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

namespace {

using mqa::PathArgs;

constexpr int kMaxDevices = 64;
constexpr int kRowsPerCta = 8;       // must match the kernels' row tile
constexpr int kMaxAutoSplits = 64;

struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int cus = 0;
  bool pool_ready = false;
};

std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

// Probes (once) whether `dev` is a gfx950 and how many CUs it has.
int32_t device_info(int dev, DeviceInfo* out) {
  if (dev < 0 || dev >= kMaxDevices) return MQA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return MQA_ERR_HIP;
    }
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.probed = true;
  }
  if (!d.pool_ready && d.gfx950) {
    // keep freed scratch in the device's default pool instead of returning it
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t thr = ~0ull;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    (void)hipGetLastError();
    d.pool_ready = true;
  }
  *out = d;
  return d.gfx950 ? MQA_OK : MQA_ERR_DEVICE;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int saved = -1;
  bool changed = false;
  int32_t enter(int dev) {
    if (hipGetDevice(&saved) != hipSuccess) {
      (void)hipGetLastError();
      return MQA_ERR_HIP;
    }
    if (saved != dev) {
      if (hipSetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return MQA_ERR_HIP;
      }
      changed = true;
    }
    return MQA_OK;
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(saved);
  }
};

int32_t stream_device(hipStream_t st, int* dev) {
  const bool ok = (st == nullptr ? hipGetDevice(dev) : hipStreamGetDevice(st, dev)) == hipSuccess;
  if (!ok) (void)hipGetLastError();   // reported through the return code only
  return ok ? MQA_OK : st == nullptr ? MQA_ERR_HIP : MQA_ERR_DEVICE;
}

// A non-null pointer must be device (or managed) memory of device `dev`.
int32_t check_ptr_device(const void* p, int dev) {
  if (p == nullptr) return MQA_OK;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return MQA_ERR_DEVICE;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return MQA_ERR_DEVICE;
  if (attr.device != dev) return MQA_ERR_DEVICE;
  return MQA_OK;
}

struct PtrSpec {
  const void* p;
  bool required;
  uintptr_t align;
};

// Host-only pointer checks (no HIP call): presence and alignment.
int32_t check_ptrs_host(const PtrSpec* specs, int n) {
  for (int i = 0; i < n; ++i)
    if (specs[i].required && specs[i].p == nullptr) return MQA_ERR_NULL_POINTER;
  for (int i = 0; i < n; ++i)
    if (specs[i].p && reinterpret_cast<uintptr_t>(specs[i].p) % specs[i].align) return MQA_ERR_MISALIGNED;
  return MQA_OK;
}

int32_t check_ptrs_device(const PtrSpec* specs, int n, int dev) {
  for (int i = 0; i < n; ++i) {
    const int32_t rc = check_ptr_device(specs[i].p, dev);
    if (rc != MQA_OK) return rc;
  }
  return MQA_OK;
}

int32_t check_sizes(int64_t Q, int64_t P_phys, int64_t P_log) {
  if (Q < 0 || P_phys < 0 || P_log < 0) return MQA_ERR_BAD_SIZE;
  if (Q > 0x7FFFFFFFll) return MQA_ERR_BAD_SIZE;                 // grid size, row index
  if (P_log > (0x7FFFFFFFll - 512) / 64) return MQA_ERR_BAD_SIZE; // positions in int32
  if (P_phys > 0x7FFFFFFFll / 64) return MQA_ERR_BAD_SIZE;        // slots in int32
  return MQA_OK;
}

int32_t check_capture(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return MQA_ERR_HIP;
  }
  return cs == hipStreamCaptureStatusNone ? MQA_OK : MQA_ERR_CAPTURING;
}

// Context splits per row tile: enough CTAs for `per_cu` of them per CU.
int32_t auto_splits(int64_t Q, int cus, int per_cu = 2) {
  const int64_t tiles = (Q + kRowsPerCta - 1) / kRowsPerCta;
  if (tiles <= 0) return 1;
  int64_t s = (per_cu * static_cast<int64_t>(cus) + tiles - 1) / tiles;
  if (s < 1) s = 1;
  if (s > kMaxAutoSplits) s = kMaxAutoSplits;
  return static_cast<int32_t>(s);
}

// Context splits of the gated scan: as auto_splits, and at least
// min(8, blocks / 64) for a context of `blocks` 256-position blocks. Shorter
// CTAs end the launch more evenly: at Q = 8192, C4 = 196,608 (1,024 row tiles,
// one split by the CU count alone) 1 / 2 / 4 / 8 / 16 splits took 7.50 / 7.38 /
// 7.32 / 7.32 / 7.32 ms (scan kernel, same session), outputs identical; the
// calibration keeps auto_splits (its combine launch costs more than it saves
// once the row tiles fill the CUs). Where the row tiles are few, the count is
// raised to give four (split, tile) items per resident CTA (two per CU), the
// form in which the scan takes its items from a device-wide counter, as long
// as every split keeps at least 32 blocks: at Q = 1024, C4 = 196,608, 16
// splits instead of 8 took 1.105 against 1.130 ms per call (two interleaved
// runs each), unchanged at C4 = 65,536.
int32_t scan_splits(int64_t Q, int64_t P_log, int cus) {
  const int64_t blocks = (P_log * 64 + 255) / 256;
  int64_t floor_s = blocks / 64;
  if (floor_s > 8) floor_s = 8;
  int32_t s = auto_splits(Q, cus, 4);
  if (floor_s > s) s = static_cast<int32_t>(floor_s);
  const int32_t pers = auto_splits(Q, cus, 8);
  if (pers > s && pers <= blocks / 32) s = pers;
  return s;
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int32_t kDefaultTile = 4096;   // positions per tile of the context-tiled path

struct FusedScratch {
  size_t state_off, gate_off, count_off, list_off, listn_off, fbcnt_off, cand_off, total;
};

// Independent of the context length: O(Q) bookkeeping plus a bounded
// candidate buffer of candidate_cap(K) keys per row.
FusedScratch fused_scratch_layout(int64_t Q, int32_t K) {
  const size_t q = static_cast<size_t>(Q);
  FusedScratch s;
  s.state_off = 0;
  s.gate_off = s.state_off + align_up(q * sizeof(int32_t));
  s.count_off = s.gate_off + align_up(q * sizeof(uint64_t));
  s.list_off = s.count_off + align_up(q * sizeof(uint32_t));
  s.listn_off = s.list_off + align_up(q * sizeof(int32_t));
  s.fbcnt_off = s.listn_off + align_up(sizeof(int32_t));
  s.cand_off = s.fbcnt_off + align_up(q * 4 * sizeof(int32_t));
  s.total = s.cand_off + align_up(q * static_cast<size_t>(mqa::candidate_cap(K)) * sizeof(uint64_t));
  return s;
}

// Common entry checks; on success the guard holds the tensors' device.
// Order: host-only checks first (testable without a GPU), then device checks.
int32_t enter(hipStream_t st, const PtrSpec* specs, int nspecs, DeviceGuard& guard, DeviceInfo* info,
              bool allow_capture = false) {
  int32_t rc = check_ptrs_host(specs, nspecs);
  if (rc != MQA_OK) return rc;
  int dev = -1;
  rc = stream_device(st, &dev);
  if (rc != MQA_OK) return rc;
  if (!allow_capture) {
    rc = check_capture(st);
    if (rc != MQA_OK) return rc;
  }
  rc = device_info(dev, info);
  if (rc != MQA_OK) return rc;
  rc = check_ptrs_device(specs, nspecs, dev);
  if (rc != MQA_OK) return rc;
  return guard.enter(dev);
}

// Stream-ordered scratch for one call.
struct Scratch {
  void* p = nullptr;
  hipStream_t st = nullptr;
  int32_t alloc(size_t bytes, hipStream_t stream) {
    st = stream;
    if (bytes == 0) return MQA_OK;
    if (hipMallocAsync(&p, bytes, stream) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
      return MQA_ERR_HIP;
    }
    return MQA_OK;
  }
  ~Scratch() {
    if (p) (void)hipFreeAsync(p, st);
  }
};

// Stage events of the measurement hook (per host thread).
thread_local void* const* t_stage_events = nullptr;

void record_stage(int i, hipStream_t st) {
  if (t_stage_events) (void)hipEventRecord(static_cast<hipEvent_t>(t_stage_events[i]), st);
}

int32_t hip_rc(hipError_t e) {
  if (e == hipSuccess) return MQA_OK;
  (void)hipGetLastError();
  return MQA_ERR_HIP;
}

// Scratch of the allocation-free entry point: one fixed array per device, held
// until the process ends. In host code its name only stands for the variable;
// the device address of each device's copy comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[MQA_STATIC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch` (device `dev` current).
int32_t static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MQA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return MQA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MQA_OK;
}

// The fused path. use_static: scratch from the device's fixed array instead of
// a stream-ordered allocation (then nothing is allocated and a capturing
// stream is accepted; every scratch word is written by a kernel of the call
// before it is read, so the array needs no clearing between calls).
int32_t run_fused(const PathArgs& p, uint32_t flags, hipStream_t st, bool use_static = false) {
  if (p.K != 512 && p.K != 1024) return MQA_ERR_UNSUPPORTED_K;
  const uint32_t known =
      MQA_FLAG_SPLITS_MASK | MQA_FLAG_NO_PREFILTER | MQA_FLAG_FORCE_UNDERFILL | MQA_FLAG_NO_FALLBACK;
  if (flags & ~known) return MQA_ERR_BAD_FLAGS;
  if ((flags & MQA_FLAG_NO_PREFILTER) && (flags & (MQA_FLAG_FORCE_UNDERFILL | MQA_FLAG_NO_FALLBACK)))
    return MQA_ERR_BAD_FLAGS;
  int32_t rc = check_sizes(p.Q, p.P_phys, p.P_log);
  if (rc != MQA_OK) return rc;
  const FusedScratch lay = fused_scratch_layout(p.Q, p.K);
  if (use_static && lay.total > static_cast<size_t>(MQA_STATIC_SCRATCH_BYTES)) return MQA_ERR_BAD_SIZE;
  const bool rows = p.Q > 0;
  const PtrSpec specs[] = {
      {p.q, rows, 16},          {p.q_scale, rows, 4},   {p.k_pages, p.P_phys > 0, 16},
      {p.k_scale, p.P_phys > 0, 16}, {p.weights, rows, 4}, {p.page_table, p.P_log > 0, 4},
      {p.row_start, rows, 4},   {p.row_end, rows, 4},   {p.out_raw, rows, 4},
      {p.out_slot, rows, 4},    {p.out_count, rows, 4}, {p.out_score, false, 4},
  };
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info, /*allow_capture=*/use_static);
  if (rc != MQA_OK) return rc;
  if (!rows) return MQA_OK;
  const int32_t explicit_splits = static_cast<int32_t>(flags & MQA_FLAG_SPLITS_MASK);
  const int32_t splits = explicit_splits ? explicit_splits : scan_splits(p.Q, p.P_log, info.cus);
  const int32_t calib_splits = explicit_splits ? explicit_splits : auto_splits(p.Q, info.cus, 4);
  const int calib_mode = (flags & MQA_FLAG_NO_PREFILTER) ? 1 : (flags & MQA_FLAG_FORCE_UNDERFILL) ? 2 : 0;
  Scratch allocated;
  char* base = nullptr;
  if (use_static) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MQA_ERR_HIP;   // the tensors' device, current since enter()
    void* ptr = nullptr;
    rc = static_scratch(dev, &ptr);
    if (rc != MQA_OK) return rc;
    base = static_cast<char*>(ptr);
  } else {
    rc = allocated.alloc(lay.total, st);
    if (rc != MQA_OK) return rc;
    base = static_cast<char*>(allocated.p);
  }
  mqa::GatedScratch g;
  g.row_state = reinterpret_cast<int32_t*>(base + lay.state_off);
  g.gate = reinterpret_cast<uint64_t*>(base + lay.gate_off);
  g.count = reinterpret_cast<uint32_t*>(base + lay.count_off);
  g.fb_list = reinterpret_cast<int32_t*>(base + lay.list_off);
  g.fb_count = reinterpret_cast<int32_t*>(base + lay.listn_off);
  g.work = reinterpret_cast<int32_t*>(base + lay.listn_off + 128);   // same 256-byte slot, its own line
  g.fb_cnt = reinterpret_cast<int32_t*>(base + lay.fbcnt_off);
  g.cand = reinterpret_cast<uint64_t*>(base + lay.cand_off);
  record_stage(0, st);
  rc = hip_rc(mqa::launch_row_prep(p, 0, g.row_state, g.fb_count, st));
  record_stage(1, st);
  for (int stage = 0; stage < 5 && rc == MQA_OK; ++stage) {
    rc = hip_rc(mqa::launch_gated_stage(p, g, splits, calib_splits, calib_mode, (flags & MQA_FLAG_NO_FALLBACK) != 0,
                                        stage, info.cus, st));
    if (stage <= 1) record_stage(2 + stage, st);   // after calibration, after the scan
  }
  record_stage(4, st);
  return rc;
}

}  // namespace

extern "C" {

int32_t mqa_fp4_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                             const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                             const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                             const int32_t* row_start, const int32_t* row_end, int32_t K, int32_t* out_raw,
                             int32_t* out_slot, int32_t* out_count, void* stream) {
  return mqa_fp4_topk_prefill_ex(q, q_scale, num_rows, k_pages, k_scale, num_phys_pages, weights, page_table,
                                 num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count,
                                 nullptr, 0u, stream);
}

int32_t mqa_fp4_topk_prefill_ex(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                                const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                                const int32_t* row_start, const int32_t* row_end, int32_t K, int32_t* out_raw,
                                int32_t* out_slot, int32_t* out_count, float* out_score, uint32_t flags,
                                void* stream) {
  const PathArgs p{q,       q_scale,    num_rows,  k_pages,  k_scale, num_phys_pages, weights,  page_table,
                   num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  return run_fused(p, flags, static_cast<hipStream_t>(stream));
}

int32_t mqa_fp4_topk_prefill_static(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                    const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                                    const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                                    const int32_t* row_start, const int32_t* row_end, int32_t K, int32_t* out_raw,
                                    int32_t* out_slot, int32_t* out_count, float* out_score, uint32_t flags,
                                    void* stream) {
  const PathArgs p{q,       q_scale,    num_rows,  k_pages,  k_scale, num_phys_pages, weights,  page_table,
                   num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  return run_fused(p, flags, static_cast<hipStream_t>(stream), /*use_static=*/true);
}

int32_t mqa_fp4_dense_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                   const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                                   const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                                   const int32_t* row_start, const int32_t* row_end, int32_t K, float* logits,
                                   int32_t* out_raw, int32_t* out_slot, int32_t* out_count, float* out_score,
                                   void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  int32_t rc = check_sizes(num_rows, num_phys_pages, num_logical_pages);
  if (rc != MQA_OK) return rc;
  const bool rows = num_rows > 0;
  const PtrSpec specs[] = {
      {q, rows, 16},          {q_scale, rows, 4},   {k_pages, num_phys_pages > 0, 16},
      {k_scale, num_phys_pages > 0, 16}, {weights, rows, 4}, {page_table, num_logical_pages > 0, 4},
      {row_start, rows, 4},   {row_end, rows, 4},   {logits, rows && num_logical_pages > 0, 4},
      {out_raw, rows, 4},     {out_slot, rows, 4},  {out_count, rows, 4}, {out_score, false, 4},
  };
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info);
  if (rc != MQA_OK) return rc;
  if (!rows) return MQA_OK;
  const PathArgs p{q,       q_scale,    num_rows,  k_pages,  k_scale, num_phys_pages, weights,  page_table,
                   num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  Scratch buf;
  rc = buf.alloc(align_up(static_cast<size_t>(num_rows) * sizeof(int32_t)), st);
  if (rc != MQA_OK) return rc;
  int32_t* row_state = static_cast<int32_t*>(buf.p);
  record_stage(0, st);
  rc = hip_rc(mqa::launch_row_prep(p, 0, row_state, nullptr, st));
  record_stage(1, st);
  record_stage(2, st);   // no calibration on the dense path
  if (rc == MQA_OK) rc = hip_rc(mqa::launch_dense_score(p, row_state, auto_splits(num_rows, info.cus), logits, st));
  record_stage(3, st);
  if (rc == MQA_OK) rc = hip_rc(mqa::launch_logits_topk(p, logits, row_state, st));
  record_stage(4, st);
  return rc;
}

int32_t mqa_fp4_dense_logits(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows, const uint8_t* k_pages,
                             const uint8_t* k_scale, int64_t num_phys_pages, const float* weights,
                             const int32_t* page_table, int64_t num_logical_pages, const int32_t* row_start,
                             const int32_t* row_end, float* logits, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t rc = check_sizes(num_rows, num_phys_pages, num_logical_pages);
  if (rc != MQA_OK) return rc;
  const bool rows = num_rows > 0;
  const PtrSpec specs[] = {
      {q, rows, 16},          {q_scale, rows, 4},   {k_pages, num_phys_pages > 0, 16},
      {k_scale, num_phys_pages > 0, 16}, {weights, rows, 4}, {page_table, num_logical_pages > 0, 4},
      {row_start, rows, 4},   {row_end, rows, 4},   {logits, rows && num_logical_pages > 0, 4},
  };
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info);
  if (rc != MQA_OK) return rc;
  if (!rows) return MQA_OK;
  const PathArgs p{q,       q_scale, num_rows, k_pages, k_scale, num_phys_pages, weights, page_table,
                   num_logical_pages, row_start, row_end, 0, nullptr, nullptr, nullptr, nullptr};
  Scratch buf;
  rc = buf.alloc(align_up(static_cast<size_t>(num_rows) * sizeof(int32_t)), st);
  if (rc != MQA_OK) return rc;
  int32_t* row_state = static_cast<int32_t*>(buf.p);
  rc = hip_rc(mqa::launch_row_prep(p, 1, row_state, nullptr, st));
  if (rc == MQA_OK) rc = hip_rc(mqa::launch_dense_score(p, row_state, auto_splits(num_rows, info.cus), logits, st));
  return rc;
}

int32_t mqa_fp4_logits_topk(const float* logits, int64_t num_rows, const int32_t* page_table,
                            int64_t num_logical_pages, int64_t num_phys_pages, const int32_t* row_start,
                            const int32_t* row_end, int32_t K, int32_t* out_raw, int32_t* out_slot,
                            int32_t* out_count, float* out_score, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  int32_t rc = check_sizes(num_rows, num_phys_pages, num_logical_pages);
  if (rc != MQA_OK) return rc;
  const bool rows = num_rows > 0;
  const PtrSpec specs[] = {
      {logits, rows && num_logical_pages > 0, 4}, {page_table, num_logical_pages > 0, 4},
      {row_start, rows, 4}, {row_end, rows, 4}, {out_raw, rows, 4}, {out_slot, rows, 4},
      {out_count, rows, 4}, {out_score, false, 4},
  };
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info);
  if (rc != MQA_OK) return rc;
  if (!rows) return MQA_OK;
  const PathArgs p{nullptr, nullptr, num_rows, nullptr, nullptr, num_phys_pages, nullptr, page_table,
                   num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  Scratch buf;
  rc = buf.alloc(align_up(static_cast<size_t>(num_rows) * sizeof(int32_t)), st);
  if (rc != MQA_OK) return rc;
  int32_t* row_state = static_cast<int32_t*>(buf.p);
  rc = hip_rc(mqa::launch_row_prep(p, 0, row_state, nullptr, st));
  if (rc == MQA_OK) rc = hip_rc(mqa::launch_logits_topk(p, logits, row_state, st));
  return rc;
}

int32_t mqa_fp4_supported_k(int32_t* ks, int32_t capacity, int32_t* n) {
  static const int32_t kSupported[2] = {512, 1024};
  if (n == nullptr) return MQA_ERR_NULL_POINTER;
  *n = 2;
  if (ks != nullptr)
    for (int32_t i = 0; i < capacity && i < 2; ++i) ks[i] = kSupported[i];
  return MQA_OK;
}

int64_t mqa_fp4_topk_scratch_bytes(int64_t num_rows, int32_t K, int32_t device) {
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  if (num_rows < 0 || num_rows > 0x7FFFFFFFll) return MQA_ERR_BAD_SIZE;
  DeviceInfo info;
  const int32_t rc = device_info(device, &info);
  if (rc != MQA_OK) return rc;
  if (num_rows == 0) return 0;
  return static_cast<int64_t>(fused_scratch_layout(num_rows, K).total);
}

int32_t mqa_fp4_status(void* stream, int32_t* status) {
  if (status == nullptr) return MQA_ERR_NULL_POINTER;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = -1;
  int32_t rc = stream_device(st, &dev);
  if (rc != MQA_OK) return rc;
  DeviceGuard guard;
  rc = guard.enter(dev);
  if (rc != MQA_OK) return rc;
  return hip_rc(mqa::status_take(st, status));
}

int32_t mqa_fp4_set_stage_events(void* const* events, int32_t n) {
  if (events == nullptr || n == 0) {
    t_stage_events = nullptr;
    return MQA_OK;
  }
  if (n != 5) return MQA_ERR_BAD_SIZE;
  t_stage_events = events;
  return MQA_OK;
}

int32_t mqa_fp4_tiled_topk_prefill(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows,
                                   const uint8_t* k_pages, const uint8_t* k_scale, int64_t num_phys_pages,
                                   const float* weights, const int32_t* page_table, int64_t num_logical_pages,
                                   const int32_t* row_start, const int32_t* row_end, int32_t K,
                                   int32_t tile_positions, int32_t* out_raw, int32_t* out_slot,
                                   int32_t* out_count, float* out_score, void* stream) {
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  if (tile_positions == 0) tile_positions = kDefaultTile;
  if (tile_positions < 0 || tile_positions % 256 != 0 || tile_positions > (1 << 22)) return MQA_ERR_BAD_SIZE;
  int32_t rc = check_sizes(num_rows, num_phys_pages, num_logical_pages);
  if (rc != MQA_OK) return rc;
  const bool rows = num_rows > 0;
  const PtrSpec specs[] = {
      {q, rows, 16},       {q_scale, rows, 4},   {k_pages, num_phys_pages > 0, 16},
      {k_scale, num_phys_pages > 0, 16}, {weights, rows, 4}, {page_table, num_logical_pages > 0, 4},
      {row_start, rows, 4}, {row_end, rows, 4},  {out_raw, rows, 4},
      {out_slot, rows, 4}, {out_count, rows, 4}, {out_score, false, 4},
  };
  const hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info);
  if (rc != MQA_OK || !rows) return rc;
  const PathArgs p{q,       q_scale,    num_rows,  k_pages,  k_scale, num_phys_pages, weights,  page_table,
                   num_logical_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  const size_t Qz = static_cast<size_t>(num_rows);
  const size_t state_b = align_up(Qz * sizeof(int32_t));
  const size_t count_b = align_up(Qz * sizeof(int32_t));
  const size_t floor_b = align_up(Qz * sizeof(uint64_t));
  const size_t run_b = align_up(Qz * static_cast<size_t>(mqa::tile_pool_cap(K)) * sizeof(uint64_t));
  const size_t tile_b = align_up(Qz * static_cast<size_t>(tile_positions) * sizeof(float));
  Scratch buf;
  rc = buf.alloc(state_b + count_b + floor_b + run_b + tile_b, st);
  if (rc != MQA_OK) return rc;
  char* base = static_cast<char*>(buf.p);
  int32_t* row_state = reinterpret_cast<int32_t*>(base);
  int32_t* run_count = reinterpret_cast<int32_t*>(base + state_b);
  uint64_t* run_floor = reinterpret_cast<uint64_t*>(base + state_b + count_b);
  uint64_t* running = reinterpret_cast<uint64_t*>(base + state_b + count_b + floor_b);
  float* tile_logits = reinterpret_cast<float*>(base + state_b + count_b + floor_b + run_b);
  record_stage(0, st);
  rc = hip_rc(mqa::launch_row_prep(p, 0, row_state, nullptr, st));
  record_stage(1, st);
  record_stage(2, st);
  if (rc == MQA_OK)
    rc = hip_rc(mqa::launch_tiled(p, row_state, auto_splits(num_rows, info.cus), tile_positions, tile_logits,
                                  running, run_count, run_floor, st));
  record_stage(3, st);
  record_stage(4, st);
  return rc;
}

int64_t mqa_fp4_tiled_scratch_bytes(int64_t num_rows, int32_t K, int32_t tile_positions) {
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  if (tile_positions == 0) tile_positions = kDefaultTile;
  if (num_rows < 0 || tile_positions < 0 || tile_positions % 256 != 0 || tile_positions > (1 << 22))
    return MQA_ERR_BAD_SIZE;
  const size_t Qz = static_cast<size_t>(num_rows);
  return static_cast<int64_t>(2 * align_up(Qz * sizeof(int32_t)) + align_up(Qz * sizeof(uint64_t)) +
                              align_up(Qz * static_cast<size_t>(mqa::tile_pool_cap(K)) * sizeof(uint64_t)) +
                              align_up(Qz * static_cast<size_t>(tile_positions) * sizeof(float)));
}

// Context splits of the decode path: enough (row, split) waves to fill the
// four 4-wave scan blocks that fit per CU (on a 64-row batch of 32K..131K-
// position contexts, 32, 48 and 64 splits took 0.136, 0.127 and 0.125 ms).
static int32_t decode_splits(int64_t Q, int cus, int32_t requested) {
  if (requested > 0) return requested;
  const int64_t target = 16ll * cus;
  int64_t s = (target + Q - 1) / (Q > 0 ? Q : 1);
  if (s < 1) s = 1;
  if (s > mqa::kMaxDecodeSplits) s = mqa::kMaxDecodeSplits;
  return static_cast<int32_t>(s);
}

int64_t mqa_fp4_decode_workspace_bytes(int64_t num_rows, int32_t K, int32_t splits, int32_t device) {
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  if (num_rows < 0 || num_rows > 0x7FFFFFFFll || splits < 0 || splits > mqa::kMaxDecodeSplits)
    return MQA_ERR_BAD_SIZE;
  int cus = 256;
  if (splits == 0) {
    DeviceInfo info;
    const int32_t rc = device_info(device, &info);
    if (rc != MQA_OK) return rc;
    cus = info.cus;
  }
  return static_cast<int64_t>(mqa::decode_scratch_bytes(num_rows, K, decode_splits(num_rows, cus, splits)));
}

int32_t mqa_fp4_topk_decode(const uint8_t* q, const uint8_t* q_scale, int64_t num_rows, const uint8_t* k_pages,
                            const uint8_t* k_scale, int64_t num_phys_pages, const float* weights,
                            const int32_t* block_table, int64_t num_seqs, int64_t max_pages,
                            const int32_t* seq_of_row, const int32_t* row_start, const int32_t* row_end, int32_t K,
                            int32_t* out_raw, int32_t* out_slot, int32_t* out_count, float* out_score,
                            void* workspace, int64_t workspace_bytes, int32_t splits, uint32_t flags,
                            void* stream) {
  if (K != 512 && K != 1024) return MQA_ERR_UNSUPPORTED_K;
  if (flags & ~(MQA_FLAG_NO_PREFILTER | MQA_FLAG_FORCE_UNDERFILL | MQA_FLAG_NO_FALLBACK)) return MQA_ERR_BAD_FLAGS;
  if ((flags & MQA_FLAG_NO_PREFILTER) && (flags & (MQA_FLAG_FORCE_UNDERFILL | MQA_FLAG_NO_FALLBACK)))
    return MQA_ERR_BAD_FLAGS;
  const int mode = (flags & MQA_FLAG_NO_PREFILTER) ? 1 : (flags & MQA_FLAG_FORCE_UNDERFILL) ? 2 : 0;
  int32_t rc = check_sizes(num_rows, num_phys_pages, max_pages);
  if (rc != MQA_OK) return rc;
  if (num_seqs < 0 || (max_pages > 0 && num_seqs > 0x7FFFFFFFll / max_pages)) return MQA_ERR_BAD_SIZE;
  if (splits < 0 || splits > mqa::kMaxDecodeSplits || workspace_bytes < 0) return MQA_ERR_BAD_SIZE;
  const bool rows = num_rows > 0;
  const PtrSpec specs[] = {
      {q, rows, 16},          {q_scale, rows, 4},     {k_pages, num_phys_pages > 0, 16},
      {k_scale, num_phys_pages > 0, 16}, {weights, rows, 4}, {block_table, num_seqs > 0 && max_pages > 0, 4},
      {seq_of_row, rows, 4},  {row_start, rows, 4},   {row_end, rows, 4},
      {out_raw, rows, 4},     {out_slot, rows, 4},    {out_count, rows, 4},
      {out_score, false, 4},  {workspace, rows, 256},
  };
  const hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, sizeof(specs) / sizeof(specs[0]), guard, &info, /*allow_capture=*/true);
  if (rc != MQA_OK || !rows) return rc;
  const int32_t sp = decode_splits(num_rows, info.cus, splits);
  if (static_cast<size_t>(workspace_bytes) < mqa::decode_scratch_bytes(num_rows, K, sp)) return MQA_ERR_BAD_SIZE;
  PathArgs p{q,       q_scale,    num_rows,  k_pages,  k_scale, num_phys_pages, weights,  block_table,
             max_pages, row_start, row_end, K, out_raw, out_slot, out_count, out_score};
  p.seq_of_row = seq_of_row;
  p.n_seq = num_seqs;
  const mqa::DecodeScratch w = mqa::decode_scratch_layout(workspace, num_rows, K, sp);
  record_stage(0, st);
  rc = hip_rc(mqa::launch_row_prep(p, 0, w.row_state, w.fb_count, st));
  record_stage(1, st);
  if (rc == MQA_OK)
    rc = hip_rc(mqa::launch_decode(p, w, sp, mode, (flags & MQA_FLAG_NO_FALLBACK) != 0, info.cus, st,
                                   t_stage_events ? record_stage : nullptr));
  record_stage(4, st);
  return rc;
}

int32_t mqa_fp4_quantize(const float* x, int64_t n_vec, uint8_t* codes, uint8_t* scales, void* stream) {
  if (n_vec < 0 || n_vec > (static_cast<int64_t>(1) << 40)) return MQA_ERR_BAD_SIZE;
  const bool any = n_vec > 0;
  const PtrSpec specs[] = {{x, any, 16}, {codes, any, 2}, {scales, any, 1}};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard guard;
  DeviceInfo info;
  const int32_t rc = enter(st, specs, 3, guard, &info);
  if (rc != MQA_OK || !any) return rc;
  return hip_rc(mqa::launch_mx_quantize(x, n_vec, codes, scales, nullptr, nullptr, 0, 0, info.cus, st));
}

int32_t mqa_fp4_cache_write(const float* k, int64_t n, const int32_t* positions, const int32_t* page_table,
                            int64_t num_logical_pages, int64_t num_phys_pages, uint8_t* k_pages, uint8_t* k_scale,
                            void* stream) {
  if (n < 0 || n > 0x7FFFFFFFll) return MQA_ERR_BAD_SIZE;
  int32_t rc = check_sizes(0, num_phys_pages, num_logical_pages);
  if (rc != MQA_OK) return rc;
  const bool any = n > 0;
  const PtrSpec specs[] = {{k, any, 16},
                           {positions, any, 4},
                           {page_table, any && num_logical_pages > 0, 4},
                           {k_pages, any && num_phys_pages > 0, 16},
                           {k_scale, any && num_phys_pages > 0, 16}};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceGuard guard;
  DeviceInfo info;
  rc = enter(st, specs, 5, guard, &info);
  if (rc != MQA_OK || !any) return rc;
  return hip_rc(mqa::launch_mx_quantize(k, n, k_pages, k_scale, positions, page_table, num_logical_pages,
                                        num_phys_pages, info.cus, st));
}

const char* mqa_fp4_error_string(int32_t code) {
  switch (code) {
    case MQA_OK: return "ok";
    case MQA_ERR_UNSUPPORTED_K: return "unsupported K (supported: 512, 1024)";
    case MQA_ERR_NULL_POINTER: return "required pointer is NULL";
    case MQA_ERR_MISALIGNED: return "pointer misaligned";
    case MQA_ERR_BAD_SIZE: return "size out of range";
    case MQA_ERR_DEVICE: return "pointer/stream/device mismatch or device is not gfx950";
    case MQA_ERR_CAPTURING: return "stream is capturing a graph (not supported)";
    case MQA_ERR_HIP: return "HIP runtime error";
    case MQA_ERR_BAD_FLAGS: return "unknown flag bits";
    default: return "unknown error";
  }
}

int32_t mqa_fp4_abi_version(void) { return MQA_FP4_ABI_VERSION; }

}  // extern "C"
