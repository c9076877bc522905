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
};

// mode 0: TopK (answers short and invalid rows); mode 1: logits only.
hipError_t launch_row_prep(const PathArgs& p, int mode, int32_t* row_state, hipStream_t st);
hipError_t launch_fused(const PathArgs& p, const int32_t* row_state, int32_t splits, uint64_t* cand_keys,
                        int32_t* cand_count, hipStream_t st);
hipError_t launch_merge(const PathArgs& p, const int32_t* row_state, int32_t splits, const uint64_t* cand_keys,
                        const int32_t* cand_count, hipStream_t st);
hipError_t launch_dense_score(const PathArgs& p, const int32_t* row_state, int32_t splits, float* logits,
                              hipStream_t st);
hipError_t launch_logits_topk(const PathArgs& p, const float* logits, const int32_t* row_state,
                              hipStream_t st);
// Copies the sticky status word to *host_out and clears it (synchronises st).
hipError_t status_take(hipStream_t st, int32_t* host_out);
int pool_capacity();

}  // namespace mqa
