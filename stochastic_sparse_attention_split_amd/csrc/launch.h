// Host-side launchers of the HIP kernels (one per translation unit); each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace santa {

hipError_t launch_score(const Problem& p, hipStream_t st);     // score.hip
hipError_t launch_sample(const Problem& p, hipStream_t st);    // sample.hip
hipError_t launch_gather(const Problem& p, hipStream_t st);    // gather.hip

// dense baseline (dense.hip): partials [B, H, Td, d + 2] fp32 then a merge
struct DenseProblem {
  const void* q;
  const void* K;
  const void* V;
  void* out;
  int B, H, Hkv, G, d;
  int64_t nk, seq_stride, batch_stride;
  bool bf16;
  float scale;
  int Td;
  float* part;
};
constexpr int DENSE_CHUNK = 512;
hipError_t launch_dense(const DenseProblem& p, hipStream_t st);

// LDS bytes the gather kernel needs for a group of G heads with S samples each
size_t gather_lds_bytes(int G, int S);

}  // namespace santa
