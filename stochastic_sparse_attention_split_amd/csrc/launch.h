// Host-side launchers of the HIP kernels (one per translation unit); each returns the launch status.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.h"

namespace santa {

// Optional timing events of one launch. When set, HIP records them with the launch itself
// (hipExtLaunchKernel), so their elapsed time is the kernel's dispatch and execution without the gaps
// between launches (a profiler's kernel duration, which starts when the first wave runs, is shorter by
// the dispatch).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename... Args>
hipError_t launch_timed(void (*k)(Args...), dim3 grid, dim3 block, hipStream_t st, const LaunchEvents& ev,
                        Args... args) {
  if (ev.start)
    hipExtLaunchKernelGGL(k, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(k, grid, block, 0, st, args...);
  return hipGetLastError();
}

hipError_t launch_score(const Problem& p, hipStream_t st, const LaunchEvents& ev = {});     // score.hip
hipError_t launch_score_fm(const Problem& p, hipStream_t st, const LaunchEvents& ev = {});  // score_fm.hip: K^T
int score_blocks_per_cu(int d, bool bf16, int G);              // resident score blocks per CU (LDS)
hipError_t launch_chunk_cdf(const Problem& p, hipStream_t st); // score.hip
hipError_t launch_budget(const Problem& p, hipStream_t st);    // prop.hip: S²ANTA-prop tile budgets
hipError_t launch_resolve(const Problem& p, hipStream_t st);   // resolve.hip: sample + gather per chunk
hipError_t launch_merge(const Problem& p, hipStream_t st);     // resolve.hip: sum of the chunk partials
// fused.hip: the whole decode in one launch (bf16, sequence-major K, G <= 8, T <= DECODE_MAX_T); grid
// (score_blocks_per_group, Hkv, B), every block resident at once
hipError_t launch_decode(const Problem& p, hipStream_t st, const LaunchEvents& ev = {});
size_t decode_lds_bytes(int G, int n, int T, int d, bool prop);  // LDS of its sampling phase (0: does not fit)
size_t decode_lds_capacity(int d);       // LDS the score phase's K tiles provide

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
// keys per dense partial block: 128 for up to 4 heads per KV head (more blocks, fewer registers), 256 above
// (the 8-head form keeps fewer rows in flight; smaller blocks only grow its merge) — the faster of 64,
// 128 and 256 in a sweep on each form
constexpr int dense_chunk(int G) { return G <= 4 ? 128 : 256; }
constexpr int DENSE_CHUNK_MIN = 128;
hipError_t launch_dense(const DenseProblem& p, hipStream_t st);

// streaming read probe (util.hip): one XOR word per block into out[blocks]
constexpr int STREAM_READ_MAX_BLOCKS = 4096;
int stream_read_blocks(int64_t bytes, int cus);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st,
                              const LaunchEvents& ev = {});

}  // namespace santa
