// Streaming read probe: reads a buffer once with 16-byte non-temporal loads (the access the score pass
// makes to K) and folds it into one XOR word per block, so the read cannot be dropped. Timing it on the
// same bytes and under the same cache state as a decode step gives the read bandwidth the chip actually
// reaches for that size, the practical ceiling beside the published HBM peak.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int RT = 1024;  // one block of 16 waves per CU
constexpr int UNR = 8;    // loads in flight per thread: 128 KiB per CU

__global__ __launch_bounds__(RT, 1) void stream_read_kernel(const uint4* src, int64_t n16, uint32_t* out) {
  __shared__ uint32_t red[RT / 64];
  const int64_t stride = (int64_t)gridDim.x * RT;
  int64_t i = (int64_t)blockIdx.x * RT + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
    uint4 v[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) v[k] = load_stream16(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < UNR; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load_stream16(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < RT / 64; ++w) r ^= red[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

int stream_read_blocks(int64_t bytes, int cus) {
  const int64_t n16 = bytes / 16;
  int64_t b = (n16 + RT - 1) / RT;
  const int64_t cap = cus > 0 ? cus : 256;  // one block per CU: the fastest grid of a size sweep
  if (b > cap) b = cap;
  if (b > STREAM_READ_MAX_BLOCKS) b = STREAM_READ_MAX_BLOCKS;
  return (int)(b < 1 ? 1 : b);
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st,
                              const LaunchEvents& ev) {
  return launch_timed(stream_read_kernel, dim3(blocks), dim3(RT), st, ev, (const uint4*)src, bytes / 16, out);
}

}  // namespace santa
