// Dense decode attention baseline: softmax(q K^T / sqrt(dk)) V ("Stochastic Sparse Attention for
// Memory-Bound Inference", Section 2, Eq. 1), split-KV like FlashDecoding: one block per (chunk of
// DENSE_CHUNK keys, KV head, sequence) writes the chunk's (max, sum-exp, unnormalised output) for the G
// heads of the group; a merge block per (head, sequence) rescales and sums them. fp32 arithmetic on
// bf16 or fp32 inputs; reads all of K and V once.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;
constexpr int BATCH = 8;

template <bool BF16>
__device__ inline void piece_f32(const uint4& w, float* o) {
  if constexpr (BF16) {
    o[0] = bf16_lo(w.x);
    o[1] = bf16_hi(w.x);
    o[2] = bf16_lo(w.y);
    o[3] = bf16_hi(w.y);
    o[4] = bf16_lo(w.z);
    o[5] = bf16_hi(w.z);
    o[6] = bf16_lo(w.w);
    o[7] = bf16_hi(w.w);
  } else {
    o[0] = __uint_as_float(w.x);
    o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z);
    o[3] = __uint_as_float(w.w);
  }
}

template <int D, bool BF16, int GM>
__global__ __launch_bounds__(THREADS) void dense_partial_kernel(DenseProblem p) {
  constexpr int EPL = BF16 ? 8 : 4;
  constexpr int LPR = D / EPL;
  constexpr int NRG = THREADS / LPR;
  constexpr int ROWS = DENSE_CHUNK / NRG;  // rows per row group
  __shared__ float sc[GM][DENSE_CHUNK];
  __shared__ float red[THREADS / 64][GM];
  __shared__ float wsum[THREADS / 64][GM][D];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int rg = tid / LPR, pc = tid % LPR;
  const int64_t n0 = (int64_t)t * DENSE_CHUNK;
  const int len = (int)((p.nk - n0) < DENSE_CHUNK ? (p.nk - n0) : DENSE_CHUNK);
  const size_t esz = BF16 ? 2 : 4;
  const char* kb = (const char*)p.K + esz * ((int64_t)b * p.batch_stride + (n0)*p.seq_stride + (int64_t)kv * D);
  const char* vb = (const char*)p.V + esz * ((int64_t)b * p.batch_stride + (n0)*p.seq_stride + (int64_t)kv * D);
  const int64_t rs = esz * p.seq_stride;

  float qv[GM][EPL];
  {
    const char* qb = (const char*)p.q;
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = 0.f;
        if (g < G) {
          const int64_t i = ((int64_t)b * p.H + (int64_t)kv * G + g) * D + pc * EPL + e;
          x = BF16 ? __uint_as_float(((uint32_t)((const uint16_t*)qb)[i]) << 16) : ((const float*)qb)[i];
        }
        qv[g][e] = x;
      }
  }

  // scores
  for (int k0 = 0; k0 < ROWS; k0 += BATCH) {
    uint4 w[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int r = rg + (k0 + k) * NRG;
      w[k] = load_stream16((const uint4*)(kb + (r < len ? r : 0) * rs) + pc);  // tail rows masked below
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      float x[EPL];
      piece_f32<BF16>(w[k], x);
      const int r = rg + (k0 + k) * NRG;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s += qv[g][e] * x[e];
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o, 64);
        if (pc == 0) sc[g][r] = s * p.scale;
      }
    }
  }
  __syncthreads();

  // chunk max and exponentials (thread handles keys tid, tid + 256)
  float mx[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    float m = -INFINITY;
    for (int r = tid; r < len; r += THREADS) m = fmaxf(m, sc[g][r]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave][g] = m;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    float m = red[0][g];
    for (int w = 1; w < THREADS / 64; ++w) m = fmaxf(m, red[w][g]);
    mx[g] = m;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    float l = 0.f;
    for (int r = tid; r < DENSE_CHUNK; r += THREADS) {
      const float e = r < len ? __expf(sc[g][r] - mx[g]) : 0.f;
      sc[g][r] = e;
      l += e;
    }
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) red[wave][g] = l;
  }
  __syncthreads();

  // P V
  float acc[GM][EPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  for (int k0 = 0; k0 < ROWS; k0 += BATCH) {
    uint4 w[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int r = rg + (k0 + k) * NRG;
      w[k] = load_stream16((const uint4*)(vb + (r < len ? r : 0) * rs) + pc);  // tail rows masked below
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      float x[EPL];
      piece_f32<BF16>(w[k], x);
      const int r = rg + (k0 + k) * NRG;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        const float pr = sc[g][r];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += pr * x[e];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      if (lane < LPR) wsum[wave][g][pc * EPL + e] = x;
    }
  __syncthreads();
  for (int i = tid; i < G * D; i += THREADS) {
    const int g = i / D, e = i % D;
    float o = 0.f;
    for (int w = 0; w < THREADS / 64; ++w) o += wsum[w][g][e];
    float* dst = p.part + (((int64_t)b * p.H + (int64_t)kv * G + g) * p.Td + t) * (D + 2);
    dst[e] = o;
    if (e == 0) {
      float l = 0.f;
      for (int w = 0; w < THREADS / 64; ++w) l += red[w][g];
      dst[D] = mx[g];
      dst[D + 1] = l;
    }
  }
}

// merge: block per (head, sequence); chunk weights f_t = exp(m_t - m*) in LDS, then every thread sums
// a strided slice of the chunks for one output element, 8 loads in flight
constexpr int MERGE_THREADS = 256;
template <int D, bool BF16>
__global__ __launch_bounds__(MERGE_THREADS) void dense_merge_kernel(DenseProblem p) {
  __shared__ float f[MAX_CHUNKS * CHUNK / DENSE_CHUNK];
  __shared__ float red[MERGE_THREADS / 64];
  __shared__ float osum[MERGE_THREADS / D][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Td = p.Td;
  const float* src = p.part + ((int64_t)b * p.H + h) * Td * (D + 2);
  float m = -INFINITY;
  for (int t = tid; t < Td; t += MERGE_THREADS) m = fmaxf(m, src[t * (D + 2) + D]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float ms = red[0];
  for (int w = 1; w < MERGE_THREADS / 64; ++w) ms = fmaxf(ms, red[w]);
  __syncthreads();
  float l = 0.f;
  for (int t = tid; t < Td; t += MERGE_THREADS) {
    const float ft = __expf(src[t * (D + 2) + D] - ms);
    f[t] = ft;
    l += ft * src[t * (D + 2) + D + 1];
  }
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  float lsum = 0.f;
  for (int w = 0; w < MERGE_THREADS / 64; ++w) lsum += red[w];
  constexpr int SL = MERGE_THREADS / D;  // chunk slices
  const int e = tid % D, sl = tid / D;
  float o = 0.f;
  for (int t0 = sl; t0 < Td; t0 += SL * 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = t0 + k * SL;
      v[k] = t < Td ? f[t] * src[t * (D + 2) + e] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) o += v[k];
  }
  osum[sl][e] = o;
  __syncthreads();
  if (tid < D) {
    float r = 0.f;
    for (int k = 0; k < SL; ++k) r += osum[k][tid];
    r /= lsum;
    const int64_t oi = ((int64_t)b * p.H + h) * D + tid;
    if (BF16)
      ((uint16_t*)p.out)[oi] = f32_to_bf16_rne(r);
    else
      ((float*)p.out)[oi] = r;
  }
}

template <int D, bool BF16>
hipError_t launch_dense_dt(const DenseProblem& p, hipStream_t st) {
  dim3 grid(p.Td, p.Hkv, p.B);
  if (p.G <= 1)
    dense_partial_kernel<D, BF16, 1><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 2)
    dense_partial_kernel<D, BF16, 2><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 4)
    dense_partial_kernel<D, BF16, 4><<<grid, THREADS, 0, st>>>(p);
  else
    dense_partial_kernel<D, BF16, 8><<<grid, THREADS, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dense_merge_kernel<D, BF16><<<dim3(p.H, p.B), MERGE_THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense(const DenseProblem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_dense_dt<128, true>(p, st) : launch_dense_dt<128, false>(p, st);
  return p.bf16 ? launch_dense_dt<64, true>(p, st) : launch_dense_dt<64, false>(p, st);
}

}  // namespace santa
