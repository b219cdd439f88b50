// Gather-and-add with GQA deduplication: one block per (KV head, sequence).
//
// "Stochastic Sparse Attention for Memory-Bound Inference":
//   * the estimate of each query head is (1/S) sum_m V_{J_m} (Section 2, Eq. 4; Appendix A, Eq. 7):
//     additions of gathered rows only, one multiply by 1/S at the end (a shift when S = 2^k);
//   * the G heads of a KV group share V, so the emitted rows are the union of their samples and each
//     distinct row is read once and added with its per-head count c_{h,n} (Appendix O, Algorithm 5,
//     compaction of emitted rows and O_h += c_{h,n} V_n).
//
// The union is an open-addressing hash table in LDS (2*G*S slots, linear probing, LDS atomics); each
// slot carries 16-bit per-head counts, and the first insertion of a row appends its slot to a compact
// list. Lanes own 16-byte pieces of a row and issue the loads of 8 rows before using them. The
// accumulation is fp64: count * V is exact, so the sum does not depend on the order rows are visited.
// Output = round(sum / S) to the output dtype, RNE.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;
constexpr int BATCH = 8;  // rows in flight per lane

__device__ inline uint32_t hash_key(int32_t n, uint32_t ts) { return ((uint32_t)n * 2654435761u) % ts; }

// LDS layout: keys[TS] int32 | list[G*S] int32 | cnt[TS*G] uint16
template <int D, bool BF16, int GM>
__global__ __launch_bounds__(THREADS) void gather_kernel(Problem p) {
  extern __shared__ __align__(16) unsigned char smem[];
  using P = Piece<BF16>;
  constexpr int EPL = P::EPL;          // elements per 16-byte piece
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int NRG = THREADS / LPR;   // row groups per block

  const int kv = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S;
  const uint32_t TS = 2u * (uint32_t)(G * S);
  int32_t* keys = (int32_t*)smem;
  int32_t* list = keys + TS;
  uint16_t* cnt = (uint16_t*)(list + (size_t)G * S);
  __shared__ int32_t nuniq;

  if (tid == 0) nuniq = 0;
  for (uint32_t i = tid; i < TS; i += THREADS) keys[i] = -1;
  for (uint32_t i = tid; i < TS * (uint32_t)G / 2u; i += THREADS) ((uint32_t*)cnt)[i] = 0u;
  __syncthreads();

  // insert every sample (head g, point m) of the group, counting per head
  const int32_t* idx = p.idx + ((int64_t)b * p.H + (int64_t)kv * G) * S;
  for (int s = tid; s < G * S; s += THREADS) {
    const int g = s / S;
    const int32_t n = idx[s];
    if (n < 0 || (int64_t)n >= p.nk) continue;  // never address V outside the cache
    uint32_t slot = hash_key(n, TS);
    while (true) {
      const int32_t old = atomicCAS(&keys[slot], -1, n);
      if (old == -1) {
        list[atomicAdd(&nuniq, 1)] = (int32_t)slot;
        break;
      }
      if (old == n) break;
      slot = slot + 1 == TS ? 0 : slot + 1;
    }
    // 16-bit counters packed in 32-bit words: add 1 to the right half
    const uint32_t ci = slot * (uint32_t)G + (uint32_t)g;
    atomicAdd((uint32_t*)cnt + (ci >> 1), (ci & 1u) ? 0x10000u : 1u);
  }
  __syncthreads();
  const int U = nuniq;

  // gather: lane owns piece pc of rows rg, rg + NRG, ... of the compact list
  const int rg = tid / LPR, pc = tid % LPR;
  double acc[GM][EPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0;
  const char* vbase = (const char*)p.V + (BF16 ? 2 : 4) * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
  const int64_t rstride = (BF16 ? 2 : 4) * p.seq_stride;
  for (int u0 = rg; u0 < U; u0 += NRG * BATCH) {
    uint4 w[BATCH];
    int32_t sl[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = u0 + k * NRG;
      sl[k] = u < U ? list[u] : -1;
      if (sl[k] >= 0) w[k] = *((const uint4*)(vbase + (int64_t)keys[sl[k]] * rstride) + pc);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (sl[k] < 0) continue;
      double v[EPL];
      P::to_f64(w[k], v);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        if (g < G) {
          const double c = (double)cnt[(uint32_t)sl[k] * (uint32_t)G + g];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] += c * v[e];
        }
      }
    }
  }

  // reduce the row groups: inside the wave by shuffles, then across waves in LDS
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      double x = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      acc[g][e] = x;
    }
  __syncthreads();  // the hash table is dead: reuse its LDS for the per-wave sums [waves][GM][D]
  double* wsum = (double*)smem;
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) wsum[((size_t)wave * GM + g) * D + pc * EPL + e] = acc[g][e];
  }
  __syncthreads();
  const double dS = (double)S;
  for (int i = tid; i < G * D; i += THREADS) {
    const int g = i / D, e = i % D;
    double tot = 0.0;
    for (int w = 0; w < THREADS / 64; ++w) tot += wsum[((size_t)w * GM + g) * D + e];
    const double r = tot / dS;
    const int64_t o = ((int64_t)b * p.H + (int64_t)kv * G + g) * D + e;
    if (BF16)
      ((uint16_t*)p.out)[o] = f64_to_bf16_rne(r);
    else
      ((float*)p.out)[o] = (float)r;
  }
  if (tid == 0) p.unique[(int64_t)b * p.Hkv + kv] = U;
}

template <int D, bool BF16, int GM>
hipError_t launch_one(const Problem& p, hipStream_t st) {
  const size_t lds = gather_lds_bytes(p.G, p.S);
  if (lds > 64 * 1024) {
    // tables beyond the default 64 KiB of dynamic LDS need the limit raised for this kernel
    const hipError_t e = hipFuncSetAttribute((const void*)gather_kernel<D, BF16, GM>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  gather_kernel<D, BF16, GM><<<dim3(p.Hkv, p.B), THREADS, lds, st>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_dt(const Problem& p, hipStream_t st) {
  if (p.G <= 1) return launch_one<D, BF16, 1>(p, st);
  if (p.G <= 2) return launch_one<D, BF16, 2>(p, st);
  if (p.G <= 4) return launch_one<D, BF16, 4>(p, st);
  return launch_one<D, BF16, 8>(p, st);
}

}  // namespace

size_t gather_lds_bytes(int G, int S) {
  const size_t TS = 2 * (size_t)G * (size_t)S;
  const size_t table = TS * 4 + (size_t)G * S * 4 + TS * (size_t)G * 2;
  const size_t red = (size_t)(THREADS / 64) * MAX_GROUP * 128 * sizeof(double);
  return table > red ? table : red;
}

hipError_t launch_gather(const Problem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_dt<128, true>(p, st) : launch_dt<128, false>(p, st);
  return p.bf16 ? launch_dt<64, true>(p, st) : launch_dt<64, false>(p, st);
}

}  // namespace santa
