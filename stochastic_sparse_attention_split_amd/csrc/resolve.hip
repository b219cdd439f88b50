// Sampling and gather-add per chunk (one block per (chunk, KV head, sequence)), then the sum of the
// chunk partials per query head.
//
// "Stochastic Sparse Attention for Memory-Bound Inference":
//   * points: SANTA draws T_m ~ U[0,1) i.i.d. (Section 2, Eq. 4; Definition A.1); S²ANTA-strat draws
//     T_m ~ U[m/S, (m+1)/S) independently and S²ANTA-sys uses one U ~ U[0, 1/S) with T_m = U + m/S
//     (Section 2.1); here T_m = u_m, (m + u_m)/S and (m + u)/S, u from Philox4x32-10 (counter (m, h, b,
//     tag), key = seed);
//   * inverse CDF with the half-open convention 1{F(j-1) <= t < F(j)} (Appendix A.4): a point's chunk
//     is the one whose interval [C_t, C_{t+1}) of the chunk CDF contains T_m Z, and its key the first
//     key of the chunk whose scaled in-chunk prefix exceeds the residual; a point at or beyond Z
//     (rounding) takes the last key with mass of the last chunk with mass;
//   * estimate = (1/S) sum_m V_{J_m} (Eq. 4). As in the pages' per-tile value kernel (Appendix O,
//     Algorithm 5), every (KV head, chunk) works on its own: it counts the samples of each of its keys
//     per head, compacts the keys that were hit, reads each such V row once for the whole GQA group and
//     adds count * V into an fp32 accumulator per head (products of a 16-bit count and a bf16 value are
//     exact in fp32).
//
// Work split: a block owns the points that land in its chunk. For stratified / systematic sampling the
// point of index m lies in [m/S, (m+1)/S), so only m in [floor(S C_t / Z) - 1, floor(S C_{t+1} / Z) + 1]
// can land in chunk t; for i.i.d. sampling every m is tested. The chunk's keys are contiguous, so the
// per-key counters live in LDS. Instead of one shared accumulator per head, each chunk writes its
// partial sums to its own slot; a second kernel adds the T slots of each head in a fixed order and
// scales by 1/S. No atomics on global memory and no device-scope fences: on this chip a fence writes
// back the whole L2 of the XCD, and contended atomics on one address serialise.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;
static_assert(THREADS == CHUNK, "one thread per key of a chunk in the compaction");
constexpr int BATCH = 8;   // V rows in flight per lane

__device__ inline double point_of(const Problem& p, int m, int h, int b, double u_sys) {
  if (p.mode == 0) return uniform53(p.seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
  if (p.mode == 1) {
    const double u = uniform53(p.seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
    return ((double)m + u) / (double)p.S;
  }
  return ((double)m + u_sys) / (double)p.S;
}

// first j in [0, CHUNK) with P[j] * f > r, else -1 (P nondecreasing; entries past the chunk's last key
// repeat the chunk total)
__device__ inline int search_chunk(const double* P, double f, double r) {
  int lo = 0, hi = CHUNK;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] * f > r) hi = mid; else lo = mid + 1;
  }
  return lo < CHUNK ? lo : -1;
}

__device__ inline int last_positive(const double* P, int len) {
  for (int j = len - 1; j > 0; --j)
    if (P[j] > P[j - 1]) return j;
  return 0;
}

template <int D, bool BF16, int GM>
__global__ __launch_bounds__(THREADS) void resolve_kernel(Problem p) {
  using Pc = Piece<BF16>;
  constexpr int EPL = Pc::EPL;
  constexpr int LPR = D / EPL;          // lanes per V row
  constexpr int NRG = THREADS / LPR;    // row groups
  constexpr int NWAVE = THREADS / 64;
  constexpr int NCW = GM / 2;           // 32-bit words of 16-bit per-head counts
  constexpr int CW = NCW + 1;           // padded stride of the per-key counters
  static_assert((size_t)NWAVE * GM * D * sizeof(float) <= (size_t)GM * CHUNK * sizeof(double),
                "the cross-wave sums reuse the prefix tile");

  __shared__ double Pt[GM][CHUNK];      // in-chunk prefixes; later the cross-wave sums
  __shared__ uint32_t cnt[CHUNK * CW];
  __shared__ int32_t lkey[CHUNK];
  __shared__ uint32_t lcnt[CHUNK][NCW];
  __shared__ double hC0[GM], hC1[GM], hF[GM], hZ[GM], hU[GM];
  __shared__ int hLo[GM], hN[GM], hLast[GM];
  __shared__ int wsum_i[NWAVE];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S, T = p.T;
  const int h0 = kv * G;
  const int grp = b * p.Hkv + kv;
  const int64_t bh0 = (int64_t)b * p.H + h0;
  const int64_t n0 = (int64_t)t * CHUNK;
  const int len = (int)min((int64_t)CHUNK, p.nk - n0);

  // ---- every load of the sampling phase at once: the prefix tile (head clamped to G-1, key clamped to
  //      the chunk's last key, so every address is valid) and this chunk's interval of the chunk CDF
  double pv[GM];
#pragma unroll
  for (int j = 0; j < GM; ++j) {
    const int g = min(j, G - 1), k = min(tid, len - 1);
    pv[j] = p.stash[(bh0 + g) * p.nk + n0 + k];
  }
  const int hg = min(tid, G - 1);
  const double* cdf = p.cdf + (bh0 + hg) * (T + 1);
  const double c0 = cdf[t], c1 = cdf[t + 1], Z = cdf[T];
  const double f = p.cscale[(bh0 + hg) * T + t];
  const int lastc = p.lastpos[bh0 + hg];

#pragma unroll
  for (int j = 0; j < GM; ++j) Pt[j][tid] = pv[j];
  for (int i = tid; i < CHUNK * CW; i += THREADS) cnt[i] = 0u;
  if (tid < G) {
    const int g = tid;
    hC0[g] = c0;
    hC1[g] = c1;
    hZ[g] = Z;
    hF[g] = f;
    hLast[g] = lastc;
    hU[g] = p.mode == 2 ? uniform53(p.seed, 0u, (uint32_t)(h0 + g), (uint32_t)b, TAG_SYS) : 0.0;
    int lo = 0, n = 0;
    if (c1 > c0 || t == lastc) {
      if (p.mode == 0) {
        n = S;
      } else {
        const double a = floor((double)S * (c0 / Z)) - 1.0, e = floor((double)S * (c1 / Z)) + 1.0;
        const int ilo = (int)fmax(0.0, a);
        const int ihi = t == lastc ? S - 1 : (int)fmin((double)(S - 1), e);
        lo = ilo;
        n = ihi >= ilo ? ihi - ilo + 1 : 0;
      }
    }
    hLo[g] = lo;
    hN[g] = n;
  }
  __syncthreads();

  // debug: probabilities of this chunk's keys from the score pass's exponentials
  if (p.prob) {
    for (int i = tid; i < G * len; i += THREADS) {
      const int g = i / len, k = i % len;
      double* pr = p.prob + (bh0 + g) * p.nk + n0 + k;
      *pr = *pr * hF[g] / hZ[g];
    }
  }

  // ---- resolve the candidate points that land in this chunk and count them per key and head
  int total = 0;
  for (int g = 0; g < G; ++g) total += hN[g];
  for (int c = tid; c < total; c += THREADS) {
    int g = 0, off = c;
    while (off >= hN[g]) off -= hN[g++];
    const int m = hLo[g] + off;
    const double y = point_of(p, m, h0 + g, b, hU[g]) * hZ[g];
    const bool mine = y < hZ[g] ? (hC0[g] <= y && y < hC1[g]) : (t == hLast[g]);
    if (!mine) continue;
    int j;
    if (y < hZ[g]) {
      j = search_chunk(Pt[g], hF[g], y - hC0[g]);
      if (j < 0) j = last_positive(Pt[g], len);  // the residual reached the chunk total through rounding
    } else {
      j = last_positive(Pt[g], len);
    }
    p.idx[(bh0 + g) * S + m] = (int32_t)(n0 + j);
    atomicAdd(&cnt[j * CW + (g >> 1)], (g & 1) ? 0x10000u : 1u);
  }
  __syncthreads();

  // ---- compact the sampled keys (thread k owns key k)
  uint32_t mycw[NCW];
  bool any = false;
#pragma unroll
  for (int w = 0; w < NCW; ++w) {
    mycw[w] = cnt[tid * CW + w];
    any |= mycw[w] != 0u;
  }
  const uint64_t bal = __ballot(any);
  if (lane == 0) wsum_i[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, nu = 0;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    if (w < wave) before += wsum_i[w];
    nu += wsum_i[w];
  }
  if (any) {
    const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
    lkey[pos] = tid;
#pragma unroll
    for (int w = 0; w < NCW; ++w) lcnt[pos][w] = mycw[w];
  }
  if (tid == 0) p.unique[(int64_t)grp * T + t] = nu;
  float* dst = p.partial + ((int64_t)grp * T + t) * G * D;
  if (nu == 0) {  // block-uniform: nothing sampled here
    for (int i = tid; i < G * D; i += THREADS) dst[i] = 0.0f;
    return;
  }
  __syncthreads();

  // ---- gather: each listed row once, added with its per-head counts
  const int rg = tid / LPR, pc = tid % LPR;
  float acc[GM][EPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  const size_t esz = BF16 ? 2 : 4;
  const char* vbase = (const char*)p.V + esz * ((int64_t)b * p.batch_stride + n0 * p.seq_stride + (int64_t)kv * D);
  const int64_t rstride = esz * p.seq_stride;
  for (int u0 = rg; u0 < nu; u0 += NRG * BATCH) {
    // list entries past nu re-read the last entry's row and are added with count 0
    int key[BATCH];
    uint32_t cw[BATCH][NCW];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = u0 + k * NRG;
      const int uu = min(u, nu - 1);
      key[k] = lkey[uu];
#pragma unroll
      for (int w = 0; w < NCW; ++w) cw[k][w] = u < nu ? lcnt[uu][w] : 0u;
    }
    uint4 w4[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) w4[k] = load_stream16((const uint4*)(vbase + key[k] * rstride) + pc);
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      float v[EPL];
      Pc::to_f32(w4[k], v);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        const uint32_t c32 = cw[k][g >> 1];
        const float c = (float)((g & 1) ? (c32 >> 16) : (c32 & 0xFFFFu));
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += c * v[e];
      }
    }
  }
  // reduce the row groups: inside the wave by lane permutes, then across waves in LDS
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      acc[g][e] = x;
    }
  float* wsum = reinterpret_cast<float*>(&Pt[0][0]);  // [NWAVE][GM][D]; Pt is dead after the last sync
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) wsum[((size_t)wave * GM + g) * D + pc * EPL + e] = acc[g][e];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += THREADS) {
    const int g = i / D, e = i % D;
    float s = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < NWAVE; ++w2) s += wsum[((size_t)w2 * GM + g) * D + e];
    dst[i] = s;
  }
}

// out[b, h] = round((sum over chunks of the partials of head h) / S); fp64 sum in chunk order
template <int D, bool BF16>
__global__ __launch_bounds__(THREADS) void merge_kernel(Problem p) {
  constexpr int V4 = D / 4;            // float4 pieces per row
  constexpr int TS = THREADS / V4;     // chunk slices
  constexpr int MB = 16;               // loads in flight per thread
  __shared__ double red[TS][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int G = p.G, T = p.T;
  const int kv = h / G, g = h % G;
  const int c = tid % V4, ts = tid / V4;
  const float* base = p.partial + ((int64_t)(b * p.Hkv + kv) * T * G + g) * D + 4 * c;
  const int64_t tstride = (int64_t)G * D;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  for (int t0 = ts; t0 < T; t0 += TS * MB) {
    float4 v[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int tt = min(t0 + k * TS, T - 1);
      v[k] = *(const float4*)(base + tt * tstride);
    }
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      if (t0 + k * TS < T) {
        a0 += v[k].x;
        a1 += v[k].y;
        a2 += v[k].z;
        a3 += v[k].w;
      }
    }
  }
  red[ts][4 * c + 0] = a0;
  red[ts][4 * c + 1] = a1;
  red[ts][4 * c + 2] = a2;
  red[ts][4 * c + 3] = a3;
  __syncthreads();
  if (tid < D) {
    double tot = 0.0;
#pragma unroll
    for (int s = 0; s < TS; ++s) tot += red[s][tid];
    const double r = tot / (double)p.S;
    const int64_t o = ((int64_t)b * p.H + h) * D + tid;
    if (BF16)
      ((uint16_t*)p.out)[o] = f64_to_bf16_rne(r);
    else
      ((float*)p.out)[o] = (float)r;
  }
}

template <int D, bool BF16>
hipError_t launch_resolve_dt(const Problem& p, hipStream_t st) {
  dim3 grid(p.T, p.Hkv, p.B);
  if (p.G <= 2)
    resolve_kernel<D, BF16, 2><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 4)
    resolve_kernel<D, BF16, 4><<<grid, THREADS, 0, st>>>(p);
  else
    resolve_kernel<D, BF16, 8><<<grid, THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_resolve(const Problem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_resolve_dt<128, true>(p, st) : launch_resolve_dt<128, false>(p, st);
  return p.bf16 ? launch_resolve_dt<64, true>(p, st) : launch_resolve_dt<64, false>(p, st);
}

hipError_t launch_merge(const Problem& p, hipStream_t st) {
  dim3 grid(p.H, p.B);
  if (p.d == 128) {
    if (p.bf16) merge_kernel<128, true><<<grid, THREADS, 0, st>>>(p);
    else merge_kernel<128, false><<<grid, THREADS, 0, st>>>(p);
  } else {
    if (p.bf16) merge_kernel<64, true><<<grid, THREADS, 0, st>>>(p);
    else merge_kernel<64, false><<<grid, THREADS, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace santa
