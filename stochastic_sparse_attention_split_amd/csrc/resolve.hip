// Sampling (one block per (chunk, KV head, sequence)) and gather-add (one block per (KV head, sequence)).
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
//   * estimate = (1/S) sum_m V_{J_m} (Eq. 4), each distinct row of a GQA group read once and added with
//     its per-head count (Appendix O, Algorithm 5: emitted-row compaction, O_h += c_{h,n} V_n).
//
// Work split: a block owns the points that land in its chunk. For stratified / systematic sampling the
// point of index m lies in [m/S, (m+1)/S), so only m in [floor(S C_t / Z) - 1, floor(S C_{t+1} / Z) + 1]
// can land in chunk t; for i.i.d. sampling every m is tested. The chunk's keys are contiguous, so the
// deduplication is a per-key counter in LDS; the chunk appends (key, per-head counts) records to its
// group's list (an atomic length per group). The gather kernel then reads each group's list, loads
// each row once (8 rows in flight per lane), accumulates count * V in fp64 (exact products,
// order-independent sums), and writes round(sum / S) in the output dtype. Work passes from one
// kernel to the next through the kernel boundary: on this chip a device-scope fence inside a kernel
// writes back the whole L2 of the XCD, which is far more expensive than one boundary.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;
constexpr int BATCH = 8;   // V rows in flight per lane in the group tail

__device__ inline double point_of(const Problem& p, int m, int h, int b, double u_sys) {
  if (p.mode == 0) return uniform53(p.seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
  if (p.mode == 1) {
    const double u = uniform53(p.seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
    return ((double)m + u) / (double)p.S;
  }
  return ((double)m + u_sys) / (double)p.S;
}

// first j in [0, len) with P[j] * f > r, else -1 (P nondecreasing up to rounding)
__device__ inline int search_chunk(const double* P, int len, double f, double r) {
  int lo = 0, hi = len;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] * f > r) hi = mid; else lo = mid + 1;
  }
  return lo < len ? lo : -1;
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
  constexpr size_t RESOLVE_BYTES = (size_t)GM * CHUNK * sizeof(double) + (size_t)CHUNK * (GM / 2 + 1) * 4;
  constexpr size_t TAIL_BYTES = (size_t)NWAVE * GM * D * sizeof(double);
  __shared__ __align__(16) unsigned char smem[RESOLVE_BYTES > TAIL_BYTES ? RESOLVE_BYTES : TAIL_BYTES];
  double (*Pt)[CHUNK] = reinterpret_cast<double (*)[CHUNK]>(smem);                 // [GM][CHUNK]
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + (size_t)GM * CHUNK * sizeof(double));  // [CHUNK][GM/2+1]
  constexpr int CW = GM / 2 + 1;  // 32-bit words of 16-bit counters per key

  __shared__ double hC0[GM], hC1[GM], hF[GM], hZ[GM], hU[GM];
  __shared__ int hLo[GM], hN[GM], hLast[GM];
  __shared__ int s_owned, s_nuniq, s_base;
  __shared__ int wsum_i[NWAVE];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S, T = p.T;
  const int h0 = kv * G;
  const int grp = b * p.Hkv + kv;
  const int64_t n0 = (int64_t)t * CHUNK;
  const int len = (int)min((int64_t)CHUNK, p.nk - n0);

  // ---- this chunk's interval of the chunk CDF, per head, and the candidate points
  if (tid < G) {
    const int g = tid;
    const int64_t bh = (int64_t)b * p.H + h0 + g;
    const double* cdf = p.cdf + bh * (T + 1);
    const double c0 = cdf[t], c1 = cdf[t + 1], Z = cdf[T];
    const int lastc = p.lastpos[bh];
    hC0[g] = c0;
    hC1[g] = c1;
    hZ[g] = Z;
    hF[g] = p.cscale[bh * T + t];
    hLast[g] = lastc;
    hU[g] = p.mode == 2 ? uniform53(p.seed, 0u, (uint32_t)(h0 + g), (uint32_t)b, TAG_SYS) : 0.0;
    int lo = 0, n = 0;
    const bool has_mass = c1 > c0 || t == lastc;
    if (has_mass) {
      if (p.mode == 0) {
        lo = 0;
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
  if (tid == 0) {
    s_owned = 0;
    s_nuniq = 0;
  }
  __syncthreads();

  // debug: probabilities of this chunk's keys from the score pass's exponentials
  if (p.prob) {
    for (int i = tid; i < G * len; i += THREADS) {
      const int g = i / len, k = i % len;
      double* pr = p.prob + ((int64_t)b * p.H + h0 + g) * p.nk + n0 + k;
      *pr = *pr * hF[g] / hZ[g];
    }
  }

  int total = 0;
  for (int g = 0; g < G; ++g) total += hN[g];

  // pass 1: does any candidate land in this chunk?
  auto owned = [&](int g, double y) {
    return y < hZ[g] ? (hC0[g] <= y && y < hC1[g]) : (t == hLast[g]);
  };
  int mine = 0;
  for (int c = tid; c < total; c += THREADS) {
    int g = 0, off = c;
    while (off >= hN[g]) off -= hN[g++];
    const int m = hLo[g] + off;
    const double y = point_of(p, m, h0 + g, b, hU[g]) * hZ[g];
    mine |= owned(g, y) ? 1 : 0;
  }
  if (mine) atomicOr(&s_owned, 1);
  __syncthreads();

  if (s_owned) {
    // the chunk's in-chunk prefixes and zeroed counters in LDS
    for (int i = tid; i < G * CHUNK; i += THREADS) {
      const int g = i / CHUNK, k = i % CHUNK;
      Pt[g][k] = k < len ? p.stash[((int64_t)b * p.H + h0 + g) * p.nk + n0 + k] : 0.0;
    }
    for (int i = tid; i < CHUNK * CW; i += THREADS) cnt[i] = 0u;
    __syncthreads();
    // pass 2: resolve the owned points
    for (int c = tid; c < total; c += THREADS) {
      int g = 0, off = c;
      while (off >= hN[g]) off -= hN[g++];
      const int m = hLo[g] + off;
      const double y = point_of(p, m, h0 + g, b, hU[g]) * hZ[g];
      if (!owned(g, y)) continue;
      int j;
      if (y < hZ[g]) {
        j = search_chunk(Pt[g], len, hF[g], y - hC0[g]);
        if (j < 0) j = last_positive(Pt[g], len);  // residual reached the chunk total through rounding
      } else {
        j = last_positive(Pt[g], len);
      }
      p.idx[((int64_t)b * p.H + h0 + g) * S + m] = (int32_t)(n0 + j);
      atomicAdd(&cnt[j * CW + (g >> 1)], (g & 1) ? 0x10000u : 1u);
    }
    __syncthreads();
    // compact the chunk's sampled keys into the group's row list
    const int k = tid;  // THREADS == CHUNK
    bool any = false;
    if (k < len) {
#pragma unroll
      for (int w = 0; w < CW; ++w) any |= cnt[k * CW + w] != 0u;
    }
    const uint64_t bal = __ballot(any);
    const int rank_w = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum_i[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, nu = 0;
    for (int w = 0; w < NWAVE; ++w) {
      if (w < wave) before += wsum_i[w];
      nu += wsum_i[w];
    }
    if (tid == 0) s_base = atomicAdd(&p.counters[grp], nu);
    __syncthreads();
    if (any) {
      const int slot = s_base + before + rank_w;
      if (slot < G * S) {  // a group never has more distinct rows than samples
        RowRecord rec;
        rec.key = (int32_t)(n0 + k);
#pragma unroll
        for (int w = 0; w < 4; ++w) rec.counts[w] = w < CW ? cnt[k * CW + w] : 0u;
        rec.pad[0] = rec.pad[1] = rec.pad[2] = 0;
        p.rows[(int64_t)grp * G * S + slot] = rec;
      }
    }
  }

}

template <int D, bool BF16, int GM>
__global__ __launch_bounds__(THREADS) void gather_kernel(Problem p) {
  using Pc = Piece<BF16>;
  constexpr int EPL = Pc::EPL;
  constexpr int LPR = D / EPL;          // lanes per V row
  constexpr int NRG = THREADS / LPR;    // row groups
  constexpr int NWAVE = THREADS / 64;
  __shared__ __align__(16) unsigned char smem[(size_t)NWAVE * GM * D * sizeof(double)];
  const int kv = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S;
  const int h0 = kv * G;
  const int grp = b * p.Hkv + kv;
  const int U = min(p.counters[grp], G * S);
  const RowRecord* recs = p.rows + (int64_t)grp * G * S;
  const int rg = tid / LPR, pc = tid % LPR;
  double acc[GM][EPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0;
  const size_t esz = BF16 ? 2 : 4;
  const char* vbase = (const char*)p.V + esz * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
  const int64_t rstride = esz * p.seq_stride;
  for (int u0 = rg; u0 < U; u0 += NRG * BATCH) {
    // records first, then every row load back to back (entries past U re-read the first record's row
    // and are added with count 0), then the accumulation
    constexpr int NCW = GM / 2;  // count words used
    int32_t key[BATCH];
    uint32_t cw[BATCH][NCW];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = u0 + k * NRG;
      const RowRecord* rr = recs + (u < U ? u : 0);
      key[k] = rr->key;
#pragma unroll
      for (int w = 0; w < NCW; ++w) cw[k][w] = u < U ? rr->counts[w] : 0u;
    }
    uint4 w4[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int64_t row = min((int64_t)max(key[k], 0), p.nk - 1);  // never address V outside the cache
      w4[k] = load_stream16((const uint4*)(vbase + row * rstride) + pc);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      double v[EPL];
      Pc::to_f64(w4[k], v);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        const uint32_t c32 = cw[k][g >> 1];
        const double c = (double)((g & 1) ? (c32 >> 16) : (c32 & 0xFFFFu));
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
      double x = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      acc[g][e] = x;
    }
  __syncthreads();
  double* wsum = reinterpret_cast<double*>(smem);  // [NWAVE][GM][D]
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
    for (int w2 = 0; w2 < NWAVE; ++w2) tot += wsum[((size_t)w2 * GM + g) * D + e];
    const double r = tot / dS;
    const int64_t o = ((int64_t)b * p.H + h0 + g) * D + e;
    if (BF16)
      ((uint16_t*)p.out)[o] = f64_to_bf16_rne(r);
    else
      ((float*)p.out)[o] = (float)r;
  }
  if (tid == 0) {
    p.unique[grp] = U;
    p.counters[grp] = 0;  // the list is consumed: ready for the next call
  }
}

template <int D, bool BF16>
hipError_t launch_dt(const Problem& p, hipStream_t st) {
  dim3 grid(p.T, p.Hkv, p.B);
  if (p.G <= 2)
    resolve_kernel<D, BF16, 2><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 4)
    resolve_kernel<D, BF16, 4><<<grid, THREADS, 0, st>>>(p);
  else
    resolve_kernel<D, BF16, 8><<<grid, THREADS, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_gather_dt(const Problem& p, hipStream_t st) {
  dim3 grid(p.Hkv, p.B);
  if (p.G <= 2)
    gather_kernel<D, BF16, 2><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 4)
    gather_kernel<D, BF16, 4><<<grid, THREADS, 0, st>>>(p);
  else
    gather_kernel<D, BF16, 8><<<grid, THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_resolve(const Problem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_dt<128, true>(p, st) : launch_dt<128, false>(p, st);
  return p.bf16 ? launch_dt<64, true>(p, st) : launch_dt<64, false>(p, st);
}

hipError_t launch_gather(const Problem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_gather_dt<128, true>(p, st) : launch_gather_dt<128, false>(p, st);
  return p.bf16 ? launch_gather_dt<64, true>(p, st) : launch_gather_dt<64, false>(p, st);
}

}  // namespace santa
