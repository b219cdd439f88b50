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
constexpr int BATCH = 2;   // V rows in flight per lane

// Compaction of the keys counted in `cnt` (16-bit per-head counts, thread k owns key k), gather of their
// V rows (each row once for the whole group, count * V into fp32 accumulators), and the chunk's partial
// sums per head (App. O, Algorithm 5, its value-accumulation step). Ends with every thread past a barrier; `Pt` is reused
// for the cross-wave sums.
template <int D, bool BF16, int GM>
__device__ inline void chunk_gather(const Problem& p, int t, int kv, int b, int len, uint32_t* cnt,
                                    int32_t* lkey, uint32_t (*lcnt)[GM / 2], int* wsum_i, double (*Pt)[CHUNK]) {
  // 4 elements per lane (8 bytes of bf16 or 16 of fp32): the per-head accumulators stay small enough for
  // eight resident blocks per CU, which large grids need more than wide loads for a handful of rows
  constexpr int EPL = 4;
  constexpr int LPR = D / EPL;          // lanes per V row
  constexpr int NRG = THREADS / LPR;    // row groups
  constexpr int NWAVE = THREADS / 64;
  constexpr int NCW = GM / 2;
  constexpr int CW = NCW + 1;
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, T = p.T;
  const int grp = b * p.Hkv + kv;
  const int64_t n0 = (int64_t)t * CHUNK;
  const size_t esz = BF16 ? 2 : 4;
  const char* vbase = (const char*)p.V + esz * ((int64_t)b * p.batch_stride + n0 * p.seq_stride + (int64_t)kv * D);
  const int64_t rstride = esz * p.seq_stride;
  (void)len;
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
    float vv[BATCH][EPL];
    if constexpr (BF16) {
      u32x2_t w2[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k)
        w2[k] = __builtin_nontemporal_load((const u32x2_t*)(vbase + key[k] * rstride) + pc);
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        vv[k][0] = bf16_lo(w2[k].x);
        vv[k][1] = bf16_hi(w2[k].x);
        vv[k][2] = bf16_lo(w2[k].y);
        vv[k][3] = bf16_hi(w2[k].y);
      }
    } else {
#pragma unroll
      for (int k = 0; k < BATCH; ++k) Piece<false>::to_f32(load_stream16((const uint4*)(vbase + key[k] * rstride) + pc), vv[k]);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const float* v = vv[k];
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

// PER > 0: the chunk CDF is computed here from the chunk statistics (T <= 64 * PER, the same arithmetic
// as the chunk CDF kernel, so every block of a head sees the same edges); PER == 0: it is read from the
// chunk CDF kernel's output. Wave w handles heads w and w + 4 of the group up to the key counts, so a
// wave searches only the prefix rows it wrote itself.
template <int D, bool BF16, int GM, int PER>
__global__ __launch_bounds__(THREADS) void resolve_kernel(Problem p) {
  using Pc = Piece<BF16>;
  constexpr int EPL = Pc::EPL;
  constexpr int LPR = D / EPL;          // lanes per V row
  constexpr int NRG = THREADS / LPR;    // row groups
  constexpr int NWAVE = THREADS / 64;
  constexpr int HPW = (GM + NWAVE - 1) / NWAVE;  // heads per wave
  constexpr int NCW = GM / 2;           // 32-bit words of 16-bit per-head counts
  constexpr int CW = NCW + 1;           // padded stride of the per-key counters
  constexpr int ROWB = D * (BF16 ? 2 : 4);
  constexpr int PFL = ROWB >= 128 ? ROWB / 128 : 1;  // 128-byte lines per V row
  constexpr int PERL = PER > 0 ? PER : 1;
  static_assert((size_t)NWAVE * GM * D * sizeof(float) <= (size_t)GM * CHUNK * sizeof(double),
                "the cross-wave sums reuse the prefix tile");

  __shared__ double Pt[GM][CHUNK];      // in-chunk prefixes; later the cross-wave sums
  __shared__ uint32_t cnt[CHUNK * CW];
  __shared__ int32_t lkey[CHUNK];
  __shared__ uint32_t lcnt[CHUNK][NCW];
  __shared__ int wsum_i[NWAVE];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S, T = p.T;
  const int h0 = kv * G;
  const int grp = b * p.Hkv + kv;
  const int64_t bh0 = (int64_t)b * p.H + h0;
  const int64_t n0 = (int64_t)t * CHUNK;
  const int len = (int)min((int64_t)CHUNK, p.nk - n0);
  const size_t esz = BF16 ? 2 : 4;
  const char* vbase = (const char*)p.V + esz * ((int64_t)b * p.batch_stride + n0 * p.seq_stride + (int64_t)kv * D);
  const int64_t rstride = esz * p.seq_stride;

  // ---- the loads of the sampling phase (heads clamped to G - 1 and keys to the chunk's last key, so every
  //      address is valid): this wave's heads' chunk CDF inputs first, then, when the chunk CDF is built
  //      here, its prefix rows at once (with a precomputed chunk CDF they are read per head once a point
  //      is known to fall in the chunk).
  //      Loads complete in issue order as far as the wait counter is concerned, so the chunk CDF can be
  //      built as soon as its few inputs have landed, while the prefix rows (the bulk of the bytes every
  //      block requests at once) are still in flight.
  double pv[HPW][4];
  double cm[HPW][PERL], cl[HPW][PERL];
  double e0[HPW], e1[HPW], eZ[HPW], eF[HPW];
  int eL[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int64_t bh = bh0 + min(wave + NWAVE * hh, G - 1);
    if constexpr (PER > 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int tt = min(lane * PER + j, T - 1);
        cm[hh][j] = p.cmax[bh * T + tt];
        cl[hh][j] = p.csum[bh * T + tt];
      }
    } else {
      const double* cdf = p.cdf + bh * (T + 1);
      e0[hh] = cdf[t];
      e1[hh] = cdf[t + 1];
      eZ[hh] = cdf[T];
      eF[hh] = p.cscale[bh * T + t];
      eL[hh] = p.lastpos[bh];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the prefix-row loads behind the statistics loads
  if constexpr (PER > 0) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int64_t bh = bh0 + min(wave + NWAVE * hh, G - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[hh][i] = p.stash[bh * p.stash_stride + n0 + min(4 * lane + i, len - 1)];
    }
  }
  for (int i = tid; i < CHUNK * CW; i += THREADS) cnt[i] = 0u;
  __syncthreads();  // counters zeroed before any wave counts (does not wait for the loads above)

  int jpf[HPW];  // a sampled key of each of this lane's heads (key 0 if none), for cache warming
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) jpf[hh] = 0;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int g = wave + NWAVE * hh;
    if (g >= G) break;  // wave-uniform
    double c0, c1, Z, f;
    int lastc;
    if constexpr (PER > 0) {
      ChunkCdf<PER> o;
      chunk_cdf_wave<PER>(cm[hh], cl[hh], T, lane, o);
      c0 = readlane_f64(pick<PER>(o.c, t % PER), t / PER);
      c1 = t + 1 < T ? readlane_f64(pick<PER>(o.c, (t + 1) % PER), (t + 1) / PER) : o.top;
      f = readlane_f64(pick<PER>(o.f, t % PER), t / PER);
      Z = o.top;
      lastc = o.last;
    } else {
      c0 = e0[hh];
      c1 = e1[hh];
      Z = eZ[hh];
      f = eF[hh];
      lastc = eL[hh];
    }
    // this head's prefix row, written and then searched by this wave only
    if constexpr (PER > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Pt[g][4 * lane + i] = pv[hh][i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    if (p.prob) {  // debug: probabilities of this chunk's keys from the score pass's exponentials
      double* pr = p.prob + (bh0 + g) * p.nk + n0;
      for (int k = lane; k < len; k += 64) pr[k] = pr[k] * f / Z;
    }
    const double u_sys = p.mode == 2 ? uniform53(p.seed, 0u, (uint32_t)(h0 + g), (uint32_t)b, TAG_SYS) : 0.0;
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
    if constexpr (PER <= 0) {
      // with the chunk CDF known from the start, the prefix row is read only when one of the head's
      // points falls in this chunk (many chunks hold none): the points are tested first, then found again
      bool any = false;
      for (int c = lane; c < n; c += 64) {
        const double y = point_of(p.seed, p.mode, p.S, lo + c, h0 + g, b, u_sys) * Z;
        any = any || (y < Z ? (c0 <= y && y < c1) : (t == lastc));
      }
      if (__ballot(any) == 0ull) continue;  // wave-uniform
      const int64_t bh = bh0 + g;
      double v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = p.stash[bh * p.stash_stride + n0 + min(4 * lane + i, len - 1)];
#pragma unroll
      for (int i = 0; i < 4; ++i) Pt[g][4 * lane + i] = v[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    for (int c = lane; c < n; c += 64) {
      const int m = lo + c;
      const double y = point_of(p.seed, p.mode, p.S, m, h0 + g, b, u_sys) * Z;
      const bool mine = y < Z ? (c0 <= y && y < c1) : (t == lastc);
      if (!mine) continue;
      int j;
      if (y < Z) {
        j = search_chunk(Pt[g], f, y - c0);
        if (j < 0) j = last_positive(Pt[g], len);  // the residual reached the chunk total through rounding
      } else {
        j = last_positive(Pt[g], len);
      }
      j = min(j, len - 1);  // keeps the gather inside the cache even if the score pass flagged a timeout
      p.idx[(bh0 + g) * S + m] = (int32_t)(n0 + j);
      atomicAdd(&cnt[j * CW + (g >> 1)], (g & 1) ? 0x10000u : 1u);
      jpf[hh] = j;
    }
  }
  // warm the caches with rows the gather below will read; the values are consumed only at the very end,
  // so nothing waits for these loads before the gather's own loads of the same lines
  uint32_t warm[HPW][PFL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int L = 0; L < PFL; ++L) warm[hh][L] = *(const uint32_t*)(vbase + jpf[hh] * rstride + L * 128);
  __syncthreads();

  chunk_gather<D, BF16, GM>(p, t, kv, b, len, cnt, lkey, lcnt, wsum_i, Pt);
  uint32_t sink = 0u;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int L = 0; L < PFL; ++L) sink ^= warm[hh][L];
  if (lane == 0) p.sink[(int64_t)grp * T + t] = sink;  // keeps the cache-warming loads
}

// S²ANTA-prop, pass 2 (Appendix O, Algorithm 5): the chunk (= tile) of each head has budget S_t; with
// x_n = (S_t / l_t) u_n and a0 ~ U(0,1) from Philox counter (t, h, b, 3), key n of the tile is sampled
// c_n = floor(a0 + P_n) - floor(a0 + P_{n-1}) times, P_n = (S_t / l_t) * (in-chunk prefix of u up to n)
// (the running sum p of Algorithm 5, taken from the score pass's prefix). Thread n owns key n for every
// head, so the counts need no atomics; the sampled keys fill idx slots
// [off_t + floor(a0 + P_{n-1}), off_t + floor(a0 + P_n)) of the head's list.
// PER > 0: each wave computes the budgets of its heads itself (tile_budget_wave, T <= 64 * PER), so the
// budget kernel is not launched; PER == 0: the budgets come from the budget kernel.
// PER < 0: S²ANTA-flash, kernel 1 ("Stochastic Sparse Attention for Memory-Bound Inference", Section 3.3
// and Appendix P, Algorithm 7): every tile has the same budget S_tile, its slots are [t S_tile, (t+1)
// S_tile), a0 comes from Philox counter (t, h, b, 4), and the partials are reweighted by the merge.
template <int D, bool BF16, int GM, int PER>
__global__ __launch_bounds__(THREADS) void resolve_prop_kernel(Problem p) {
  constexpr bool FLASH = PER < 0;
  constexpr int NCW = GM / 2;
  constexpr int CW = NCW + 1;
  constexpr int NWAVE = THREADS / 64;
  constexpr int HPW = (GM + NWAVE - 1) / NWAVE;  // heads per wave
  constexpr int PL = PER > 0 ? PER : 1;
  __shared__ double Pt[GM][CHUNK];
  __shared__ uint32_t cnt[CHUNK * CW];
  __shared__ int32_t lkey[CHUNK];
  __shared__ uint32_t lcnt[CHUNK][NCW];
  __shared__ int wsum_i[NWAVE];
  __shared__ double hInv[GM], hA0[GM], hF[GM], hZ[GM];
  __shared__ int hS[GM], hOff[GM];
  __shared__ int hist[PER > 0 ? NWAVE : 1][256];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, S = p.S, T = p.T;
  const int h0 = kv * G;
  const int64_t bh0 = (int64_t)b * p.H + h0;
  const int64_t n0 = (int64_t)t * CHUNK;
  const int len = (int)min((int64_t)CHUNK, p.nk - n0);

  // every load at once (heads clamped to G - 1, keys to the chunk's last key, tiles to T - 1): the tile
  // statistics and budgets first, the prefix rows (the bulk of the bytes) last, so that the budgets can
  // be formed while the prefix rows are still in flight (wait counters retire loads in issue order)
  double pv[HPW][4];
  double cm[HPW][PL], cl[HPW][PL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int64_t bh = bh0 + min(wave + NWAVE * hh, G - 1);
    if constexpr (PER > 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int tt = min(lane * PER + j, T - 1);
        cm[hh][j] = p.cmax[bh * T + tt];
        cl[hh][j] = p.csum[bh * T + tt];
      }
    }
  }
  const int64_t bhg = bh0 + min(tid, G - 1);
  const double lt = p.csum[bhg * T + t];
  int Bt = 0, off = 0;
  double f = 0.0, Z = 0.0;
  if constexpr (FLASH) {
    Bt = p.S_tile;
    off = t * p.S_tile;
  } else if constexpr (PER == 0) {
    Bt = p.budget[bhg * T + t];
    off = p.boff[bhg * T + t];
    f = p.cscale[bhg * T + t];
    Z = p.cdf[bhg * (T + 1) + T];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the prefix-row loads behind the statistics loads
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int64_t bh = bh0 + min(wave + NWAVE * hh, G - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[hh][i] = p.stash[bh * p.stash_stride + n0 + min(4 * lane + i, len - 1)];
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int g = wave + NWAVE * hh;
    if constexpr (PER > 0) {
      if (g < G) {
        const TileBudget r = tile_budget_wave<PER>(cm[hh], cl[hh], T, S, t, lane, hist[wave]);
        if (lane == 0) {
          hS[g] = r.st;
          hOff[g] = r.off;
          hF[g] = r.f;
          hZ[g] = r.Z;
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int g = wave + NWAVE * hh;
    if (g < GM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Pt[g][4 * lane + i] = pv[hh][i];
    }
  }
  if (tid < G) {
    if constexpr (PER <= 0) {
      hS[tid] = Bt;
      hOff[tid] = off;
      hF[tid] = f;
      hZ[tid] = Z;
    }
    hA0[tid] = uniform53(p.seed, (uint32_t)t, (uint32_t)(h0 + tid), (uint32_t)b, FLASH ? TAG_FLASH : TAG_PROP);
  }
  __syncthreads();
  if (tid < G) hInv[tid] = hS[tid] > 0 ? (double)hS[tid] / lt : 0.0;
  __syncthreads();

  if (!FLASH && p.prob) {  // debug: probabilities of this chunk's keys from the score pass's exponentials
    for (int i = tid; i < G * len; i += THREADS) {
      const int g = i / len, k = i % len;
      double* pr = p.prob + (bh0 + g) * p.nk + n0 + k;
      *pr = *pr * hF[g] / hZ[g];
    }
  }

  uint32_t w[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) w[i] = 0u;
  if (tid < len) {
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= G || hS[g] == 0) continue;
      const double inv = hInv[g], a0 = hA0[g];
      const double ylo = a0 + inv * (tid > 0 ? Pt[g][tid - 1] : 0.0);
      const double yhi = a0 + inv * Pt[g][tid];
      const int lo = (int)floor(ylo), hi = (int)floor(yhi);
      const int c = hi > lo ? min(hi - lo, hS[g]) : 0;
      int32_t* dst = p.idx + (bh0 + g) * p.L + hOff[g];
      for (int i = 0; i < c; ++i)  // slots outside the tile's budget are never written
        if (lo + i >= 0 && lo + i < hS[g]) dst[lo + i] = (int32_t)(n0 + tid);
      w[g >> 1] += (g & 1) ? ((uint32_t)c << 16) : (uint32_t)c;
    }
  }
#pragma unroll
  for (int i = 0; i < NCW; ++i) cnt[tid * CW + i] = w[i];
  __syncthreads();
  chunk_gather<D, BF16, GM>(p, t, kv, b, len, cnt, lkey, lcnt, wsum_i, Pt);
}

// Whether a bounded wait of the streaming score kernel gave up in one of group grp's blocks (their
// handshake flags); the merge then writes NaN for the group's heads. `writer` (one block per group)
// records the outcome in the group's status word, which every call writes. Block-uniform; ends with a
// barrier.
__device__ inline bool group_flagged(const Problem& p, int grp, bool writer) {
  int f = 0;
  if (p.check_sync) {
    const int P = p.score_blocks_per_group;
    for (int i = threadIdx.x; i < P; i += blockDim.x) f |= p.sync_err[(int64_t)grp * P + i];
  }
  const bool any = __syncthreads_or(f != 0) != 0;
  if (writer && threadIdx.x == 0) p.status[grp] = any ? 1 : 0;
  return any;
}

// out[b, h] = round((sum over chunks of the partials of head h) / S). One block per (head, sequence, group
// of MCOLS columns of the head dimension), so a head's partials are read by D / MCOLS CUs: MCOLS / 4
// float4 columns x TS chunk slices (TS = 4096 / D); slice ts adds chunks ts, ts + TS, ... in fp64 in that
// order (MB loads in flight per thread, one round for T <= TS * MB), then the slices are added in order:
// a fixed order for every call.
constexpr int MTHREADS = 1024;  // threads over a whole row: sets the slice count
constexpr int MCOLS = 32;       // head-dimension columns per block
template <int D>
constexpr int merge_slices() { return MTHREADS / (D / 4); }
template <int D>
constexpr int merge_threads() { return MCOLS / 4 * merge_slices<D>(); }
template <int D, bool BF16, int MB>
__global__ __launch_bounds__(merge_threads<D>()) void merge_kernel(Problem p) {
  constexpr int V4 = MCOLS / 4;          // float4 pieces per block row
  constexpr int TS = merge_slices<D>();  // chunk slices
  __shared__ double red[TS][MCOLS];
  const int h = blockIdx.x, b = blockIdx.y, col0 = blockIdx.z * MCOLS;
  const int tid = threadIdx.x;
  const int G = p.G, T = p.T;
  const int kv = h / G, g = h % G;
  const bool poisoned = group_flagged(p, b * p.Hkv + kv, g == 0 && blockIdx.z == 0);
  const int c = tid % V4, ts = tid / V4;
  const float* base = p.partial + ((int64_t)(b * p.Hkv + kv) * T * G + g) * D + col0 + 4 * c;
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
  if (tid < MCOLS) {
    double tot = 0.0;
#pragma unroll 8
    for (int s2 = 0; s2 < TS; ++s2) tot += red[s2][tid];
    const double r = tot / (double)p.S;
    const int64_t o = ((int64_t)b * p.H + h) * D + col0 + tid;
    if (BF16)
      ((uint16_t*)p.out)[o] = poisoned ? (uint16_t)0x7FC0u : f64_to_bf16_rne(r);
    else
      ((float*)p.out)[o] = poisoned ? __uint_as_float(0x7FC00000u) : (float)r;
  }
}

// S²ANTA-flash, kernel 2 ("Stochastic Sparse Attention for Memory-Bound Inference", Appendix P,
// Algorithm 8), one block per (query head, sequence): m* = max_t m_t, W_t = exp(m_t - m*) l_t,
// Z = sum_t W_t, and out = (sum_t W_t Otilde_t) / (Z S_tile) with Otilde_t the fp32 tile partials; the
// weighted sums run in fp64 in tile order within each of the TS slices, the slices are added in order.
template <int D, bool BF16>
__global__ __launch_bounds__(THREADS) void merge_flash_kernel(Problem p) {
  constexpr int V4 = D / 4;            // float4 pieces per row
  constexpr int TS = THREADS / V4;     // tile slices
  constexpr int MB = 16;               // loads in flight per thread
  constexpr int NW = THREADS / 64;
  __shared__ double red[TS][D];
  __shared__ double wt[MAX_CHUNKS];
  __shared__ double bred[NW];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, T = p.T;
  const int kv = h / G, g = h % G;
  const int64_t bh = (int64_t)b * p.H + h;
  const bool poisoned = group_flagged(p, b * p.Hkv + kv, g == 0);

  double mx = -INFINITY;
  for (int t = tid; t < T; t += THREADS) mx = fmax(mx, p.cmax[bh * T + t]);
  const double ms = block_max_f64<NW>(mx, bred, lane, wave);
  double part = 0.0;
  for (int t = tid; t < T; t += THREADS) {
    const double w = exp_f64(p.cmax[bh * T + t] - ms) * p.csum[bh * T + t];
    wt[t] = w;
    part += w;
  }
  const double Z = block_sum_f64<NW>(part, bred, lane, wave);  // its barriers also publish wt[]

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
      const int tt = t0 + k * TS;
      if (tt < T) {
        const double w = wt[tt];
        a0 += w * (double)v[k].x;
        a1 += w * (double)v[k].y;
        a2 += w * (double)v[k].z;
        a3 += w * (double)v[k].w;
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
    const double r = tot / (Z * (double)p.S_tile);
    const int64_t o = bh * D + tid;
    if (BF16)
      ((uint16_t*)p.out)[o] = poisoned ? (uint16_t)0x7FC0u : f64_to_bf16_rne(r);
    else
      ((float*)p.out)[o] = poisoned ? __uint_as_float(0x7FC00000u) : (float)r;
  }
  if (p.fused && p.want_unique && g == 0) {
    // per chunk: distinct sampled keys (union of the heads' key bits) and V rows actually read (every head
    // reads its own sampled rows, so the sum of the heads' bit counts), the latter after all B * Hkv * T
    const int grp = b * p.Hkv + kv;
    for (int t = tid; t < T; t += THREADS) {
      const uint64_t* bm = p.bmap + ((int64_t)grp * T + t) * 16;
      int u = 0, rd = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint64_t w = 0;
        for (int gg = 0; gg < G; ++gg) {
          w |= bm[gg * 4 + i];
          rd += __popcll(bm[gg * 4 + i]);
        }
        u += __popcll(w);
      }
      p.unique[(int64_t)grp * T + t] = u;
      p.unique[(int64_t)p.B * p.Hkv * T + (int64_t)grp * T + t] = rd;
    }
  }
  if (p.prob) {  // debug: probabilities from the score pass's exponentials, exp(s - m_t) exp(m_t - m*) / Z
    double* pr = p.prob + bh * p.nk;
    for (int64_t n = tid; n < p.nk; n += THREADS) {
      const int t = (int)(n / CHUNK);
      pr[n] = pr[n] * exp_f64(p.cmax[bh * T + t] - ms) / Z;
    }
  }
}

template <int D, bool BF16, int GM>
hipError_t launch_resolve_g(const Problem& p, hipStream_t st) {
  const dim3 grid(p.T, p.Hkv, p.B);
  if (p.cdf_done)
    resolve_kernel<D, BF16, GM, 0><<<grid, THREADS, 0, st>>>(p);
  else if (p.T <= 64)
    resolve_kernel<D, BF16, GM, 1><<<grid, THREADS, 0, st>>>(p);
  else if (p.T <= FUSED_CDF_MAX_T)
    resolve_kernel<D, BF16, GM, 2><<<grid, THREADS, 0, st>>>(p);
  else
    return hipErrorInvalidValue;  // T > FUSED_CDF_MAX_T always runs the chunk CDF kernel first
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_resolve_dt(const Problem& p, hipStream_t st) {
  if (p.G <= 2) return launch_resolve_g<D, BF16, 2>(p, st);
  if (p.G <= 4) return launch_resolve_g<D, BF16, 4>(p, st);
  return launch_resolve_g<D, BF16, 8>(p, st);
}

}  // namespace

template <int D, bool BF16, int GM>
hipError_t launch_prop_g(const Problem& p, hipStream_t st) {
  const dim3 grid(p.T, p.Hkv, p.B);
  if (p.mode == 4)
    resolve_prop_kernel<D, BF16, GM, -1><<<grid, THREADS, 0, st>>>(p);
  else if (p.T <= 64)
    resolve_prop_kernel<D, BF16, GM, 1><<<grid, THREADS, 0, st>>>(p);
  else if (p.T <= FUSED_CDF_MAX_T)
    resolve_prop_kernel<D, BF16, GM, 2><<<grid, THREADS, 0, st>>>(p);
  else
    resolve_prop_kernel<D, BF16, GM, 0><<<grid, THREADS, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_prop_dt(const Problem& p, hipStream_t st) {
  if (p.G <= 2) return launch_prop_g<D, BF16, 2>(p, st);
  if (p.G <= 4) return launch_prop_g<D, BF16, 4>(p, st);
  return launch_prop_g<D, BF16, 8>(p, st);
}

hipError_t launch_resolve(const Problem& p, hipStream_t st) {
  if (p.mode == 3 || p.mode == 4) {
    if (p.d == 128) return p.bf16 ? launch_prop_dt<128, true>(p, st) : launch_prop_dt<128, false>(p, st);
    return p.bf16 ? launch_prop_dt<64, true>(p, st) : launch_prop_dt<64, false>(p, st);
  }
  if (p.d == 128) return p.bf16 ? launch_resolve_dt<128, true>(p, st) : launch_resolve_dt<128, false>(p, st);
  return p.bf16 ? launch_resolve_dt<64, true>(p, st) : launch_resolve_dt<64, false>(p, st);
}

hipError_t launch_merge(const Problem& p, hipStream_t st) {
  dim3 grid(p.H, p.B);
  if (p.mode == 4) {
    if (p.d == 128) {
      if (p.bf16) merge_flash_kernel<128, true><<<grid, THREADS, 0, st>>>(p);
      else merge_flash_kernel<128, false><<<grid, THREADS, 0, st>>>(p);
    } else {
      if (p.bf16) merge_flash_kernel<64, true><<<grid, THREADS, 0, st>>>(p);
      else merge_flash_kernel<64, false><<<grid, THREADS, 0, st>>>(p);
    }
    return hipGetLastError();
  }
  // loads in flight per thread: one round for up to 128 chunks (d = 128: 32 slices x 4), else 16 per round
  const bool small = p.T <= MTHREADS / 32 * 4;
  const dim3 mgrid(p.H, p.B, p.d / MCOLS);
  if (p.d == 128) {
    constexpr int NT = merge_threads<128>();
    if (small) {
      if (p.bf16) merge_kernel<128, true, 4><<<mgrid, NT, 0, st>>>(p);
      else merge_kernel<128, false, 4><<<mgrid, NT, 0, st>>>(p);
    } else {
      if (p.bf16) merge_kernel<128, true, 16><<<mgrid, NT, 0, st>>>(p);
      else merge_kernel<128, false, 16><<<mgrid, NT, 0, st>>>(p);
    }
  } else {
    constexpr int NT = merge_threads<64>();
    if (small) {
      if (p.bf16) merge_kernel<64, true, 4><<<mgrid, NT, 0, st>>>(p);
      else merge_kernel<64, false, 4><<<mgrid, NT, 0, st>>>(p);
    } else {
      if (p.bf16) merge_kernel<64, true, 16><<<mgrid, NT, 0, st>>>(p);
      else merge_kernel<64, false, 16><<<mgrid, NT, 0, st>>>(p);
    }
  }
  return hipGetLastError();
}

}  // namespace santa
