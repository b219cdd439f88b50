// Split-K score pass: blocks pinned to one (KV head, sequence) group, each looping over a strided set
// of CHUNK-key chunks of that group.
//
// "Stochastic Sparse Attention for Memory-Bound Inference", Appendix O, Algorithm 3 (pass-1 tile
// statistics with the optional stash) and Section 3.2 ("Pass 1"): for every query head h of the GQA
// group, s_{h,n} = q_h . K_n / sqrt(dk) (Eq. 1), the chunk max m_{h,t}, and the in-chunk exponentials
// exp(s_{h,n} - m_{h,t}). This pass stores their in-chunk inclusive prefix sums (the chunk's CDF up to
// the chunk's own scale) and l_{h,t} = the chunk total, which is what the sampler's inverse CDF needs.
//
// Two forms. The streaming form (bf16 caches, the usual case; described above score_stream_kernel)
// copies K tiles into LDS with global_load_lds and splits the work into copy, matrix-core and
// exponential waves. The register form below (fp32 caches) works as follows.
//
// MI355X design of the register form:
//   * K is streamed once with non-temporal 16-byte loads in full-row order (16 lanes cover a 256-byte
//     row), the next chunk's loads in flight while the current chunk is computed. The current chunk
//     sits in a padded LDS tile (row stride + 16 bytes), from which the matrix-core layout is read
//     without bank conflicts.
//   * Dot products run on the fp64 matrix cores (v_mfma_f64_4x4x4_4b: 4 blocks of 4 keys x 4 dims x
//     4 heads): lane l supplies key (l & 15) at dim slot (l >> 4) for A and head (l & 3) at dim slot
//     (l >> 4) for B, and receives the score of key 4*((l >> 2) & 3) + (l >> 4), head (l & 3); no
//     cross-lane reduction. Products of bf16 (or fp32) inputs are exact in fp64 and accumulate in fp64,
//     which the sampler's index parity needs. Four independent accumulation chains per wave.
//   * Softmax bookkeeping: a wave owns a head, a lane owns 4 consecutive keys: local max / exp /
//     prefix, then DPP wavefront max and scan (fp64).
//   * With the Bernoulli ternary query (Section 5, Eq. 5; Appendix C, Eqs. 8-9) the B operand holds
//     qhat in {-1, 0, +1} and the score is (qhat . K) * norm * (1/sqrt(dk)).

#include "common.h"
#include "launch.h"
#include "stream_kernel.h"

namespace santa {

namespace {

using namespace sk;

constexpr int THREADS = 256;   // 4 waves; 64 keys per wave, 16 keys per MFMA group
constexpr int GROUPS_PER_WAVE = 4;
static_assert(THREADS / 64 * GROUPS_PER_WAVE * 16 == CHUNK, "a block covers one chunk per iteration");
static_assert(4 * 64 == CHUNK, "a wave covers one chunk with 4 keys per lane in the softmax step");


template <int D, bool BF16>
struct Geo {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int ROWB = D * ESZ;              // bytes per K row
  static constexpr int NPR = ROWB / 16;             // 16-byte pieces per row
  static constexpr int RSTRIDE = ROWB + 16;         // padded LDS row stride (conflict-free MFMA reads)
  static constexpr int NLD = CHUNK * NPR / THREADS; // 16-byte loads per thread per chunk
  static constexpr int RPI = THREADS / NPR;         // rows covered by one block-wide load instruction
  static constexpr int EPL = 16 / ESZ;              // elements per piece
  static constexpr int PP = NPR / 4;                // pieces per lane per row in the MFMA layout
  static constexpr int LDS_K = CHUNK * RSTRIDE;
};

// full-row loads of chunk rows [n0, n0+len): load i covers row i*RPI + tid/NPR, piece tid%NPR; rows past
// the end re-read row n0 (always valid) so every load is unconditional; those keys are masked later.
// Loads [I0, I0 + N) only, so that a prefetch can be spread over the MFMA loop.
template <int D, bool BF16, int I0 = 0, int N = Geo<D, BF16>::NLD>
__device__ inline void load_rows(uint4* r, const char* kbase, int64_t seq_bytes, int64_t n0, int len, int tid) {
  using Gm = Geo<D, BF16>;
  const int piece = tid % Gm::NPR, row0 = tid / Gm::NPR;
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) {
    const int row = i * Gm::RPI + row0;
    r[i] = load_stream16(kbase + (n0 + (row < len ? row : 0)) * seq_bytes + piece * 16);
  }
}

template <int D, bool BF16>
__device__ inline void store_rows(unsigned char* ks, const uint4* r, int tid) {
  using Gm = Geo<D, BF16>;
  const int piece = tid % Gm::NPR, row0 = tid / Gm::NPR;
#pragma unroll
  for (int i = 0; i < Gm::NLD; ++i) *(uint4*)(ks + (i * Gm::RPI + row0) * Gm::RSTRIDE + piece * 16) = r[i];
}

// Chunk CDF (Appendix O, Algorithm 4: m* = max_t m_t, W_t = l_t exp(m_t - m*), Z = sum_t W_t) of the
// one (query head, sequence) per one-wave block, so every head's CDF is built at once: lane l owns a
// contiguous run of chunks; the prefix is exclusive, then made monotone by a running maximum so that
// the chunks' intervals [cdf_t, cdf_{t+1}) partition [0, Z) exactly. cdf[T] = Z.
// Register form: T <= 64 * PER and lane l owns chunks [l*PER, l*PER + PER), held in registers, so the statistics
// are read in one round trip. The plain form below takes any T: lane l owns a contiguous run of ceil(T/64)
// chunks, re-read from memory between the steps.
template <int PER>
__global__ __launch_bounds__(64) void chunk_cdf_reg_kernel(Problem p) {
  const int lane = threadIdx.x;
  const int T = p.T;
  const int t0 = lane * PER;
  {
    const int64_t bh = (int64_t)blockIdx.y * p.H + blockIdx.x;
    double m[PER], l[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int tt = min(t0 + j, T - 1);  // every lane loads a valid address; extra entries are masked
      m[j] = p.cmax[bh * T + tt];
      l[j] = p.csum[bh * T + tt];
    }
    ChunkCdf<PER> o;
    chunk_cdf_wave<PER>(m, l, T, lane, o);
    double* cdf = p.cdf + bh * (T + 1);
    double* csc = p.cscale + bh * T;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (t0 + j < T) {
        cdf[t0 + j] = o.c[j];
        csc[t0 + j] = o.f[j];
      }
    }
    if (lane == 0) {
      cdf[T] = o.top;
      p.lastpos[bh] = o.last;
    }
  }
}

__global__ __launch_bounds__(64) void chunk_cdf_kernel(Problem p) {
  const int lane = threadIdx.x;
  const int T = p.T;
  const int per = (T + 63) / 64;
  const int t0 = min(T, lane * per), t1 = min(T, t0 + per);
  {
    const int64_t bh = (int64_t)blockIdx.y * p.H + blockIdx.x;
    const double* cm = p.cmax + bh * T;
    const double* cs = p.csum + bh * T;
    double* cdf = p.cdf + bh * (T + 1);
    double* csc = p.cscale + bh * T;
    double mx = -INFINITY;
    for (int t = t0; t < t1; ++t) mx = fmax(mx, cm[t]);
    const double ms = readlane_f64(wave_incl_max_dpp(mx), 63);
    double run = 0.0;
    int lp = -1;
    for (int t = t0; t < t1; ++t) {
      const double f = exp_f64(cm[t] - ms);
      const double w = cs[t] * f;
      csc[t] = f;
      cdf[t] = run;  // local exclusive prefix, offset below
      run += w;
      if (w > 0.0) lp = t;
    }
    const double incl = wave_incl_scan_dpp(run);
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    double lmax = 0.0;
    for (int t = t0; t < t1; ++t) {
      const double c = fmax(excl + cdf[t], lmax);
      cdf[t] = c;
      lmax = c;
    }
    // running maximum across lanes: lane l's values are raised to the maximum of all earlier lanes
    const double pmax = wave_incl_max_dpp(t1 > t0 ? lmax : 0.0);
    double before = __shfl_up(pmax, 1, 64);
    if (lane == 0) before = 0.0;
    for (int t = t0; t < t1; ++t) cdf[t] = fmax(cdf[t], before);
    const double Z = readlane_f64(incl, 63);
    const double top = readlane_f64(pmax, 63);
    if (lane == 0) cdf[T] = fmax(Z, top);
    const double lpd = readlane_f64(wave_incl_max_dpp((double)lp), 63);
    if (lane == 0) p.lastpos[bh] = (int32_t)lpd;
  }
}

// NQ = number of 4-head quads (1: G <= 4, 2: G <= 8); MINB = resident blocks per CU the LDS allows
template <int D, bool BF16, int NQ, int MINB>
__global__ __launch_bounds__(THREADS, MINB) void score_kernel(Problem p) {
  using Gm = Geo<D, BF16>;
  constexpr int EPL = Gm::EPL, PP = Gm::PP;
  constexpr int HMAX = 4 * NQ;
  static_assert(CHUNK >= D + 2, "the query staging aliases the score tile");

  __shared__ __align__(16) unsigned char ks[Gm::LDS_K];
  __shared__ double sc[HMAX][CHUNK];
  __shared__ double hnorm[HMAX];
  double (*qe)[D + 2] = reinterpret_cast<double (*)[D + 2]>(&sc[0][0]);  // prologue only

  const int kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int h0 = kv * G;
  const int T = p.T;
  const int step = gridDim.x;
  int t = blockIdx.x;
  if (t >= T) return;

  const int64_t seq_bytes = (int64_t)Gm::ESZ * p.seq_stride;
  const char* kbase = (const char*)p.K + (int64_t)Gm::ESZ * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
  auto chunk_len = [&](int tt) { return (int)min((int64_t)CHUNK, p.nk - (int64_t)tt * CHUNK); };

  // ---- first chunk's loads before anything else
  uint4 r[Gm::NLD];
  load_rows<D, BF16>(r, kbase, seq_bytes, (int64_t)t * CHUNK, chunk_len(t), tid);

  // ---- effective query of each head of the group, fp64, staged in LDS then kept in registers
  using P = Piece<BF16>;
  const char* qbase = (const char*)p.q;
  for (int i = tid; i < HMAX * D; i += THREADS) {
    const int g = i / D, e = i % D;
    double v = 0.0;
    if (g < G) v = P::elem(qbase, ((int64_t)b * p.H + h0 + g) * D + e);
    qe[g][e] = v;
  }
  __syncthreads();
  if (p.ternary) {
    if (tid < HMAX) {
      double m = 0.0;
      for (int e = 0; e < D; ++e) m = fmax(m, fabs(qe[tid][e]));
      hnorm[tid] = m;
    }
    __syncthreads();
    for (int i = tid; i < HMAX * D; i += THREADS) {
      const int g = i / D, e = i % D;
      const double v = qe[g][e];
      const double nrm = hnorm[g];
      double rr = 0.0;
      if (g < G && nrm > 0.0) {
        const double u = uniform53(p.seed, (uint32_t)e, (uint32_t)(h0 + g), (uint32_t)b, TAG_BERNOULLI);
        if (u < fabs(v) / nrm) rr = v > 0.0 ? 1.0 : (v < 0.0 ? -1.0 : 0.0);
      }
      qe[g][e] = rr;
    }
    __syncthreads();
  }
  // B operand of lane l: head (quad*4 + (l & 3)), dim EPL*(4*pp + slot) + e
  const int slot = lane >> 4;
  double qb[NQ][PP][EPL];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qb[qd][pp][e] = qe[qd * 4 + (lane & 3)][EPL * (4 * pp + slot) + e];
  double mul[NQ];  // score multipliers of the heads this wave finalises (wave, wave + 4)
#pragma unroll
  for (int j = 0; j < NQ; ++j) mul[j] = p.ternary ? hnorm[wave + 4 * j] : 1.0;
  __syncthreads();  // the staging area is reused for scores

  // Results of a chunk (stash prefixes, chunk max and sum) are held in registers and stored after the
  // next chunk's K tile has reached LDS and before its prefetch is issued: stores issued behind a full
  // queue of streaming loads would stall the wave until those loads drain.
  double pend[NQ][4];
  double pend_m[NQ], pend_l[NQ];
  int64_t pend_n0 = -1;
  int pend_len = 0, pend_t = 0;
  auto flush = [&]() {
    if (pend_n0 < 0) return;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int g = wave + 4 * j;
      if (g >= G) break;
      const int64_t bh = (int64_t)b * p.H + h0 + g;
      double* dst = p.stash + bh * p.stash_stride + pend_n0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * lane + i < pend_len) dst[4 * lane + i] = pend[j][i];
      if (lane == 63) {
        p.cmax[bh * T + pend_t] = pend_m[j];
        p.csum[bh * T + pend_t] = pend_l[j];
      }
    }
  };

  for (; t < T; t += step) {
    const int len = chunk_len(t);
    const int64_t n0 = (int64_t)t * CHUNK;
    store_rows<D, BF16>(ks, r, tid);
    __syncthreads();
    flush();
    const int tn = t + step;
    const bool more = tn < T;
    const int64_t nn0 = (int64_t)tn * CHUNK;
    const int nlen = more ? chunk_len(tn) : 0;

    // ---- fp64 MFMA chains: one per 16-key group and head quad, interleaved; the next chunk's loads
    //      are spread over the pieces
    double acc[GROUPS_PER_WAVE][NQ];
#pragma unroll
    for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi)
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) acc[gi][qd] = 0.0;
    static_assert(Gm::NLD % PP == 0, "prefetch split over the pieces");
    constexpr int LPP = Gm::NLD / PP;
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      if (more) {
        switch (pp) {  // compile-time ranges; pp is unrolled
#define SANTA_PF(k) case k: if constexpr (k < PP) load_rows<D, BF16, k * LPP, LPP>(r, kbase, seq_bytes, nn0, nlen, tid); break;
          SANTA_PF(0) SANTA_PF(1) SANTA_PF(2) SANTA_PF(3) SANTA_PF(4) SANTA_PF(5) SANTA_PF(6) SANTA_PF(7)
#undef SANTA_PF
        }
      }
      uint4 a4[GROUPS_PER_WAVE];
#pragma unroll
      for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi)
        a4[gi] = *(const uint4*)(ks + (wave * 64 + gi * 16 + (lane & 15)) * Gm::RSTRIDE + (4 * pp + slot) * 16);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi) {
          const double a = piece_elem<BF16>(a4[gi], e);
#pragma unroll
          for (int qd = 0; qd < NQ; ++qd)
            acc[gi][qd] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, qb[qd][pp][e], acc[gi][qd], 0, 0, 0);
        }
    }
#pragma unroll
    for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi) {
      const int key = wave * 64 + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) sc[qd * 4 + (lane & 3)][key] = acc[gi][qd];
    }
    __syncthreads();

    // ---- per-head chunk max, exponentials, in-chunk prefix: wave owns heads wave, wave + 4;
    //      lane owns keys 4*lane .. 4*lane + 3
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int g = wave + 4 * j;
      if (g >= G) break;
      double s[4];
      double lmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * lane + i;
        double v = sc[g][k];
        if (p.ternary) v = v * mul[j];
        v = v * p.scale;
        s[i] = k < len ? v : -INFINITY;
        lmax = fmax(lmax, s[i]);
      }
      const double m = readlane_f64(wave_incl_max_dpp(lmax), 63);
      double ex[4], pre[4], run = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ex[i] = (4 * lane + i) < len ? exp_f64(s[i] - m) : 0.0;
        run += ex[i];
        pre[i] = run;
      }
      const double incl = wave_incl_scan_dpp(run);
      double excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) pend[j][i] = excl + pre[i];
      pend_m[j] = m;
      pend_l[j] = incl;
      if (p.prob) {
        double* pr = p.prob + ((int64_t)b * p.H + h0 + g) * p.nk + n0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * lane + i < len) pr[4 * lane + i] = ex[i];
      }
    }
    pend_n0 = n0;
    pend_len = len;
    pend_t = t;
    __syncthreads();  // ks and sc are rewritten by the next chunk
  }
  flush();
}

// ---------------------------------------------------------------------------------------------

template <int D, bool BF16, int NQ>
constexpr int blocks_per_cu() {
  constexpr size_t lds = (size_t)Geo<D, BF16>::LDS_K + 4 * NQ * CHUNK * sizeof(double) + 4 * NQ * sizeof(double);
  return lds * 2 <= 160 * 1024 ? 2 : 1;
}

template <int D, bool BF16, int NQ>
hipError_t launch_q(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  constexpr int MINB = blocks_per_cu<D, BF16, NQ>();
  return launch_timed(score_kernel<D, BF16, NQ, MINB>, dim3(p.score_blocks_per_group, p.Hkv, p.B), dim3(THREADS), st,
                      ev, p);
}

template <int D, bool BF16>
hipError_t launch_d(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  if constexpr (BF16) {
    const dim3 grid(p.score_blocks_per_group, p.Hkv, p.B);
    if (p.G <= 4) {
      if (p.fused) return launch_timed(score_stream_kernel<D, 1, KM_FLASH>, grid, dim3(STHREADS), st, ev, p);
      return launch_timed(score_stream_kernel<D, 1, KM_SCORE>, grid, dim3(STHREADS), st, ev, p);
    }
    return launch_timed(score_stream_kernel<D, 2, KM_SCORE>, grid, dim3(STHREADS), st, ev, p);
  }
  return p.G <= 4 ? launch_q<D, BF16, 1>(p, st, ev) : launch_q<D, BF16, 2>(p, st, ev);
}

}  // namespace

int score_blocks_per_cu(int d, bool bf16, int G) {
  if (bf16) return 1;  // streaming form (G <= 8): one block per CU (two K tiles fill most of the LDS)
  const bool q1 = G <= 4;
  if (d == 128) {
    if (bf16) return q1 ? blocks_per_cu<128, true, 1>() : blocks_per_cu<128, true, 2>();
    return q1 ? blocks_per_cu<128, false, 1>() : blocks_per_cu<128, false, 2>();
  }
  if (bf16) return q1 ? blocks_per_cu<64, true, 1>() : blocks_per_cu<64, true, 2>();
  return q1 ? blocks_per_cu<64, false, 1>() : blocks_per_cu<64, false, 2>();
}

hipError_t launch_score(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  if (p.d == 128) return p.bf16 ? launch_d<128, true>(p, st, ev) : launch_d<128, false>(p, st, ev);
  return p.bf16 ? launch_d<64, true>(p, st, ev) : launch_d<64, false>(p, st, ev);
}

hipError_t launch_chunk_cdf(const Problem& p, hipStream_t st) {
  const dim3 grid(p.H, p.B);  // one wave per (query head, sequence)
  if (p.T <= 64)
    chunk_cdf_reg_kernel<1><<<grid, 64, 0, st>>>(p);
  else if (p.T <= 128)
    chunk_cdf_reg_kernel<2><<<grid, 64, 0, st>>>(p);
  else if (p.T <= 256)
    chunk_cdf_reg_kernel<4><<<grid, 64, 0, st>>>(p);
  else if (p.T <= 512)
    chunk_cdf_reg_kernel<8><<<grid, 64, 0, st>>>(p);
  else if (p.T <= 1024)
    chunk_cdf_reg_kernel<16><<<grid, 64, 0, st>>>(p);
  else
    chunk_cdf_kernel<<<grid, 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace santa
