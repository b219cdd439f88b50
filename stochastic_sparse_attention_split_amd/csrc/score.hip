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

namespace santa {

namespace {

constexpr int THREADS = 256;   // 4 waves; 64 keys per wave, 16 keys per MFMA group
constexpr int GROUPS_PER_WAVE = 4;
static_assert(THREADS / 64 * GROUPS_PER_WAVE * 16 == CHUNK, "a block covers one chunk per iteration");
static_assert(4 * 64 == CHUNK, "a wave covers one chunk with 4 keys per lane in the softmax step");

// element e of a 16-byte piece, widened exactly to fp64
template <bool BF16>
__device__ inline double piece_elem(const uint4& w, int e) {
  if constexpr (BF16) {
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (double)((e & 1) ? bf16_hi(x) : bf16_lo(x));
  } else {
    const uint32_t x = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
    return (double)__uint_as_float(x);
  }
}

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
// Streaming form for bf16 caches (one block per CU). The memory system copies each chunk's K tile
// straight into LDS (global_load_lds: 16 bytes per lane, no register staging), two tiles in flight: the
// copy of chunk k+2 starts as soon as chunk k's matrix-core pass has finished reading its tile, so the
// HBM stream does not pause for the exponentials and stores. The compiler does not track these copies;
// the block waits for them with explicit vmcnt waits whose counts are derived in the loop below.

// the LDS address of a __shared__ object, as the 32-bit offset M0 takes
__device__ inline uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// one wave-wide copy global -> LDS: lane l's 16 bytes at `g` land at LDS address lds + 16 l
__device__ inline void copy_to_lds16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ inline void wait_vm() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (N == 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else if constexpr (N == 64) asm volatile("s_waitcnt vmcnt(63)" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}

constexpr int SQUART = 4;                // key quarters of a chunk (64 keys each): one matrix wave each
constexpr int SSOFT = 4;                 // exponential waves: one head each (two for G = 5..8)
constexpr int SCOPY = 4;                 // copy waves: two per K tile
constexpr int STHREADS = 64 * (SQUART + SSOFT + SCOPY);  // 12 waves: three per SIMD
constexpr int SPIN_LIMIT = 1 << 22;      // bounded waits: a stuck handshake ends the kernel, flagged

template <int D>
struct SGeo {
  static constexpr int ROWB = D * 2;         // bytes per bf16 K row
  static constexpr int PPR = ROWB / 16;      // 16-byte pieces per row (16 or 8)
  static constexpr int TILE = CHUNK * ROWB;  // bytes per chunk tile (64 or 32 KiB)
  static constexpr int CPW = TILE / 1024 / 2;  // wave-wide 1 KiB copies per copy wave per chunk (32 or 16)
  static constexpr int RPS = 1024 / ROWB;    // rows per 1 KiB copy (4 or 8)
  static constexpr int PP = PPR / 4;         // pieces per lane per row in the matrix-core layout
  static constexpr int PPH = PP / 2;         // of which one half of the head dimension holds
};

// byte offset of piece `pc` of row `row` in a tile: pieces are XOR-swizzled by the row, so the 16 rows a
// quarter-wave reads in the matrix-core layout fall in distinct LDS banks
template <int D>
__device__ inline int tile_off(int row, int pc) {
  return row * SGeo<D>::ROWB + ((pc ^ (row % SGeo<D>::PPR)) << 4);
}

// LDS handshake counters. signal(): this wave's earlier LDS writes (and, for copy waves, the copies
// waited for) are complete, then one lane adds 1. wait_ge(): poll until the counter reaches `target`;
// false after SPIN_LIMIT polls (the caller then abandons the block and flags it).
__device__ inline void signal(int* ctr, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// A polling wave keeps its issue priority: a poll is a few instructions per sleep, and a waiting wave
// at the lowest priority is starved by the MFMA waves sharing its SIMD and notices its counter late.
__device__ inline bool wait_ge(int* ctr, int target) {
  int spins = 0;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (++spins > SPIN_LIMIT) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::: "memory");
  return true;
}

// Streaming score pass for bf16 caches and G <= 8, one block of 12 waves per CU (one wave of each role
// per SIMD), three roles that meet only through LDS counters (no block-wide barrier after the start), so
// the K stream, the matrix cores and the exponentials overlap:
//   * waves 0..3: fp64 MFMA over key quarter w (64 keys: four 16-key groups) and the whole head dimension
//     (element parity gives eight independent accumulation chains per head group), writing complete
//     scores. Two half-row waves per SIMD keep the matrix pipe busier on their own, but beside the K
//     stream writing into LDS one whole-row wave is no slower, and no partial rows need adding. For
//     G = 5..8 (HG = 2) the wave scores both head groups: each K element is converted once for the
//     MFMAs of the eight heads, and the query operands are read from LDS per 4-piece step to stay within
//     the register budget of three waves per SIMD;
//   * waves 4..7: chunk max, exponentials, in-chunk prefix and the stores of head w - 4 (and w for
//     G = 5..8);
//   * waves 8..11: global -> LDS copies (global_load_lds) of the K tiles, waves 8-9 tile 0 with the
//     block's even chunks, 10-11 tile 1 with the odd ones (wave 10 first copies the queries). The first
//     chunk of tile 1 is requested only once tile 0 has landed, so across the device the first tiles
//     arrive before any second one and the matrix cores start half a pass earlier.
// Counters (chunk k lives in tile k & 1; its fill index there is k >> 1):
//   ld[j] +1 per copy wave when its half of tile j's current chunk has landed;
//   use[j] +1 per MFMA wave when its reads of tile j are done;  pr +1 per MFMA wave per chunk whose
//   scores are written;  pc +1 per exponential wave per chunk whose scores it has read;  qr queries
//   landed;  pb prologue barrier;  fin waves finished (the last one publishes the block's handshake
//   status).
// HG = head groups of four (G <= 4 * HG).
// FL: S²ANTA-flash kernel 1 ("Stochastic Sparse Attention for Memory-Bound Inference", Section 3.3 and
// Appendix P, Algorithm 7) fused in: right after a chunk's exponentials, the exponential wave of head g
// takes the tile's systematic counts with the uniform budget S_tile (c_n = floor(a0 + inv P_n) -
// floor(a0 + inv P_{n-1}), inv = S_tile / l_t, P the in-chunk prefix it has just formed, a0 from Philox
// counter (t, h, b, 4)), writes the index slots and the tile's sampled-key bits, and issues the loads of
// its sampled V rows; one chunk later (the loads have landed meanwhile) it adds count x row into the fp32
// tile partial and stores it. Only the merge kernel follows: two launches per decode step.
template <int D, int HG, bool FL>
__global__ __launch_bounds__(STHREADS, 1) void score_stream_kernel(Problem p) {
  static_assert(!FL || HG == 1, "the fused S²ANTA-flash form covers G <= 4");
  constexpr int NMF = SQUART;  // matrix-core waves
  constexpr int NTH = 64 * (NMF + SSOFT + SCOPY);
  using Sg = SGeo<D>;
  constexpr int EPL = 8, PPH = Sg::PPH, CPW = Sg::CPW;
  constexpr int KPW = CHUNK / SQUART;  // keys per MFMA wave
  constexpr int NGR = KPW / 16;       // 16-key groups per MFMA wave
  constexpr int HM = 4 * HG;          // heads held
  constexpr int NPW = 2 * PPH;       // 4-piece steps of a row per MFMA wave
  static_assert(D * 2 * HM <= 1024 * HG, "the queries of a group fit HG 1 KiB copies");

  __shared__ __align__(16) unsigned char kt[2][Sg::TILE];
  __shared__ __align__(16) double part[HG][4][CHUNK];  // scores: [head group][head][key]
  __shared__ __align__(16) double qe[HM][D + 2];
  __shared__ double hnorm[HM];
  __shared__ __align__(16) unsigned char qs[1024 * HG];
  __shared__ int rl[FL ? 4 : 1][FL ? CHUNK : 1];  // fused S²ANTA-flash: sampled rows (key | count << 8) per head
  constexpr int NCTR = 10;
  __shared__ int ctr[NCTR];
  int* ld = &ctr[0];   // [2]
  int* use = &ctr[2];  // [2]
  int* pr = &ctr[4];
  int* pc = &ctr[5];
  int* qr = &ctr[6];
  int* pb = &ctr[7];
  int* fin = &ctr[8];
  int* bad = &ctr[9];

  const int kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int h0 = kv * G;
  const int T = p.T;
  const int step = gridDim.x;
  const int t0 = blockIdx.x;
  if (t0 >= T) return;
  const int n = (T - 1 - t0) / step + 1;  // this block's chunks: t0, t0 + step, ...
  int* err = p.sync_err + ((int64_t)b * gridDim.y + kv) * gridDim.x + t0;

  if (tid < NCTR) ctr[tid] = 0;
  __syncthreads();  // the only block-wide barrier

  const int64_t seq_bytes = 2 * p.seq_stride;
  const char* kbase = (const char*)p.K + 2 * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
  auto chunk_len = [&](int tt) { return (int)min((int64_t)CHUNK, p.nk - (int64_t)tt * CHUNK); };
  bool ok = true;
  // every wave ends here: the last one to finish publishes whether any handshake timed out
  auto finish = [&]() {
    if (lane == 0) {
      if (!ok) __hip_atomic_fetch_or(bad, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const int before = __hip_atomic_fetch_add(fin, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (before == NTH / 64 - 1)
        __hip_atomic_store(err, __hip_atomic_load(bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  if (wave >= NMF + SSOFT) {
    // ---- copy waves: at most one chunk's copies in flight per wave, so vmcnt(0) means all landed.
    // Highest issue priority on their SIMD: they issue rarely and the whole block waits on them.
    __builtin_amdgcn_s_setprio(3);
    const int j = (wave - NMF - SSOFT) >> 1, hf = (wave - NMF - SSOFT) & 1;
    if (j == 1 && hf == 0) {
      const char* qsrc = (const char*)p.q + ((int64_t)b * p.H + h0) * D * 2;
#pragma unroll
      for (int c = 0; c < HG; ++c)  // bytes past the group's queries re-read its last piece (never used)
        copy_to_lds16(qsrc + min(c * 1024 + lane * 16, G * D * 2 - 16), lds_addr(qs) + c * 1024);
      wait_vm<0>();
      signal(qr, lane);
    }
    for (int k = j, m = 0; k < n && ok; k += 2, ++m) {
      if (m > 0) ok = wait_ge(&use[j], NMF * m);  // the tile's previous chunk is no longer read
      if (m == 0 && j == 1) ok = wait_ge(&ld[0], 2);  // the block's first chunk goes first
      if (!ok) break;
      const int t = t0 + k * step;
      const int64_t n0 = (int64_t)t * CHUNK;
      const int len = chunk_len(t);
      const uint32_t base = lds_addr(&kt[j][0]);
#pragma unroll 4
      for (int i = 0; i < CPW; ++i) {
        const int q = hf * CPW + i;
        const int row = q * Sg::RPS + lane / Sg::PPR;
        const int pc = (lane % Sg::PPR) ^ (row % Sg::PPR);
        const int grow = row < len ? row : 0;  // rows past the end re-read row 0 (masked later)
        copy_to_lds16(kbase + (n0 + grow) * seq_bytes + pc * 16, base + q * 1024);
      }
      wait_vm<0>();
      signal(&ld[j], lane);
    }
    wait_vm<0>();  // no copy may land after the block ends
    finish();
    return;
  }

  // ---- prologue of the MFMA and exponential waves (12 waves, counter barrier pb)
  int np = 0;
  auto pbar = [&]() {
    signal(pb, lane);
    ++np;
    ok = ok && wait_ge(pb, (NMF + SSOFT) * np);
  };
  ok = wait_ge(qr, 1);
  if (ok) {
    for (int i = tid; i < HM * D; i += (NMF + SSOFT) * 64) {
      const int g = i / D, e = i % D;
      double v = 0.0;
      if (g < G) v = (double)__uint_as_float(((uint32_t)((const uint16_t*)qs)[g * D + e]) << 16);
      qe[g][e] = v;
    }
  }
  pbar();
  if (p.ternary) {
    if (ok && tid < HM) {
      double m = 0.0;
      for (int e = 0; e < D; ++e) m = fmax(m, fabs(qe[tid][e]));
      hnorm[tid] = m;
    }
    pbar();
    if (ok) {
      for (int i = tid; i < HM * D; i += (NMF + SSOFT) * 64) {
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
    }
    pbar();
  }

  if (wave >= NMF) {
    // ---- exponential waves: heads w - 4 (+ 4) of every chunk, lane owns keys 4*lane .. 4*lane + 3. Issue
    // priority above the MFMA waves sharing their SIMD, whose instruction stream would otherwise starve them.
    __builtin_amdgcn_s_setprio(2);
    const int g0 = wave - NMF;
    // fused S²ANTA-flash state: V-row loads of the previous chunk still in flight
    constexpr int LPR = D / 8;     // lanes per V row (16-byte pieces)
    constexpr int RPI = 64 / LPR;  // rows per load instruction
    constexpr int NPEND = 4;       // load instructions carried over to the next chunk
    uint4 vpend[NPEND];
    float cpend[NPEND];
    int npend = 0, tpend = -1;
    const int grp = b * p.Hkv + kv;
    const int64_t rstride = 2 * p.seq_stride;
    const char* vgrp = (const char*)p.V + 2 * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
    // count x row sums of one chunk: reduce the RPI row lanes, store the head's fp32 tile partial
    auto store_partial = [&](float* acc, int tt) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) acc[e] += __shfl_xor(acc[e], o, 64);
      if (lane < LPR) {
        float4* dst = (float4*)(p.partial + (((int64_t)grp * T + tt) * G + g0) * D + lane * 8);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    };
    auto flush = [&]() {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int bi = 0; bi < NPEND; ++bi) {
        if (bi < npend) {  // wave-uniform
          float v[8];
          Piece<true>::to_f32(vpend[bi], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += cpend[bi] * v[e];
        }
      }
      store_partial(acc, tpend);
      npend = 0;
      tpend = -1;
    };
    for (int k = 0; k < n && ok; ++k) {
      ok = wait_ge(pr, NMF * (k + 1));  // chunk k's partials are complete
      if (!ok) break;
      double raw[HG][4];
#pragma unroll
      for (int hx = 0; hx < HG; ++hx) {
        const double2* lo = (const double2*)&part[hx][g0][4 * lane];
        const double2 l0 = lo[0], l1 = lo[1];
        raw[hx][0] = l0.x;
        raw[hx][1] = l0.y;
        raw[hx][2] = l1.x;
        raw[hx][3] = l1.y;
      }
      signal(pc, lane);  // the partial rows have been read
      const int t = t0 + k * step;
      const int len = chunk_len(t);
      const int64_t n0 = (int64_t)t * CHUNK;
#pragma unroll
      for (int hx = 0; hx < HG; ++hx) {
        const int g = g0 + 4 * hx;
        if (g >= G) continue;  // wave-uniform
        const double nrm = p.ternary ? hnorm[g] : 1.0;
        const int64_t bh = (int64_t)b * p.H + h0 + g;
        double sv[4];
        double lmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 4 * lane + i;
          double v = raw[hx][i];
          if (p.ternary) v = v * nrm;  // (qhat . K) * norm, then * (1/sqrt(dk))
          v = v * p.scale;
          sv[i] = kk < len ? v : -INFINITY;
          lmax = fmax(lmax, sv[i]);
        }
        const double m = readlane_f64(wave_incl_max_dpp(lmax), 63);
        double ex[4], pre[4], run = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ex[i] = exp_f64(sv[i] - m);  // keys past the end: -inf -> 0
          run += ex[i];
          pre[i] = run;
        }
        const double incl = wave_incl_scan_dpp(run);
        double excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.0;
        // stash rows are CHUNK-padded: the whole chunk is stored, keys past the end repeat the total (the
        // fused S²ANTA-flash samples here and needs no stash). Non-temporal stores: the rows leave the
        // caches as they are written instead of as dirty lines written back at the end of the kernel; the
        // sampling kernel reads them only after its chunk CDF and points.
        if constexpr (!FL) {
          typedef double f64x2_t __attribute__((ext_vector_type(2)));
          f64x2_t* dst = (f64x2_t*)(p.stash + bh * p.stash_stride + n0 + 4 * lane);
          const f64x2_t v0 = {excl + pre[0], excl + pre[1]};
          const f64x2_t v1 = {excl + pre[2], excl + pre[3]};
          __builtin_nontemporal_store(v0, dst);
          __builtin_nontemporal_store(v1, dst + 1);
        }
        if (lane == 0) {
          p.cmax[bh * T + t] = m;
          p.csum[bh * T + t] = readlane_f64(incl, 63);
        }
        if (p.prob) {
          double* pr = p.prob + bh * p.nk + n0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * lane + i < len) pr[4 * lane + i] = ex[i];
        }
        if constexpr (FL) {
          if (tpend >= 0) flush();  // the previous chunk's rows have landed
          const int St = p.S_tile;
          const double inv = (double)St / readlane_f64(incl, 63);
          const double a0 = uniform53(p.seed, (uint32_t)t, (uint32_t)(h0 + g), (uint32_t)b, TAG_FLASH);
          // the prefix value before each key: the stored prefix of the previous key (0 before key 0)
          double prevP = __shfl_up(excl + pre[3], 1, 64);
          if (lane == 0) prevP = 0.0;
          int32_t* idst = p.idx + bh * p.L + (int64_t)t * St;
          int cn[4];
          uint64_t bm[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const double P = excl + pre[i];
            const int lo = (int)floor(a0 + inv * prevP), hi = (int)floor(a0 + inv * P);
            int c = hi > lo ? hi - lo : 0;
            if (4 * lane + i >= len) c = 0;
            if (p.want_idx)
              for (int j = 0; j < c; ++j)
                if (lo + j < St) idst[lo + j] = (int32_t)(n0 + 4 * lane + i);
            cn[i] = c;
            prevP = P;
            bm[i] = __ballot(c > 0);
          }
          if (p.want_unique && lane == 0) {
            uint64_t* bd = p.bmap + (((int64_t)grp * T + t) * 4 + g) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) bd[i] = bm[i];
          }
          // this head's sampled rows in key-slot order (i-major), then their loads
          int nrows = 0, pos = -1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (cn[i] > 0) {
              pos = nrows + __popcll(bm[i] & ((1ull << lane) - 1ull));
              rl[g][pos] = (4 * lane + i) | (cn[i] << 8);
            }
            nrows += __popcll(bm[i]);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int r = lane / LPR, pcs = lane % LPR;
          const char* vch = vgrp + n0 * rstride + pcs * 16;
          if (nrows <= NPEND * RPI) {
            npend = (nrows + RPI - 1) / RPI;
            tpend = t;
#pragma unroll
            for (int bi = 0; bi < NPEND; ++bi) {
              if (bi < npend) {  // wave-uniform
                const int row = bi * RPI + r;
                const int ent = rl[g][min(row, nrows - 1)];  // rows past the list re-read its last row
                cpend[bi] = row < nrows ? (float)(ent >> 8) : 0.0f;
                vpend[bi] = load_stream16(vch + (ent & 255) * rstride);
              }
            }
          } else {  // many sampled rows: gathered here
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int r0 = 0; r0 < nrows; r0 += RPI * NPEND) {
              uint4 w[NPEND];
              float cw[NPEND];
#pragma unroll
              for (int bi = 0; bi < NPEND; ++bi) {
                const int row = r0 + bi * RPI + r;
                const int ent = rl[g][min(row, nrows - 1)];
                cw[bi] = row < nrows ? (float)(ent >> 8) : 0.0f;
                w[bi] = load_stream16(vch + (ent & 255) * rstride);
              }
#pragma unroll
              for (int bi = 0; bi < NPEND; ++bi) {
                float v[8];
                Piece<true>::to_f32(w[bi], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += cw[bi] * v[e];
              }
            }
            store_partial(acc, t);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the list is rewritten next chunk
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
    }
    if constexpr (FL) {
      if (tpend >= 0) flush();
    }
    finish();
    return;
  }

  // ---- MFMA waves: 16-key groups x element parity = independent accumulation chains
  const int slot = lane >> 4;
  if constexpr (HG == 2) {
    const int quart = wave;
    for (int k = 0; k < n && ok; ++k) {
      ok = wait_ge(&ld[k & 1], 2 * ((k >> 1) + 1));  // chunk k's tile has landed
      if (!ok) break;
      const unsigned char* ks = &kt[k & 1][0];
      double acc[HG][NGR][2];  // [head group][key group][element parity]
#pragma unroll
      for (int hx = 0; hx < HG; ++hx)
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi) acc[hx][gi][0] = acc[hx][gi][1] = 0.0;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        uint4 a4[NGR];
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi)
          a4[gi] = *(const uint4*)(ks + tile_off<D>(quart * KPW + gi * 16 + (lane & 15), 4 * pp + slot));
        double qv[HG][EPL];
#pragma unroll
        for (int hx = 0; hx < HG; ++hx)
#pragma unroll
          for (int e = 0; e < EPL; ++e) qv[hx][e] = qe[4 * hx + (lane & 3)][EPL * (4 * pp + slot) + e];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int gi = 0; gi < NGR; ++gi) {
            const double a = piece_elem<true>(a4[gi], e);
#pragma unroll
            for (int hx = 0; hx < HG; ++hx)
              acc[hx][gi][e & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, qv[hx][e], acc[hx][gi][e & 1], 0, 0, 0);
          }
      }
      signal(&use[k & 1], lane);  // this wave's reads of tile k & 1 are complete
      if (k >= 1) ok = wait_ge(pc, SSOFT * k);  // chunk k - 1's partials were read
      if (!ok) break;
#pragma unroll
      for (int hx = 0; hx < HG; ++hx)
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi) {
          const int key = quart * KPW + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
          part[hx][lane & 3][key] = acc[hx][gi][0] + acc[hx][gi][1];
        }
      signal(pr, lane);
    }
    finish();
    return;
  }
  // key quarter over the whole head dimension (HG = 1)
  const int quart = wave;
  const int qrow = lane & 3;
  double qb[NPW][EPL];
#pragma unroll
  for (int pp = 0; pp < NPW; ++pp)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qb[pp][e] = qe[qrow][EPL * (4 * pp + slot) + e];
  for (int k = 0; k < n && ok; ++k) {
    ok = wait_ge(&ld[k & 1], 2 * ((k >> 1) + 1));  // chunk k's tile has landed
    if (!ok) break;
    const unsigned char* ks = &kt[k & 1][0];
    double acc[NGR][2];  // [group][element parity]
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) acc[gi][0] = acc[gi][1] = 0.0;
#pragma unroll
    for (int pp = 0; pp < NPW; ++pp) {
      uint4 a4[NGR];
#pragma unroll
      for (int gi = 0; gi < NGR; ++gi)
        a4[gi] = *(const uint4*)(ks + tile_off<D>(quart * KPW + gi * 16 + (lane & 15), 4 * pp + slot));
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi)
          acc[gi][e & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(piece_elem<true>(a4[gi], e), qb[pp][e],
                                                               acc[gi][e & 1], 0, 0, 0);
    }
    signal(&use[k & 1], lane);  // this wave's reads of tile k & 1 are complete
    if (k >= 1) ok = wait_ge(pc, SSOFT * k);  // chunk k - 1's partials were read
    if (!ok) break;
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) {
      const int key = quart * KPW + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
      part[0][lane & 3][key] = acc[gi][0] + acc[gi][1];
    }
    signal(pr, lane);
  }
  finish();
}

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
      if (p.fused) return launch_timed(score_stream_kernel<D, 1, true>, grid, dim3(STHREADS), st, ev, p);
      return launch_timed(score_stream_kernel<D, 1, false>, grid, dim3(STHREADS), st, ev, p);
    }
    return launch_timed(score_stream_kernel<D, 2, false>, grid, dim3(STHREADS), st, ev, p);
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
