// Split-K score pass: one block per (chunk of CHUNK keys, KV head, sequence).
//
// "Stochastic Sparse Attention for Memory-Bound Inference", Appendix O, Algorithm 3 (pass-1 tile
// statistics with the optional stash) and Section 3.2 ("Pass 1"): for every query head h of the GQA
// group, s_{h,n} = q_h . K_n / sqrt(dk) (Eq. 1), chunk max m_{h,t}, and the in-chunk exponentials
// exp(s_{h,n} - m_{h,t}). This pass stores their in-chunk inclusive prefix sums (the chunk's CDF up to
// the chunk's own scale) and l_{h,t} = the chunk total, which is what the sampler's inverse CDF needs.
//
// MI355X design:
//   * K is read once, 16 bytes per lane per load, every row shared by the G heads of its group.
//   * The dot products run on the fp64 matrix cores (v_mfma_f64_4x4x4_4b: 4 blocks of 4 keys x 4 dims
//     x 4 heads), so a 16-key group needs no cross-lane reduction: lane l holds key (l & 15) at dim
//     slot (l >> 4) for A, head (l & 3) at dim slot (l >> 4) for B, and receives the score of key
//     4*((l >> 2) & 3) + (l >> 4), head (l & 3). Products of bf16 (or fp32) inputs are exact in fp64
//     and accumulate in fp64, which the sampler's index parity needs.
//   * exp, max and the prefix scan are fp64 wavefront operations on 256 keys per block.
//   * With the Bernoulli ternary query (Section 5, Eq. 5; Appendix C, Eqs. 8-9) the B operand holds
//     qhat in {-1, 0, +1} and the score is (qhat . K) * norm * (1/sqrt(dk)).

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;   // 4 waves; 64 keys per wave, 16 keys per MFMA group
constexpr int GROUPS_PER_WAVE = 4;

__device__ inline double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// NQ = number of 4-head quads (1: G <= 4, 2: G <= 8)
template <int D, bool BF16, int NQ>
__global__ __launch_bounds__(THREADS) void score_kernel(Problem p) {
  using P = Piece<BF16>;
  constexpr int EPL = P::EPL;
  constexpr int NPIECE = D / EPL;     // 16-byte pieces per row
  constexpr int PP = NPIECE / 4;      // pieces per lane per row (lane takes pieces 4*pp + slot)
  constexpr int HMAX = 4 * NQ;

  __shared__ double sc[HMAX][CHUNK];
  __shared__ double qe[HMAX][D];
  __shared__ double red[THREADS / 64][HMAX];
  __shared__ double hnorm[HMAX];

  const int t = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int h0 = kv * G;
  const int64_t n0 = (int64_t)t * CHUNK;
  const int len = (int)((p.nk - n0) < CHUNK ? (p.nk - n0) : CHUNK);

  // ---- issue the K loads first: lane (slot = lane >> 4, key = lane & 15) of each 16-key group
  const int slot = lane >> 4;
  const char* kbase = (const char*)p.K;
  const size_t esz = BF16 ? 2 : 4;
  uint4 kw[GROUPS_PER_WAVE][PP];
#pragma unroll
  for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi) {
    const int r = wave * 64 + gi * 16 + (lane & 15);
    const bool ok = r < len;
    const int64_t row = n0 + (ok ? r : 0);
    const uint4* rp = (const uint4*)(kbase + esz * ((int64_t)b * p.batch_stride + row * p.seq_stride + (int64_t)kv * D));
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      kw[gi][pp] = ok ? rp[4 * pp + slot] : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- effective query of each head of the group, fp64 in LDS
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
      double r = 0.0;
      if (g < G && nrm > 0.0) {
        const double u = uniform53(p.seed, (uint32_t)e, (uint32_t)(h0 + g), (uint32_t)b, TAG_BERNOULLI);
        if (u < fabs(v) / nrm) r = v > 0.0 ? 1.0 : (v < 0.0 ? -1.0 : 0.0);
      }
      qe[g][e] = r;
    }
    __syncthreads();
  }

  // ---- B operand registers: head (quad*4 + (lane & 3)), dims EPL*(4*pp + slot) + e
  double qb[NQ][PP][EPL];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qb[qd][pp][e] = qe[qd * 4 + (lane & 3)][EPL * (4 * pp + slot) + e];

  // ---- fp64 MFMA chains, one per 16-key group
#pragma unroll
  for (int gi = 0; gi < GROUPS_PER_WAVE; ++gi) {
    double acc[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) acc[qd] = 0.0;
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      double a[EPL];
      P::to_f64(kw[gi][pp], a);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd) acc[qd] = __builtin_amdgcn_mfma_f64_4x4x4f64(a[e], qb[qd][pp][e], acc[qd], 0, 0, 0);
    }
    const int key = wave * 64 + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) sc[qd * 4 + (lane & 3)][key] = acc[qd];
  }
  __syncthreads();

  // ---- per-head chunk max, exponentials and in-chunk prefix (thread = key)
  const bool valid = tid < len;
  double s[HMAX];
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    double v = sc[g][tid];
    if (p.ternary) v = v * hnorm[g];
    v = v * p.scale;
    s[g] = valid ? v : -INFINITY;
  }
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    const double m = wave_max(s[g]);
    if (lane == 0) red[wave][g] = m;
  }
  __syncthreads();
  double cm[HMAX];
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    double m = red[0][g];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w) m = fmax(m, red[w][g]);
    cm[g] = m;
  }
  __syncthreads();
  double ex[HMAX], pre[HMAX];
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    ex[g] = valid ? exp(s[g] - cm[g]) : 0.0;
    pre[g] = wave_incl_scan(ex[g], lane);
    if (lane == 63) red[wave][g] = pre[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += red[w][g];
    pre[g] += off;
  }
  const int64_t T = p.T;
#pragma unroll
  for (int g = 0; g < HMAX; ++g) {
    if (g >= G) break;
    const int64_t bh = (int64_t)b * p.H + h0 + g;
    if (valid) {
      p.stash[bh * p.nk + n0 + tid] = pre[g];
      if (p.prob) p.prob[bh * p.nk + n0 + tid] = ex[g];
    }
    if (tid == len - 1) {
      p.cmax[bh * T + t] = cm[g];
      p.csum[bh * T + t] = pre[g];
    }
  }
}

template <int D, bool BF16>
hipError_t launch_d(const Problem& p, hipStream_t st) {
  dim3 grid(p.T, p.Hkv, p.B);
  if (p.G <= 4)
    score_kernel<D, BF16, 1><<<grid, THREADS, 0, st>>>(p);
  else
    score_kernel<D, BF16, 2><<<grid, THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Problem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_d<128, true>(p, st) : launch_d<128, false>(p, st);
  return p.bf16 ? launch_d<64, true>(p, st) : launch_d<64, false>(p, st);
}

}  // namespace santa
