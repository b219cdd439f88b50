// Reduce/CDF + sampler: one block per (query head, sequence).
//
// "Stochastic Sparse Attention for Memory-Bound Inference":
//   * chunk masses: m* = max_t m_t, W_t = l_t exp(m_t - m*), Z = sum_t W_t (Appendix O, Algorithm 4,
//     lines for m*, W and Z; Section 3.2 "Global budget allocation"), and their exclusive prefix C_t,
//     the chunk-level CDF of the softmax up to the factor Z;
//   * points: SANTA draws T_m ~ U[0,1) i.i.d. (Section 2, Eq. 4; Definition A.1); S²ANTA-strat draws
//     T_m ~ U[m/S, (m+1)/S) independently and S²ANTA-sys uses one U ~ U[0, 1/S) with T_m = U + m/S
//     (Section 2.1); here T_m = u_m, (m + u_m)/S and (m + u)/S respectively, u from Philox4x32-10;
//   * inverse CDF with the half-open convention 1{F(j-1) <= t < F(j)} (Appendix A.4): the chunk t with
//     C_t <= T Z < C_{t+1}, then the first key j of the chunk whose scaled in-chunk prefix exceeds the
//     residual T Z - C_t. A point at or beyond the total (rounding) takes the last key with nonzero mass.
//
// Everything is fp64. The chunk CDF lives in LDS; the in-chunk search reads the score pass's prefix
// stash with a two-level 16-ary search (16 independent loads, then one 128-byte line).

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;

// last key with nonzero mass in chunk `base[0..len)` (inclusive prefix sums)
__device__ inline int last_positive(const double* base, int len) {
  for (int j = len - 1; j > 0; --j)
    if (base[j] > base[j - 1]) return j;
  return 0;
}

__global__ __launch_bounds__(THREADS) void sample_kernel(Problem p) {
  __shared__ double C[MAX_CHUNKS + 1];   // exclusive prefix of W_t; C[T] = Z
  __shared__ double F[MAX_CHUNKS];       // exp(m_t - m*)
  __shared__ double red[THREADS / 64];
  __shared__ double part[THREADS / 64];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T;
  const int64_t bh = (int64_t)b * p.H + h;
  const double* cmax = p.cmax + bh * T;
  const double* csum = p.csum + bh * T;

  // m* = max_t m_t
  double m = -INFINITY;
  for (int t = tid; t < T; t += THREADS) m = fmax(m, cmax[t]);
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  double mstar = red[0];
  for (int w = 1; w < THREADS / 64; ++w) mstar = fmax(mstar, red[w]);

  // W_t and its exclusive prefix: each thread owns a contiguous run of chunks
  const int per = (T + THREADS - 1) / THREADS;
  const int t0 = tid * per, t1 = min(T, t0 + per);
  double run = 0.0;
  for (int t = t0; t < t1; ++t) {
    const double f = exp(cmax[t] - mstar);
    F[t] = f;
    C[t] = run;  // local exclusive prefix for now
    run += csum[t] * f;
  }
  // exclusive prefix of the per-thread totals: wavefront scans, then the wave totals
  double incl = run;
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  double woff = 0.0, total = 0.0;
  for (int w = 0; w < THREADS / 64; ++w) {
    if (w < wave) woff += part[w];
    total += part[w];
  }
  const double off = woff + excl;
  for (int t = t0; t < t1; ++t) C[t] += off;
  if (tid == 0) C[T] = total;
  __syncthreads();
  const double Z = C[T];

  // debug: rescale the score pass's in-chunk exponentials to probabilities
  if (p.prob) {
    double* pr = p.prob + bh * p.nk;
    for (int64_t n = tid; n < p.nk; n += THREADS) pr[n] = pr[n] * F[n / CHUNK] / Z;
  }

  const double* stash = p.stash + bh * p.nk;
  double u_sys = 0.0;
  if (p.mode == 2) u_sys = uniform53(p.seed, 0u, (uint32_t)h, (uint32_t)b, TAG_SYS);
  for (int mi = tid; mi < p.S; mi += THREADS) {
    double pt;
    if (p.mode == 0) {
      pt = uniform53(p.seed, (uint32_t)mi, (uint32_t)h, (uint32_t)b, TAG_POINT);
    } else if (p.mode == 1) {
      const double u = uniform53(p.seed, (uint32_t)mi, (uint32_t)h, (uint32_t)b, TAG_POINT);
      pt = ((double)mi + u) / (double)p.S;
    } else {
      pt = ((double)mi + u_sys) / (double)p.S;
    }
    const double y = pt * Z;
    int t;
    int j = -1;
    if (!(y < Z)) {
      // rounding put the point at or past the total: last chunk with mass, its last key with mass
      t = T - 1;
      while (t > 0 && !(C[t + 1] > C[t])) --t;
      const int len = (int)min((int64_t)CHUNK, p.nk - (int64_t)t * CHUNK);
      j = last_positive(stash + (int64_t)t * CHUNK, len);
    } else {
      // last chunk with C_t <= y (C_0 = 0 <= y)
      int lo = 0, hi = T;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (C[mid] <= y) lo = mid; else hi = mid;
      }
      t = lo;
      const double r = y - C[t];
      const double f = F[t];
      const int len = (int)min((int64_t)CHUNK, p.nk - (int64_t)t * CHUNK);
      const double* base = stash + (int64_t)t * CHUNK;
      // level 1: how many complete 16-key blocks end at or below the residual
      const int nb = (len + 15) >> 4;
      double v1[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v1[k] = base[min(16 * k + 15, len - 1)];
      int sb = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) sb += (k < nb && v1[k] * f <= r) ? 1 : 0;
      if (sb < nb) {
        const int j0 = 16 * sb;
        double v2[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v2[i] = base[min(j0 + i, len - 1)];
        int c = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) c += (j0 + i < len && v2[i] * f <= r) ? 1 : 0;
        if (j0 + c < len) j = j0 + c;
      }
      if (j < 0) j = last_positive(base, len);  // residual reached the chunk total through rounding
    }
    p.idx[bh * p.S + mi] = (int32_t)((int64_t)t * CHUNK + j);
  }
}

}  // namespace

hipError_t launch_sample(const Problem& p, hipStream_t st) {
  sample_kernel<<<dim3(p.H, p.B), THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace santa
