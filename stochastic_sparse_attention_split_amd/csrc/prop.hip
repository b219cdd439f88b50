// S²ANTA-prop tile budgets, one block per (query head, sequence).
//
// "Stochastic Sparse Attention for Memory-Bound Inference", Section 3.2 and Appendix O, Algorithm 4:
// m* = max_t m_t, W_t = exp(m_t - m*) l_t, Z = sum_t W_t, q_t = S W_t / Z, S_t = floor(q_t), and the
// S - sum_t S_t samples left over go to the tiles with the largest fractional parts of q_t (largest
// remainder; equal fractions go to the lower tile). Tiles are the 256-key chunks of the score pass.
// Also written: the exclusive prefix of the budgets (each tile's first slot in the head's index list),
// exp(m_t - m*) and Z (for the debug probabilities).
//
// The remainder ranks are counted directly: rank_t = #{t' : r_t' > r_t or (r_t' = r_t and t' < t)} and
// tile t gets a sample more iff rank_t < S - sum S_t; the remainders sit in LDS and every thread scans
// them in the same order (LDS broadcast reads).

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int BT = 256;
constexpr int NW = BT / 64;
constexpr int TPT = MAX_CHUNKS / BT;  // tiles per thread at most (t = tid + BT * k)

__device__ inline double block_max(double v, double* red, int lane, int wave) {
  v = readlane_f64(wave_incl_max_dpp(v), 63);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmax(r, red[w]);
  __syncthreads();
  return r;
}

// sum in a fixed order: lanes by the DPP scan tree, then waves in index order
__device__ inline double block_sum(double v, double* red, int lane, int wave) {
  v = readlane_f64(wave_incl_scan_dpp(v), 63);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += red[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(BT) void budget_kernel(Problem p) {
  __shared__ double rem[MAX_CHUNKS];
  __shared__ int st[MAX_CHUNKS];
  __shared__ double red[NW];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, S = p.S;
  const int64_t bh = (int64_t)b * p.H + h;
  const double* cm = p.cmax + bh * T;
  const double* cs = p.csum + bh * T;

  double m[TPT], l[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int tt = min(tid + BT * k, T - 1);  // valid address; entries past T are masked
    m[k] = cm[tt];
    l[k] = cs[tt];
  }
  double mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < TPT; ++k)
    if (tid + BT * k < T) mx = fmax(mx, m[k]);
  const double ms = block_max(mx, red, lane, wave);

  double w[TPT], part = 0.0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    w[k] = tid + BT * k < T ? exp(m[k] - ms) * l[k] : 0.0;
    part += w[k];
  }
  const double Z = block_sum(part, red, lane, wave);

  int fl[TPT];
  double flsum = 0.0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = tid + BT * k;
    if (t < T) {
      const double q = ((double)S * w[k]) / Z;
      const double f = floor(q);
      fl[k] = (int)f;
      rem[t] = q - f;
      flsum += f;
      p.cscale[bh * T + t] = exp(m[k] - ms);
    } else {
      fl[k] = 0;
    }
  }
  const int R = S - (int)block_sum(flsum, red, lane, wave);  // block_sum's barrier also publishes rem[]

#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = tid + BT * k;
    if (t >= T) continue;
    const double r = rem[t];
    int rank = 0;
    for (int u = 0; u < T; ++u) {
      const double ru = rem[u];
      rank += (ru > r || (ru == r && u < t)) ? 1 : 0;
    }
    const int s_t = fl[k] + (rank < R ? 1 : 0);
    st[t] = s_t;
    p.budget[bh * T + t] = s_t;
  }
  if (tid == 0) p.cdf[bh * (T + 1) + T] = Z;
  __syncthreads();

  // exclusive prefix of the budgets in tile order: wave 0, lane l owns tiles [l*per, l*per + per)
  if (wave == 0) {
    const int per = (T + 63) / 64;
    const int t0 = min(T, lane * per), t1 = min(T, t0 + per);
    int run = 0;
    for (int t = t0; t < t1; ++t) run += st[t];
    const int incl = (int)wave_incl_scan_dpp((double)run);  // integer sums are exact in fp64
    int excl = incl - run;
    for (int t = t0; t < t1; ++t) {
      p.boff[bh * T + t] = excl;
      excl += st[t];
    }
  }
}

}  // namespace

hipError_t launch_budget(const Problem& p, hipStream_t st) {
  budget_kernel<<<dim3(p.H, p.B), BT, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace santa
