// S²ANTA-prop tile budgets, one block per (query head, sequence).
//
// "Stochastic Sparse Attention for Memory-Bound Inference", Section 3.2 and Appendix O, Algorithm 4:
// m* = max_t m_t, W_t = exp(m_t - m*) l_t, Z = sum_t W_t, q_t = S W_t / Z, S_t = floor(q_t), and the
// R = S - sum_t S_t samples left over go to the tiles with the largest fractional parts of q_t (largest
// remainder; equal fractions go to the lower tile). Tiles are the 256-key chunks of the score pass.
// Also written: the exclusive prefix of the budgets (each tile's first slot in the head's index list),
// exp(m_t - m*) and Z (for the debug probabilities).
//
// The R winners are found by a most-significant-digit radix select over the 80-bit keys
// (bits of the fractional part, then 0xFFFF - t), which are all distinct and whose unsigned order is
// the largest-remainder order with ties to the lower tile (a non-negative double's bit pattern orders
// like its value). Each pass histograms one byte of the keys still in the running, picks the byte of
// the R-th largest key, and stops as soon as every key left in that bin is a winner (usually after two
// or three passes; at most ten). Work per thread is linear in the tiles it owns.

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int BT = 256;
constexpr int NW = BT / 64;
constexpr int NPASS = 10;  // 8 bytes of the fraction, 2 bytes of the reversed tile index

__device__ inline int key_byte(uint64_t frac_bits, int t, int pass) {
  return pass < 8 ? (int)((frac_bits >> (56 - 8 * pass)) & 255u)
                  : (int)(((uint32_t)(0xFFFF - t) >> (8 * (NPASS - 1 - pass))) & 255u);
}

// TPT = tiles per thread (tile t = tid + BT * k), T <= BT * TPT
template <int TPT>
__global__ __launch_bounds__(BT) void budget_kernel(Problem p) {
  __shared__ int st[MAX_CHUNKS];
  __shared__ int hist[256];
  __shared__ int sel[3];
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
  const double ms = block_max_f64<NW>(mx, red, lane, wave);

  double w[TPT], part = 0.0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const double e = exp_f64(m[k] - ms);
    w[k] = tid + BT * k < T ? e * l[k] : 0.0;
    part += w[k];
    if (tid + BT * k < T) p.cscale[bh * T + tid + BT * k] = e;
  }
  const double Z = block_sum_f64<NW>(part, red, lane, wave);

  int fl[TPT];
  uint64_t key[TPT];
  uint32_t cand = 0;
  double flsum = 0.0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const double q = ((double)S * w[k]) / Z;
    const double f = floor(q);
    fl[k] = (int)f;
    key[k] = (uint64_t)__double_as_longlong(q - f);
    if (tid + BT * k < T) {
      flsum += f;
      cand |= 1u << k;
    }
  }
  int need = S - (int)block_sum_f64<NW>(flsum, red, lane, wave);  // the R leftover samples

  uint32_t above = 0;  // keys already known to be among the R largest
  if (need > 0) {
    for (int pass = 0; pass < NPASS; ++pass) {
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (cand >> k & 1u) atomicAdd(&hist[key_byte(key[k], tid + BT * k, pass)], 1);
      __syncthreads();
      if (wave == 0) {
        // lane owns bins 4 lane .. 4 lane + 3; keys in bins above bin i number total - (prefix through i)
        int c[4], loc = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = hist[4 * lane + i];
          loc += c[i];
        }
        const double incl = wave_incl_scan_dpp((double)loc);  // counts <= 4096 are exact
        const int total = (int)readlane_f64(incl, 63);
        int through = (int)incl - loc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          through += c[i];
          const int hi = total - through;  // keys in higher bins
          if (hi < need && need <= hi + c[i]) {
            sel[0] = 4 * lane + i;
            sel[1] = need - hi;
            sel[2] = c[i];
          }
        }
      }
      __syncthreads();
      const int d = sel[0], bin = sel[2];
      need = sel[1];
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        if (!(cand >> k & 1u)) continue;
        const int kb = key_byte(key[k], tid + BT * k, pass);
        if (kb > d) above |= 1u << k;
        if (kb != d) cand &= ~(1u << k);
      }
      if (need == bin) break;  // block-uniform; holds at the last pass, where every bin has one key
    }
    above |= cand;
  } else {
    above = 0;
  }

#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int t = tid + BT * k;
    if (t >= T) continue;
    const int s_t = fl[k] + (int)(above >> k & 1u);
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
  const dim3 grid(p.H, p.B);
  if (p.T <= BT) budget_kernel<1><<<grid, BT, 0, st>>>(p);
  else if (p.T <= 2 * BT) budget_kernel<2><<<grid, BT, 0, st>>>(p);
  else if (p.T <= 4 * BT) budget_kernel<4><<<grid, BT, 0, st>>>(p);
  else if (p.T <= 8 * BT) budget_kernel<8><<<grid, BT, 0, st>>>(p);
  else budget_kernel<16><<<grid, BT, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace santa
