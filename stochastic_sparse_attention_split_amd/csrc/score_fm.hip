// Score pass over a feature-major key cache K^T [batch][kv_heads][d][row stride] ("Stochastic Sparse
// Attention for Memory-Bound Inference", Section 5.1 and Appendix C.2): one block per (KPT / 4 chunks,
// KV group, sequence). A feature row holds one head dimension of consecutive keys, so a score estimator that
// needs only some features reads only those rows.
//
// Query weights w[g][i] (the score of head g is s_{g,n} = (sum_i w[g][i] K_{n,i}) / sqrt(dk)):
//   * exact scores (Eq. 1): w[g][i] = q_{g,i};
//   * Bernoulli ternary query per head (Section 5, Eq. 5; Appendix C, Eqs. 8-9, B = 1):
//     w[g][i] = norm_g qhat_{g,i}, norm_g = max_i |q_{g,i}|, qhat from Philox counter (i, h, b, 2);
//   * mean-group query (Section 5.1, Eq. 6; Appendix C.2, Eqs. 10-13): m_i = (1/G) sum_g |q_{g,i}|,
//     norm = max_i m_i, stratified Bernoulli counts c_i = #{n < B : (n + U_{i,n}) / B < m_i / norm} with
//     U_{i,n} from Philox counter (i, kv, b, 5 + 256 n), w[g][i] = ((norm c_i) / B) / m_i * q_{g,i}.
// Features with w[.][i] = 0 for every head of the group are not read. The block's 256 threads are
// 64 groups of KPT consecutive keys (one 16-byte load per feature row for bf16 and KPT = 8) x 4 feature
// slices, so a block covers KPT / 4 chunks; each slice accumulates its features in fp64 (bf16 and fp32
// values are exact in fp64), the slices are added in a fixed order. The softmax bookkeeping and the
// stores (chunk max, sum, in-chunk prefix) are those of the sequence-major score pass.
//
// The pass is bound by HBM (selected features x nk x element bytes); the fp64 VALU work is 5 operations
// per element and head group (one conversion, four FMAs for four heads).

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int FM_THREADS = 256;
constexpr int FM_SLICES = FM_THREADS / 64;  // feature slices; each wave is one slice
constexpr int UNR = 8;                      // feature rows in flight per thread

// KPT consecutive elements of a feature row as raw 32-bit words (non-temporal: each row is read once)
template <bool BF16, int KPT>
struct Raw {
  static constexpr int NW = BF16 ? KPT / 2 : KPT;
  uint32_t w[NW];
};

template <bool BF16, int KPT>
__device__ inline Raw<BF16, KPT> load_raw(const void* base, int64_t off) {
  Raw<BF16, KPT> r;
  const uint32_t* src = (const uint32_t*)((const char*)base + off * (BF16 ? 2 : 4));
  if constexpr (Raw<BF16, KPT>::NW == 4) {
    const uint4 v = load_stream16(src);
    r.w[0] = v.x;
    r.w[1] = v.y;
    r.w[2] = v.z;
    r.w[3] = v.w;
  } else {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)src);
    r.w[0] = v.x;
    r.w[1] = v.y;
  }
  return r;
}

template <bool BF16, int KPT>
__device__ inline double raw_elem(const Raw<BF16, KPT>& r, int k) {
  if constexpr (BF16) return (double)((k & 1) ? bf16_hi(r.w[k >> 1]) : bf16_lo(r.w[k >> 1]));
  else return (double)__uint_as_float(r.w[k]);
}

template <bool BF16>
__device__ inline double load1(const void* base, int64_t off) {
  if constexpr (BF16) return (double)__uint_as_float((uint32_t)((const uint16_t*)base)[off] << 16);
  else return (double)((const float*)base)[off];
}

template <int D, bool BF16, int GM, int KPT>
__global__ __launch_bounds__(FM_THREADS) void score_fm_kernel(Problem p) {
  constexpr int KPB = 64 * KPT;        // keys per block
  constexpr int CPB = KPB / CHUNK;     // chunks per block
  static_assert(KPB % CHUNK == 0, "a block covers whole chunks");
  __shared__ double w[GM][D];
  __shared__ double qv[GM][D];
  __shared__ double red[FM_SLICES][GM][KPB];
  __shared__ int sel[D];
  __shared__ int wcnt[FM_THREADS / 64];
  __shared__ double hn[GM];
  __shared__ double bred[FM_THREADS / 64];

  const int tb = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, T = p.T;
  const int h0 = kv * G;
  const int64_t nb0 = (int64_t)tb * KPB;  // first key of the block

  // ---- query weights of the group (every block recomputes them: d x G values and d x B generator calls)
  for (int i = tid; i < GM * D; i += FM_THREADS) {
    const int g = i / D, e = i % D;
    qv[g][e] = g < G ? load1<BF16>(p.q, ((int64_t)b * p.H + h0 + g) * D + e) : 0.0;
  }
  __syncthreads();
  bool keep = false;
  if (p.group_bern) {
    double m = 0.0;
    if (tid < D) {
      for (int g = 0; g < G; ++g) m += fabs(qv[g][tid]);
      m = m / (double)G;
    }
    const double norm = block_max_f64<FM_THREADS / 64>(tid < D ? m : 0.0, bred, lane, wave);
    if (tid < D) {
      int c = 0;
      if (norm > 0.0) {
        const double pi = m / norm;
        for (int n = 0; n < p.bern; ++n) {
          const double u = uniform53(p.seed, (uint32_t)tid, (uint32_t)kv, (uint32_t)b, TAG_GROUP + 256u * n);
          c += (((double)n + u) / (double)p.bern < pi) ? 1 : 0;
        }
      }
      const double ratio = (m > 0.0 && c > 0) ? ((norm * (double)c) / (double)p.bern) / m : 0.0;
      for (int g = 0; g < GM; ++g) w[g][tid] = g < G ? ratio * qv[g][tid] : 0.0;
      keep = ratio != 0.0;
    }
  } else if (p.ternary) {
    if (tid < G) {
      double nrm = 0.0;
      for (int e = 0; e < D; ++e) nrm = fmax(nrm, fabs(qv[tid][e]));
      hn[tid] = nrm;
    }
    __syncthreads();
    if (tid < D) {
      for (int g = 0; g < GM; ++g) {
        double v = 0.0;
        if (g < G && hn[g] > 0.0) {
          const double qe = qv[g][tid];
          const double u = uniform53(p.seed, (uint32_t)tid, (uint32_t)(h0 + g), (uint32_t)b, TAG_BERNOULLI);
          if (u < fabs(qe) / hn[g]) v = (qe > 0.0 ? 1.0 : (qe < 0.0 ? -1.0 : 0.0)) * hn[g];
        }
        w[g][tid] = v;
        keep = keep || v != 0.0;
      }
    }
  } else if (tid < D) {
    for (int g = 0; g < GM; ++g) {
      w[g][tid] = qv[g][tid];
      keep = keep || qv[g][tid] != 0.0;
    }
  }
  // compact the kept features in increasing order (threads tid < D, D <= 128: waves 0 and 1)
  const uint64_t bal = __ballot(keep);
  if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
  __syncthreads();
  const int before = (wave > 0 ? wcnt[0] : 0) + (wave > 1 ? wcnt[1] : 0) + (wave > 2 ? wcnt[2] : 0);
  if (keep) sel[before + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = tid;
  const int nsel = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  if (tb == 0 && tid == 0) p.kfeat[(int64_t)b * p.Hkv + kv] = nsel;
  __syncthreads();

  // ---- feature rows: thread (slice, key group) accumulates KPT keys x GM heads over its features
  const int kg = tid & 63, sl = tid >> 6;
  const int64_t nkp = (p.nk + KPT - 1) / KPT * KPT;
  // in bounds: rows hold >= nk rounded up to 8 >= nkp; groups past the end re-read the last one (masked)
  const int64_t kofs = min(nb0 + KPT * kg, nkp - KPT);
  const int64_t rbase = (int64_t)b * p.kt_batch_stride + (int64_t)kv * D * p.kt_row_stride + kofs;
  double acc[GM][KPT];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int k = 0; k < KPT; ++k) acc[g][k] = 0.0;
  for (int j0 = sl; j0 < nsel; j0 += FM_SLICES * UNR) {
    Raw<BF16, KPT> x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = min(j0 + FM_SLICES * u, nsel - 1);  // valid feature; duplicates are skipped below
      x[u] = load_raw<BF16, KPT>(p.K, rbase + (int64_t)sel[j] * p.kt_row_stride);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + FM_SLICES * u;
      if (j < nsel) {
        const int f = sel[j];
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
          const double xv = raw_elem<BF16, KPT>(x[u], k);
#pragma unroll
          for (int g = 0; g < GM; ++g) acc[g][k] = fma(w[g][f], xv, acc[g][k]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int k = 0; k < KPT; ++k) red[sl][g][KPT * kg + k] = acc[g][k];
  __syncthreads();

  // ---- per (chunk, head): chunk max, exponentials, in-chunk prefix (a wave per pair, 4 keys per lane)
  for (int pr = wave; pr < CPB * G; pr += FM_THREADS / 64) {
    const int c = pr / G, g = pr % G;
    const int t = tb * CPB + c;
    if (t >= T) continue;  // wave-uniform
    const int64_t n0 = (int64_t)t * CHUNK;
    const int len = (int)min((int64_t)CHUNK, p.nk - n0);
    const int64_t bh = (int64_t)b * p.H + h0 + g;
    double sv[4], lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = 4 * lane + i;
      const int rk = c * CHUNK + kk;
      const double raw = ((red[0][g][rk] + red[1][g][rk]) + red[2][g][rk]) + red[3][g][rk];
      sv[i] = kk < len ? raw * p.scale : -INFINITY;
      lmax = fmax(lmax, sv[i]);
    }
    const double m = readlane_f64(wave_incl_max_dpp(lmax), 63);
    double ex[4], pre[4], run = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = (4 * lane + i) < len ? exp_f64(sv[i] - m) : 0.0;
      run += ex[i];
      pre[i] = run;
    }
    const double incl = wave_incl_scan_dpp(run);
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    double2* dst = (double2*)(p.stash + bh * p.stash_stride + n0 + 4 * lane);
    dst[0] = make_double2(excl + pre[0], excl + pre[1]);
    dst[1] = make_double2(excl + pre[2], excl + pre[3]);
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
  }
}

template <int D, bool BF16, int GM, int KPT>
hipError_t launch_fm(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  constexpr int CPB = 64 * KPT / CHUNK;
  const dim3 grid((p.T + CPB - 1) / CPB, p.Hkv, p.B);
  return launch_timed(score_fm_kernel<D, BF16, GM, KPT>, grid, dim3(FM_THREADS), st, ev, p);
}

template <int D, bool BF16>
hipError_t launch_fm_dt(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  // bf16 with G <= 4: 8 keys per thread (one 16-byte load per feature row); otherwise 4 keys per thread
  if (p.G > 4) return launch_fm<D, BF16, 8, 4>(p, st, ev);
  if constexpr (BF16) return launch_fm<D, BF16, 4, 8>(p, st, ev);
  else return launch_fm<D, BF16, 4, 4>(p, st, ev);
}

}  // namespace

hipError_t launch_score_fm(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  if (p.d == 128) return p.bf16 ? launch_fm_dt<128, true>(p, st, ev) : launch_fm_dt<128, false>(p, st, ev);
  return p.bf16 ? launch_fm_dt<64, true>(p, st, ev) : launch_fm_dt<64, false>(p, st, ev);
}

}  // namespace santa
