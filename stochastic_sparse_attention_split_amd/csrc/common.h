// Shared device/host definitions of the SANTA / S²ANTA HIP path (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

// Keys per chunk: the unit of the split-K score pass and of the per-chunk (max, sum-exp) statistics
// (the tile of "Stochastic Sparse Attention for Memory-Bound Inference", Appendix O, Algorithm 3).
// The estimator is defined by the global CDF, so results do not depend on this choice.
constexpr int CHUNK = 256;
constexpr int MAX_CHUNKS = 4096;          // nk <= 2^20 per sequence
constexpr int MAX_GROUP = 8;              // query heads per KV head handled by one score block
constexpr int FUSED_CDF_MAX_T = 128;  // up to this many chunks the sampling kernel builds the chunk CDF itself
// Above this many sampling blocks (B * kv_heads * T; 8 per CU) the chunk CDF is built once per head by its
// own kernel even for T <= FUSED_CDF_MAX_T: every sampling block would otherwise rebuild all T chunk
// entries of its heads, fp64 work that then outweighs the extra launch.
constexpr int64_t SEPARATE_CDF_MIN_BLOCKS = 2048;
// One-launch decode (score, chunk CDF, sampling, gather and the output sum in one kernel): the blocks of
// a (KV head, sequence) group meet at barriers in device memory, so every block of the grid must be
// resident at once (one block per CU). Sizes of the synchronisation region at the start of every
// workspace, and the largest chunk count per sequence the in-kernel chunk CDF takes (8 chunks per lane).
constexpr int SYNC_MAX_BLOCKS = 1024;
constexpr int SYNC_MAX_GROUPS = 1024;
constexpr int DECODE_MAX_T = 512;
constexpr int DECODE_MAX_CHUNKS = 32;  // chunks per block: the sampled-key bitmap (4 words per lane) is scanned by one wave
constexpr int SPIN_LIMIT_DEFAULT = 1 << 22;  // polls before a bounded wait gives up

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):
// two 32x32->64 products per round, counter (c0,c1,c2,c3) <- (hi1^c1^k0, lo1, hi0^c3^k1, lo0), key
// advanced by the Weyl constants between rounds.
struct Philox4 {
  uint32_t x0, x1, x2, x3;
};

__host__ __device__ inline uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

__host__ __device__ inline Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = mulhi32(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = mulhi32(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return {c0, c1, c2, c3};
}

// 53-bit uniform in [0,1) from the first two output words: top 53 bits of (x0:x1), times 2^-53 (exact).
__host__ __device__ inline double uniform53(uint64_t seed, uint32_t m, uint32_t h, uint32_t b, uint32_t tag) {
  const Philox4 r = philox4x32_10(m, h, b, tag, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t w = ((uint64_t)r.x0 << 32) | (uint64_t)r.x1;
  return (double)(w >> 11) * 0x1.0p-53;
}

constexpr uint32_t TAG_POINT = 0;      // i.i.d. / stratified point m
constexpr uint32_t TAG_SYS = 1;        // systematic offset (m = 0)
constexpr uint32_t TAG_PROP = 3;       // S²ANTA-prop tile offset a0
constexpr uint32_t TAG_FLASH = 4;      // S²ANTA-flash tile offset a0
constexpr uint32_t TAG_GROUP = 5;      // mean-group Bernoulli feature m (+256 n for sample n)
constexpr uint32_t TAG_BERNOULLI = 2;  // ternary-query element m (+256 n for Bernoulli sample n)

// ---------------------------------------------------------------------------------------------
// e^x in fp64 for the softmax arguments x = s - max <= 0 (also correct for x up to ~709); x < -746 and
// x = -inf give +0. Derived from the mathematics: x = k ln2 + r with k = rint(x / ln2), |r| <= ln2 / 2;
// ln2 = LN2_HI + LN2_LO where LN2_HI keeps 32 significant bits, so k * LN2_HI is exact for |k| < 2^21;
// e^r by its Taylor series through r^13 (the remainder is below 2^-57 relative on |r| <= ln2 / 2), in
// Horner form with the coefficients 1/n! rounded to fp64; then the factor 2^k by ldexp. Straight-line
// code with no branch: a call costs 19 fp64 operations. Accuracy: within a few units in the last place of
// the correctly rounded result; e^0 = 1 exactly.
__host__ __device__ inline double exp_f64(double x) {
  constexpr double INV_LN2 = 0x1.71547652b82fep+0;   // 1 / ln 2
  constexpr double LN2_HI = 0x1.62e42ff000000p-1;    // ln 2 to 32 significant bits
  constexpr double LN2_LO = -0x1.718432a1b0e26p-35;  // ln 2 - LN2_HI
  const double k = fmax(rint(x * INV_LN2), -1100.0);  // -inf and huge negative x: clamped (result 0 below)
  double r = fma(-k, LN2_HI, x);
  r = fma(-k, LN2_LO, r);
  double q = 0x1.6124613a86d09p-33;       // 1/13!
  q = fma(q, r, 0x1.1eed8eff8d898p-29);   // 1/12!
  q = fma(q, r, 0x1.ae64567f544e4p-26);   // 1/11!
  q = fma(q, r, 0x1.27e4fb7789f5cp-22);   // 1/10!
  q = fma(q, r, 0x1.71de3a556c734p-19);   // 1/9!
  q = fma(q, r, 0x1.a01a01a01a01ap-16);   // 1/8!
  q = fma(q, r, 0x1.a01a01a01a01ap-13);   // 1/7!
  q = fma(q, r, 0x1.6c16c16c16c17p-10);   // 1/6!
  q = fma(q, r, 0x1.1111111111111p-7);    // 1/5!
  q = fma(q, r, 0x1.5555555555555p-5);    // 1/4!
  q = fma(q, r, 0x1.5555555555555p-3);    // 1/3!
  q = fma(q, r, 0.5);                     // 1/2!
  q = fma(q, r, 1.0);                     // 1/1!
  q = fma(q, r, 1.0);                     // 1/0!
  const double y = ldexp(q, (int)k);
  return x >= -746.0 ? y : 0.0;
}

// ---------------------------------------------------------------------------------------------
// 16-byte streaming load that does not allocate in the caches (K and V are read once per step; a
// non-temporal load also avoids evicting dirty lines from the Infinity Cache)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------------------------
// element conversions

// bf16 pair packed in a 32-bit word -> two floats (exact: bf16 is the top half of an fp32)
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp64 -> bf16 bits, round to nearest even, directly from the double (no intermediate fp32 rounding).
// Values are expected in the normal fp32 exponent range.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  uint64_t bits = (uint64_t)__double_as_longlong(x);
  const uint64_t lsb = (bits >> 45) & 1u;  // lowest kept mantissa bit (7 kept of 52)
  bits += 0x0FFFFFFFFFFFull + lsb;          // 2^44 - 1 + lsb: ties go to even
  bits &= ~0x1FFFFFFFFFFFull;               // clear the 45 dropped bits
  const float f = (float)__longlong_as_double((long long)bits);  // exact: fits in bf16 precision
  return (uint16_t)(__float_as_uint(f) >> 16);
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A 16-byte piece of a row: 8 bf16 or 4 fp32 elements, widened exactly to fp64.
template <bool BF16>
struct Piece;

template <>
struct Piece<true> {
  static constexpr int EPL = 8;
  __device__ static inline void to_f64(const uint4& w, double* o) {
    o[0] = (double)bf16_lo(w.x);
    o[1] = (double)bf16_hi(w.x);
    o[2] = (double)bf16_lo(w.y);
    o[3] = (double)bf16_hi(w.y);
    o[4] = (double)bf16_lo(w.z);
    o[5] = (double)bf16_hi(w.z);
    o[6] = (double)bf16_lo(w.w);
    o[7] = (double)bf16_hi(w.w);
  }
  __device__ static inline void to_f32(const uint4& w, float* o) {
    o[0] = bf16_lo(w.x);
    o[1] = bf16_hi(w.x);
    o[2] = bf16_lo(w.y);
    o[3] = bf16_hi(w.y);
    o[4] = bf16_lo(w.z);
    o[5] = bf16_hi(w.z);
    o[6] = bf16_lo(w.w);
    o[7] = bf16_hi(w.w);
  }
  __device__ static inline double elem(const void* base, int64_t i) {
    return (double)__uint_as_float(((uint32_t)((const uint16_t*)base)[i]) << 16);
  }
};

template <>
struct Piece<false> {
  static constexpr int EPL = 4;
  __device__ static inline void to_f64(const uint4& w, double* o) {
    o[0] = (double)__uint_as_float(w.x);
    o[1] = (double)__uint_as_float(w.y);
    o[2] = (double)__uint_as_float(w.z);
    o[3] = (double)__uint_as_float(w.w);
  }
  __device__ static inline void to_f32(const uint4& w, float* o) {
    o[0] = __uint_as_float(w.x);
    o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z);
    o[3] = __uint_as_float(w.w);
  }
  __device__ static inline double elem(const void* base, int64_t i) { return (double)((const float*)base)[i]; }
};

// ---------------------------------------------------------------------------------------------
// fp64 wavefront operations with DPP (row shifts within 16-lane rows, then row broadcasts 15 / 31):
// six dependent VALU steps instead of LDS-latency lane permutes.
template <int CTRL, int ROW_MASK>
__device__ inline double dpp_f64(double old, double src) {
  const long long o = __double_as_longlong(old), s = __double_as_longlong(src);
  const int lo = __builtin_amdgcn_update_dpp((int)o, (int)s, CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(o >> 32), (int)(s >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// inclusive prefix sum over the 64 lanes (lane i gets the sum of lanes 0..i)
__device__ inline double wave_incl_scan_dpp(double v) {
  v += dpp_f64<0x111, 0xf>(0.0, v);  // row_shr:1
  v += dpp_f64<0x112, 0xf>(0.0, v);  // row_shr:2
  v += dpp_f64<0x114, 0xf>(0.0, v);  // row_shr:4
  v += dpp_f64<0x118, 0xf>(0.0, v);  // row_shr:8
  v += dpp_f64<0x142, 0xa>(0.0, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xc>(0.0, v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// running maximum over the lanes; lane 63 holds the wave maximum
__device__ inline double wave_incl_max_dpp(double v) {
  const double ninf = -INFINITY;
  v = fmax(v, dpp_f64<0x111, 0xf>(ninf, v));
  v = fmax(v, dpp_f64<0x112, 0xf>(ninf, v));
  v = fmax(v, dpp_f64<0x114, 0xf>(ninf, v));
  v = fmax(v, dpp_f64<0x118, 0xf>(ninf, v));
  v = fmax(v, dpp_f64<0x142, 0xa>(ninf, v));
  v = fmax(v, dpp_f64<0x143, 0xc>(ninf, v));
  return v;
}

// value of lane `l` (wave-uniform), fp64
__device__ inline double readlane_f64(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)x, l);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// ---------------------------------------------------------------------------------------------
// Chunk CDF of one head, computed by one wave ("Stochastic Sparse Attention for Memory-Bound Inference",
// Appendix O, Algorithm 4: m* = max_t m_t, W_t = l_t exp(m_t - m*), Z = sum_t W_t). Lane l owns chunks
// [l*PER, l*PER + PER) (T <= 64 * PER). The exclusive prefix is made monotone by a running maximum so
// that the intervals [C_t, C_{t+1}) partition [0, C_T) exactly; C_T = max(Z, that maximum). The inputs
// m[j], l[j] are the lane's chunk statistics (entries at t >= T are ignored).
template <int PER>
struct ChunkCdf {
  double c[PER];  // C_t
  double f[PER];  // exp(m_t - m*)
  double top;     // C_T (wave-uniform)
  int last;       // last chunk with W_t > 0 (wave-uniform)
};

template <int PER>
__device__ inline void chunk_cdf_wave(const double* m, const double* l, int T, int lane, ChunkCdf<PER>& o) {
  const int t0 = lane * PER;
  double mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (t0 + j < T) mx = fmax(mx, m[j]);
  const double ms = readlane_f64(wave_incl_max_dpp(mx), 63);
  double loc[PER], run = 0.0;
  int lp = -1;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool valid = t0 + j < T;
    o.f[j] = valid ? exp_f64(m[j] - ms) : 0.0;
    const double w = l[j] * o.f[j];
    loc[j] = run;  // local exclusive prefix, offset below
    run += w;
    if (valid && w > 0.0) lp = t0 + j;
  }
  const double incl = wave_incl_scan_dpp(run);
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  double lmax = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const double c = fmax(excl + loc[j], lmax);
    loc[j] = c;
    lmax = c;
  }
  // running maximum across lanes: lane l's values are raised to the maximum of all earlier lanes
  const double pmax = wave_incl_max_dpp(t0 < T ? lmax : 0.0);
  double before = __shfl_up(pmax, 1, 64);
  if (lane == 0) before = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) o.c[j] = fmax(loc[j], before);
  o.top = fmax(readlane_f64(incl, 63), readlane_f64(pmax, 63));
  o.last = (int)readlane_f64(wave_incl_max_dpp((double)lp), 63);
}

// ---------------------------------------------------------------------------------------------
// Points and the in-chunk search shared by the sampling kernels.

// T_m of point m of query head h in sequence b: i.i.d. u_m, stratified (m + u_m)/S, systematic (m + u)/S
// with one u per head ("Stochastic Sparse Attention for Memory-Bound Inference", Section 2 Eq. 4 and
// Section 2.1)
__device__ inline double point_of(uint64_t seed, int mode, int S, int m, int h, int b, double u_sys) {
  if (mode == 0) return uniform53(seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
  if (mode == 1) {
    const double u = uniform53(seed, (uint32_t)m, (uint32_t)h, (uint32_t)b, TAG_POINT);
    return ((double)m + u) / (double)S;
  }
  return ((double)m + u_sys) / (double)S;
}

// Where entry e of a prefix row is stored: RowAt is the plain layout; RowSwz, the layout of the prefix rows
// a block keeps in LDS, permutes each 16-entry block by (block index ^ k), k the row's chunk slot in the
// block, so that the reads of a search over several rows (the same entry of different rows, or entry j
// of different 16-entry blocks) fall in different LDS banks.
struct RowAt {
  __device__ int operator()(int e) const { return e; }
};
struct RowSwz {
  int k;
  __device__ int operator()(int e) const { return (e & ~15) | ((e ^ (e >> 4) ^ k) & 15); }
};

// search_chunk (below) in two rounds of independent loads (fewer dependent round trips, in LDS or in
// device memory): the first 16-entry block whose last entry exceeds r (15 probes), then the first
// entry of that block that does. at(e) is where entry e is stored.
template <class At = RowAt>
__device__ inline int search_chunk16(const double* P, double f, double r, At at = At()) {
  static_assert(CHUNK == 256, "16 blocks of 16 entries");
  double v[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) v[i] = P[at(16 * i + 15)];
  int bi = 15;  // no earlier block qualifies: the answer, if any, is in the last one
#pragma unroll
  for (int i = 14; i >= 0; --i)
    if (v[i] * f > r) bi = i;
  double w[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) w[j] = P[at(16 * bi + j)];
  int j0 = 16;
#pragma unroll
  for (int j = 15; j >= 0; --j)
    if (w[j] * f > r) j0 = j;
  const int res = 16 * bi + j0;
  return res < CHUNK ? res : -1;
}

// first j in [0, CHUNK) with P[j] * f > r, else -1 (P nondecreasing; entries past the chunk's last key
// repeat the chunk total): the half-open inverse-CDF convention 1{F(j-1) <= t < F(j)} (Appendix A.4)
__device__ inline int search_chunk(const double* P, double f, double r) {
  int lo = 0, hi = CHUNK;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] * f > r) hi = mid; else lo = mid + 1;
  }
  return lo < CHUNK ? lo : -1;
}

// last key of a chunk whose prefix grows (its last key with mass; 0 if none); at(e) as above
template <class At = RowAt>
__device__ inline int last_positive(const double* P, int len, At at = At()) {
  for (int j = len - 1; j > 0; --j)
    if (P[at(j)] > P[at(j - 1)]) return j;
  return 0;
}

// block-wide maximum and sum over NW waves (every thread passes its value; all get the result). The sum
// is taken in a fixed order: lanes by the DPP scan tree, then the waves in index order. `red` holds NW
// doubles of LDS; both end with a barrier, so `red` may be reused at once.
template <int NW>
__device__ inline double block_max_f64(double v, double* red, int lane, int wave) {
  v = readlane_f64(wave_incl_max_dpp(v), 63);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmax(r, red[w]);
  __syncthreads();
  return r;
}

template <int NW>
__device__ inline double block_sum_f64(double v, double* red, int lane, int wave) {
  v = readlane_f64(wave_incl_scan_dpp(v), 63);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += red[w];
  __syncthreads();
  return r;
}

// inclusive prefix sum of an int over the wave (DPP row shifts and broadcasts)
__device__ inline int wave_incl_scan_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// a compile-time int as a value (selects a template instance inside a generic lambda)
template <int N>
struct IntC {
  static constexpr int value = N;
};

// element j (wave-uniform) of a small register array
template <int N>
__device__ inline double pick(const double* a, int j) {
  double v = a[0];
#pragma unroll
  for (int i = 1; i < N; ++i)
    if (j == i) v = a[i];
  return v;
}

// S²ANTA-prop budgets of one head, computed by one wave (Appendix O, Algorithm 4; T <= 64 * PER, lane l
// owns tiles [l*PER, l*PER + PER)): m* = max m_t, W_t = exp(m_t - m*) l_t, Z = sum W_t, q_t = S W_t / Z,
// S_t = floor(q_t) plus one for the R = S - sum floor(q_t) largest fractional parts (ties to the lower
// tile). The winners come from a radix select over the 80-bit keys (fraction bits, 0xFFFF - t), one byte
// per pass, in a 256-bin LDS histogram owned by this wave; it stops once every key left in the chosen
// bin wins. Gives every tile's S_t, its first slot sum_{t' < t} S_t', exp(m_t - m*), and Z.
struct TileBudget {
  int st, off;
  double f, Z;
};

__device__ inline int prop_key_byte(uint64_t frac_bits, int t, int pass) {
  return pass < 8 ? (int)((frac_bits >> (56 - 8 * pass)) & 255u)
                  : (int)(((uint32_t)(0xFFFF - t) >> (8 * (9 - pass))) & 255u);
}

// every tile's values, each held by the lane that owns the tile
template <int PER>
struct TileBudgets {
  double st[PER];   // S_t
  double off[PER];  // first slot of the tile in the head's index list
  double e[PER];    // exp(m_t - m*)
  double Z;
};

template <int PER>
__device__ inline void tile_budgets_wave(const double* m, const double* l, int T, int S, int lane, int* hist,
                                         TileBudgets<PER>& o) {
  const int t0 = lane * PER;
  double mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (t0 + j < T) mx = fmax(mx, m[j]);
  const double ms = readlane_f64(wave_incl_max_dpp(mx), 63);
  double e[PER], w[PER], run = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    e[j] = exp_f64(m[j] - ms);
    w[j] = t0 + j < T ? e[j] * l[j] : 0.0;
    run += w[j];
  }
  const double Z = readlane_f64(wave_incl_scan_dpp(run), 63);
  int fl[PER];
  uint64_t key[PER];
  uint32_t cand = 0u;
  double flsum = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const double q = ((double)S * w[j]) / Z;
    const double f = floor(q);
    fl[j] = (int)f;
    key[j] = (uint64_t)__double_as_longlong(q - f);
    if (t0 + j < T) {
      flsum += f;
      cand |= 1u << j;
    }
  }
  int need = S - (int)readlane_f64(wave_incl_scan_dpp(flsum), 63);
  uint32_t above = 0u;
  if (need > 0) {
    // a byte that every key shares would put every candidate in one bin and change nothing: the passes
    // start at the first byte in which the keys differ (the tile bytes if every fraction is equal)
    const uint64_t ref = (uint64_t)__shfl((long long)key[0], 0, 64);  // tile 0 always exists
    uint64_t dif = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (cand >> j & 1u) dif |= key[j] ^ ref;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dif |= (uint64_t)__shfl_xor((long long)dif, o, 64);
    const int first = dif == 0 ? 8 : __builtin_clzll(dif) / 8;
    for (int pass = first; pass < 10; ++pass) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (cand >> j & 1u) atomicAdd(&hist[prop_key_byte(key[j], t0 + j, pass)], 1);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      int c[4], loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[4 * lane + i];
        loc += c[i];
      }
      const int incl = wave_incl_scan_i32(loc);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      int through = incl - loc, sd = 0, sneed = 0, sbin = 0;
      bool found = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        through += c[i];
        const int hi = total - through;  // keys in higher bins
        if (hi < need && need <= hi + c[i]) {
          found = true;
          sd = 4 * lane + i;
          sneed = need - hi;
          sbin = c[i];
        }
      }
      const int owner = __builtin_ctzll(__ballot(found));  // exactly one lane finds the bin
      const int d = __builtin_amdgcn_readlane(sd, owner), bin = __builtin_amdgcn_readlane(sbin, owner);
      need = __builtin_amdgcn_readlane(sneed, owner);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (!(cand >> j & 1u)) continue;
        const int kb = prop_key_byte(key[j], t0 + j, pass);
        if (kb > d) above |= 1u << j;
        if (kb != d) cand &= ~(1u << j);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // histogram reads done before the next clear
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (need == bin) break;  // wave-uniform; holds at the last pass, where every bin has one key
    }
    above |= cand;
  }
  double offv[PER], acc = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    o.st[j] = (double)(fl[j] + (int)(above >> j & 1u));
    offv[j] = acc;  // local exclusive prefix
    acc += t0 + j < T ? o.st[j] : 0.0;
  }
  const double inc = wave_incl_scan_dpp(acc);  // integer sums are exact in fp64
  const double before = inc - acc;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    o.off[j] = before + offv[j];
    o.e[j] = e[j];
  }
  o.Z = Z;
}

// the values of tile t (wave-uniform)
template <int PER>
__device__ inline TileBudget tile_budget_wave(const double* m, const double* l, int T, int S, int t, int lane,
                                              int* hist) {
  TileBudgets<PER> o;
  tile_budgets_wave<PER>(m, l, T, S, lane, hist, o);
  const int ol = t / PER, oj = t % PER;
  TileBudget r;
  r.st = (int)readlane_f64(pick<PER>(o.st, oj), ol);
  r.off = (int)readlane_f64(pick<PER>(o.off, oj), ol);
  r.f = readlane_f64(pick<PER>(o.e, oj), ol);
  r.Z = o.Z;
  return r;
}

// S²ANTA-flash uniform tile budget ("Stochastic Sparse Attention for Memory-Bound Inference", Appendix P,
// Algorithm 6: S_tile ~ S / T, rounded): halves round up, at least one sample per tile
inline int flash_tile_budget(int S, int64_t T) {
  const int64_t st = (2 * (int64_t)S + T) / (2 * T);
  return st < 1 ? 1 : (int)st;
}

// ---------------------------------------------------------------------------------------------
// problem description passed to kernels

struct Problem {
  const void* q;
  const void* K;
  const void* V;
  void* out;
  int B, H, Hkv, G, d;
  int64_t nk;
  int64_t seq_stride;    // elements
  int64_t batch_stride;  // elements
  int S;
  int mode;              // 0 iid, 1 strat, 2 sys, 3 prop, 4 flash
  int S_tile;            // S²ANTA-flash: samples per tile
  int L;                 // sampled keys listed per head (S; T * S_tile for S²ANTA-flash)
  bool ternary;
  bool group_bern;       // mean-group-query Bernoulli scores (feature-major K only)
  int bern;              // Bernoulli samples B of the mean-group query
  bool kfm;              // K is feature-major: K^T [B][Hkv][d][kt_row_stride]
  int64_t kt_row_stride;    // elements between feature rows of K^T
  int64_t kt_batch_stride;  // elements between sequences of K^T
  bool bf16;
  uint64_t seed;
  double scale;          // 1/sqrt(d), formed on the host in fp64
  int T;                 // chunks per sequence
  int score_blocks_per_group;  // score blocks per (KV head, sequence); each loops over chunks
  // workspace (no initial contents required: every call writes what it later reads)
  double* stash;         // [B, H, stash_stride] in-chunk inclusive prefix of exp(s - m_t)
  int64_t stash_stride;  // T * CHUNK: rows padded to whole chunks
  double* cmax;          // [B, H, T] chunk max m_t
  double* csum;          // [B, H, T] chunk sum-exp l_t
  double* cdf;           // [B, H, T+1] exclusive prefix of W_t = l_t exp(m_t - m*); cdf[T] = Z
  double* cscale;        // [B, H, T] exp(m_t - m*)
  int32_t* lastpos;      // [B, H] last chunk with W_t > 0
  float* partial;        // [B, Hkv, T, G, d] per-chunk sums of count * V (fp32, exact products)
  int32_t* idx;          // [B, H, L]
  int32_t* unique;       // [B, Hkv, T] distinct sampled keys of each chunk; then [B, Hkv, T] V rows read (fused flash)
  uint32_t* sink;        // [B, Hkv, T] values of the cache-warming loads (never read)
  int32_t* sync_err;     // [B, Hkv, T] per score block: 1 if an LDS handshake timed out
  int32_t* budget;       // [B, H, T] S²ANTA-prop tile budgets S_t
  int32_t* boff;         // [B, H, T] exclusive prefix of the budgets (first idx slot of each tile)
  double* prob;          // optional [B, H, nk]
  int32_t* kfeat;        // [B, Hkv] feature rows of K^T read by the feature-major score pass
  bool fused;            // S²ANTA-flash sampled and gathered inside the streaming score pass
  bool want_unique;      // fill unique[] (the stats path reads it); the fused S²ANTA-flash skips it otherwise
  bool want_idx;         // the caller asked for idx_out (the fused S²ANTA-flash writes idx only then)
  bool cdf_done;         // the chunk CDF kernel has run: the sampling kernel reads cdf / cscale / lastpos
  uint64_t* bmap;        // [B, Hkv, T, 4, 4] fused S²ANTA-flash: sampled keys of each (chunk, head) as bits
  int spin_limit;        // polls before a bounded wait gives up (the block then flags itself)
  int32_t* status;       // [B, Hkv] per call: 0, or 1 if a bounded wait of the group's blocks gave up
  bool check_sync;       // the merge reads the streaming score blocks' handshake flags (sync_err)
  // one-launch decode (KM_DECODE): epoch per group and started flag per block (grid index
  // (b * Hkv + kv) * P + r); the chunk statistics are cmax / csum, the per-block partial output sums
  // live in `partial` as [blocks, G, d]
  uint64_t* sync_epoch;  // [SYNC_MAX_GROUPS]
  uint64_t* sync_start;  // [SYNC_MAX_BLOCKS] started flags: the block's published words are VOID
  bool one_launch;       // the whole decode runs in the score kernel
  int lds_nb, lds_cnt, lds_list, lds_bits, lds_cdf, lds_scl, lds_rows, lds_hist;  // its sampling phase's LDS plan
};

// LDS plan of the sampling phase of the one-launch decode for G heads, n chunks per block and T chunks
// per sequence, inside the `cap` bytes of the score phase's K tiles: per-key 16-bit counts per head, the
// list and bitmap of the sampled keys, each head's chunk CDF C_0..C_T and chunk scales, and for G <= 4,
// n <= 4 the prefix rows of the block's nb = n chunks per head (total = 0: does not fit). Computed on
// the host, which passes the offsets to the kernel.
struct DecodeLds {
  int nb;
  size_t cnt, list, bits, cdf, scl, rows, hist, total;
};
// prop: S²ANTA-prop, whose head waves also need a 256-bin histogram each for the tile budgets
__host__ __device__ inline DecodeLds decode_lds_plan(int G, int n, int T, size_t cap, bool prop) {
  const size_t gm = G <= 4 ? 4 : 8, ncw = gm / 2;
  DecodeLds L;
  L.cnt = 0;
  L.list = L.cnt + (size_t)n * CHUNK * ncw * 4;
  L.bits = L.list + (size_t)n * CHUNK * 4;
  L.cdf = L.bits + ((size_t)n * CHUNK / 8 + 15) / 16 * 16;
  L.scl = L.cdf + ((size_t)G * (T + 1) * 8 + 15) / 16 * 16;
  L.rows = L.scl + (size_t)G * T * 8;
  // the prefix rows go to LDS only where the score phase kept them in registers (G <= 4, n <= 4); with
  // more chunks or heads they are searched where they are, in device memory
  const size_t per_chunk = (size_t)G * CHUNK * 8;
  const size_t want_nb = (G <= 4 && n <= 4) ? (size_t)n : 0;
  const size_t fit = cap > L.rows ? (cap - L.rows) / per_chunk : 0;
  L.nb = (int)(fit < want_nb ? fit : want_nb);
  L.hist = L.rows + (size_t)L.nb * per_chunk;
  L.total = L.hist + (prop ? gm * 256 * 4 : 0);
  if (L.nb < (int)want_nb || L.total > cap) L.total = 0;  // does not fit
  return L;
}

// sampling modes, as numbered in the C header (SANTA_IID ... SANTA_FLASH)
constexpr int MODE_IID = 0, MODE_STRAT = 1, MODE_SYS = 2, MODE_PROP = 3, MODE_FLASH = 4;

// forms of the streaming score kernel
constexpr int KM_SCORE = 0;   // scores, statistics and prefix rows for the separate sampling kernel
constexpr int KM_FLASH = 1;   // S²ANTA-flash kernel 1 fused in
constexpr int KM_DECODE = 2;  // the whole decode step in one launch
constexpr int KM_DECODE_PROP = 3;   // the same for S²ANTA-prop (tile budgets and per-key counts, no points)
constexpr int KM_DECODE_FLASH = 4;  // the same for S²ANTA-flash (uniform tile budget, weighted gather)

}  // namespace santa
