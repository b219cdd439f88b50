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
constexpr uint32_t TAG_BERNOULLI = 2;  // ternary-query element m (+256 n for Bernoulli sample n)

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
  __device__ static inline double elem(const void* base, int64_t i) { return (double)((const float*)base)[i]; }
};

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
  int mode;              // 0 iid, 1 strat, 2 sys
  bool ternary;
  bool bf16;
  uint64_t seed;
  double scale;          // 1/sqrt(d), formed on the host in fp64
  int T;                 // chunks per sequence
  // workspace
  double* stash;         // [B, H, nk] in-chunk inclusive prefix of exp(s - m_t)
  double* cmax;          // [B, H, T] chunk max m_t
  double* csum;          // [B, H, T] chunk sum-exp l_t
  int32_t* idx;          // [B, H, S]
  int32_t* unique;       // [B, Hkv]
  double* prob;          // optional [B, H, nk]
};

}  // namespace santa
