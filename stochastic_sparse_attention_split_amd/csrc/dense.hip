// Dense decode attention baseline: softmax(q K^T / sqrt(dk)) V ("Stochastic Sparse Attention for
// Memory-Bound Inference", Section 2, Eq. 1), split-KV like FlashDecoding: one block per (chunk of
// dense_chunk(G) keys, KV head, sequence) writes the chunk's (max, sum-exp, unnormalised output) for the G
// heads of the group; a merge block per (head, sequence) rescales and sums them. fp32 arithmetic on
// bf16 or fp32 inputs; for bf16 the products use v_dot2 on bf16 pairs (the attention weights rounded to
// bf16 for the V sum, as in FlashAttention-style kernels); reads all of K and V once.

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace santa {

namespace {

constexpr int THREADS = 256;

template <bool BF16>
__device__ inline void piece_f32(const uint4& w, float* o) {
  if constexpr (BF16) {
    o[0] = bf16_lo(w.x);
    o[1] = bf16_hi(w.x);
    o[2] = bf16_lo(w.y);
    o[3] = bf16_hi(w.y);
    o[4] = bf16_lo(w.z);
    o[5] = bf16_hi(w.z);
    o[6] = bf16_lo(w.w);
    o[7] = bf16_hi(w.w);
  } else {
    o[0] = __uint_as_float(w.x);
    o[1] = __uint_as_float(w.y);
    o[2] = __uint_as_float(w.z);
    o[3] = __uint_as_float(w.w);
  }
}

// One block per (chunk of CH keys, KV head, sequence); each of the 4 waves owns CH / 4 consecutive
// keys of the chunk. LPR lanes hold one key row (16 bytes each), NRG rows side by side per load step. A
// wave issues the K and V loads of up to RB rows per lane at once (V does not depend on the scores), then
// keeps its own running max / sum-exp / weighted V sum, so the only block-wide step is the final merge of
// the 4 waves' partials.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs, fp32 accumulation (v_dot2)
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// two floats rounded to nearest-even bf16, packed (x in the low half)
__device__ inline uint32_t pack_bf16x2(float x, float y) {
  const bf16x2_t v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}

// Sum over aligned groups of N lanes (N = 2, 4, ..., 64), the result in every lane of the group. Up to 16
// lanes it uses DPP (quad permutes, then the half-row and row mirrors, each pairing a lane with one in
// the other half of its group), which needs no LDS round trip; every lane adds the same two values, so
// all lanes of a group hold the same bits.
template <int N>
__device__ inline float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  if constexpr (N >= 2) x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

template <int D, bool BF16, int GM, int CH>
__global__ __launch_bounds__(THREADS) void dense_partial_kernel(DenseProblem p) {
  constexpr int EPL = BF16 ? 8 : 4;        // elements per 16-byte piece
  constexpr int LPR = D / EPL;             // lanes per key row
  constexpr int NRG = 64 / LPR;            // rows per wave load step
  constexpr int WROWS = CH / (THREADS / 64);
  constexpr int R = WROWS / NRG;           // rows per lane
  constexpr int RBM = GM <= 4 ? 16 : 4;    // rows per lane in flight (fewer for 8 heads: registers)
  constexpr int RB = R < RBM ? R : RBM;
  __shared__ float wm[THREADS / 64][GM];
  __shared__ float wl[THREADS / 64][NRG][GM];
  __shared__ float wacc[THREADS / 64][NRG][GM][D];

  // the KV heads of a position are adjacent in memory: blocks of one chunk for every KV head run side by
  // side (grid x = KV head), so the rows they stream share DRAM pages
  const int kv = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int rg = lane / LPR, pc = lane % LPR;
  const int64_t n0 = (int64_t)t * CH;
  const int len = (int)((p.nk - n0) < CH ? (p.nk - n0) : CH);
  const size_t esz = BF16 ? 2 : 4;
  const int64_t base = (int64_t)b * p.batch_stride + n0 * p.seq_stride + (int64_t)kv * D;
  const char* kb = (const char*)p.K + esz * base;
  const char* vb = (const char*)p.V + esz * base;
  const int64_t rs = esz * p.seq_stride;
  const int r0 = wave * WROWS + rg;  // row of step k: r0 + k * NRG

  // the lane's 16-byte piece of every query of the group, all loads in flight at once (heads past G
  // read head 0 of the group and are zeroed)
  uint4 qw[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    const int64_t row = (int64_t)b * p.H + (int64_t)kv * G + (g < G ? g : 0);
    qw[g] = *((const uint4*)((const char*)p.q + esz * row * D) + pc);
  }

  float m[GM], l[GM], acc[GM][EPL];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int k0 = 0; k0 < R; k0 += RB) {
    uint4 kw[RB], vw[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int r = r0 + (k0 + k) * NRG;
      kw[k] = load_stream16((const uint4*)(kb + (r < len ? r : 0) * rs) + pc);  // rows past len masked below
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int r = r0 + (k0 + k) * NRG;
      vw[k] = load_stream16((const uint4*)(vb + (r < len ? r : 0) * rs) + pc);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every K and V load of the batch issued before the math
    float s[GM][RB];
    if constexpr (BF16) {  // bf16 pairs straight into v_dot2 (fp32 accumulation), scaled after the sum
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const bool ok = r0 + (k0 + k) * NRG < len;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          float d = 0.f;
          d = dot2_bf16(kw[k].x, g < G ? qw[g].x : 0u, d);
          d = dot2_bf16(kw[k].y, g < G ? qw[g].y : 0u, d);
          d = dot2_bf16(kw[k].z, g < G ? qw[g].z : 0u, d);
          d = dot2_bf16(kw[k].w, g < G ? qw[g].w : 0u, d);
          d = group_sum<LPR>(d) * p.scale;
          s[g][k] = ok ? d : -INFINITY;
        }
      }
    } else {
      float qv[GM][EPL];
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        piece_f32<BF16>(qw[g], qv[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] = g < G ? qv[g][e] * p.scale : 0.f;
      }
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float x[EPL];
        piece_f32<BF16>(kw[k], x);
        const bool ok = r0 + (k0 + k) * NRG < len;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d += qv[g][e] * x[e];
          d = group_sum<LPR>(d);
          s[g][k] = ok ? d : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      float mb = s[g][0];
#pragma unroll
      for (int k = 1; k < RB; ++k) mb = fmaxf(mb, s[g][k]);
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o, 64));
      const float mn = fmaxf(m[g], mb);
      if (mn != -INFINITY) {  // else no valid row yet: nothing to rescale or add
        const float c = __expf(m[g] - mn);  // 0 while m is -inf
        l[g] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= c;
        m[g] = mn;
      }
    }
    if constexpr (BF16) {  // two rows at a time: (row k, row k+1) pairs of each element against bf16 weights
#pragma unroll
      for (int k = 0; k < RB; k += 2) {
        const uint32_t a[4] = {vw[k].x, vw[k].y, vw[k].z, vw[k].w};
        const uint32_t c[4] = {vw[k + 1].x, vw[k + 1].y, vw[k + 1].z, vw[k + 1].w};
        uint32_t pk[EPL];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[2 * i] = __builtin_amdgcn_perm(c[i], a[i], 0x05040100u);      // low halves: element 2i
          pk[2 * i + 1] = __builtin_amdgcn_perm(c[i], a[i], 0x07060302u);  // high halves: element 2i + 1
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          const float p0 = s[g][k] == -INFINITY ? 0.f : __expf(s[g][k] - m[g]);
          const float p1 = s[g][k + 1] == -INFINITY ? 0.f : __expf(s[g][k + 1] - m[g]);
          l[g] += p0 + p1;
          const uint32_t pp = pack_bf16x2(p0, p1);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = dot2_bf16(pk[e], pp, acc[g][e]);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        float x[EPL];
        piece_f32<BF16>(vw[k], x);
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          const float pr = s[g][k] == -INFINITY ? 0.f : __expf(s[g][k] - m[g]);
          l[g] += pr;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] += pr * x[e];
        }
      }
    }
  }

  // every row group's sums go to LDS as they are (no cross-lane reduction); one pass then folds the
  // 4 waves x NRG row groups of each (head, element)
  if (pc == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) wl[wave][rg][g] = l[g];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) wm[wave][g] = m[g];
  }
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) wacc[wave][rg][g][pc * EPL + e] = acc[g][e];
  __syncthreads();
  for (int i = tid; i < G * D; i += THREADS) {
    const int g = i / D, e = i % D;
    float M = wm[0][g];
    for (int w = 1; w < THREADS / 64; ++w) M = fmaxf(M, wm[w][g]);
    float o = 0.f, L = 0.f;
    for (int w = 0; w < THREADS / 64; ++w) {
      const float f = wm[w][g] == -INFINITY ? 0.f : __expf(wm[w][g] - M);  // a wave with no valid row adds 0
      float ow = 0.f, lw = 0.f;
#pragma unroll
      for (int r = 0; r < NRG; ++r) {
        ow += wacc[w][r][g][e];
        lw += wl[w][r][g];
      }
      o += f * ow;
      L += f * lw;
    }
    float* dst = p.part + (((int64_t)b * p.H + (int64_t)kv * G + g) * p.Td + t) * (D + 2);
    dst[e] = o;
    if (e == 0) {
      dst[D] = M;
      dst[D + 1] = L;
    }
  }
}

// merge: block per (head, sequence, MCOLS columns). Thread (slice sl, column e) folds chunks sl, sl + SL,
// ... into a running (max, sum-exp, weighted sum) with the loads of MB chunks in flight at once; the SL
// slices are then combined the same way.
constexpr int MERGE_THREADS = 512;
constexpr int MCOLS = 32;
constexpr int MB = 16;
template <int D, bool BF16>
__global__ __launch_bounds__(MERGE_THREADS) void dense_merge_kernel(DenseProblem p) {
  constexpr int SL = MERGE_THREADS / MCOLS;
  __shared__ float sm[SL];
  __shared__ float sls[SL];
  __shared__ float so[SL][MCOLS];
  const int h = blockIdx.x, b = blockIdx.y, c0 = blockIdx.z * MCOLS;
  const int tid = threadIdx.x, e = c0 + tid % MCOLS, sl = tid / MCOLS;
  const int Td = p.Td;
  const float* src = p.part + ((int64_t)b * p.H + h) * Td * (D + 2);
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int t0 = sl; t0 < Td; t0 += SL * MB) {
    float mt[MB], lt[MB], vt[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int t = t0 + k * SL;
      const float* r = src + (int64_t)(t < Td ? t : t0) * (D + 2);  // chunks past Td re-read t0, weight 0
      mt[k] = r[D];
      lt[k] = r[D + 1];
      vt[k] = r[e];
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < MB; ++k)
      if (t0 + k * SL < Td) mb = fmaxf(mb, mt[k]);  // finite: chunk t0 holds at least one key
    const float c = __expf(M - mb);                  // 0 while M is -inf
    L *= c;
    O *= c;
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const float f = t0 + k * SL < Td ? __expf(mt[k] - mb) : 0.f;
      L += f * lt[k];
      O += f * vt[k];
    }
    M = mb;
  }
  so[sl][tid % MCOLS] = O;
  if (tid % MCOLS == 0) {
    sm[sl] = M;
    sls[sl] = L;
  }
  __syncthreads();
  if (tid < MCOLS) {
    float Mx = sm[0];
    for (int k = 1; k < SL; ++k) Mx = fmaxf(Mx, sm[k]);
    float r = 0.f, l = 0.f;
    for (int k = 0; k < SL; ++k) {
      const float f = sm[k] == -INFINITY ? 0.f : __expf(sm[k] - Mx);  // a slice with no chunk adds 0
      r += f * so[k][tid];
      l += f * sls[k];
    }
    r /= l;
    const int64_t oi = ((int64_t)b * p.H + h) * D + c0 + tid;
    if (BF16)
      ((uint16_t*)p.out)[oi] = f32_to_bf16_rne(r);
    else
      ((float*)p.out)[oi] = r;
  }
}

template <int D, bool BF16>
hipError_t launch_dense_dt(const DenseProblem& p, hipStream_t st) {
  dim3 grid(p.Hkv, p.Td, p.B);
  if (p.G <= 1)
    dense_partial_kernel<D, BF16, 1, dense_chunk(1)><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 2)
    dense_partial_kernel<D, BF16, 2, dense_chunk(2)><<<grid, THREADS, 0, st>>>(p);
  else if (p.G <= 4)
    dense_partial_kernel<D, BF16, 4, dense_chunk(4)><<<grid, THREADS, 0, st>>>(p);
  else
    dense_partial_kernel<D, BF16, 8, dense_chunk(8)><<<grid, THREADS, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dense_merge_kernel<D, BF16><<<dim3(p.H, p.B, D / MCOLS), MERGE_THREADS, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense(const DenseProblem& p, hipStream_t st) {
  if (p.d == 128) return p.bf16 ? launch_dense_dt<128, true>(p, st) : launch_dense_dt<128, false>(p, st);
  return p.bf16 ? launch_dense_dt<64, true>(p, st) : launch_dense_dt<64, false>(p, st);
}

}  // namespace santa
