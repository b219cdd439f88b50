// Streaming score pass for bf16 caches: one block of 16 waves per CU with copy, matrix-core and
// exponential roles (described above score_stream_kernel). Three forms share it:
//   KM_SCORE:  scores, chunk statistics and the in-chunk prefix rows ("stash") for the sampling kernel;
//   KM_FLASH:  S²ANTA-flash kernel 1 fused in (samples and gathers each tile right after its exponentials);
//   KM_DECODE: the whole decode step in one launch: after the score phase the blocks of a (KV head,
//              sequence) group exchange their chunk statistics, then every block samples and gathers its
//              own chunks and the group's output is summed (the tail of score_stream_kernel);
//   KM_DECODE_PROP, KM_DECODE_FLASH: the same for S²ANTA-prop and -flash (tile budgets and per-key
//              counts instead of points).
#pragma once

#include "common.h"
#include "launch.h"

namespace santa {
namespace sk {

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

// Streaming form for bf16 caches (one block per CU). The memory system copies K straight into LDS
// (global_load_lds: 16 bytes per lane, no register staging) in half-chunk buffers, two chunks in flight:
// the copy of a buffer's next half-chunk starts as soon as the matrix waves have finished reading it, so
// the HBM stream does not pause for the exponentials and stores. The compiler does not track these
// copies; the copy waves wait for them with explicit vmcnt waits.

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
// one wave-wide 4-byte copy global -> LDS (lane l's dword at `g` lands at lds + 4 l): brings the line
// of `g` into the caches without a register result
__device__ inline void touch_to_lds4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
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

constexpr int SQUART = 8;                // matrix waves: four per half of a chunk (32 keys each), two per SIMD
constexpr int SSOFT = 4;                 // exponential waves: one head each (two for G = 5..8)
constexpr int SCOPY = 4;                 // copy waves: one per half-chunk K buffer
constexpr int NBUF = 4;                  // half-chunk K buffers in LDS (two chunks in flight)
constexpr int HALF = CHUNK / 2;          // keys per buffer
constexpr int SPH = SQUART / 2;          // matrix waves per half
constexpr int STHREADS = 64 * (SQUART + SSOFT + SCOPY);  // 16 waves: four per SIMD

template <int D>
struct SGeo {
  static constexpr int ROWB = D * 2;         // bytes per bf16 K row
  static constexpr int PPR = ROWB / 16;      // 16-byte pieces per row (16 or 8)
  static constexpr int HTILE = HALF * ROWB;  // bytes per half-chunk buffer (32 or 16 KiB)
  static constexpr int CPH = HTILE / 1024;   // wave-wide 1 KiB copies per half chunk (32 or 16)
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

// Bounded poll of n flags in device memory (one wave; flags are read with coherent device-scope loads):
// calls done(true) once every flag equals `target`, done(false) after `limit` checks. Up to 64 flags: four
// rounds of loads, issued spaced in time and checked in order. (The compiler's wait at the head of the
// loop covers every round in flight, so from the second sweep on the four rounds are checked together;
// keeping them spaced by unrolling the first sweeps, here and in the decode's other polls, was measured
// no faster: the extra device-scope loads cost about what the earlier sight of the words gains.) The
// rounds still in flight when the flags are seen are retired after done() (a use of their registers, so
// the compiler's own wait lands there): code that joins this wave's path afterwards finds no load of it
// outstanding.
__device__ inline uint64_t ld_flag(const uint64_t* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class Done>
__device__ inline void poll_flags(const uint64_t* flags, int n, uint64_t target, int lane, int limit, Done&& done) {
  if (n <= 64) {
    const uint64_t* f = flags + (lane < n ? lane : n - 1);
    uint64_t v0 = ld_flag(f);
    __builtin_amdgcn_s_sleep(4);
    uint64_t v1 = ld_flag(f);
    __builtin_amdgcn_s_sleep(4);
    uint64_t v2 = ld_flag(f);
    __builtin_amdgcn_s_sleep(4);
    uint64_t v3 = ld_flag(f);
    bool seen = false;
    for (int spins = 0; spins < limit; spins += 4) {
      if ((seen = __ballot(v0 != target) == 0ull)) break;
      v0 = ld_flag(f);
      if ((seen = __ballot(v1 != target) == 0ull)) break;
      v1 = ld_flag(f);
      if ((seen = __ballot(v2 != target) == 0ull)) break;
      v2 = ld_flag(f);
      if ((seen = __ballot(v3 != target) == 0ull)) break;
      v3 = ld_flag(f);
    }
    done(seen);
    asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3));
    return;
  }
  for (int spins = 0;; ++spins) {
    bool mine = true;
    for (int i = lane; i < n; i += 64) mine = (ld_flag(flags + i) == target) && mine;
    if (__ballot(!mine) == 0ull) return done(true);
    if (spins >= limit) return done(false);
    __builtin_amdgcn_s_sleep(1);
  }
}

// One-launch decode: the words that blocks of a group exchange (chunk statistics, partial sums) hold
// VOID until this call writes them, or FAIL when their block gave up. Both are signalling NaNs with
// low payload bits set, which no computation here yields: arithmetic returns quiet NaNs, and NaNs
// carried over from bf16 inputs have all low payload bits clear. Words are compared as bit patterns.
constexpr uint64_t D_VOID = 0xFFF4C0DE00000001ull, D_FAIL = 0xFFF4C0DE00000002ull;
constexpr uint32_t F_VOID = 0xFFA00001u, F_FAIL = 0xFFA00002u;

__device__ inline uint64_t ld_word(const double* f) {
  return __hip_atomic_load((const uint64_t*)f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_word(double* f, uint64_t v) {
  __hip_atomic_store((uint64_t*)f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One-launch decode: the chunk CDF of one head (Appendix O, Algorithm 4) from the chunk statistics the
// blocks of its group publish: loads every word once, then reloads (bounded) the words still VOID; lane
// l owns chunks [l PER, (l + 1) PER). The
// edges C_0..C_T and the chunk scales exp(m_t - m*) go to LDS (cg, sg), (Z, last chunk with mass) to
// zl, and the lane's statistics m_t, l_t to mo, lo (without the CDF if CDF is false). Returns 0, or 1 if
// a block reported FAIL or the wait gave up.
template <int PER, bool CDF = true>
__device__ inline int cdf_poll_to_lds(const double* cm, const double* cs, int T, int lane, int limit,
                                      double* cg, double* sg, double2* zl, double* mo, double* lo) {
  uint64_t wm[PER], wl[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {  // lanes past T re-read the last chunk
    const int tt = min(lane * PER + j, T - 1);
    wm[j] = ld_word(cm + tt);
    wl[j] = ld_word(cs + tt);
  }
  for (int spins = 0;; ++spins) {
    bool vd = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) vd = vd || wm[j] == D_VOID || wl[j] == D_VOID;
    if (__ballot(vd) == 0ull) break;
    if (spins >= limit) return 1;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < PER; ++j) {  // only the words still VOID are read again
      const int tt = min(lane * PER + j, T - 1);
      if (wm[j] == D_VOID) wm[j] = ld_word(cm + tt);
      if (wl[j] == D_VOID) wl[j] = ld_word(cs + tt);
    }
  }
  bool fl = false;
  double m[PER], l[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    fl = fl || wm[j] == D_FAIL || wl[j] == D_FAIL;
    m[j] = __longlong_as_double((long long)wm[j]);
    l[j] = __longlong_as_double((long long)wl[j]);
  }
  if (__ballot(fl) != 0ull) return 1;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    mo[j] = m[j];
    lo[j] = l[j];
  }
  if constexpr (!CDF) return 0;
  ChunkCdf<PER> o;
  chunk_cdf_wave<PER>(m, l, T, lane, o);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int t = lane * PER + j;
    if (t < T) {
      cg[t] = o.c[j];
      sg[t] = o.f[j];
    }
  }
  if (lane == 0) cg[T] = o.top;  // the last chunk ends at the total
  *zl = make_double2(o.top, (double)o.last);
  return 0;
}

// LDS handshake counters. signal(): this wave's earlier LDS writes (and, for copy waves, the copies
// waited for) are complete, then one lane adds 1. wait_ge(): poll until the counter reaches `target`;
// false after `limit` polls (the caller then abandons the block and flags it).
__device__ inline void signal(int* ctr, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// A polling wave keeps its issue priority: a poll is a few instructions per sleep, and a waiting wave
// at the lowest priority is starved by the MFMA waves sharing its SIMD and notices its counter late.
__device__ inline bool wait_ge(int* ctr, int target, int limit) {
  int spins = 0;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (++spins > limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::: "memory");
  return true;
}

// Streaming score pass for bf16 caches and G <= 8, one block of 16 waves per CU (four per SIMD), three
// roles that meet only through LDS counters (no block-wide barrier after the start), so the K stream, the
// matrix cores and the exponentials overlap:
//   * waves 0..7: fp64 MFMA, two per SIMD: waves 0..3 score the first half of every chunk, waves 4..7 the
//     second (32 keys each: two 16-key groups) over the whole head dimension (element parity gives four
//     independent accumulation chains per head group), writing complete scores. Two matrix waves per SIMD
//     keep the fp64 matrix pipe busier than one (one wave alone issues an MFMA only every ~46 cycles).
//     For G = 5..8 (HG = 2) the wave scores both head groups: each K element is converted once for the
//     MFMAs of the eight heads, and the query operands are read from LDS per 4-piece step to stay within
//     the register budget of four waves per SIMD;
//   * waves 8..11: chunk max, exponentials, in-chunk prefix and the stores of head w - 8 (and w - 4 for
//     G = 5..8);
//   * waves 12..15: global -> LDS copies (global_load_lds) into four half-chunk K buffers: copy wave j
//     fills buffer j with half (j & 1) of the block's chunks (j >> 1), (j >> 1) + 2, ... (wave 15 first
//     copies the queries). Half-chunk buffers are released as soon as their half is scored, so the next
//     copy starts half a chunk earlier than with whole-chunk tiles. The block's second chunk is requested
//     only once its first has landed, so across the device the first chunks arrive before any second one.
// Counters (chunk k's half h lives in buffer 2 (k & 1) + h; its fill index there is k >> 1):
//   ld[j] +1 when buffer j's current half-chunk has landed;  use[j] +1 per MFMA wave when its reads of
//   buffer j are done;  pr +1 per MFMA wave per chunk whose scores are written;  pc +1 per exponential
//   wave per chunk whose scores it has read;  qr queries landed;  pb prologue barrier;  fin waves finished
//   (the last one publishes the block's handshake status).
// HG = head groups of four (G <= 4 * HG).
// FL: S²ANTA-flash kernel 1 ("Stochastic Sparse Attention for Memory-Bound Inference", Section 3.3 and
// Appendix P, Algorithm 7) fused in: right after a chunk's exponentials, the exponential wave of head g
// takes the tile's systematic counts with the uniform budget S_tile (c_n = floor(a0 + inv P_n) -
// floor(a0 + inv P_{n-1}), inv = S_tile / l_t, P the in-chunk prefix it has just formed, a0 from Philox
// counter (t, h, b, 4)), writes the index slots and the tile's sampled-key bits, and issues the loads of
// its sampled V rows; one chunk later (the loads have landed meanwhile) it adds count x row into the fp32
// tile partial and stores it. Only the merge kernel follows: two launches per decode step.
// end of a role's score phase: the block is done (KM_SCORE, KM_FLASH) or goes on to the sampling and
// gather phase of the one-launch decode
#define SK_PHASE1_DONE()        \
  do {                          \
    if constexpr (!DEC) {       \
      finish();                 \
      return;                   \
    } else {                    \
      goto decode_tail;         \
    }                           \
  } while (0)

// KM_DECODE(_PROP): the whole decode step in one launch; NREG > 0 keeps each exponential wave's prefix rows of
// the block's (at most NREG) chunks in registers instead of storing them (G <= 4). The sampling and
// gather phase after the score phase is described at the start of that phase (decode_tail) below.
template <int D, int HG, int KM, int NREG = 0>
__global__ __launch_bounds__(STHREADS, 1) void score_stream_kernel(Problem p) {
  constexpr bool FL = KM == KM_FLASH;
  constexpr bool DEC = KM == KM_DECODE || KM == KM_DECODE_PROP || KM == KM_DECODE_FLASH;
  constexpr bool DPROP = KM == KM_DECODE_PROP, DFLASH = KM == KM_DECODE_FLASH;
  static_assert(!FL || HG == 1, "the fused S²ANTA-flash form covers G <= 4");
  static_assert(NREG == 0 || (DEC && HG == 1), "register prefix rows: one-launch decode with G <= 4");
  constexpr int NRX = NREG > 0 ? NREG : 1;
  constexpr int NMF = SQUART;  // matrix-core waves
  constexpr int NTH = 64 * (NMF + SSOFT + SCOPY);
  using Sg = SGeo<D>;
  constexpr int EPL = 8, PPH = Sg::PPH, CPH = Sg::CPH;
  constexpr int KPW = HALF / SPH;     // keys per MFMA wave
  constexpr int NGR = KPW / 16;       // 16-key groups per MFMA wave
  constexpr int HM = 4 * HG;          // heads held
  constexpr int NPW = 2 * PPH;       // 4-piece steps of a row per MFMA wave
  static_assert(D * 2 * HM <= 1024 * HG, "the queries of a group fit HG 1 KiB copies");

  __shared__ __align__(16) unsigned char kt[NBUF][Sg::HTILE];
  __shared__ __align__(16) double part[HG][4][CHUNK];  // scores: [head group][head][key]
  __shared__ __align__(16) double qe[HM][D + 2];
  __shared__ double hnorm[HM];
  __shared__ __align__(16) unsigned char qs[1024 * HG];
  __shared__ int rl[FL ? 4 : 1][FL ? CHUNK : 1];  // fused S²ANTA-flash: sampled rows (key | count << 8) per head
  constexpr int NCTR = 16;
  __shared__ int ctr[NCTR];
  int* ld = &ctr[0];   // [NBUF]
  int* use = &ctr[4];  // [NBUF]
  int* pr = &ctr[8];
  int* pc = &ctr[9];
  int* qr = &ctr[10];
  int* pb = &ctr[11];
  int* fin = &ctr[12];
  int* bad = &ctr[13];
  int* ivd = &ctr[14];  // one-launch decode: copy waves whose VOID stores are complete
  int* stc = &ctr[15];  // one-launch decode: the started flags of the group have been polled
  __shared__ int dstat[3];      // one-launch decode: statistics failed, output poisoned, started flags seen
  __shared__ uint64_t depoch;   // one-launch decode: the group's epoch at the start of this call
  __shared__ uint32_t pfsink[DEC ? 64 : 1];  // one-launch decode: landing place of V-row prefetch copies
  // one-launch decode, more than 4 chunks per block: first candidate point and exclusive prefix of the
  // candidate counts of each chunk, per head
  __shared__ int rlo[DEC ? 8 : 1][DEC ? DECODE_MAX_CHUNKS : 1], rpre[DEC ? 8 : 1][DEC ? DECODE_MAX_CHUNKS + 1 : 1];
  __shared__ int wcnt[STHREADS / 64];
  // one-launch S²ANTA-flash: weight W_t / (Z S_tile) of each head's count in each of the block's tiles
  __shared__ float fw[KM == KM_DECODE_FLASH ? 8 : 1][KM == KM_DECODE_FLASH ? DECODE_MAX_CHUNKS : 1];
  double pv[NRX][4];            // one-launch decode, NREG > 0: this exponential wave's prefix rows

  // (chunk slot, KV head, sequence) of this block. The one-launch decode numbers the blocks XCD by XCD:
  // the dispatcher sends block l (in x, y, z order) to XCD l mod 8, so the blocks of a group share an
  // XCD when its blocks fit in one, and their exchanges through device memory take the shorter trip
  // (about 0.5 against 0.75 us per store-to-load hop, measured). Any placement gives the same results.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if constexpr (DEC) {
    const int nb = gridDim.x * gridDim.y * gridDim.z;
    if ((nb & 7) == 0) {
      const int l = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
      const int m = (l & 7) * (nb >> 3) + (l >> 3);
      bx = m % gridDim.x;
      by = (m / gridDim.x) % gridDim.y;
      bz = m / (gridDim.x * gridDim.y);
    }
  }
  const int kv = by, b = bz;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int h0 = kv * G;
  const int T = p.T;
  const int step = gridDim.x;
  const int t0 = bx;
  if (t0 >= T) return;
  const int n = (T - 1 - t0) / step + 1;  // this block's chunks: t0, t0 + step, ...
  int* err = p.sync_err + ((int64_t)b * gridDim.y + kv) * gridDim.x + t0;

  if (tid < NCTR) ctr[tid] = 0;
  if (tid < 3) dstat[tid] = 0;
  __syncthreads();  // the only block-wide barrier of the score phase

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
    // ---- copy waves: copy wave j fills buffer j with half (j & 1) of the block's chunks k = (j >> 1),
    // (j >> 1) + 2, ...; at most one half-chunk's copies in flight per wave, so vmcnt(0) means all
    // landed. Highest issue priority on their SIMD: they issue rarely and the whole block waits on them.
    __builtin_amdgcn_s_setprio(3);
    const int j = wave - NMF - SSOFT, hh = j & 1;
    if (j == SCOPY - 1) {
      const char* qsrc = (const char*)p.q + ((int64_t)b * p.H + h0) * D * 2;
#pragma unroll
      for (int c = 0; c < HG; ++c)  // bytes past the group's queries re-read its last piece (never used)
        copy_to_lds16(qsrc + min(c * 1024 + lane * 16, G * D * 2 - 16), lds_addr(qs) + c * 1024);
      wait_vm<0>();
      signal(qr, lane);
    }
    // One-launch decode: right after its first copies every copy wave sets its share of the words this
    // block will publish (chunk statistics, partial sums) to VOID; the wait for those copies completes
    // the stores too. Once all four waves have, the block announces that it has started. A block reads
    // another block's words only after it has seen that block's started flag, so it sees VOID or this
    // call's value, never a value left by an earlier call. Block 0 clears the group's status word the
    // same way.
    const int grp = b * p.Hkv + kv, me = grp * step + t0;
    if constexpr (DEC) {
      // the group's epoch (it changes only after every block of the group has published its partial
      // sums), read by the last copy wave, whose first copies wait for another wave's anyway, and put in
      // LDS at once: no load of it is left in flight where the roles join the sampling phase
      if (j == SCOPY - 1) {
        const uint64_t e = __hip_atomic_load(p.sync_epoch + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) depoch = e;
      }
    }
    bool voided = !DEC, announced = !DEC;
    auto set_void = [&]() {
      // statistics words of chunk k: set by the copy wave of its first half, so the wait that precedes
      // the chunk's scores (and so its genuine statistics) completes them
      if (hh == 0) {
        const int nk = n > (j >> 1) ? (n - (j >> 1) + 1) / 2 : 0;  // chunks k = (j >> 1) + 2 m < n
        for (int i = lane; i < nk * 2 * G; i += 64) {
          const int k = (j >> 1) + 2 * (i / (2 * G)), g = (i >> 1) % G;
          st_word(((i & 1) ? p.csum : p.cmax) + ((int64_t)b * p.H + h0 + g) * T + t0 + k * step, D_VOID);
        }
      }
      uint32_t* gpart = reinterpret_cast<uint32_t*>(p.partial) + (int64_t)me * G * D;
      for (int i = j * 64 + lane; i < G * D; i += SCOPY * 64)
        __hip_atomic_store(gpart + i, F_VOID, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j == 0 && t0 == 0 && lane == 0)
        __hip_atomic_store(p.status + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      voided = true;
    };
    auto announce = [&]() {  // this wave's VOID stores are complete
      if (lane == 0) {
        // the last copy wave wrote depoch before its own increment of ivd
        const int before = __hip_atomic_fetch_add(ivd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (before == SCOPY - 1)
          __hip_atomic_store(p.sync_start + me, ((depoch + 1) << 10) | (uint64_t)grp, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      announced = true;
    };
    for (int k = j >> 1, m = 0; k < n && ok; k += 2, ++m) {
      if (m > 0) ok = wait_ge(&use[j], SPH * m, p.spin_limit);  // the buffer's previous half is no longer read
      // the block's second chunk is requested once the same half of its first has landed, so across the
      // device every block's first chunk arrives before any second one
      if (m == 0 && j >= 2) ok = wait_ge(&ld[j - 2], 1, p.spin_limit);
      if (!ok) break;
      const int t = t0 + k * step;
      const int64_t c0 = (int64_t)t * CHUNK, h0k = c0 + hh * HALF;
      const uint32_t base = lds_addr(&kt[j][0]);
#pragma unroll 4
      for (int i = 0; i < CPH; ++i) {
        const int row = i * Sg::RPS + lane / Sg::PPR;  // row of the half
        const int pc = (lane % Sg::PPR) ^ (row % Sg::PPR);
        const int64_t key = h0k + row < p.nk ? h0k + row : c0;  // keys past the end re-read the chunk's first
        copy_to_lds16(kbase + key * seq_bytes + pc * 16, base + i * 1024);
      }
      if (!voided) set_void();
      wait_vm<0>();
      signal(&ld[j], lane);
      if (!announced) announce();
    }
    if (!voided) set_void();
    wait_vm<0>();  // no copy may land after the block ends
    if constexpr (DEC) {
      if (!announced) announce();
      if (j == SCOPY - 1) {  // the started flags of the group, seen before the sampling phase needs them
        const uint64_t target = ((depoch + 1) << 10) | (uint64_t)grp;
        auto done = [&](bool seen) {
          if (lane == 0) dstat[2] = seen ? 1 : 2;
          signal(stc, lane);
        };
        if (wait_ge(ivd, SCOPY, p.spin_limit))
          poll_flags(p.sync_start + (int64_t)grp * step, step, target, lane, p.spin_limit, done);
        else
          done(false);
      }
    }
    SK_PHASE1_DONE();
  }

  {
  // ---- prologue of the MFMA and exponential waves (counter barrier pb)
  int np = 0;
  auto pbar = [&]() {
    signal(pb, lane);
    ++np;
    ok = ok && wait_ge(pb, (NMF + SSOFT) * np, p.spin_limit);
  };
  ok = wait_ge(qr, 1, p.spin_limit);
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
      ok = wait_ge(pr, NMF * (k + 1), p.spin_limit);  // chunk k's partials are complete
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
        // One-launch decode: the rows stay in this wave's registers (NREG > 0), or are stored with plain
        // stores so that this CU reads them back from its L2 after the group barrier.
        if constexpr (DEC && NREG > 0) {
#pragma unroll
          for (int kk = 0; kk < NREG; ++kk)
            if (kk == k)
#pragma unroll
              for (int i = 0; i < 4; ++i) pv[kk][i] = excl + pre[i];
        } else if constexpr (!FL) {
          typedef double f64x2_t __attribute__((ext_vector_type(2)));
          f64x2_t* dst = (f64x2_t*)(p.stash + bh * p.stash_stride + n0 + 4 * lane);
          const f64x2_t v0 = {excl + pre[0], excl + pre[1]};
          const f64x2_t v1 = {excl + pre[2], excl + pre[3]};
          if constexpr (DEC) {
            dst[0] = v0;
            dst[1] = v1;
          } else {
            __builtin_nontemporal_store(v0, dst);
            __builtin_nontemporal_store(v1, dst + 1);
          }
        }
        if (lane == 0) {
          if constexpr (DEC) {  // read by every block of the group after the barrier: coherent device-scope stores
            __hip_atomic_store(p.cmax + bh * T + t, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.csum + bh * T + t, readlane_f64(incl, 63), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          } else {
            p.cmax[bh * T + t] = m;
            p.csum[bh * T + t] = readlane_f64(incl, 63);
          }
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
            int c = hi > lo ? min(hi - lo, St) : 0;
            if (4 * lane + i >= len) c = 0;
            if (p.want_idx)
              for (int j = 0; j < c; ++j)
                if (lo + j >= 0 && lo + j < St) idst[lo + j] = (int32_t)(n0 + 4 * lane + i);
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
    SK_PHASE1_DONE();
  }

  // ---- MFMA waves: 16-key groups x element parity = independent accumulation chains
  const int slot = lane >> 4;
  const int mh = wave / SPH, quart = wave % SPH;  // this wave's half of each chunk and key slice in it
  if (mh == 1) __builtin_amdgcn_s_setprio(1);  // second halves land later and gate the next copies
  if constexpr (HG == 2) {
    for (int k = 0; k < n && ok; ++k) {
      const int jb = 2 * (k & 1) + mh;
      ok = wait_ge(&ld[jb], (k >> 1) + 1, p.spin_limit);  // chunk k's half has landed
      if (!ok) break;
      const unsigned char* ks = &kt[jb][0];
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
      signal(&use[jb], lane);  // this wave's reads of the buffer are complete
      if (k >= 1) ok = wait_ge(pc, SSOFT * k, p.spin_limit);  // chunk k - 1's partials were read
      if (!ok) break;
#pragma unroll
      for (int hx = 0; hx < HG; ++hx)
#pragma unroll
        for (int gi = 0; gi < NGR; ++gi) {
          const int key = mh * HALF + quart * KPW + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
          part[hx][lane & 3][key] = acc[hx][gi][0] + acc[hx][gi][1];
        }
      signal(pr, lane);
    }
    SK_PHASE1_DONE();
  }
  // key slice over the whole head dimension (HG = 1)
  const int qrow = lane & 3;
  double qb[NPW][EPL];
#pragma unroll
  for (int pp = 0; pp < NPW; ++pp)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qb[pp][e] = qe[qrow][EPL * (4 * pp + slot) + e];
  for (int k = 0; k < n && ok; ++k) {
    const int jb = 2 * (k & 1) + mh;
    ok = wait_ge(&ld[jb], (k >> 1) + 1, p.spin_limit);  // chunk k's half has landed
    if (!ok) break;
    const unsigned char* ks = &kt[jb][0];
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
    signal(&use[jb], lane);  // this wave's reads of the buffer are complete
    if (k >= 1) ok = wait_ge(pc, SSOFT * k, p.spin_limit);  // chunk k - 1's partials were read
    if (!ok) break;
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) {
      const int key = mh * HALF + quart * KPW + gi * 16 + 4 * ((lane >> 2) & 3) + (lane >> 4);
      part[0][lane & 3][key] = acc[gi][0] + acc[gi][1];
    }
    signal(pr, lane);
  }
  SK_PHASE1_DONE();
  }

decode_tail: __attribute__((unused));
  if constexpr (DEC) {
    // ==== one-launch decode: sampling and gather after the score phase ====
    // ("Stochastic Sparse Attention for Memory-Bound Inference", Section 3.1: the global barrier between
    // the split-K statistics and the sampling; Appendix O, Algorithms 4 and 5.) The blocks of a (KV head,
    // sequence) group share nothing but device memory: each publishes its chunk statistics, builds the
    // chunk CDF of each head from every block's statistics, resolves the points that fall in its own
    // chunks from its own prefix rows, gathers each sampled V row once for the group and publishes its
    // per-head partial sums; each block then adds the group's partials of a slice of the outputs in
    // block order (fp64) and scales by 1/S.
    // Cross-block data travel only as device-scope relaxed atomic stores and loads, which this chip keeps
    // coherent across its L2s without a cache write-back. The published words are VOID until written
    // (see the start of the exponential waves), so a reader waits for the data themselves instead of for
    // a flag stored after them. Started flags carry ((epoch + 1) << 10 | group): the epoch of a group is
    // read by every block at its start and advanced once every block of the group has published its
    // partial sums, so flags left by earlier calls never match and the workspace needs no initial contents.
    __builtin_amdgcn_s_setprio(0);
    if (!ok && lane == 0) __hip_atomic_fetch_or(bad, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // The matrix waves are done (their last LDS reads are behind them): they end here, and the sampling
    // phase runs on the exponential and copy waves. A wave that has ended is not waited for at a barrier.
    if (wave < NMF) return;
    constexpr int NW = SSOFT + SCOPY;  // waves of the sampling phase
    constexpr int TT = 64 * NW;        // its threads
    const int tw = wave - NMF, ttid = tid - 64 * NMF;
    // prefix rows (NREG = 0) and debug probabilities stored above are read back below, partly by other
    // waves: this wave's stores must be complete first
    if (NREG == 0 || p.prob != nullptr) wait_vm<0>();
    __syncthreads();
    constexpr int GM = 4 * HG;      // head slots of the counters
    constexpr int NCW = GM / 2;     // 32-bit words of 16-bit per-head counts per key
    const int P = step, r = t0;
    const int grp = b * p.Hkv + kv;
    const int me = grp * P + r;
    const bool failed = *bad != 0;  // block-uniform: a wait of the score phase gave up
    // the K tiles are free now (layout: decode_lds_plan for the group's largest chunk count, computed on
    // the host)
    struct {
      int nb;
    } LP = {p.lds_nb};
    unsigned char* lds = &kt[0][0];
    uint32_t* cnt = reinterpret_cast<uint32_t*>(lds + p.lds_cnt);    // [n][CHUNK][NCW]
    int32_t* list = reinterpret_cast<int32_t*>(lds + p.lds_list);    // sampled keys, slot k * CHUNK + j
    uint32_t* bits = reinterpret_cast<uint32_t*>(lds + p.lds_bits);  // [n * CHUNK / 32] sampled-key bitmap
    double* cdfl = reinterpret_cast<double*>(lds + p.lds_cdf);       // [G][T + 1] chunk CDF C_t of each head
    double* scl = reinterpret_cast<double*>(lds + p.lds_scl);        // [G][T] chunk scales exp(m_t - m*)
    double* rows = reinterpret_cast<double*>(lds + p.lds_rows);      // [G][nb][CHUNK] prefix rows (NREG > 0),
                                                                     // entry e of slot k at RowSwz{k}(e)
    const int nbits = (n * CHUNK + 31) / 32;
    for (int i = ttid; i < n * CHUNK * NCW; i += TT) cnt[i] = 0u;
    for (int i = ttid; i < nbits; i += TT) bits[i] = 0u;
    // the head of this wave: the exponential waves take heads 0..3 (whose prefix rows they hold), the copy
    // waves heads 4..7
    const int hw = tw < SSOFT ? tw : (HG == 2 ? tw - SSOFT + 4 : -1);
    const bool headwave = hw >= 0 && hw < G;
    const int64_t bhw = (int64_t)b * p.H + h0 + (headwave ? hw : 0);
    // the prefix rows of this head's chunks (at most 4), kept in the exponential wave's registers by the
    // score phase, into LDS (with more chunks they stay in device memory, in this CU's L2)
    auto put_rows = [&]() {
      if constexpr (NREG > 0) {
        double* rowg = rows + (size_t)(headwave ? hw : 0) * LP.nb * CHUNK;
#pragma unroll
        for (int kk = 0; kk < NREG; ++kk)
          if (kk < n)
#pragma unroll
            for (int i = 0; i < 4; ++i) rowg[kk * CHUNK + RowSwz{kk}(4 * lane + i)] = pv[kk][i];
      }
    };

    // a block whose score phase gave up publishes FAIL for its chunks, so no reader waits for them
    if (failed && headwave && lane < 2 * n)
      st_word(((lane & 1) ? p.csum : p.cmax) + bhw * T + t0 + (lane >> 1) * P, D_FAIL);
    const double u_sys =
        headwave && p.mode == 2 ? uniform53(p.seed, 0u, (uint32_t)(h0 + hw), (uint32_t)b, TAG_SYS) : 0.0;
    if (headwave) put_rows();
    __syncthreads();  // the counters and the bitmap are clear

    // -- each head's chunk CDF from the group's statistics, then the points of the head that fall in this
    // block's chunks (one wave per head)
    int hst = 1;  // wave-uniform: 0 once this head wave's chunk CDF is in LDS
    const int64_t vstride = 2 * p.seq_stride;
    const char* vbase = (const char*)p.V + 2 * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
    double2 zl = make_double2(0.0, 0.0);
    // Per-tile systematic counts (KM_DECODE_PROP / _FLASH): tile t of head g with budget st > 0 gives key n of the
    // block's chunk k the count c_n = floor(a0 + P_n st / l_t) - floor(a0 + P_{n-1} st / l_t) (lane l: keys
    // 4 l .. 4 l + 3, P the in-chunk prefix), index slots [off + floor(..)) of the head's list, and its
    // count and key bit for the gather.
    auto count_tile = [&](int k, int t, int st, int off, double inv, double a0) {
      const int g = hw, len = chunk_len(t);
      const double* rw = NREG > 0 ? rows + ((size_t)g * LP.nb + k) * CHUNK
                                  : p.stash + bhw * p.stash_stride + (int64_t)t * CHUNK;
      auto at = [&](int e) { return NREG > 0 ? RowSwz{k}(e) : e; };  // (the LDS rows' layout)
      int32_t* dst = p.idx + bhw * p.L + off;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 4 * lane + i;
        if (x >= len) continue;
        const double ylo = a0 + inv * (x > 0 ? rw[at(x - 1)] : 0.0);
        const double yhi = a0 + inv * rw[at(x)];
        const int lo_ = (int)floor(ylo), hi_ = (int)floor(yhi);
        const int c = hi_ > lo_ ? min(hi_ - lo_, st) : 0;
        if (c == 0) continue;
        if (p.want_idx)
          for (int q = 0; q < c; ++q)  // slots outside the tile's budget are never written
            if (lo_ + q >= 0 && lo_ + q < st) dst[lo_ + q] = (int32_t)((int64_t)t * CHUNK + x);
        const char* vrow = vbase + ((int64_t)t * CHUNK + x) * vstride;  // into the caches for the gather
        touch_to_lds4(vrow, lds_addr(pfsink));
        if constexpr (D * 2 > 128) touch_to_lds4(vrow + 128, lds_addr(pfsink));
        const int slot = k * CHUNK + x;
        atomicAdd(&cnt[slot * NCW + (g >> 1)], (g & 1) ? ((uint32_t)c << 16) : (uint32_t)c);
        atomicOr(&bits[slot >> 5], 1u << (slot & 31));
      }
    };
    // S²ANTA-prop ("Stochastic Sparse Attention for Memory-Bound Inference", Section 3.2; Appendix O,
    // Algorithms 4 and 5): the head's tile budgets S_t from every chunk's statistics (largest remainder,
    // the multi-launch path's own code), a0 from Philox counter (t, h, b, 3), the tile's first slot the
    // budgets' exclusive prefix. The outputs are (1/S) sum c_n v_n.
    auto prop_counts = [&](auto per, const double* mo, const double* lo) {
      constexpr int PER = decltype(per)::value;
      TileBudgets<PER> tb;
      tile_budgets_wave<PER>(mo, lo, T, p.S, lane, reinterpret_cast<int*>(lds + p.lds_hist) + hw * 256, tb);
      const int g = hw, h = h0 + hw;
      for (int k = 0; k < n; ++k) {
        const int t = t0 + k * P;
        const int ol = t / PER, oj = t % PER;
        if (__builtin_expect(p.prob != nullptr, 0)) {  // for the debug probabilities below
          const double et = readlane_f64(pick<PER>(tb.e, oj), ol);  // (every lane forms its pick first)
          if (lane == 0) scl[(size_t)g * T + t] = et;
        }
        const int st = (int)readlane_f64(pick<PER>(tb.st, oj), ol);
        if (st == 0) continue;  // wave-uniform
        const int off = (int)readlane_f64(pick<PER>(tb.off, oj), ol);
        const double inv = (double)st / readlane_f64(pick<PER>(lo, oj), ol);
        count_tile(k, t, st, off, inv, uniform53(p.seed, (uint32_t)t, (uint32_t)h, (uint32_t)b, TAG_PROP));
      }
      zl = make_double2(tb.Z, 0.0);  // (read by the debug probabilities only)
    };
    // S²ANTA-flash (Section 3.3; Appendix P, Algorithms 6-8): every tile has the budget S_tile, slots
    // [t S_tile, (t + 1) S_tile), a0 from Philox counter (t, h, b, 4); the gather weights the tile's counts
    // by W_t / (Z S_tile), W_t = exp(m_t - m*) l_t from the chunk CDF's scales, and the outputs are the sums.
    auto flash_counts = [&](auto per, const double* lo) {
      constexpr int PER = decltype(per)::value;
      const int g = hw, h = h0 + hw;
      const int st = p.S_tile;
      const double* sg = scl + (size_t)g * T;
      for (int k = 0; k < n; ++k) {
        const int t = t0 + k * P;
        const double lt = readlane_f64(pick<PER>(lo, t % PER), t / PER);
        if (lane == 0) fw[g][k] = (float)((sg[t] * lt) / (zl.x * (double)st));
        count_tile(k, t, st, t * st, (double)st / lt,
                   uniform53(p.seed, (uint32_t)t, (uint32_t)h, (uint32_t)b, TAG_FLASH));
      }
    };
    if (!failed && headwave) {
      double* cg = cdfl + (size_t)hw * (T + 1);
      double* sg = scl + (size_t)hw * T;
      // every block's started flag has been seen (exponential wave 0 of this block)
      if (wait_ge(stc, 1, p.spin_limit) && dstat[2] == 1) {
        // lane l owns chunks [l PER, (l + 1) PER) with PER the power of two the multi-launch path uses
        // for this T (the same edges, bit for bit)
        const double* cmg = p.cmax + bhw * T;
        const double* csg = p.csum + bhw * T;
        auto poll = [&](auto per) {
          constexpr int PER = decltype(per)::value;
          double mo[PER], lo[PER];
          int r;
          if constexpr (DFLASH) {
            r = cdf_poll_to_lds<PER>(cmg, csg, T, lane, p.spin_limit, cg, sg, &zl, mo, lo);
            if (r == 0) flash_counts(per, lo);
          } else if constexpr (DPROP) {  // S²ANTA-prop: budgets, no chunk CDF
            r = cdf_poll_to_lds<PER, false>(cmg, csg, T, lane, p.spin_limit, cg, sg, &zl, mo, lo);
            if (r == 0) prop_counts(per, mo, lo);
          } else {
            r = cdf_poll_to_lds<PER>(cmg, csg, T, lane, p.spin_limit, cg, sg, &zl, mo, lo);
          }
          return r;
        };
        if (T <= 64) hst = poll(IntC<1>());
        else if (T <= 128) hst = poll(IntC<2>());
        else if (T <= 256) hst = poll(IntC<4>());
        else hst = poll(IntC<8>());
      }
      if (hst != 0 && lane == 0) __hip_atomic_fetch_or(&dstat[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (hst == 0) {
      const int g = hw, h = h0 + hw;
      double* cg = cdfl + (size_t)g * (T + 1);
      double* sg = scl + (size_t)g * T;
      const double Z = zl.x;
      const int lastc = (int)zl.y;
      // (the products with 1/Z may round differently from the quotients; the +-1 margin of the candidate
      // range covers that, and each candidate is then tested exactly)
      const double invZ = 1.0 / Z;
      if (__builtin_expect(p.prob != nullptr, 0)) {  // debug: probabilities from the score phase's exponentials
        for (int kk = 0; kk < n; ++kk) {
          const int t = t0 + kk * P, len = chunk_len(t);
          const double f = sg[t];
          double* prb = p.prob + bhw * p.nk + (int64_t)t * CHUNK;
          for (int x = lane; x < len; x += 64) prb[x] = prb[x] * f / Z;
        }
      }
      // the candidate points of the block's chunks, lane kk for chunk t0 + kk P: every point for i.i.d.
      // sampling (its chunk found from the CDF); for stratified / systematic sampling point m lies in
      // [m/S, (m+1)/S), so chunk t can only hold m in [floor(S C_t / Z) - 1, floor(S C_{t+1} / Z) + 1]
      int lo = 0, np = 0;
      if (lane < n && p.mode != 0 && !DPROP && !DFLASH) {  // (S²ANTA-prop and -flash have no points)
        const int t = t0 + lane * P;
        const double c0 = cg[t], c1 = cg[t + 1];
        if (c1 > c0 || t == lastc) {
          const double a = floor((double)p.S * (c0 * invZ)) - 1.0, e = floor((double)p.S * (c1 * invZ)) + 1.0;
          const int ilo = (int)fmax(0.0, a);
          const int ihi = t == lastc ? p.S - 1 : (int)fmin((double)(p.S - 1), e);
          lo = ilo;
          np = ihi >= ilo ? ihi - ilo + 1 : 0;
        }
      }
      int clo[4], cpre[5];  // up to 4 chunks: in registers
      cpre[0] = 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        clo[kk] = __builtin_amdgcn_readlane(lo, kk);
        cpre[kk + 1] = cpre[kk] + __builtin_amdgcn_readlane(np, kk);
      }
      int total = p.mode == 0 ? p.S : cpre[4];
      if (n > 4) {  // more chunks: first points and exclusive prefix of the counts in LDS (int DPP scan)
        int incl = np;
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, false);  // row_shr:1
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, false);  // row_shr:2
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, false);  // row_shr:4
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, false);  // row_shr:8
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xa, 0xf, false);  // row_bcast:15
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xc, 0xf, false);  // row_bcast:31
        if (lane < n) {
          rlo[g][lane] = lo;
          rpre[g][lane + 1] = incl;
        }
        if (lane == 0) rpre[g][0] = 0;
        if (p.mode != 0) total = __builtin_amdgcn_readlane(incl, n - 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      for (int c = lane; c < total; c += 64) {
        int k = 0, m = c;
        if (p.mode != 0) {
          if (n <= 4) {
#pragma unroll
            for (int x = 1; x < 4; ++x)
              if (c >= cpre[x]) k = x;
            m = clo[k] + (c - cpre[k]);
          } else {  // the last chunk whose first candidate is at or before c
            int kl = 0, kh = n - 1;
            while (kl < kh) {
              const int mid = (kl + kh + 1) >> 1;
              if (rpre[g][mid] <= c) kl = mid; else kh = mid - 1;
            }
            k = kl;
            m = rlo[g][k] + (c - rpre[g][k]);
          }
        }
        const double y = point_of(p.seed, p.mode, p.S, m, h, b, u_sys) * Z;
        if (p.mode == 0) {  // the chunk holding y, if it is one of this block's
          int tt;
          if (y < Z) {  // the last edge at or below y (edges are nondecreasing)
            int el = 0, eh = T - 1;
            while (el < eh) {
              const int mid = (el + eh + 1) >> 1;
              if (cg[mid] <= y) el = mid; else eh = mid - 1;
            }
            tt = el;
          } else {
            tt = lastc;
          }
          if (tt < t0 || (tt - t0) % P != 0) continue;
          k = (tt - t0) / P;
        }
        const int t = t0 + k * P, len = chunk_len(t);
        const double c0 = cg[t], c1 = cg[t + 1];
        const bool mine = y < Z ? (c0 <= y && y < c1) : (t == lastc);
        if (!mine) continue;
        // the block's prefix rows: in LDS (NREG > 0), else in its own stores in device memory (its L2)
        const double* rw = NREG > 0 ? rows + ((size_t)g * LP.nb + k) * CHUNK
                                    : p.stash + bhw * p.stash_stride + (int64_t)t * CHUNK;
        int j;
        if constexpr (NREG > 0) {  // (the LDS rows' layout)
          j = y < Z ? search_chunk16(rw, sg[t], y - c0, RowSwz{k}) : -1;
          if (__builtin_expect(j < 0, 0)) j = last_positive(rw, len, RowSwz{k});  // at or beyond the total
        } else {
          j = y < Z ? search_chunk16(rw, sg[t], y - c0) : -1;
          if (__builtin_expect(j < 0, 0)) j = last_positive(rw, len);  // at or beyond the total through rounding
        }
        j = min(j, len - 1);
        p.idx[bhw * p.S + m] = (int32_t)((int64_t)t * CHUNK + j);
        // the key's V row, brought into the caches now for the gather below: copies into a sink in LDS
        // that nothing reads, so nothing waits for them (the waves wait for their copies before ending)
        const char* vrow = vbase + ((int64_t)t * CHUNK + j) * vstride;
        touch_to_lds4(vrow, lds_addr(pfsink));
        if constexpr (D * 2 > 128) touch_to_lds4(vrow + 128, lds_addr(pfsink));
        const int slot = k * CHUNK + j;
        atomicAdd(&cnt[slot * NCW + (g >> 1)], (g & 1) ? 0x10000u : 1u);
        atomicOr(&bits[slot >> 5], 1u << (slot & 31));
      }
    }
    __syncthreads();
    const bool good = !failed && dstat[0] == 0;  // block-uniform

    // -- compaction (one wave): the block's sampled keys in slot order, distinct keys per chunk
    if (tw == 0) {
      int cw = 0;
      uint32_t wv[4];  // bitmap words 4 lane .. 4 lane + 3 (at most 32 chunks of 8 words)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int wi = 4 * lane + x;
        wv[x] = wi < nbits ? bits[wi] : 0u;
        cw += __popc(wv[x]);
      }
      int incl = cw;  // inclusive prefix of the counts over the lanes (DPP row shifts and broadcasts)
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, false);
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, false);
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, false);
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, false);
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xa, 0xf, false);
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xc, 0xf, false);
      int pos = incl - cw;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        uint32_t w = wv[x];
        while (w) {
          list[pos++] = (4 * lane + x) * 32 + __builtin_ctz(w);
          w &= w - 1u;
        }
      }
      // chunk k owns words 8k .. 8k + 7, i.e. lanes 2k and 2k + 1: its distinct keys are the scan's
      // difference between lane 2k + 1 and lane 2k - 1
      const int before2 = __shfl_up(incl, 2, 64);
      if ((lane & 1) == 1 && lane / 2 < n)
        p.unique[(int64_t)grp * T + t0 + (lane / 2) * P] = incl - (lane >= 2 ? before2 : 0);
      if (lane == 63) wcnt[0] = incl;
    }
    __syncthreads();
    const int nu = good ? wcnt[0] : 0;

    // -- gather: each sampled row of the block's chunks read once, count x row into fp32 per head
    constexpr int EPG = 4;              // elements per lane (8 bytes of bf16)
    constexpr int LPR = D / EPG;        // lanes per V row
    constexpr int NRG = TT / LPR;       // rows per pass
    const int rg = ttid / LPR, pcl = ttid % LPR;
    float acc[GM][EPG];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < EPG; ++e) acc[g][e] = 0.0f;
    {
      typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
      const int64_t rstride = 2 * p.seq_stride;
      const char* vgrp = (const char*)p.V + 2 * ((int64_t)b * p.batch_stride + (int64_t)kv * D);
      for (int u0 = rg; u0 < nu; u0 += 2 * NRG) {
        int64_t key[2];
        uint32_t cw[2][NCW];
        int kc[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {  // entries past the list re-read its last row, added with count 0
          const int u = u0 + k2 * NRG;
          const int s = list[min(u, nu - 1)];
          kc[k2] = s / CHUNK;
          key[k2] = (int64_t)(t0 + (s / CHUNK) * P) * CHUNK + s % CHUNK;
#pragma unroll
          for (int w = 0; w < NCW; ++w) cw[k2][w] = u < nu ? cnt[s * NCW + w] : 0u;
        }
        u32x2_t w2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          w2[k2] = __builtin_nontemporal_load((const u32x2_t*)(vgrp + key[k2] * rstride) + pcl);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const float v[4] = {bf16_lo(w2[k2].x), bf16_hi(w2[k2].x), bf16_lo(w2[k2].y), bf16_hi(w2[k2].y)};
#pragma unroll
          for (int g = 0; g < GM; ++g) {
            const uint32_t c32 = cw[k2][g >> 1];
            float c = (float)((g & 1) ? (c32 >> 16) : (c32 & 0xFFFFu));
            if constexpr (DFLASH) c *= fw[g < G ? g : 0][kc[k2]];  // S²ANTA-flash: times the tile weight
#pragma unroll
            for (int e = 0; e < EPG; ++e) acc[g][e] += c * v[e];
          }
        }
      }
    }
    // row groups: down to two per wave by lane permutes (d = 64 only), then every row group in order
    // through LDS
    constexpr int KEEP = 2;              // row groups per wave kept for the LDS sum
    constexpr int NRGS = NW * KEEP;      // row-group sums added per output element
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < EPG; ++e) {
        float x = acc[g][e];
#pragma unroll
        for (int o2 = LPR * KEEP; o2 < 64; o2 <<= 1) x += __shfl_xor(x, o2, 64);
        acc[g][e] = x;
      }
    __syncthreads();  // every wave is done with the counters and the list
    float* wsum = reinterpret_cast<float*>(lds);  // [NW * KEEP][GM][D]
    if (lane < LPR * KEEP) {
      const int rgs = tw * KEEP + lane / LPR;
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < EPG; ++e) wsum[((size_t)rgs * GM + g) * D + pcl * EPG + e] = acc[g][e];
    }
    __syncthreads();
    const int GD = G * D;
    uint32_t* gpart = reinterpret_cast<uint32_t*>(p.partial) + (int64_t)me * GD;
    for (int i = ttid; i < GD; i += TT) {
      const int g = i / D, e = i % D;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NRGS; ++w) sum += wsum[((size_t)w * GM + g) * D + e];
      __hip_atomic_store(gpart + i, good ? __float_as_uint(sum) : F_FAIL, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // wsum has been read: its LDS is reused below

    // -- outputs: block r adds the group's P partials of outputs [r per, (r + 1) per) (fp64, in a fixed
    // order), times 1/S, waiting (bounded) for each partial word while it is VOID. A FAIL word, or a wait
    // that gave up, makes the block's outputs NaN and sets the group's status word: by block 0, which
    // cleared it, or by a block that has seen block 0's started flag, stored after that clear.
    const int per = (GD + P - 1) / P;
    const int o0 = r * per, no = max(0, min(GD - o0, per));
    float* fin = reinterpret_cast<float*>(lds);  // [P][no]
    const uint32_t* gparts = reinterpret_cast<const uint32_t*>(p.partial) + (int64_t)grp * P * GD + o0;
    bool fbad = false;
    for (int j = ttid; j < no * P; j += TT) {
      const int i = j / no, e = j - i * no;
      const uint32_t* src = gparts + (int64_t)i * GD + e;
      uint32_t v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int spins = 0; v == F_VOID && spins < p.spin_limit; ++spins) {
        __builtin_amdgcn_s_sleep(2);
        v = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      fbad = fbad || v == F_VOID || v == F_FAIL;
      fin[j] = __uint_as_float(v);
    }
    if (fbad) __hip_atomic_fetch_or(&dstat[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    const bool poisoned = dstat[1] != 0;  // block-uniform
    for (int e0 = ttid >> 4; e0 < no; e0 += TT / 16) {  // 16 threads per output, a fixed tree
      const int q = ttid & 15;
      double sum = 0.0;
      for (int i = q; i < P; i += 16) sum += (double)fin[i * no + e0];
      sum += dpp_f64<0xB1, 0xf>(0.0, sum);   // quad_perm [1,0,3,2]
      sum += dpp_f64<0x4E, 0xf>(0.0, sum);   // quad_perm [2,3,0,1]
      sum += dpp_f64<0x141, 0xf>(0.0, sum);  // row_half_mirror
      sum += dpp_f64<0x140, 0xf>(0.0, sum);  // row_mirror
      if (q == 0) {
        const int o2 = o0 + e0, g = o2 / D, e = o2 % D;
        const int64_t dst = ((int64_t)b * p.H + h0 + g) * D + e;
        const double o = DFLASH ? sum : sum / (double)p.S;  // (S²ANTA-flash: weighted already)
        ((uint16_t*)p.out)[dst] = poisoned ? (uint16_t)0x7FC0u : f64_to_bf16_rne(o);
      }
    }
    if (ttid == 0) {
      if (poisoned && (r == 0 || dstat[2] == 1))
        __hip_atomic_fetch_or(p.status + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // block 0 has seen every block's partial words (its slice reads all P blocks), so every block of
      // the group has read the epoch: it may advance
      if (r == 0) __hip_atomic_store(p.sync_epoch + grp, depoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vm<0>();  // no V-row copy into the LDS sink may land after the block ends
  }
}

#undef SK_PHASE1_DONE

}  // namespace sk
}  // namespace santa
