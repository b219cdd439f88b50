/*
 * santa.h — C ABI of the MI355X (gfx950) SANTA / S²ANTA decode-attention library (libsanta.so).
 *
 * One decode step of stochastic sparse attention, as defined in "Stochastic Sparse Attention for
 * Memory-Bound Inference" (Lee et al., arXiv:2605.01910):
 *   1. scores s = q K^T / sqrt(dk) over the whole KV cache (Section 2, Eq. 1), exact, or with the
 *      Bernoulli ternary query of Section 5 (Eq. 5) and Appendix C (Eqs. 8-9);
 *   2. the softmax over the nk keys and its CDF, built from per-chunk max / sum-exp statistics
 *      (Section 3.1, split-KV; Appendix O, Algorithms 3-4);
 *   3. S indices drawn from the post-softmax categorical by inverse CDF: i.i.d. (SANTA, Section 2,
 *      Eq. 4), stratified or systematic (S²ANTA, Section 2.1), with the half-open convention
 *      1{F(j-1) <= t < F(j)} of Appendix A.4;
 *   4. a gather-and-add of the sampled V rows, each row read once per GQA group and weighted by its
 *      sample count, per (KV head, chunk) with an fp32 accumulator (Appendix O, Algorithm 5), then the
 *      chunk sums added per head and scaled by 1/S (Section 2, Eq. 4).
 *
 * Conventions shared by every entry point:
 *   - Device pointers are caller-owned; the library never frees or retains them past the call.
 *   - Layouts are row-major: q and out are [batch, heads, d]; K and V are sequence-major caches
 *     [batch, nk, kv_heads, d] (Appendix Q), element (b, n, k, i) at
 *     b*kv_batch_stride + n*kv_seq_stride + k*d + i. Query head h reads KV head h / (heads/kv_heads)
 *     (Appendix O, Algorithm 2).
 *   - K and V rows and q must be 16-byte aligned (base pointers and strides).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default stream). Results are valid
 *     after the stream is synchronised. Debug outputs that live on the host (stats, stage times) make
 *     the call synchronise the stream before it returns.
 *   - Every call validates its arguments on the host before it makes any HIP call, and returns a
 *     status code (SANTA_OK or a SANTA_ERR_*); nothing is thrown across the ABI. A description of the
 *     last failure on the calling thread is available from santa_last_error().
 *   - The result is a pure function of (inputs, S, mode, seed): the random numbers are Philox4x32-10
 *     (Salmon et al., SC'11) keyed by (seed mod 2^32, seed >> 32) with counter (m, h, b, tag): tag 0 for
 *     the m-th i.i.d./stratified point of query head h in batch b, tag 1 for the systematic offset, tag
 *     2 + 256n for the Bernoulli decision of query element m in Bernoulli sample n. A uniform is
 *     ((x0 << 32 | x1) >> 11) * 2^-53.
 *   - Inputs must be finite; NaN and Inf are not checked and propagate.
 */
#ifndef SANTA_H_
#define SANTA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SANTA_OK 0
#define SANTA_ERR_INVALID_ARG 1     /* null pointer, heads % kv_heads != 0, S < 1, nk < 1, bad mode bits ... */
#define SANTA_ERR_UNSUPPORTED 2     /* d not in {64, 128}, dtype, G > 8, nk > 2^20, S > 65535 */
#define SANTA_ERR_WORKSPACE 3       /* workspace_bytes smaller than santa_workspace_bytes() */
#define SANTA_ERR_HIP 4             /* a HIP runtime call or launch failed (see santa_last_error) */
#define SANTA_ERR_TIMEOUT 5         /* a bounded in-kernel wait gave up (blocks of one launch that were not all
                                       resident, or a handshake that never completed); the outputs of the
                                       affected query heads are NaN. Reported by santa_status() and by calls
                                       with stats_out. */

/* sampling modes (low byte) and flags */
#define SANTA_IID 0                 /* SANTA: T_m ~ U[0,1) i.i.d. (Section 2, Eq. 4) */
#define SANTA_STRAT 1               /* S²ANTA-strat: T_m ~ U[m/S, (m+1)/S) independently (Section 2.1) */
#define SANTA_SYS 2                 /* S²ANTA-sys: one U ~ U[0, 1/S), T_m = U + m/S (Section 2.1) */
#define SANTA_PROP 3                /* S²ANTA-prop (Section 3.2; Appendix O, Algorithms 2-5): 256-key tiles get
                                       largest-remainder budgets S_t ~ S W_t / Z, then systematic counts
                                       c_n = floor(a0 + p + x_n) - floor(a0 + p) within the tile, with
                                       x_n = S_t exp(s_n - m_t) / l_t and a0 ~ U(0,1) per (tile, head) from
                                       Philox counter (t, h, b, 3). idx_out lists each head's sampled keys in
                                       increasing order with multiplicity. */
#define SANTA_FLASH 4               /* S²ANTA-flash (Section 3.3; Appendix P, Algorithms 6-8): every 256-key tile
                                       gets the same budget S_tile = max(1, round(S / T)) (halves up), its own
                                       systematic counts with a0 ~ U(0,1) from Philox counter (t, h, b, 4) and
                                       an fp32 partial sum_n c_n V_n; the merge returns
                                       (sum_t W_t partial_t) / (Z S_tile), W_t = exp(m_t - m*) l_t. idx_out lists
                                       T * S_tile keys per head (santa_samples_per_head), tile t's in slots
                                       [t S_tile, (t+1) S_tile), increasing within a tile. */
#define SANTA_TERNARY_Q 0x100       /* Bernoulli ternary query for the score stage (Section 5, Eq. 5; B = 1,
                                       norm = max_i |q_i| per (batch, head)) */
#define SANTA_GROUP_BERNOULLI_Q 0x200 /* mean-group-query Bernoulli scores (Section 5.1, Eq. 6; Appendix C.2,
                                       Eqs. 10-13): per KV group m_i = mean over its heads of |q_i|,
                                       norm = max_i m_i, c_i = #{n < B : (n + U_{i,n}) / B < m_i / norm}
                                       (stratified, U from Philox counter (i, kv, b, 5 + 256 n)), score of head
                                       g = (sum_i ((norm c_i / B) / m_i) q_{g,i} K_i) / sqrt(dk); features with
                                       c_i = 0 are not read. Needs SANTA_K_FEATURE_MAJOR and bern_samples = B;
                                       excludes SANTA_TERNARY_Q */
#define SANTA_K_FEATURE_MAJOR 0x400 /* K is given feature-major, K^T [batch][kv_heads][d][kt_row_stride]:
                                       element (b, kv, i, n) at K[b * kt_batch_stride + (kv * d + i) *
                                       kt_row_stride + n]; V keeps the sequence-major layout. The score pass
                                       then reads only the feature rows with a non-zero query weight. */
#define SANTA_MULTI_LAUNCH 0x800    /* use the multi-launch path (score, sampling and merge kernels) even where
                                       the one-launch decode applies; same results up to the order of the fp32
                                       partial sums (a measurement and diagnosis option) */

/* element types of q, K, V and out */
#define SANTA_BF16 0
#define SANTA_F32 1

typedef struct santa_stats {
  int32_t launches;      /* kernels launched by the call */
  int64_t bytes_k;       /* K bytes streamed: batch * nk * kv_heads * d * elt (feature-major K: only the
                            feature rows read, sum over groups of rows * nk * elt) */
  int64_t bytes_v;       /* V bytes gathered: (sum over (b, kv) of distinct sampled rows) * d * elt; in the
                            two-launch S²ANTA-flash every head reads its own sampled rows of each tile, so
                            there the sum runs over (b, head, tile) of that head's distinct rows in the tile */
  int64_t bytes_qo;      /* q read + out written: 2 * batch * heads * d * elt */
  int64_t unique_rows;   /* sum over (b, kv) of the distinct sampled rows */
  int64_t* group_unique_rows;  /* optional host array [batch * kv_heads] (NULL to skip): the distinct sampled
                                  rows of each (sequence, KV head), the rows its gather reads (Appendix O,
                                  Algorithm 5, the emitted rows of the group) */
} santa_stats;

typedef struct santa_args {
  const void* q;             /* [batch, heads, d] device */
  const void* K;             /* [batch, nk, kv_heads, d] device (strided, see above); with
                                SANTA_K_FEATURE_MAJOR the K^T layout described there */
  const void* V;             /* same layout as K */
  void* out;                 /* [batch, heads, d] device, same dtype as the inputs */
  int32_t batch;
  int32_t heads;
  int32_t kv_heads;
  int32_t d;                 /* head dimension: 64 or 128 */
  int64_t nk;                /* keys attended per sequence (the current token included) */
  int64_t kv_seq_stride;     /* elements between consecutive positions; 0 means kv_heads * d */
  int64_t kv_batch_stride;   /* elements between sequences; 0 means nk * kv_seq_stride */
  int32_t S;                 /* samples per query head, >= 1 */
  int32_t mode;              /* SANTA_IID | SANTA_STRAT | SANTA_SYS | SANTA_PROP | SANTA_FLASH, optionally
                                | SANTA_TERNARY_Q or SANTA_GROUP_BERNOULLI_Q, | SANTA_K_FEATURE_MAJOR */
  int32_t dtype;             /* SANTA_BF16 or SANTA_F32 */
  int32_t bern_samples;      /* B of SANTA_GROUP_BERNOULLI_Q, 1..64; ignored otherwise */
  uint64_t seed;
  void* stream;              /* hipStream_t, NULL = default stream */
  void* workspace;           /* device scratch of at least santa_workspace_bytes() bytes; no initial contents
                                are required (every call writes each part before reading it); calls that
                                share it must not overlap */
  size_t workspace_bytes;
  /* optional debug outputs; NULL to skip */
  int32_t* idx_out;          /* device [batch, heads, L], L = santa_samples_per_head(nk, S, mode) (= S except
                                for SANTA_FLASH): sampled key index of each point, in point order */
  double* prob_out;          /* device [batch, heads, nk]: softmax probabilities */
  santa_stats* stats_out;    /* host; the call synchronises the stream to fill it */
  float* stage_ms;           /* host float[4], milliseconds; synchronises the stream. [0]: time of the
                                score kernel (events HIP records with its launch, hipExtLaunchKernel: its
                                dispatch and execution; the whole decode for the one-launch form); [1]:
                                from the end of the score kernel to an event after the chunk CDF and
                                resolve launches; [2]: from there to an event after the merge launch; [3]:
                                from the score kernel's start event to that last event */
  /* SANTA_K_FEATURE_MAJOR only (elements); rows must hold at least nk rounded up to 8 and start 16-byte
     aligned */
  int64_t kt_row_stride;     /* between feature rows; 0 means nk rounded up to 8 */
  int64_t kt_batch_stride;   /* between sequences; 0 means kv_heads * d * kt_row_stride */
  int32_t debug_spin_limit;  /* polls before a bounded in-kernel wait gives up; 0 = the library default (a
                                wait of seconds). Tests set small values to force the timeout path, whose
                                outputs are NaN and whose status is SANTA_ERR_TIMEOUT. */
} santa_args;

/*
 * santa_status — the outcome of the last call that used this workspace with these sizes: synchronises
 * a->stream, then returns SANTA_OK, or SANTA_ERR_TIMEOUT if a bounded in-kernel wait of any (sequence, KV
 * head) group gave up in that call (those heads' outputs are NaN). a->workspace NULL means the scratch of
 * santa_decode_noalloc on the current device. Every decode call writes these status words, so the
 * default path needs no stats_out to detect the failure.
 */
int santa_status(const santa_args* a);

/*
 * santa_decode — one SANTA / S²ANTA decode step in its simplest form: batch 1, bf16 q/K/V/out,
 * contiguous [nk, kv_heads, d] caches, the default stream, and a workspace the library
 * allocates on first use and keeps (grow-only, per device) until santa_release(). Calls on one device
 * share that workspace and must not overlap. Returns a status code.
 */
int santa_decode(const void* q, const void* K, const void* V, int64_t nk, int heads, int kv_heads, int d, int S,
                 int mode, uint64_t seed, void* out);

/*
 * santa_decode_ex — the full form. Caller-owned workspace (`workspace`, `workspace_bytes`); never
 * allocates device memory. Calls sharing one workspace must not overlap.
 * One launch where it applies (bf16, sequence-major K, any of the five modes, at most one block
 * per CU for the whole grid, up to 512 chunks of 256 keys per sequence and 32 per block, and the block's
 * chunks fit the sampling phase's LDS): the split-K score pass, then, after an exchange of the chunk
 * statistics between the blocks of each (KV head, sequence) group (Section 3.1's global barrier, per
 * group; the blocks wait for the published values themselves), the chunk CDF, the points that fall in
 * each block's chunks (SANTA_PROP: every head's tile budgets, then the per-key counts of the block's
 * tiles; SANTA_FLASH: the uniform per-tile budget, no CDF), the gather of each distinct sampled row once
 * per group into fp32 sums per head (SANTA_FLASH: each count weighted by W_t / (Z S_tile)), and the sum of
 * the blocks' partials per head times 1/S (SANTA_FLASH: the plain sum). These barriers need every block
 * of the launch resident at once; if other work keeps blocks from running, the bounded waits give up
 * and the call reports SANTA_ERR_TIMEOUT (santa_status) with NaN outputs.
 * Otherwise three or four kernels on `stream`: the split-K score pass; for more than 128 chunks of 256
 * keys, the chunk CDF per KV group (SANTA_PROP: the tile budgets per query head; SANTA_FLASH needs neither),
 * which the next kernel otherwise builds itself; the sampling and gather-add per (chunk, KV group) (each
 * distinct sampled row read once and added with its per-head counts into an fp32 chunk partial); and the
 * merge that adds the chunk partials of each head and scales by 1/S (SANTA_FLASH: weights each partial by
 * W_t / (Z S_tile)).
 */
int santa_decode_ex(const santa_args* a);

/*
 * santa_decode_noalloc — santa_decode_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes the same arguments but
 * ignores `workspace` / `workspace_bytes`: its workspace is a SANTA_NOALLOC_MAX_BYTES device array of
 * the library (one per device, created when the library's code object is loaded on that device and held
 * until the process ends; its address is looked up once per device on the first call there). The call
 * allocates nothing. The caller still passes q, K, V, out and the optional device idx_out / prob_out.
 * Errors: SANTA_ERR_WORKSPACE when santa_workspace_bytes() for these sizes exceeds
 * SANTA_NOALLOC_MAX_BYTES; SANTA_ERR_INVALID_ARG when stats_out or stage_ms is set (they synchronise and
 * create events); otherwise as santa_decode_ex. Every call on one device shares that device's array, so
 * calls that overlap on one device (other streams, other threads) race; calls in one stream do not.
 * No initial contents are required: each call writes every part of the array it later reads.
 */
#define SANTA_NOALLOC_MAX_BYTES (64u << 20)
int santa_decode_noalloc(const santa_args* a);

/* Workspace bytes santa_decode_ex needs for these sizes (0 if the sizes are invalid or d is unsupported). */
size_t santa_workspace_bytes(int batch, int64_t nk, int heads, int kv_heads, int d, int S, int mode);

/*
 * Number of sampled keys listed per head for these sizes: S for SANTA_IID/STRAT/SYS/PROP, T * S_tile for
 * SANTA_FLASH (T = ceil(nk / 256), S_tile as defined there). -1 if nk < 1, S < 1 or the mode is unknown.
 * idx_out must hold batch * heads * this many int32.
 */
int64_t santa_samples_per_head(int64_t nk, int S, int mode);

/*
 * santa_dense_decode — dense decode attention softmax(q K^T / sqrt(dk)) V (Section 2, Eq. 1) over the
 * same layouts, fp32 accumulation, output in the input dtype. A measurement baseline that reads all of
 * K and V (split-KV partials and a merge, as in FlashDecoding-style decoding). S, mode, seed and the
 * debug outputs of `a` are ignored; the workspace must hold santa_dense_workspace_bytes() bytes.
 */
int santa_dense_decode(const santa_args* a);
size_t santa_dense_workspace_bytes(int batch, int64_t nk, int heads, int kv_heads, int d);

/*
 * santa_philox4x32_10 — host-side evaluation of the library's own Philox4x32-10 (the same inline code
 * the kernels run), for known-answer tests: out = Philox(ctr, key).
 */
void santa_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/*
 * santa_exp_f64 — host-side evaluation of the library's own fp64 exponential (the same inline code the
 * kernels run for every softmax weight exp(s - max) and chunk scale exp(m_t - m*), Section 2, Eq. 1), for
 * accuracy tests: e^x within a few units in the last place for -746 <= x <= 709, +0 below -746 and for
 * -inf, exactly 1 at 0. No GPU is touched.
 */
double santa_exp_f64(double x);

/*
 * santa_stream_read — diagnostic: reads `bytes` of device memory at `src` once with 16-byte non-temporal
 * loads (the loads the score pass streams K with; one block of 1024 threads per CU, 128 KiB in flight per
 * CU), writing one XOR word per block into `scratch` (device memory of santa_stream_read_scratch_bytes()
 * bytes, contents meaningless): the read bandwidth the device reaches for that size and cache state.
 * bytes must be a positive multiple of 16 and src 16-byte aligned; asynchronous like the decode calls,
 * unless kernel_ms (host, optional) is given: then the call synchronises and stores the kernel's time
 * in milliseconds from events HIP records with its launch (its dispatch and execution).
 */
int santa_stream_read(const void* src, size_t bytes, void* scratch, size_t scratch_bytes, void* stream,
                      float* kernel_ms);
size_t santa_stream_read_scratch_bytes(void);

const char* santa_status_string(int status);
const char* santa_last_error(void);   /* thread-local description of the last failure, "" if none */
const char* santa_version(void);
void santa_release(void);            /* frees the workspace santa_decode allocated, on every device */

#ifdef __cplusplus
}
#endif

#endif /* SANTA_H_ */
