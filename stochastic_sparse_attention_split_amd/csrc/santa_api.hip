// C ABI of libsanta.so: argument validation (before any HIP call), workspace layout, and the launch
// sequence score -> chunk CDF -> resolve (sample + gather per chunk) -> merge on the caller's stream.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/santa.h"
#include "common.h"
#include "launch.h"

using namespace santa;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SANTA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  size_t sync, status, stash, cmax, csum, cdf, cscale, lastpos, partial, idx, unique, sink, sync_err, budget, boff,
      kfeat, bmap, total;
};

// the synchronisation region of the one-launch decode, at offset 0 of every workspace: epochs per group
// and started flags per block
constexpr size_t SYNC_BYTES = SYNC_MAX_GROUPS * sizeof(uint64_t) + SYNC_MAX_BLOCKS * sizeof(uint64_t);

// every region is written by the call before it is read: no initial contents are required
// sampled keys listed per head: S, or T * S_tile for S²ANTA-flash
int64_t list_len(int64_t nk, int S, int mode) {
  const int64_t T = (nk + CHUNK - 1) / CHUNK;
  return (mode & 0xFF) == SANTA_FLASH ? T * flash_tile_budget(S, T) : (int64_t)S;
}

Layout layout(int64_t B, int64_t nk, int64_t H, int64_t Hkv, int64_t d, int64_t S, int mode) {
  const int64_t T = (nk + CHUNK - 1) / CHUNK;
  const int64_t G = H / Hkv;
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.sync = take(SYNC_BYTES);
  L.status = take((size_t)(B * Hkv) * sizeof(int32_t));
  L.stash = take((size_t)(B * H * T * CHUNK) * sizeof(double));
  L.cmax = take((size_t)(B * H * T) * sizeof(double));
  L.csum = take((size_t)(B * H * T) * sizeof(double));
  L.cdf = take((size_t)(B * H * (T + 1)) * sizeof(double));
  L.cscale = take((size_t)(B * H * T) * sizeof(double));
  L.lastpos = take((size_t)(B * H) * sizeof(int32_t));
  L.partial = take((size_t)(B * Hkv * T * G * d) * sizeof(float));
  L.idx = take((size_t)(B * H * list_len(nk, (int)S, mode)) * sizeof(int32_t));
  L.unique = take((size_t)(2 * B * Hkv * T) * sizeof(int32_t));  // distinct keys, then rows read (fused flash)
  L.sink = take((size_t)(B * Hkv * T) * sizeof(uint32_t));
  L.sync_err = take((size_t)(B * Hkv * T) * sizeof(int32_t));
  L.budget = take((size_t)(B * H * T) * sizeof(int32_t));
  L.boff = take((size_t)(B * H * T) * sizeof(int32_t));
  L.kfeat = take((size_t)(B * Hkv) * sizeof(int32_t));
  L.bmap = (mode & 0xFF) == SANTA_FLASH ? take((size_t)(B * Hkv * T) * 16 * sizeof(uint64_t)) : off;
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// shape checks shared by the sampled and the dense entry points
int validate_common(const santa_args* a, int64_t* seq, int64_t* bstride) {
  if (!a) return fail(SANTA_ERR_INVALID_ARG, "args is NULL");
  if (!a->q || !a->K || !a->V || !a->out) return fail(SANTA_ERR_INVALID_ARG, "q, K, V and out must be non-NULL");
  if (a->batch < 1 || a->heads < 1 || a->kv_heads < 1 || a->nk < 1)
    return fail(SANTA_ERR_INVALID_ARG, "batch, heads, kv_heads and nk must be >= 1");
  if (a->heads % a->kv_heads) return fail(SANTA_ERR_INVALID_ARG, "heads (%d) must be a multiple of kv_heads (%d)",
                                           a->heads, a->kv_heads);
  if (a->dtype != SANTA_BF16 && a->dtype != SANTA_F32)
    return fail(SANTA_ERR_UNSUPPORTED, "dtype %d is not SANTA_BF16 or SANTA_F32", a->dtype);
  if (a->d != 64 && a->d != 128) return fail(SANTA_ERR_UNSUPPORTED, "head dimension %d is not 64 or 128", a->d);
  if (a->heads / a->kv_heads > MAX_GROUP)
    return fail(SANTA_ERR_UNSUPPORTED, "GQA group %d exceeds %d heads per KV head", a->heads / a->kv_heads, MAX_GROUP);
  if (a->nk > (int64_t)MAX_CHUNKS * CHUNK)
    return fail(SANTA_ERR_UNSUPPORTED, "nk %lld exceeds %d", (long long)a->nk, MAX_CHUNKS * CHUNK);
  const int64_t row = (int64_t)a->kv_heads * a->d;
  const int64_t s = a->kv_seq_stride ? a->kv_seq_stride : row;
  if (s < row) return fail(SANTA_ERR_INVALID_ARG, "kv_seq_stride %lld < kv_heads*d", (long long)s);
  const int64_t bs = a->kv_batch_stride ? a->kv_batch_stride : s * a->nk;
  if (a->batch > 1 && bs < s * a->nk)
    return fail(SANTA_ERR_INVALID_ARG, "kv_batch_stride %lld < nk*kv_seq_stride", (long long)bs);
  const int64_t esz = a->dtype == SANTA_BF16 ? 2 : 4;
  if ((s * esz) % 16 || (bs * esz) % 16 || !aligned16(a->q) || !aligned16(a->K) || !aligned16(a->V))
    return fail(SANTA_ERR_INVALID_ARG, "q, K, V and the K/V strides must be 16-byte aligned");
  *seq = s;
  *bstride = bs;
  return SANTA_OK;
}

// rows of a feature-major K^T hold at least nk rounded up to 8 elements (4-key vector loads stay inside)
int64_t kt_row_min(int64_t nk) { return (nk + 7) & ~(int64_t)7; }

int validate_sampled(const santa_args* a, int64_t* seq, int64_t* bstride, int64_t* kt_row, int64_t* kt_batch) {
  int st = validate_common(a, seq, bstride);
  if (st) return st;
  if (a->S < 1) return fail(SANTA_ERR_INVALID_ARG, "S must be >= 1 (got %d)", a->S);
  const int base = a->mode & 0xFF, flags = a->mode & ~0xFF;
  if (base > SANTA_FLASH || base < 0 ||
      (flags & ~(SANTA_TERNARY_Q | SANTA_GROUP_BERNOULLI_Q | SANTA_K_FEATURE_MAJOR | SANTA_MULTI_LAUNCH)))
    return fail(SANTA_ERR_INVALID_ARG, "mode 0x%x has unknown bits", (unsigned)a->mode);
  if ((flags & SANTA_TERNARY_Q) && (flags & SANTA_GROUP_BERNOULLI_Q))
    return fail(SANTA_ERR_INVALID_ARG, "SANTA_TERNARY_Q and SANTA_GROUP_BERNOULLI_Q exclude each other");
  if ((flags & SANTA_GROUP_BERNOULLI_Q) && !(flags & SANTA_K_FEATURE_MAJOR))
    return fail(SANTA_ERR_INVALID_ARG, "SANTA_GROUP_BERNOULLI_Q needs SANTA_K_FEATURE_MAJOR");
  if ((flags & SANTA_GROUP_BERNOULLI_Q) && (a->bern_samples < 1 || a->bern_samples > 64))
    return fail(SANTA_ERR_INVALID_ARG, "bern_samples %d is not in 1..64", a->bern_samples);
  if (a->S > 65535) return fail(SANTA_ERR_UNSUPPORTED, "S %d exceeds 65535", a->S);
  if (a->debug_spin_limit < 0) return fail(SANTA_ERR_INVALID_ARG, "debug_spin_limit %d < 0", a->debug_spin_limit);
  *kt_row = 0;
  *kt_batch = 0;
  if (flags & SANTA_K_FEATURE_MAJOR) {
    const int64_t esz = a->dtype == SANTA_BF16 ? 2 : 4;
    const int64_t r = a->kt_row_stride ? a->kt_row_stride : kt_row_min(a->nk);
    if (r < kt_row_min(a->nk))
      return fail(SANTA_ERR_INVALID_ARG, "kt_row_stride %lld < nk rounded up to 8 (%lld)", (long long)r,
                  (long long)kt_row_min(a->nk));
    const int64_t bs = a->kt_batch_stride ? a->kt_batch_stride : (int64_t)a->kv_heads * a->d * r;
    if (a->batch > 1 && bs < (int64_t)a->kv_heads * a->d * r)
      return fail(SANTA_ERR_INVALID_ARG, "kt_batch_stride %lld < kv_heads*d*kt_row_stride", (long long)bs);
    if ((r * esz) % 16 || (bs * esz) % 16)
      return fail(SANTA_ERR_INVALID_ARG, "K^T rows and sequences must start 16-byte aligned");
    *kt_row = r;
    *kt_batch = bs;
  }
  return SANTA_OK;
}

// compute units of the current device (queried once per device)
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// as many score blocks as fit on the device at once, spread over the (KV head, sequence) groups
int score_blocks_per_group(int groups, int T, int per_cu) {
  const int target = per_cu * device_cus();
  int per = (target + groups - 1) / groups;
  return per < 1 ? 1 : (per > T ? T : per);
}

static_assert(MODE_IID == SANTA_IID && MODE_STRAT == SANTA_STRAT && MODE_SYS == SANTA_SYS &&
                  MODE_PROP == SANTA_PROP && MODE_FLASH == SANTA_FLASH,
              "the kernels number the sampling modes as the C header does");

// The one-launch decode applies when the streaming score kernel runs (bf16, sequence-major K, G <= 8), the
// sampling is any of the five modes, every block of the grid fits on the device at once (one per CU), the
// chunk CDF fits the in-kernel form and the sampling phase's LDS fits the K tiles.
// Returns the blocks per group, or 0 when the multi-launch path runs.
int one_launch_blocks(const Problem& p, int cus) {
  if (!p.bf16 || p.kfm || p.group_bern || p.mode > SANTA_FLASH || p.G > MAX_GROUP || p.T > DECODE_MAX_T) return 0;
  const int groups = p.B * p.Hkv;
  if (groups > cus || groups > SYNC_MAX_GROUPS) return 0;
  const int per = std::min(p.T, cus / groups);
  if ((int64_t)per * groups > SYNC_MAX_BLOCKS) return 0;
  const int n = (p.T + per - 1) / per;
  if (n > DECODE_MAX_CHUNKS || decode_lds_bytes(p.G, n, p.T, p.d, p.mode == SANTA_PROP) == 0) return 0;
  if (p.mode == SANTA_IID && (int64_t)n * p.S > 32768) return 0;  // i.i.d. points are tested in every chunk
  return per;
}

struct Events {
  hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};
  bool on = false;
  ~Events() {
    for (auto& x : e)
      if (x) (void)hipEventDestroy(x);
  }
};

// the per-group status words a call leaves in its workspace (stream already synchronised)
int read_status(const int32_t* status, int batch, int kv_heads) {
  const int groups = batch * kv_heads;
  std::vector<int32_t> v((size_t)groups);
  const hipError_t e = hipMemcpy(v.data(), status, v.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(status)");
  for (int g = 0; g < groups; ++g)
    if (v[g] != 0)
      return fail(SANTA_ERR_TIMEOUT, "a bounded in-kernel wait gave up for sequence %d, KV head %d; the outputs "
                  "of its query heads are NaN", g / kv_heads, g % kv_heads);
  return SANTA_OK;
}

}  // namespace

extern "C" {

size_t santa_workspace_bytes(int batch, int64_t nk, int heads, int kv_heads, int d, int S, int mode) {
  if (batch < 1 || nk < 1 || heads < 1 || kv_heads < 1 || S < 1 || heads % kv_heads) return 0;
  if (d != 64 && d != 128) return 0;
  return layout(batch, nk, heads, kv_heads, d, S, mode).total;
}

int64_t santa_samples_per_head(int64_t nk, int S, int mode) {
  if (nk < 1 || S < 1 || (mode & 0xFF) < 0 || (mode & 0xFF) > SANTA_FLASH) return -1;
  return list_len(nk, S, mode);
}

int santa_decode_ex(const santa_args* a) {
  g_err.clear();
  int64_t seq = 0, bstride = 0, kt_row = 0, kt_batch = 0;
  int st = validate_sampled(a, &seq, &bstride, &kt_row, &kt_batch);
  if (st) return st;
  const Layout L = layout(a->batch, a->nk, a->heads, a->kv_heads, a->d, a->S, a->mode);
  if (!a->workspace || a->workspace_bytes < L.total)
    return fail(SANTA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", a->workspace_bytes,
                L.total);

  char* ws = (char*)a->workspace;
  Problem p;
  p.q = a->q;
  p.K = a->K;
  p.V = a->V;
  p.out = a->out;
  p.B = a->batch;
  p.H = a->heads;
  p.Hkv = a->kv_heads;
  p.G = a->heads / a->kv_heads;
  p.d = a->d;
  p.nk = a->nk;
  p.seq_stride = seq;
  p.batch_stride = bstride;
  p.S = a->S;
  p.mode = a->mode & 0xFF;
  p.ternary = (a->mode & SANTA_TERNARY_Q) != 0;
  p.group_bern = (a->mode & SANTA_GROUP_BERNOULLI_Q) != 0;
  p.bern = p.group_bern ? a->bern_samples : 0;
  p.kfm = (a->mode & SANTA_K_FEATURE_MAJOR) != 0;
  p.kt_row_stride = kt_row;
  p.kt_batch_stride = kt_batch;
  p.bf16 = a->dtype == SANTA_BF16;
  p.seed = a->seed;
  p.scale = 1.0 / std::sqrt((double)a->d);
  p.T = (int)((a->nk + CHUNK - 1) / CHUNK);
  p.S_tile = flash_tile_budget(a->S, p.T);
  p.L = (int)list_len(a->nk, a->S, a->mode);
  p.score_blocks_per_group = score_blocks_per_group(p.B * p.Hkv, p.T, score_blocks_per_cu(p.d, p.bf16, p.G));
  p.stash = (double*)(ws + L.stash);
  p.stash_stride = (int64_t)p.T * CHUNK;
  p.cmax = (double*)(ws + L.cmax);
  p.csum = (double*)(ws + L.csum);
  p.cdf = (double*)(ws + L.cdf);
  p.cscale = (double*)(ws + L.cscale);
  p.lastpos = (int32_t*)(ws + L.lastpos);
  p.partial = (float*)(ws + L.partial);
  p.idx = a->idx_out ? a->idx_out : (int32_t*)(ws + L.idx);
  p.unique = (int32_t*)(ws + L.unique);
  p.sink = (uint32_t*)(ws + L.sink);
  p.sync_err = (int32_t*)(ws + L.sync_err);
  p.budget = (int32_t*)(ws + L.budget);
  p.boff = (int32_t*)(ws + L.boff);
  p.prob = a->prob_out;
  p.kfeat = (int32_t*)(ws + L.kfeat);
  p.bmap = (uint64_t*)(ws + L.bmap);
  // S²ANTA-flash with bf16 and G <= 4 on the sequence-major cache: sampled inside the score pass
  p.fused = p.mode == SANTA_FLASH && p.bf16 && p.G <= 4 && !p.kfm;
  p.want_unique = a->stats_out != nullptr;
  p.want_idx = a->idx_out != nullptr;
  p.spin_limit = a->debug_spin_limit > 0 ? a->debug_spin_limit : SPIN_LIMIT_DEFAULT;
  p.status = (int32_t*)(ws + L.status);
  p.check_sync = p.bf16 && !p.kfm;  // the streaming score kernel flags its blocks' handshakes
  p.sync_epoch = (uint64_t*)(ws + L.sync);
  p.sync_start = p.sync_epoch + SYNC_MAX_GROUPS;
  const int one = (a->mode & SANTA_MULTI_LAUNCH) ? 0 : one_launch_blocks(p, device_cus());
  p.one_launch = one > 0;
  if (p.one_launch) {
    p.fused = false;  // S²ANTA-flash too runs in the one launch
    p.score_blocks_per_group = one;
    // the sampling phase's LDS plan for the largest chunk count of a block (checked to fit above)
    const DecodeLds L =
        decode_lds_plan(p.G, (p.T + one - 1) / one, p.T, decode_lds_capacity(p.d), p.mode == SANTA_PROP);
    p.lds_nb = L.nb;
    p.lds_cnt = (int)L.cnt;
    p.lds_list = (int)L.list;
    p.lds_bits = (int)L.bits;
    p.lds_cdf = (int)L.cdf;
    p.lds_scl = (int)L.scl;
    p.lds_rows = (int)L.rows;
    p.lds_hist = (int)L.hist;
  }

  hipStream_t stream = (hipStream_t)a->stream;
  Events ev;
  if (a->stage_ms) {
    ev.on = true;
    for (auto& x : ev.e) {
      hipError_t e = hipEventCreate(&x);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  }
  hipError_t e;
  (void)hipGetLastError();  // start from a clean error state
  // with stage timing, HIP records e[0] and e[1] with the score kernel's launch (its dispatch and execution)
  LaunchEvents sev;
  if (ev.on) sev = LaunchEvents{ev.e[0], ev.e[1]};
  if (p.one_launch) {
    if ((e = launch_decode(p, stream, sev)) != hipSuccess) return hip_fail(e, "one-launch decode kernel launch");
  } else if ((e = p.kfm ? launch_score_fm(p, stream, sev) : launch_score(p, stream, sev)) != hipSuccess) {
    return hip_fail(e, "score kernel launch");
  }
  const bool prop = p.mode == SANTA_PROP;
  // for T <= FUSED_CDF_MAX_T the sampling kernel builds the chunk CDF (or the prop tile budgets) itself;
  // S²ANTA-flash needs neither
  const bool cdf_kernel = !p.one_launch && p.mode != SANTA_FLASH &&
                          (p.T > FUSED_CDF_MAX_T ||
                           (!prop && (int64_t)p.B * p.Hkv * p.T > SEPARATE_CDF_MIN_BLOCKS));
  p.cdf_done = cdf_kernel && !prop;
  if (cdf_kernel && !prop && (e = launch_chunk_cdf(p, stream)) != hipSuccess)
    return hip_fail(e, "chunk CDF kernel launch");
  if (cdf_kernel && prop && (e = launch_budget(p, stream)) != hipSuccess) return hip_fail(e, "budget kernel launch");
  if (!p.one_launch && !p.fused && (e = launch_resolve(p, stream)) != hipSuccess)
    return hip_fail(e, "resolve kernel launch");
  if (ev.on && (e = hipEventRecord(ev.e[2], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (!p.one_launch && (e = launch_merge(p, stream)) != hipSuccess) return hip_fail(e, "merge kernel launch");
  if (ev.on && (e = hipEventRecord(ev.e[3], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");

  if (a->stats_out) {
    std::vector<int32_t> u((size_t)a->batch * a->kv_heads * p.T);
    if ((e = hipMemcpyAsync(u.data(), p.unique, u.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream)) !=
        hipSuccess)
      return hip_fail(e, "hipMemcpyAsync(unique)");
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int64_t U = 0;
    for (int32_t x : u) U += x;
    int64_t R = U;  // V rows read: each distinct row once per (sequence, KV head) ...
    if (p.fused) {  // ... except in the fused S²ANTA-flash, where every head reads its own sampled rows
      std::vector<int32_t> rd(u.size());
      if ((e = hipMemcpy(rd.data(), p.unique + u.size(), rd.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) !=
          hipSuccess)
        return hip_fail(e, "hipMemcpy(rows read)");
      R = 0;
      for (int32_t x : rd) R += x;
    }
    const int64_t esz = p.bf16 ? 2 : 4;
    int64_t kbytes = (int64_t)a->batch * a->nk * a->kv_heads * a->d * esz;
    if (p.kfm) {  // feature rows actually read by the feature-major score pass
      std::vector<int32_t> kf((size_t)a->batch * a->kv_heads);
      if ((e = hipMemcpy(kf.data(), p.kfeat, kf.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_fail(e, "hipMemcpy(feature rows)");
      kbytes = 0;
      for (int32_t x : kf) kbytes += (int64_t)x * a->nk * esz;
    }
    santa_stats* s = a->stats_out;
    s->launches = p.one_launch ? 1 : (p.fused ? 2 : (cdf_kernel ? 4 : 3));
    s->bytes_k = kbytes;
    s->bytes_v = R * a->d * esz;
    s->bytes_qo = 2 * (int64_t)a->batch * a->heads * a->d * esz;
    s->unique_rows = U;
    if (s->group_unique_rows)
      for (int g = 0; g < a->batch * a->kv_heads; ++g) {
        int64_t ug = 0;
        for (int t = 0; t < p.T; ++t) ug += u[(size_t)g * p.T + t];
        s->group_unique_rows[g] = ug;
      }
    if ((st = read_status(p.status, a->batch, a->kv_heads)) != SANTA_OK) return st;
  }
  if (ev.on) {
    if ((e = hipEventSynchronize(ev.e[3])) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (int i = 0; i < 3; ++i) {
      float ms = 0.f;
      if ((e = hipEventElapsedTime(&ms, ev.e[i], ev.e[i + 1])) != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      a->stage_ms[i] = ms;
    }
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, ev.e[0], ev.e[3])) != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    a->stage_ms[3] = ms;
  }
  return SANTA_OK;
}

// ---- library-owned workspace for the simple entry point

namespace {
std::mutex g_ws_mu;
struct DevWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::vector<DevWs> g_ws;
}  // namespace

int santa_decode(const void* q, const void* K, const void* V, int64_t nk, int heads, int kv_heads, int d, int S,
                 int mode, uint64_t seed, void* out) {
  g_err.clear();
  santa_args a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.K = K;
  a.V = V;
  a.out = out;
  a.batch = 1;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.d = d;
  a.nk = nk;
  a.S = S;
  a.mode = mode;
  a.dtype = SANTA_BF16;
  a.seed = seed;
  int64_t seq, bs, ktr, ktb;
  int st = validate_sampled(&a, &seq, &bs, &ktr, &ktb);
  if (st) return st;
  const size_t need = layout(1, nk, heads, kv_heads, d, S, mode).total;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DevWs& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr) {
      (void)hipDeviceSynchronize();
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if ((e = hipMalloc(&w.ptr, need)) != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    w.bytes = need;
  }
  a.workspace = w.ptr;
  a.workspace_bytes = w.bytes;
  return santa_decode_ex(&a);
}

// ---- entry point without allocation: the workspace is the library's own device array

// One copy per device, zero-initialised when the code object is loaded and held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SANTA_NOALLOC_MAX_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: the device address of `scratch`

// device address of `scratch` on the current device, looked up once per device with that device current
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SANTA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SANTA_OK;
}
}  // namespace

int santa_decode_noalloc(const santa_args* a) {
  g_err.clear();
  if (!a) return fail(SANTA_ERR_INVALID_ARG, "args is NULL");
  if (a->stats_out || a->stage_ms)
    return fail(SANTA_ERR_INVALID_ARG, "santa_decode_noalloc takes no host debug outputs (stats_out, stage_ms)");
  int64_t seq = 0, bstride = 0, kt_row = 0, kt_batch = 0;
  int st = validate_sampled(a, &seq, &bstride, &kt_row, &kt_batch);
  if (st) return st;
  const size_t need = layout(a->batch, a->nk, a->heads, a->kv_heads, a->d, a->S, a->mode).total;
  if (need > (size_t)SANTA_NOALLOC_MAX_BYTES)
    return fail(SANTA_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; santa_decode_noalloc holds %zu",
                need, (size_t)SANTA_NOALLOC_MAX_BYTES);
  void* ptr = nullptr;
  if ((st = scratch_address(&ptr))) return st;
  santa_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = SANTA_NOALLOC_MAX_BYTES;
  return santa_decode_ex(&b);
}

int santa_status(const santa_args* a) {
  g_err.clear();
  if (!a) return fail(SANTA_ERR_INVALID_ARG, "args is NULL");
  int64_t seq = 0, bstride = 0, kt_row = 0, kt_batch = 0;
  santa_args b = *a;
  const void* ws = a->workspace;
  int st;
  if (!ws) {  // santa_decode_noalloc's scratch of the current device
    void* ptr = nullptr;
    if ((st = scratch_address(&ptr))) return st;
    b.workspace = ptr;
    b.workspace_bytes = SANTA_NOALLOC_MAX_BYTES;
  }
  if ((st = validate_sampled(&b, &seq, &bstride, &kt_row, &kt_batch))) return st;
  const Layout L = layout(b.batch, b.nk, b.heads, b.kv_heads, b.d, b.S, b.mode);
  if (b.workspace_bytes < L.total)
    return fail(SANTA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", b.workspace_bytes,
                L.total);
  const hipError_t e = hipStreamSynchronize((hipStream_t)b.stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return read_status((const int32_t*)((const char*)b.workspace + L.status), b.batch, b.kv_heads);
}

void santa_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  for (size_t dev = 0; dev < g_ws.size(); ++dev) {
    if (!g_ws[dev].ptr) continue;
    if (hipSetDevice((int)dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws[dev].ptr);
    }
    g_ws[dev] = DevWs{};
  }
  if (cur >= 0) (void)hipSetDevice(cur);
}

// ---- dense baseline

size_t santa_dense_workspace_bytes(int batch, int64_t nk, int heads, int kv_heads, int d) {
  if (batch < 1 || nk < 1 || heads < 1 || kv_heads < 1 || heads % kv_heads || (d != 64 && d != 128)) return 0;
  const int64_t Td = (nk + DENSE_CHUNK_MIN - 1) / DENSE_CHUNK_MIN;  // the most partials of any chunk size
  return align_up((size_t)(batch * (int64_t)heads * Td * (d + 2)) * sizeof(float));
}

int santa_dense_decode(const santa_args* a) {
  g_err.clear();
  int64_t seq = 0, bs = 0;
  int st = validate_common(a, &seq, &bs);
  if (st) return st;
  const size_t need = santa_dense_workspace_bytes(a->batch, a->nk, a->heads, a->kv_heads, a->d);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(SANTA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", a->workspace_bytes, need);
  DenseProblem p;
  p.q = a->q;
  p.K = a->K;
  p.V = a->V;
  p.out = a->out;
  p.B = a->batch;
  p.H = a->heads;
  p.Hkv = a->kv_heads;
  p.G = a->heads / a->kv_heads;
  p.d = a->d;
  p.nk = a->nk;
  p.seq_stride = seq;
  p.batch_stride = bs;
  p.bf16 = a->dtype == SANTA_BF16;
  p.scale = (float)(1.0 / std::sqrt((double)a->d));
  const int ch = p.G <= 4 ? dense_chunk(4) : dense_chunk(8);
  p.Td = (int)((a->nk + ch - 1) / ch);
  p.part = (float*)a->workspace;
  (void)hipGetLastError();
  const hipError_t e = launch_dense(p, (hipStream_t)a->stream);
  if (e != hipSuccess) return hip_fail(e, "dense kernel launch");
  return SANTA_OK;
}

// ---- diagnostics

size_t santa_stream_read_scratch_bytes(void) { return (size_t)STREAM_READ_MAX_BLOCKS * sizeof(uint32_t); }

int santa_stream_read(const void* src, size_t bytes, void* scratch, size_t scratch_bytes, void* stream,
                      float* kernel_ms) {
  g_err.clear();
  if (!src || !scratch) return fail(SANTA_ERR_INVALID_ARG, "src and scratch must be non-NULL");
  if (bytes < 16 || bytes % 16 || (uintptr_t)src % 16)
    return fail(SANTA_ERR_INVALID_ARG, "bytes (%zu) must be a positive multiple of 16 and src 16-byte aligned", bytes);
  if (scratch_bytes < santa_stream_read_scratch_bytes())
    return fail(SANTA_ERR_WORKSPACE, "scratch of %zu bytes is smaller than the %zu needed", scratch_bytes,
                santa_stream_read_scratch_bytes());
  (void)hipGetLastError();
  const int blocks = stream_read_blocks((int64_t)bytes, device_cus());
  Events ev;
  LaunchEvents lev;
  hipError_t e;
  if (kernel_ms) {
    for (int i = 0; i < 2; ++i)
      if ((e = hipEventCreate(&ev.e[i])) != hipSuccess) return hip_fail(e, "hipEventCreate");
    lev = LaunchEvents{ev.e[0], ev.e[1]};
  }
  e = launch_stream_read(src, (int64_t)bytes, (uint32_t*)scratch, blocks, (hipStream_t)stream, lev);
  if (e != hipSuccess) return hip_fail(e, "stream read kernel launch");
  if (kernel_ms) {
    if ((e = hipEventSynchronize(ev.e[1])) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    if ((e = hipEventElapsedTime(kernel_ms, ev.e[0], ev.e[1])) != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  }
  return SANTA_OK;
}

void santa_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const Philox4 r = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  out[0] = r.x0;
  out[1] = r.x1;
  out[2] = r.x2;
  out[3] = r.x3;
}

double santa_exp_f64(double x) { return santa::exp_f64(x); }

const char* santa_status_string(int status) {
  switch (status) {
    case SANTA_OK: return "ok";
    case SANTA_ERR_INVALID_ARG: return "invalid argument";
    case SANTA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SANTA_ERR_WORKSPACE: return "workspace too small";
    case SANTA_ERR_HIP: return "HIP runtime error";
    case SANTA_ERR_TIMEOUT: return "a bounded in-kernel wait gave up";
    default: return "unknown status";
  }
}

const char* santa_last_error(void) { return g_err.c_str(); }

const char* santa_version(void) { return "santa-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
