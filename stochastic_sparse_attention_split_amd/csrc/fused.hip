// One-launch decode: the streaming score kernel in its KM_DECODE form (score phase, then chunk CDF,
// sampling, gather and the output sum after in-kernel barriers between the blocks of each group).

#include "common.h"
#include "launch.h"
#include "stream_kernel.h"

namespace santa {

namespace {

template <int D>
hipError_t launch_decode_d(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  const dim3 grid(p.score_blocks_per_group, p.Hkv, p.B);
  const int n = (p.T + p.score_blocks_per_group - 1) / p.score_blocks_per_group;  // chunks of block 0
  const dim3 th(sk::STHREADS);
  if (p.mode == MODE_PROP) {
    if (p.G <= 4) {
      if (n <= 4) return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE_PROP, 4>, grid, th, st, ev, p);
      return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE_PROP, 0>, grid, th, st, ev, p);
    }
    return launch_timed(sk::score_stream_kernel<D, 2, KM_DECODE_PROP, 0>, grid, th, st, ev, p);
  }
  if (p.mode == MODE_FLASH) {
    if (p.G <= 4) {
      if (n <= 4) return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE_FLASH, 4>, grid, th, st, ev, p);
      return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE_FLASH, 0>, grid, th, st, ev, p);
    }
    return launch_timed(sk::score_stream_kernel<D, 2, KM_DECODE_FLASH, 0>, grid, th, st, ev, p);
  }
  if (p.G <= 4) {
    if (n <= 4) return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE, 4>, grid, th, st, ev, p);
    return launch_timed(sk::score_stream_kernel<D, 1, KM_DECODE, 0>, grid, th, st, ev, p);
  }
  return launch_timed(sk::score_stream_kernel<D, 2, KM_DECODE, 0>, grid, th, st, ev, p);
}

}  // namespace

// LDS the sampling phase of the one-launch decode needs for G heads, n chunks per block and T chunks per
// sequence (0 if it does not fit the score phase's K tiles of head dimension d)
size_t decode_lds_bytes(int G, int n, int T, int d, bool prop) {
  return decode_lds_plan(G, n, T, decode_lds_capacity(d), prop).total;
}

size_t decode_lds_capacity(int d) { return 2 * (size_t)CHUNK * d * 2; }

hipError_t launch_decode(const Problem& p, hipStream_t st, const LaunchEvents& ev) {
  if (!p.bf16 || p.kfm || p.G > 8 || p.T > DECODE_MAX_T) return hipErrorInvalidValue;
  return p.d == 128 ? launch_decode_d<128>(p, st, ev) : launch_decode_d<64>(p, st, ev);
}

}  // namespace santa
