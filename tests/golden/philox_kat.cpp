// Known-answer source for the Philox4x32-10 pin: the open-source rocRAND engine (MIT / D. E. Shaw BSD),
// compiled host-only from /opt/rocm/include. Reads "c0 c1 c2 c3 k0 k1" lines, prints the 4 output words.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Exposed : rocrand_device::philox4x32_10_engine {
  static uint4 run(uint4 c, uint2 k) {
    Exposed e;
    return e.ten_rounds(c, k);
  }
};

int main() {
  unsigned a, b, c, d, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &a, &b, &c, &d, &k0, &k1) == 6) {
    uint4 r = Exposed::run(make_uint4(a, b, c, d), make_uint2(k0, k1));
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
