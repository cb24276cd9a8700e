// Test helper: prints rocRAND's Philox-4x32-10 block for counter/key triples
// read from stdin (one "c0 c1 c2 c3 k0 k1" line each). Calls the library's
// own engine; used only to pin the CPU oracle's Philox.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return this->ten_rounds(c, k); }
};

int main() {
  Probe pr;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 o = pr.block(make_uint4(c0, c1, c2, c3), make_uint2(k0, k1));
    std::printf("%u %u %u %u\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
