// Test-only host program: prints rocRAND's Philox4x32-10 block for each
// (counter, key) read from stdin, one "c0 c1 c2 c3 k0 k1" line (hex) each.
// rocRAND is an independent implementation of the published generator
// (Salmon et al., SC'11); the oracle's own Philox is checked against it.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

namespace {
struct Engine : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};
}  // namespace

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  Engine e;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 r = e.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
