// Test-only host program: prints rocRAND's Philox4x32 block for each line
// "c0 c1 c2 c3 k0 k1 R" (hex words, decimal round count) read from stdin.
// rocRAND is an independent implementation of the published generator
// (Salmon et al., SC'11); the oracle's own Philox is checked against it.
//   R == 10: rocRAND's ten-round block as it ships.
//   other R: R applications of rocRAND's own single round, its own Weyl key
//            bump between consecutive rounds (the published R-round
//            construction), so round counts other than 10 are pinned to the
//            same round function and key schedule.
//   R < 0:   that composition for -R rounds (R = -10 checks the composition
//            against the shipped ten-round block).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

namespace {
using Engine10 = rocrand_device::philox4x32_10_engine;

struct Engine : Engine10 {
  uint4 block(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

// The engine's round and key bump are private static members.  An explicit
// instantiation may name private members (access checking does not apply to
// the names in an explicit instantiation), and the instantiated friend
// function hands their addresses out.
struct RoundTag {
  using type = uint4 (*)(uint4, uint2);
  friend type get(RoundTag);
};
struct BumpTag {
  using type = uint2 (*)(uint2);
  friend type get(BumpTag);
};
template <typename Tag, typename Tag::type F>
struct Expose {
  friend typename Tag::type get(Tag) { return F; }
};
template struct Expose<RoundTag, &Engine10::single_round>;
template struct Expose<BumpTag, &Engine10::bumpkey>;

uint4 r_rounds(uint4 ctr, uint2 key, int rounds) {
  const auto round = get(RoundTag{});
  const auto bump = get(BumpTag{});
  for (int i = 0; i < rounds; ++i) {
    if (i > 0) key = bump(key);
    ctr = round(ctr, key);
  }
  return ctr;
}
}  // namespace

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  int rounds;
  Engine e;
  while (std::scanf("%x %x %x %x %x %x %d", &c0, &c1, &c2, &c3, &k0, &k1, &rounds) == 7) {
    const uint4 c{c0, c1, c2, c3};
    const uint2 k{k0, k1};
    const uint4 r = rounds == 10 ? e.block(c, k) : r_rounds(c, k, rounds < 0 ? -rounds : rounds);
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
