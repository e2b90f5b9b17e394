// Prints Philox4x32-10 blocks computed by rocRAND's header-only engine, used
// on the host only.  The oracle's Philox is pinned against it: rocRAND maps
// (seed, subsequence, offset) to key = (lo32 seed, hi32 seed) and counter =
// (lo32(offset/4), hi32(offset/4), lo32 subsequence, hi32 subsequence).
// Input lines: "seed subsequence block"; output: four hex words per line.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, subseq, block;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &block) == 3) {
    rocrand_device::philox4x32_10_engine eng(seed, subseq, block * 4ull);
    unsigned w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
