// Host-side reference words from rocRAND's philox4x32_10 (its device API is
// also callable on the host).  Reads "seed index step" triples on stdin and
// prints the 32-bit word rocRAND returns at that offset of subsequence
// `step`.  Used only to pin the oracle's Philox; it links nothing of ours.
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed, index;
  unsigned step;
  while (std::scanf("%llu %llu %u", &seed, &index, &step) == 3) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, step, index, &st);
    std::printf("%u\n", rocrand(&st));
  }
  return 0;
}
