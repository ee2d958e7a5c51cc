// Host-side dump of rocRAND's Philox4x32-10 engine (an independent,
// library implementation used only to pin the oracle's Philox).
// Usage: rocrand_philox_dump SEED SUBSEQUENCE COUNTER_LO_START N
// Prints, for c = COUNTER_LO_START .. +N-1, the four output words of
// Philox4x32-10 at counter (c, 0, SUBSEQUENCE low, SUBSEQUENCE high) and key
// (SEED low, SEED high): the engine reached by skipping 4*c outputs.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  unsigned long long subseq = std::strtoull(argv[2], nullptr, 0);
  unsigned long long c0 = std::strtoull(argv[3], nullptr, 0);
  unsigned long long n = std::strtoull(argv[4], nullptr, 0);
  for (unsigned long long c = c0; c < c0 + n; ++c) {
    rocrand_device::philox4x32_10_engine eng(seed, subseq, 4ull * c);
    unsigned int w0 = eng.next(), w1 = eng.next(), w2 = eng.next(), w3 = eng.next();
    std::printf("%llu %u %u %u %u\n", c, w0, w1, w2, w3);
  }
  return 0;
}
