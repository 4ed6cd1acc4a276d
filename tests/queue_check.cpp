// Host check of the LM-head kernel's work queues (csrc/rlk_queue.h): for each launch geometry
// given on the command line as "n_vb n_tt rb" triples, every queue is drained the way the kernel's
// blocks drain it, and every (vocab block, row tile) item of the launch must come out exactly
// once. Prints one line per geometry; the exit status is the number of failed geometries.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rlk_queue.h"

int main(int argc, char** argv) {
  int failed = 0;
  for (int i = 1; i + 2 < argc; i += 3) {
    const long n_vb = std::atol(argv[i]), n_tt = std::atol(argv[i + 1]), rb = std::atol(argv[i + 2]);
    rlk::LmheadArgs a{};
    rlk::queue_setup(a, n_vb, n_tt, rb);
    std::vector<int> seen((size_t)(n_vb * n_tt), 0);
    long bad = 0, handed = 0, longest = 0, shortest = -1;
    for (int x = 0; x < rlk::kQueues; ++x) {
      long len = 0;
      for (uint32_t c = 0;; ++c) {
        int vb = -1, tt = -1;
        if (!rlk::queue_item(a, x, c, vb, tt)) break;
        ++len;
        ++handed;
        if (vb < 0 || vb >= n_vb || tt < 0 || tt >= n_tt) ++bad;
        else ++seen[(size_t)tt * n_vb + vb];
        if (len > n_vb * n_tt) break;  // a queue that never ends
      }
      longest = len > longest ? len : longest;
      shortest = (shortest < 0 || len < shortest) ? len : shortest;
    }
    long missing = 0, twice = 0;
    for (int s : seen) {
      missing += s == 0;
      twice += s > 1;
    }
    const bool ok = bad == 0 && missing == 0 && twice == 0 && handed == n_vb * n_tt;
    std::printf("%s n_vb=%ld n_tt=%ld rb=%ld items=%ld handed=%ld out_of_range=%ld missing=%ld "
                "repeated=%ld queue_len=%ld..%ld\n", ok ? "OK" : "FAIL", n_vb, n_tt, rb,
                n_vb * n_tt, handed, bad, missing, twice, shortest, longest);
    failed += !ok;
  }
  return failed;
}
