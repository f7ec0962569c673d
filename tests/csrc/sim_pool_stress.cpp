// Stress test of the planner's worker pool (host only; built by
// tests/test_host_sanitizers.py with and without ThreadSanitizer).
//
// Many batches of random sizes run back to back from one caller thread, while
// a second thread keeps calling the same pool (it finds the pool busy and runs
// its items itself). Each batch owns a freshly allocated counter array that
// the items increment through a lambda capturing it by reference; after run()
// returns, every counter of the batch must be exactly 1: an item run twice, an
// item of one batch run under another batch's function, or a run() that
// returned before its items finished all show up as a count other than 1 (or,
// under the sanitizer, as a race or a use after scope).
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <thread>
#include <vector>

#include "sim_pool.hpp"

int main(int argc, char** argv) {
  const int batches = argc > 1 ? std::atoi(argv[1]) : 20000;
  const unsigned threads = argc > 2 ? (unsigned)std::atoi(argv[2]) : 8;
  skv::SimPool pool(threads);
  std::atomic<long> bad{0}, done_items{0};
  std::atomic<bool> stop{false};

  auto one_batch = [&](std::mt19937& rng) {
    const size_t n = 1 + rng() % 300;
    const int spin = (int)(rng() % 4);
    auto hits = std::make_unique<std::atomic<int>[]>(n);
    for (size_t i = 0; i < n; ++i) hits[i].store(0);
    pool.run(n, [&](size_t i) {
      if (i >= n) {
        bad.fetch_add(1);
        return;
      }
      for (volatile int s = 0; s < spin * 50; ++s) {
      }
      hits[i].fetch_add(1);
    });
    for (size_t i = 0; i < n; ++i)
      if (hits[i].load() != 1) bad.fetch_add(1);
    done_items.fetch_add((long)n);
  };

  std::thread other([&] {
    std::mt19937 rng(7);
    while (!stop.load()) one_batch(rng);
  });
  std::mt19937 rng(1);
  for (int k = 0; k < batches; ++k) one_batch(rng);
  stop.store(true);
  other.join();
  std::printf("batches %d items %ld bad %ld threads %zu\n", batches, done_items.load(), bad.load(),
              pool.threads());
  return bad.load() == 0 ? 0 : 1;
}
