// Worker threads for the planner's independent simulations, shared by every
// planner call in the process.
//
// run(count, fn) calls fn(i) exactly once for every i in [0, count) and
// returns after all of them have finished. The caller takes part; results are
// written by index, so the outcome does not depend on which thread ran what. A
// call made while another thread is using the pool, a small batch, or a call
// in a process forked from the one that made the pool runs its items on the
// calling thread.
//
// Batches are isolated by one 64-bit word: generation (32 bits) | count (16) |
// next index (16). An item is claimed only by a compare-and-swap that finds
// the word of its own generation with next < count and advances next by one.
// A worker still inside the loop of a finished batch therefore cannot take an
// item of the next one (its generation no longer matches), and every index of
// a batch is claimed once: within a generation next only grows, and the word
// is replaced only after every item of the batch has completed.
#pragma once

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include <unistd.h>

namespace skv {

class SimPool {
 public:
  // threads = 0: one per hardware thread, at most 16 (the caller included)
  explicit SimPool(unsigned threads = 0) {
    unsigned n = threads;
    if (n == 0) n = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    for (unsigned i = 1; i < n; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~SimPool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_.store(true);
    }
    cv_.notify_all();
    for (auto& w : workers_) w.join();
  }
  SimPool(const SimPool&) = delete;
  SimPool& operator=(const SimPool&) = delete;

  size_t threads() const { return workers_.size() + 1; }

  void run(size_t count, const std::function<void(size_t)>& fn) {
    if (count == 0) return;
    std::unique_lock<std::mutex> busy(busy_, std::try_to_lock);
    if (workers_.empty() || count < 4 || count > kMaxCount || !busy.owns_lock() ||
        getpid() != pid_) {
      for (size_t i = 0; i < count; ++i) fn(i);
      return;
    }
    const uint32_t gen = ++gen_;   // only the owner of busy_ changes it
    fn_.store(&fn);
    pending_.store(count);
    {
      std::lock_guard<std::mutex> g(mu_);
      word_.store(pack(gen, (uint32_t)count, 0));
      if (sleepers_ > 0) cv_.notify_all();
    }
    work(gen);
    // the search issues many short batches: wait briefly by polling first
    if (!spin_until([this] { return pending_.load() == 0; })) {
      std::unique_lock<std::mutex> g(mu_);
      done_cv_.wait(g, [this] { return pending_.load() == 0; });
    }
  }

 private:
  static constexpr size_t kMaxCount = 0xFFFF;
  static uint64_t pack(uint32_t gen, uint32_t count, uint32_t next) {
    return ((uint64_t)gen << 32) | ((uint64_t)count << 16) | next;
  }
  static uint32_t gen_of(uint64_t w) { return (uint32_t)(w >> 32); }
  static uint32_t count_of(uint64_t w) { return (uint32_t)(w >> 16) & 0xFFFF; }
  static uint32_t next_of(uint64_t w) { return (uint32_t)w & 0xFFFF; }

  template <class Pred>
  static bool spin_until(Pred p) {
    const auto t0 = std::chrono::steady_clock::now();
    for (unsigned i = 1;; ++i) {
      if (p()) return true;
      if ((i & 63) == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(200))
        return false;
    }
  }

  // Claim and run items of generation gen until none is left.
  void work(uint32_t gen) {
    uint64_t w = word_.load();
    for (;;) {
      if (gen_of(w) != gen || next_of(w) >= count_of(w)) return;
      if (!word_.compare_exchange_weak(w, w + 1)) continue;   // w now holds the current word
      // the batch cannot finish (nor fn_ change) before this item is done
      (*fn_.load())(next_of(w));
      if (pending_.fetch_sub(1) == 1) {
        std::lock_guard<std::mutex> g(mu_);
        done_cv_.notify_all();
      }
      w = word_.load();
    }
  }

  void loop() {
    uint32_t seen = 0;
    for (;;) {
      auto fresh = [&] { return stop_.load() || gen_of(word_.load()) != seen; };
      if (!spin_until(fresh)) {
        std::unique_lock<std::mutex> g(mu_);
        ++sleepers_;
        cv_.wait(g, fresh);
        --sleepers_;
      }
      if (stop_.load()) return;
      seen = gen_of(word_.load());
      work(seen);
    }
  }

  std::vector<std::thread> workers_;
  std::mutex busy_, mu_;
  std::condition_variable cv_, done_cv_;
  std::atomic<const std::function<void(size_t)>*> fn_{nullptr};
  std::atomic<uint64_t> word_{0};
  std::atomic<size_t> pending_{0};
  std::atomic<bool> stop_{false};
  uint32_t gen_ = 0;
  int sleepers_ = 0;
  const pid_t pid_ = getpid();
};

}  // namespace skv
