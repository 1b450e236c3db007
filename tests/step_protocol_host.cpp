// Host model of the single-launch step's work protocol (qk_norm_rope_amd/csrc/
// step_protocol.h): the kernel's own protocol code, run_step_protocol, over the
// same control-word layout held in std::atomic ints, with one host thread per
// workgroup and at most `resident` of them running at once (the GPU holds only so
// many workgroups; the others start when one leaves). Items sleep for random
// short times so the interleavings vary from run to run.
//
// Checked per configuration: the run ends (a watchdog fails a run that has not
// ended within its limit); every item runs exactly once; every prefill and decode
// item sees every append chunk's and the plan's writes; the control words are zero
// again at the end, so the next call (run on the same words) starts clean; a lost
// publication (an append chunk that never publishes) ends the wait at its bound,
// records the fault, skips phase 2, and every workgroup still leaves.
//
// Usage: step_protocol_host  (exit status 0: every configuration passed)
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "step_protocol.h"

using namespace qknr;
using Clock = std::chrono::steady_clock;

struct Config {
  int grid, resident, n_append, n_prefill, n_decode;
  int lose_append;        // an append chunk that never publishes (-1: none)
  int calls;              // consecutive calls on the same control words
  unsigned seed;
};

struct Shared {
  std::atomic<int> ctl[kCtlInts];
  std::vector<std::atomic<int>> append_runs, append_written, prefill_runs, decode_runs;
  std::atomic<int> plan_runs{0}, plan_written{0}, unready_reads{0};
  int lose_append = -1;
  std::chrono::milliseconds wait_bound{200};
  // residency: at most `resident` workgroups run at once
  std::mutex mu;
  std::condition_variable cv;
  int running = 0;
  explicit Shared(const Config& c)
      : append_runs(c.n_append), append_written(c.n_append), prefill_runs(c.n_prefill), decode_runs(c.n_decode) {
    for (auto& w : ctl) w.store(0);
  }
  void reset_items() {
    for (auto& a : append_runs) a.store(0);
    for (auto& a : append_written) a.store(0);
    for (auto& a : prefill_runs) a.store(0);
    for (auto& a : decode_runs) a.store(0);
    plan_runs.store(0);
    plan_written.store(0);
    unready_reads.store(0);
  }
};

struct HostEnv {
  Shared& sh;
  const StepWork& w;
  std::mt19937 rng;

  void jitter() {
    const int us = std::uniform_int_distribution<int>(0, 200)(rng);
    if (us > 150) std::this_thread::sleep_for(std::chrono::microseconds(us - 150));
    else if (us > 100) std::this_thread::yield();
  }
  int take(int word) {
    jitter();
    return sh.ctl[word].fetch_add(1, std::memory_order_relaxed);
  }
  void publish(int word) {
    sh.ctl[word].fetch_add(1, std::memory_order_release);
  }
  bool wait_ready(int n_append, int n_plan) {
    const auto end = Clock::now() + sh.wait_bound;
    int a = 0, p = 0;
    for (;;) {
      a = sh.ctl[kAppendDone].load(std::memory_order_relaxed);
      p = sh.ctl[kPlanDone].load(std::memory_order_relaxed);
      if (a >= n_append && p >= n_plan) {
        std::atomic_thread_fence(std::memory_order_acquire);
        return true;
      }
      if (Clock::now() > end) break;
      std::this_thread::yield();
    }
    sh.ctl[kFault].store(1, std::memory_order_relaxed);
    sh.ctl[kSeenAppend].store(a, std::memory_order_relaxed);
    sh.ctl[kSeenPlan].store(p, std::memory_order_relaxed);
    return false;
  }
  int leave() { return sh.ctl[kExited].fetch_add(1, std::memory_order_acq_rel); }
  void clear() {
    for (int i = 0; i < kFault; ++i) sh.ctl[i].store(0, std::memory_order_relaxed);
  }
  void plan() {
    jitter();
    sh.plan_runs.fetch_add(1);
    sh.plan_written.store(1, std::memory_order_relaxed);
  }
  void append(int i) {
    jitter();
    sh.append_runs[i].fetch_add(1);
    sh.append_written[i].store(1, std::memory_order_relaxed);
    if (i == sh.lose_append) {   // this chunk's publication never happens: undo the protocol's add
      sh.ctl[kAppendDone].fetch_sub(1, std::memory_order_relaxed);
    }
  }
  void check_ready() {   // what a prefill or decode item reads must already be written
    bool ok = sh.plan_written.load(std::memory_order_relaxed) == 1;
    for (auto& a : sh.append_written) ok &= a.load(std::memory_order_relaxed) == 1;
    if (!ok) sh.unready_reads.fetch_add(1);
  }
  void prefill(int i) {
    check_ready();
    jitter();
    sh.prefill_runs[i].fetch_add(1);
  }
  void decode(int i) {
    check_ready();
    jitter();
    sh.decode_runs[i].fetch_add(1);
  }
};

// A lost chunk's add is undone after the protocol's own add (append runs before
// publish), which never lets kAppendDone reach n_append: the wait must time out.
static bool run_config(const Config& c) {
  Shared sh(c);
  sh.lose_append = c.lose_append;
  StepWork w{c.n_append, c.n_prefill, c.n_decode, c.grid};
  for (int call = 0; call < c.calls; ++call) {
    sh.reset_items();
    std::vector<std::thread> threads;
    for (int g = 0; g < c.grid; ++g) {
      threads.emplace_back([&, g]() {
        {
          std::unique_lock<std::mutex> lk(sh.mu);
          sh.cv.wait(lk, [&] { return sh.running < c.resident; });
          ++sh.running;
        }
        HostEnv e{sh, w, std::mt19937(c.seed * 7919u + call * 131u + g)};
        run_step_protocol(e, w);
        {
          std::lock_guard<std::mutex> lk(sh.mu);
          --sh.running;
        }
        sh.cv.notify_all();
      });
    }
    for (auto& t : threads) t.join();
    // outcome
    bool fault = sh.ctl[kFault].load() != 0;
    bool ok = true;
    auto fail = [&](const char* what) {
      std::printf("FAIL grid=%d resident=%d append=%d prefill=%d decode=%d lose=%d call=%d seed=%u: %s\n",
                  c.grid, c.resident, c.n_append, c.n_prefill, c.n_decode, c.lose_append, call, c.seed, what);
      ok = false;
    };
    if (sh.plan_runs.load() != 1) fail("the plan ran other than once");
    for (auto& a : sh.append_runs)
      if (a.load() != 1) fail("an append chunk ran other than once");
    for (int i = 0; i < kFault; ++i)
      if (sh.ctl[i].load() != 0) fail("a control word is not zero after the call");
    if (c.lose_append < 0) {
      if (fault) fail("fault recorded without a lost publication");
      if (sh.unready_reads.load() != 0) fail("a phase-2 item ran before every write was published");
      for (auto& a : sh.prefill_runs)
        if (a.load() != 1) fail("a prefill item ran other than once");
      for (auto& a : sh.decode_runs)
        if (a.load() != 1) fail("a decode item ran other than once");
    } else {
      if (!fault) fail("a lost publication was not recorded as a fault");
      if (sh.ctl[kSeenAppend].load() != c.n_append - 1) fail("the fault does not record the publications seen");
      for (auto& a : sh.prefill_runs)
        if (a.load() != 0) fail("a prefill item ran after a failed wait");
      for (auto& a : sh.decode_runs)
        if (a.load() != 0) fail("a decode item ran after a failed wait");
      sh.ctl[kFault].store(0);   // the caller reads and clears the fault words
      sh.ctl[kSeenAppend].store(0);
      sh.ctl[kSeenPlan].store(0);
    }
    if (!ok) return false;
  }
  return true;
}

int main() {
  std::vector<Config> cfgs;
  unsigned seed = 1;
  // grid x resident x items, consecutive calls on the same words
  const int shapes[][5] = {
      {1, 1, 5, 3, 2},     {4, 1, 7, 9, 4},     {8, 3, 20, 16, 16}, {16, 16, 3, 40, 32},
      {32, 4, 64, 64, 64}, {12, 5, 1, 0, 7},    {9, 9, 0, 5, 0},    {6, 2, 33, 0, 0},
      {64, 8, 100, 128, 128}, {5, 5, 200, 1, 1},
  };
  for (const auto& s : shapes)
    for (int rep = 0; rep < 3; ++rep) cfgs.push_back({s[0], s[1], s[2], s[3], s[4], -1, 3, seed++});
  // a lost publication: the wait ends at its bound, phase 2 is skipped, all leave
  cfgs.push_back({8, 3, 10, 6, 6, 4, 2, seed++});
  cfgs.push_back({4, 1, 3, 2, 2, 0, 1, seed++});

  std::atomic<bool> done{false};
  std::thread watchdog([&] {   // a hang is a failure, not a stuck test
    const auto end = Clock::now() + std::chrono::seconds(120);
    while (!done.load()) {
      if (Clock::now() > end) {
        std::printf("FAIL: the protocol did not finish within 120 s (a hang)\n");
        std::fflush(stdout);
        std::_Exit(2);
      }
      std::this_thread::sleep_for(std::chrono::milliseconds(20));
    }
  });
  int failed = 0;
  for (const auto& c : cfgs) failed += !run_config(c);
  done.store(true);
  watchdog.join();
  std::printf("%zu configurations, %d failed\n", cfgs.size(), failed);
  return failed ? 1 : 0;
}
