// A CPU model of the fused kernel's fetch/flag protocol, for ThreadSanitizer (test
// infrastructure; it shares no code with the GPU library). It follows the protocol the ROCm/iris
// issue "Fused all-gather+GEMM HBM-buffer kernel for iris.ops" describes (opening summary:
// fetchers copy A tiles into a staging buffer and set per-tile ready flags; GEMM workers wait
// on those flags, so no whole-gather barrier is needed), in the form the library implements:
//   - fetcher threads claim units from one counter (fetch_add), copy the unit's rows from
//     its shard into staging with plain stores, then publish: flags[u] += 1 with release;
//   - worker threads take output tiles; before reading a unit they poll flags[u] (relaxed)
//     until it equals the run's epoch, with a bounded spin, then acquire and read staging
//     with plain loads. The GPU acquires with a fence after its relaxed polls; ThreadSanitizer
//     does not model standalone fences, so here the acquire is one acquire re-read of the
//     flag once the polls have seen the epoch (the same ordering: every write published
//     before the flag reached the epoch happens before the reads that follow);
//   - flags hold the epoch (one increment per run), never reset; every run writes new data.
// Each worker checks every element it reads against the value the current run wrote, so a
// read of the previous run's data (a publish seen too early) is detected even where no data
// race is reported.
//
// Modes (argv[1]): ok | drop (one unit is never published: its waiters must time out and
// report it) | delay (fetchers sleep random amounts: results must be unchanged) | double (one
// unit published twice: waiters must detect the flag past the epoch) | race (the publish and
// the acquire are relaxed: ThreadSanitizer must report a data race).
// Exit status 0 means the mode behaved as expected; the test also checks the printed line.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

struct Model {
  int units = 48, unit_elems = 256, fetchers = 3, workers = 5, runs = 4;
  std::vector<int> shard;                       // source data, rewritten every run
  std::vector<int> staging;                     // [units][unit_elems]
  std::vector<std::atomic<unsigned>> flags;     // epoch of the last publish
  std::atomic<int> next_unit{0};
  std::atomic<int> timeouts{0}, over_epoch{0}, stale{0};
  std::string mode;
  int drop_unit = 17, double_unit = 9;
  long spin_limit = 2000000;

  explicit Model(const std::string& m) : shard(units * unit_elems), staging(units * unit_elems),
                                         flags(units), mode(m) {
    for (auto& f : flags) f.store(0, std::memory_order_relaxed);
  }

  static int value(unsigned epoch, int u, int i) { return (int)(epoch * 1000003u) ^ (u * 4099 + i); }

  void fetcher(unsigned epoch, int id) {
    std::mt19937 rng(epoch * 131 + id);
    const bool relaxed = mode == "race";
    for (;;) {
      const int u = next_unit.fetch_add(1, std::memory_order_relaxed);
      if (u >= units) break;
      if (mode == "delay") std::this_thread::sleep_for(std::chrono::microseconds(rng() % 300));
      for (int i = 0; i < unit_elems; ++i) staging[u * unit_elems + i] = shard[u * unit_elems + i];
      if (mode == "drop" && u == drop_unit) continue;
      flags[u].fetch_add(1, relaxed ? std::memory_order_relaxed : std::memory_order_release);
      if (mode == "double" && u == double_unit)
        flags[u].fetch_add(1, std::memory_order_release);
    }
  }

  void worker(unsigned epoch, int id) {
    const bool relaxed = mode == "race";
    for (int u = id; u < units; u += workers) {  // a tile needs units u (its m-tile x k-groups)
      long polls = 0;
      unsigned v = flags[u].load(std::memory_order_relaxed);
      while (v != epoch && polls < spin_limit) {
        if (v > epoch) break;
        ++polls;
        std::this_thread::yield();
        v = flags[u].load(std::memory_order_relaxed);
      }
      if (v > epoch) {
        over_epoch.fetch_add(1);
        continue;
      }
      if (v != epoch) {
        timeouts.fetch_add(1);
        continue;
      }
      if (!relaxed && flags[u].load(std::memory_order_acquire) != epoch) {
        over_epoch.fetch_add(1);
        continue;
      }
      for (int i = 0; i < unit_elems; ++i)
        if (staging[u * unit_elems + i] != value(epoch, u, i)) {
          stale.fetch_add(1);
          break;
        }
    }
  }

  void run(unsigned epoch) {
    for (int u = 0; u < units; ++u)
      for (int i = 0; i < unit_elems; ++i) shard[u * unit_elems + i] = value(epoch, u, i);
    next_unit.store(0);
    std::vector<std::thread> ts;
    for (int f = 0; f < fetchers; ++f) ts.emplace_back(&Model::fetcher, this, epoch, f);
    for (int w = 0; w < workers; ++w) ts.emplace_back(&Model::worker, this, epoch, w);
    for (auto& t : ts) t.join();
  }
};

}  // namespace

int main(int argc, char** argv) {
  const std::string mode = argc > 1 ? argv[1] : "ok";
  Model m(mode);
  int runs = m.runs;
  if (mode == "drop" || mode == "double") {
    runs = 1;
    m.spin_limit = 20000;
  }
  for (int e = 1; e <= runs; ++e) m.run((unsigned)e);
  const int to = m.timeouts.load(), oe = m.over_epoch.load(), st = m.stale.load();
  std::printf("mode=%s runs=%d timeouts=%d over_epoch=%d stale=%d\n", mode.c_str(), runs, to, oe,
              st);
  if (mode == "ok" || mode == "delay" || mode == "race") return (to || oe || st) ? 1 : 0;
  if (mode == "drop") return (to == 1 && !oe && !st) ? 0 : 1;     // exactly the dropped unit
  if (mode == "double") return (oe == 1 && !to && !st) ? 0 : 1;   // exactly the doubled unit
  return 2;
}
