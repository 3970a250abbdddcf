// CPU model of the persistent kernels' work-distribution protocol (a test
// fixture, not part of the library).  Each workgroup is a std::thread; a
// residency limit (`slots`) models how many workgroups the GPU runs at once:
// a workgroup that has not started waits for a free slot and a finished one
// frees its slot.  The model follows the kernels' protocol step for step:
//
//   * a workgroup's role comes from an atomic ticket taken when it starts
//     (land / reduce tickets first, then compute);
//   * work is claimed from atomic queue counters;
//   * a unit of landed data is published by an arrival counter whose last
//     arrival resets it and stores the flag's epoch with release order;
//   * a waiter spins with acquire loads until the flag holds this launch's
//     epoch, giving up on an abort or after a time limit (which records a
//     timeout and aborts the launch);
//   * the last workgroup of a launch resets the launch's counters (and,
//     after an abort, the arrival counters), so launches can follow each
//     other on the same control memory with the epoch incremented.
//
// Operations (argv[1]):
//   ag     land workgroups land the peers' items; compute tiles wait for the
//          flag of their row block's chunk (and may land items while they
//          wait, as the AllGather kernel's helpers do)
//   rs     reduce workgroups sum peers' partials per item and release the
//          item's flag; compute tiles wait for it in their epilogue;
//          n_compute = 0 is the transfer-alone mode
//   moe    every workgroup routes items, then waits until all are routed and
//          reads every item's counts itself (its own copy of the offsets);
//          ticket 0 also writes the per-item bases for the combine and
//          publishes scan_ready; every workgroup lands route items, then runs
//          tiles that wait for the flags of the items filling their rows
//          (with --static only compute workgroups run tiles); with --combine
//          every workgroup then waits for the last tile and scan_ready before
//          it combines
//   ring   land workgroups land key/value blocks; a task waits for the blocks
//          it reads; the two halves of a pair combine through a counter and a
//          flag (the first to finish publishes, the second waits and merges)
//
// Options: --grid G --slots S --land L --compute C --items N --tiles T
//   --launches K --timeout-ms M --seed X --late-us U (random start delay per
//   workgroup) --withhold I (land skips unit I: the waiters must time out)
//   --permute (units are landed in a shuffled order) --no-help --combine
//   --static (MoE: land workgroups keep their role)
//
// Output: one JSON line {"ok": ..., "err": ..., "mismatch": ..., "late":
// ..., "ms": ...}.  err is 0 or 2 (timeout); mismatch counts data a waiter
// read after its flag that was not what the producer wrote for this launch.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

using Clock = std::chrono::steady_clock;
constexpr uint32_t kErrTimeout = 2;

struct Opts {
  std::string op = "ag";
  int grid = 16, slots = 16, land = 2, compute = -1, items = 32, tiles = 48, launches = 3;
  int timeout_ms = 2000, late_us = 0, withhold = -1;
  unsigned seed = 1;
  bool permute = false, help = true, combine = false, static_roles = false;
};

// Control memory that outlives a launch (flags and arrival counters, as the
// library's handle keeps them).
struct Control {
  std::atomic<uint32_t> ticket{0}, land_ctr{0}, tile_ctr{0}, reduce_ctr{0}, route_ctr{0};
  std::atomic<uint32_t> route_done{0}, scan_ready{0}, tiles_done{0}, done{0};
  std::atomic<uint32_t> abort_epoch{0}, err_code{0};
  std::vector<std::atomic<uint32_t>> flags, cnt;
  explicit Control(size_t n) : flags(n), cnt(n) {
    for (auto &f : flags) f.store(0);
    for (auto &c : cnt) c.store(0);
  }
};

// Counting semaphore of GPU slots.
struct Slots {
  std::mutex m;
  std::condition_variable cv;
  int free;
  explicit Slots(int n) : free(n) {}
  void take() {
    std::unique_lock<std::mutex> l(m);
    cv.wait(l, [&] { return free > 0; });
    --free;
  }
  void give() {
    { std::lock_guard<std::mutex> l(m); ++free; }
    cv.notify_one();
  }
};

uint64_t stamp(uint32_t unit, uint32_t epoch) {
  return (uint64_t)epoch << 32 | (uint64_t)(unit * 2654435761u + 12345u);
}

struct Launch {
  const Opts &o;
  Control &c;
  uint32_t epoch;
  Clock::duration limit;
  std::vector<std::atomic<uint64_t>> &data;   // one word per landed unit
  std::vector<std::atomic<uint64_t>> &ws;     // reduce / merge workspace
  std::vector<int> order;                     // landing order of the units
  std::atomic<int> mismatch{0};
  std::atomic<uint64_t> bases{0};             // MoE: the item bases ticket 0 writes for the combine
  std::vector<std::vector<int>> needs;        // units each tile waits for

  bool aborted() const { return c.abort_epoch.load(std::memory_order_relaxed) == epoch; }
  void raise(uint32_t code) {
    uint32_t z = 0;
    c.err_code.compare_exchange_strong(z, code);
    c.abort_epoch.store(epoch);
  }
  // spin until flag f holds this launch's epoch
  bool wait_flag(uint32_t f) {
    const auto t0 = Clock::now();
    while (c.flags[f].load(std::memory_order_acquire) != epoch) {
      if (aborted()) return false;
      if (Clock::now() - t0 > limit) {
        raise(kErrTimeout);
        return false;
      }
      std::this_thread::yield();
    }
    return true;
  }
  template <class Pred>
  bool wait_until(Pred pred) {
    const auto t0 = Clock::now();
    while (!pred()) {
      if (aborted()) return false;
      if (Clock::now() - t0 > limit) {
        raise(kErrTimeout);
        return false;
      }
      std::this_thread::yield();
    }
    return true;
  }
  // arrival of one of `target` parts of flag f (the last one publishes)
  void arrive(uint32_t f, uint32_t target) {
    const uint32_t old = c.cnt[f].fetch_add(1, std::memory_order_acq_rel);
    if (old + 1 == target) {
      c.cnt[f].store(0, std::memory_order_relaxed);
      c.flags[f].store(epoch, std::memory_order_release);
    }
  }
  // land unit u (its data word, then its flag); a withheld unit never lands
  void land(int u) {
    if (u == o.withhold) return;
    data[u].store(stamp(u, epoch), std::memory_order_relaxed);
    arrive((uint32_t)u, 1);
  }
  void check(int u) {
    if (data[u].load(std::memory_order_relaxed) != stamp(u, epoch)) mismatch.fetch_add(1);
  }
  bool land_queue() {  // land units until the queue is empty
    for (;;) {
      const uint32_t i = c.land_ctr.fetch_add(1);
      if (i >= (uint32_t)o.items) return true;
      land(order[i]);
    }
  }
  bool run_tile(int t) {
    for (int u : needs[t]) {
      if (!wait_flag((uint32_t)u)) return false;
      check(u);
    }
    return true;
  }
  void finish() {  // the last workgroup resets the launch-scoped counters
    const uint32_t d = c.done.fetch_add(1, std::memory_order_acq_rel);
    if (d + 1 == (uint32_t)o.grid) {
      for (auto *a : {&c.ticket, &c.land_ctr, &c.tile_ctr, &c.reduce_ctr, &c.route_ctr, &c.route_done,
                      &c.tiles_done})
        a->store(0);
      if (aborted())
        for (auto &x : c.cnt) x.store(0);
      c.done.store(0, std::memory_order_release);
    }
  }

  int n_compute() const { return o.compute >= 0 ? o.compute : o.grid - o.land; }

  void wg_ag() {
    const uint32_t tk = c.ticket.fetch_add(1);
    if (tk < (uint32_t)o.land) {
      land_queue();
      // land workgroups join the tiles once nothing is left to land
    } else if (tk >= (uint32_t)(o.land + n_compute())) {
      return;
    }
    for (;;) {
      const uint32_t t = c.tile_ctr.fetch_add(1);
      if (t >= (uint32_t)o.tiles) return;
      // a helper lands queued units while its tile's units are missing
      if (o.help) {
        for (;;) {
          bool ready = true;
          for (int u : needs[t]) ready &= c.flags[u].load(std::memory_order_acquire) == epoch;
          if (ready) break;
          const uint32_t i = c.land_ctr.fetch_add(1);
          if (i >= (uint32_t)o.items) break;
          land(order[i]);
        }
      }
      if (!run_tile((int)t)) return;
    }
  }

  // rs: units are reduce items (one per tile here); the reduce role sums the
  // peers' partials (data) into ws and releases the item; a compute tile's
  // epilogue waits for its item and reads ws
  void wg_rs() {
    const uint32_t tk = c.ticket.fetch_add(1);
    const bool xfer = n_compute() == 0;
    if (tk < (uint32_t)o.land) {
      for (;;) {
        const uint32_t i = c.reduce_ctr.fetch_add(1);
        if (i >= (uint32_t)o.items) break;
        const int u = order[i];
        if (u == o.withhold) continue;
        ws[u].store(stamp(u, epoch) ^ 0x5A5A5A5Aull, std::memory_order_relaxed);
        if (!xfer) arrive((uint32_t)u, 1);
      }
      return;
    }
    if (tk >= (uint32_t)(o.land + n_compute())) return;
    for (;;) {
      const uint32_t t = c.tile_ctr.fetch_add(1);
      if (t >= (uint32_t)o.tiles) return;
      const int u = (int)t % o.items;  // the tile's reduce item
      if (!wait_flag((uint32_t)u)) return;
      if (ws[u].load(std::memory_order_relaxed) != (stamp(u, epoch) ^ 0x5A5A5A5Aull)) mismatch.fetch_add(1);
    }
  }

  void wg_moe() {
    const uint32_t tk = c.ticket.fetch_add(1);
    // route: every workgroup takes route items
    for (;;) {
      const uint32_t i = c.route_ctr.fetch_add(1);
      if (i >= (uint32_t)o.items) break;
      ws[i].store(stamp(i, epoch), std::memory_order_relaxed);  // the item's counts
      c.route_done.fetch_add(1, std::memory_order_release);
    }
    // every workgroup: all items routed, then their counts (the offsets)
    if (!wait_until([&] { return c.route_done.load(std::memory_order_acquire) >= (uint32_t)o.items; })) return;
    for (int i = 0; i < o.items; ++i)
      if (ws[i].load(std::memory_order_relaxed) != stamp(i, epoch)) mismatch.fetch_add(1);
    if (tk == 0) {  // the combine's item bases
      bases.store(stamp(7777777, epoch), std::memory_order_relaxed);
      c.scan_ready.store(epoch, std::memory_order_release);
    }
    // every workgroup lands, then compute workgroups run tiles
    land_queue();
    if ((tk >= (uint32_t)o.land || !o.static_roles) && tk < (uint32_t)(o.land + n_compute())) {
      for (;;) {
        const uint32_t t = c.tile_ctr.fetch_add(1);
        if (t >= (uint32_t)o.tiles) break;
        if (!run_tile((int)t)) return;
        c.tiles_done.fetch_add(1, std::memory_order_release);
      }
    }
    if (o.combine) {  // every tile's rows and ticket 0's bases must be final before the combine
      if (!wait_until([&] { return c.tiles_done.load(std::memory_order_acquire) >= (uint32_t)o.tiles; })) return;
      if (!wait_until([&] { return c.scan_ready.load(std::memory_order_acquire) == epoch; })) return;
      if (bases.load(std::memory_order_relaxed) != stamp(7777777, epoch)) mismatch.fetch_add(1);
    }
  }

  // ring: units are key/value blocks; tiles are tasks, task t of pair t % P,
  // half t / P; merge flags follow the block flags
  void wg_ring() {
    const uint32_t tk = c.ticket.fetch_add(1);
    if (tk < (uint32_t)o.land) land_queue();
    if (tk >= (uint32_t)(o.land + n_compute())) return;
    const int pairs = o.tiles / 2;
    for (;;) {
      const uint32_t t = c.tile_ctr.fetch_add(1);
      if (t >= (uint32_t)o.tiles) return;
      if (!run_tile((int)t)) return;
      const int pair = (int)t % pairs;
      const uint32_t f = (uint32_t)(o.items + pair);
      const uint64_t mine = stamp((uint32_t)(1000000 + t), epoch);
      if (c.cnt[f].fetch_add(1, std::memory_order_acq_rel) == 0) {
        ws[pair].store(mine, std::memory_order_relaxed);  // the first half publishes its part
        c.flags[f].store(epoch, std::memory_order_release);
      } else {
        c.cnt[f].store(0, std::memory_order_relaxed);  // for the next launch
        if (!wait_flag(f)) return;
        const uint32_t other = (t < (uint32_t)pairs) ? t + (uint32_t)pairs : t - (uint32_t)pairs;
        if (ws[pair].load(std::memory_order_relaxed) != stamp(1000000 + other, epoch)) mismatch.fetch_add(1);
      }
    }
  }
};

void parse(int argc, char **argv, Opts &o) {
  if (argc > 1) o.op = argv[1];
  for (int i = 2; i < argc; ++i) {
    const std::string a = argv[i];
    auto next = [&] { return i + 1 < argc ? std::atoi(argv[++i]) : 0; };
    if (a == "--grid") o.grid = next();
    else if (a == "--slots") o.slots = next();
    else if (a == "--land") o.land = next();
    else if (a == "--compute") o.compute = next();
    else if (a == "--items") o.items = next();
    else if (a == "--tiles") o.tiles = next();
    else if (a == "--launches") o.launches = next();
    else if (a == "--timeout-ms") o.timeout_ms = next();
    else if (a == "--late-us") o.late_us = next();
    else if (a == "--withhold") o.withhold = next();
    else if (a == "--seed") o.seed = (unsigned)next();
    else if (a == "--permute") o.permute = true;
    else if (a == "--no-help") o.help = false;
    else if (a == "--combine") o.combine = true;
    else if (a == "--static") o.static_roles = true;
    else { std::fprintf(stderr, "unknown option %s\n", a.c_str()); std::exit(2); }
  }
}

}  // namespace

int main(int argc, char **argv) {
  Opts o;
  parse(argc, argv, o);
  if (o.grid < 1 || o.slots < 1 || o.items < 1 || o.tiles < 2 || o.land < 0 || o.land > o.grid) {
    std::fprintf(stderr, "bad sizes\n");
    return 2;
  }
  Control c((size_t)o.items + (size_t)o.tiles);
  std::vector<std::atomic<uint64_t>> data((size_t)o.items), ws((size_t)std::max(o.items, o.tiles));
  for (auto &d : data) d.store(0);
  for (auto &w : ws) w.store(0);
  std::mt19937 rng(o.seed);
  uint32_t err = 0;
  int mismatch = 0;
  const auto t0 = Clock::now();
  for (int L = 0; L < o.launches; ++L) {
    Launch l{o, c, (uint32_t)(L + 1), std::chrono::milliseconds(o.timeout_ms), data, ws, {}, {}, {}};
    c.err_code.store(0);
    l.order.resize((size_t)o.items);
    for (int i = 0; i < o.items; ++i) l.order[i] = i;
    if (o.permute) std::shuffle(l.order.begin(), l.order.end(), rng);
    // each tile waits for 1..3 units (AG: its row block's chunk; MoE: the
    // route items filling its rows; ring: the blocks of its half)
    l.needs.resize((size_t)o.tiles);
    for (int t = 0; t < o.tiles; ++t) {
      const int k = 1 + (int)(rng() % 3);
      for (int j = 0; j < k; ++j) l.needs[t].push_back((int)(rng() % (uint32_t)o.items));
    }
    std::vector<int> delay((size_t)o.grid);
    for (auto &d : delay) d = o.late_us > 0 ? (int)(rng() % (uint32_t)o.late_us) : 0;
    Slots slots(o.slots);
    std::vector<std::thread> th;
    for (int g = 0; g < o.grid; ++g)
      th.emplace_back([&, g] {
        if (delay[g]) std::this_thread::sleep_for(std::chrono::microseconds(delay[g]));
        slots.take();
        if (o.op == "ag") l.wg_ag();
        else if (o.op == "rs") l.wg_rs();
        else if (o.op == "moe") l.wg_moe();
        else l.wg_ring();
        l.finish();
        slots.give();
      });
    for (auto &t : th) t.join();
    mismatch += l.mismatch.load();
    if (c.err_code.load()) err = c.err_code.load();
    // counters of a finished launch are back at zero
    if (c.ticket.load() || c.land_ctr.load() || c.tile_ctr.load() || c.done.load()) mismatch += 1000000;
    if (!c.err_code.load())
      for (auto &x : c.cnt)
        if (x.load()) { mismatch += 1000000; break; }
  }
  const double ms = std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
  std::printf("{\"ok\": %s, \"err\": %u, \"mismatch\": %d, \"ms\": %.1f}\n",
              (err == 0 && mismatch == 0) ? "true" : "false", err, mismatch, ms);
  return 0;
}
