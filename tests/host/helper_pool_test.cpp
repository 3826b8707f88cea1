// Host-only test of the helper-context pool that natsl_forward draws its
// helper stream and events from.  Several threads lease contexts of two
// devices concurrently and "use" them (stamp the fake events with their own
// id, yield, check the stamps); a context leased by two threads at once, a
// context of the wrong device, or a lost context fails the test.  Built with
// g++ under ThreadSanitizer and under AddressSanitizer + UBSan by
// test_helper_pool.py.
#include <atomic>
#include <cstdio>
#include <thread>
#include <vector>

#include "../../linear_attention_natsl_amd/csrc/helper_pool.hpp"

struct FakeCtx {
  int dev;
  std::atomic<int> holder{-1};
  int fork = -1, routed = -1, join = -1;  // the "events": last recorder's id
};

static std::atomic<int> g_made{0};
static std::atomic<int> g_errors{0};

int main() {
  natsl::HelperPool<FakeCtx, 4> pool;
  const int kThreads = 8, kIters = 3000;
  std::vector<FakeCtx*> all[4];
  std::mutex all_mu;
  auto make = [&](int dev) {
    FakeCtx* c = new FakeCtx();
    c->dev = dev;
    g_made++;
    std::lock_guard<std::mutex> lk(all_mu);
    all[dev].push_back(c);
    return c;
  };
  std::vector<std::thread> th;
  for (int t = 0; t < kThreads; ++t)
    th.emplace_back([&, t] {
      for (int i = 0; i < kIters; ++i) {
        const int dev = (t + i) & 1;
        natsl::HelperPool<FakeCtx, 4>::Lease lease;
        lease.pool = &pool;
        lease.dev = dev;
        lease.ctx = pool.acquire(dev, make);
        FakeCtx* c = lease.ctx;
        if (!c || c->dev != dev) { g_errors++; continue; }
        int expect = -1;
        if (!c->holder.compare_exchange_strong(expect, t)) { g_errors++; continue; }
        // the call's record / wait sequence on its own events
        c->fork = t;
        std::this_thread::yield();
        c->routed = t;
        std::this_thread::yield();
        c->join = t;
        if (c->fork != t || c->routed != t || c->join != t) g_errors++;
        c->holder.store(-1);
      }
    });
  for (auto& x : th) x.join();
  int bad = g_errors.load();
  // every context is back in its device's free list, none was lost or doubled
  for (int dev = 0; dev < 2; ++dev)
    if (pool.free_count(dev) != all[dev].size()) bad++;
  // no more contexts than threads per device were ever needed
  if (g_made.load() > 2 * kThreads) bad++;
  // an out-of-range device gets nothing and makes nothing
  const int made = g_made.load();
  if (pool.acquire(7, make) != nullptr || pool.acquire(-1, make) != nullptr || g_made.load() != made) bad++;
  for (int dev = 0; dev < 2; ++dev)
    for (FakeCtx* c : all[dev]) delete c;
  std::printf("helper pool: %d contexts made, %d errors\n", made, bad);
  return bad == 0 ? 0 : 1;
}
