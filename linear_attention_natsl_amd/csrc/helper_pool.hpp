// Per-device pool of helper contexts (a helper stream and its events) for
// calls that fork work onto a second stream.  Host code only, independent of
// HIP so that a host-only test can drive it with a fake context type.
//
// A call takes a context with acquire() and gives it back when it returns
// (Lease's destructor).  While one call holds a context no other call can
// obtain it, so concurrent calls never share a stream or an event; a context
// is handed out again only after its previous holder has enqueued all of its
// event waits.  Contexts are created on demand and never destroyed (work a
// call enqueued on a helper stream may still be running when it returns).
#pragma once
#include <mutex>
#include <vector>

namespace natsl {

template <typename Ctx, int MaxDevices = 64>
class HelperPool {
 public:
  // Returns a free context of device `dev`, or one made by make(dev) (which
  // returns nullptr on failure); nullptr if dev is out of range or make fails.
  template <typename Make>
  Ctx* acquire(int dev, Make&& make) {
    if (dev < 0 || dev >= MaxDevices) return nullptr;
    {
      std::lock_guard<std::mutex> lk(mu_);
      std::vector<Ctx*>& f = free_[dev];
      if (!f.empty()) {
        Ctx* c = f.back();
        f.pop_back();
        return c;
      }
    }
    return make(dev);  // outside the lock: creating streams and events is slow
  }
  void release(int dev, Ctx* c) {
    if (!c || dev < 0 || dev >= MaxDevices) return;
    std::lock_guard<std::mutex> lk(mu_);
    free_[dev].push_back(c);
  }
  // contexts currently free on a device (for tests)
  size_t free_count(int dev) {
    std::lock_guard<std::mutex> lk(mu_);
    return (dev < 0 || dev >= MaxDevices) ? 0 : free_[dev].size();
  }

  // gives the context back when the holder's scope ends
  struct Lease {
    HelperPool* pool = nullptr;
    int dev = -1;
    Ctx* ctx = nullptr;
    Lease() = default;
    Lease(const Lease&) = delete;
    Lease& operator=(const Lease&) = delete;
    ~Lease() {
      if (pool && ctx) pool->release(dev, ctx);
    }
  };

 private:
  std::mutex mu_;
  std::vector<Ctx*> free_[MaxDevices];
};

}  // namespace natsl
