// kq_host.h — host-side helpers shared by the launch code: once-per-device
// setup state, safe to use from several host threads at once.
#pragma once

#include <atomic>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kq {

// Per-device flag for a setup step that must run once on each device (a
// kernel attribute, a cached device property).  Two threads racing through
// the first call may both run the step, which must therefore be idempotent.
// Devices past the 64th run it on every call.
class DeviceOnce {
  public:
    bool done(int dev) const {
        return dev >= 0 && dev < 64 && ((mask_.load(std::memory_order_acquire) >> dev) & 1u);
    }
    void set(int dev) {
        if (dev >= 0 && dev < 64) mask_.fetch_or(uint64_t(1) << dev, std::memory_order_release);
    }

  private:
    std::atomic<uint64_t> mask_{0};
};

}  // namespace kq
