// Concurrent launch lanes: per-device side streams and fork/join events.
#include "lanes.hpp"

#include <atomic>

namespace etpc {
namespace {

std::atomic<int> g_limit{kLanes};

constexpr int kMaxDevices = 64;

struct DeviceLanes {
  std::mutex mu;
  bool tried = false;
  bool ok = false;
  hipStream_t side[kLanes] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kLanes] = {};
};

DeviceLanes g_dev[kMaxDevices];

// Lazily creates the side streams and events of the current device; holds dl.mu.
bool ensure(DeviceLanes& dl) {
  if (dl.tried) return dl.ok;
  dl.tried = true;
  bool ok = hipEventCreateWithFlags(&dl.fork, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < kLanes; ++i) {
    ok = hipStreamCreateWithFlags(&dl.side[i], hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&dl.join[i], hipEventDisableTiming) == hipSuccess;
  }
  dl.ok = ok;
  return ok;
}

}  // namespace

int lanes_limit() { return g_limit.load(); }

void set_lanes_limit(int n) { g_limit.store(n < 1 ? 1 : (n > kLanes ? kLanes : n)); }

LaneGroup::LaneGroup(hipStream_t main, int n) : main_(main) {
  const int lim = lanes_limit();
  n_ = n < 1 ? 1 : (n > lim ? lim : n);
  if (n_ == 1) return;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    n_ = 1;
    return;
  }
  DeviceLanes& dl = g_dev[dev];
  lock_ = std::unique_lock<std::mutex>(dl.mu);
  if (!ensure(dl)) {
    lock_.unlock();
    n_ = 1;
    return;
  }
  err_ = hipEventRecord(dl.fork, main_);
  for (int i = 0; i < n_ && err_ == hipSuccess; ++i) {
    side_[i] = dl.side[i];
    join_[i] = dl.join[i];
    err_ = hipStreamWaitEvent(side_[i], dl.fork, 0);
  }
  forked_ = true;
}

hipError_t LaneGroup::finish() {
  if (done_) return err_;
  done_ = true;
  if (forked_) {
    for (int i = 0; i < n_; ++i) {
      hipError_t e = hipEventRecord(join_[i], side_[i]);
      if (e == hipSuccess) e = hipStreamWaitEvent(main_, join_[i], 0);
      if (e != hipSuccess && err_ == hipSuccess) err_ = e;
    }
  }
  if (lock_.owns_lock()) lock_.unlock();
  return err_;
}

LaneGroup::~LaneGroup() { (void)finish(); }

}  // namespace etpc

extern "C" {

etpc_status etpc_set_lanes(int32_t lanes) {
  etpc::set_lanes_limit(lanes);
  return ETPC_OK;
}

int32_t etpc_get_lanes(void) { return etpc::lanes_limit(); }

}  // extern "C"
