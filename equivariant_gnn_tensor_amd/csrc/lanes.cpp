// Concurrent launch lanes: per-device side streams and fork/join events.
#include "lanes.hpp"

namespace etpc {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceLanes {
  std::mutex mu;
  bool tried = false;
  bool ok = false;
  hipStream_t side[kLanes] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kLanes] = {};
  // post stream (its own lock, held for a whole pass)
  std::mutex post_mu;
  bool post_tried = false;
  bool post_ok = false;
  hipStream_t post = nullptr;
  hipEvent_t post_follow = nullptr;
  hipEvent_t post_slot[2] = {};
  hipEvent_t post_ready[2] = {};
  hipEvent_t post_join = nullptr;
  hipEvent_t post_part[PostStream::kPostParts] = {};
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

// Lazily creates the post stream and its events; holds dl.post_mu.
bool ensure_post(DeviceLanes& dl) {
  if (dl.post_tried) return dl.post_ok;
  dl.post_tried = true;
  bool ok = hipStreamCreateWithFlags(&dl.post, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&dl.post_follow, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&dl.post_join, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < 2; ++i)
    ok = hipEventCreateWithFlags(&dl.post_slot[i], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&dl.post_ready[i], hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < PostStream::kPostParts; ++i)
    ok = hipEventCreateWithFlags(&dl.post_part[i], hipEventDisableTiming) == hipSuccess;
  dl.post_ok = ok;
  return ok;
}

}  // namespace

LaneGroup::LaneGroup(hipStream_t main, int n) : main_(main) {
  n_ = n < 1 ? 1 : (n > kLanes ? kLanes : n);
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

hipError_t LaneGroup::signal(hipStream_t target) {
  if (!forked_ || done_ || err_ != hipSuccess) return err_;
  for (int i = 0; i < n_ && err_ == hipSuccess; ++i) {
    err_ = hipEventRecord(join_[i], side_[i]);
    if (err_ == hipSuccess) err_ = hipStreamWaitEvent(target, join_[i], 0);
  }
  return err_;
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

PostStream::PostStream(hipStream_t main, bool enable) : main_(main) {
  if (!enable) return;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  DeviceLanes& dl = g_dev[dev];
  lock_ = std::unique_lock<std::mutex>(dl.post_mu);
  if (!ensure_post(dl)) {
    lock_.unlock();
    return;
  }
  post_ = dl.post;
  follow_ev_ = dl.post_follow;
  slot_ev_[0] = dl.post_slot[0];
  slot_ev_[1] = dl.post_slot[1];
  ready_ev_[0] = dl.post_ready[0];
  ready_ev_[1] = dl.post_ready[1];
  join_ev_ = dl.post_join;
  for (int i = 0; i < kPostParts; ++i) part_ev_[i] = dl.post_part[i];
  on_ = true;
}

hipError_t PostStream::follow() {
  if (!on_ || err_ != hipSuccess) return err_;
  err_ = hipEventRecord(follow_ev_, main_);
  if (err_ == hipSuccess) err_ = hipStreamWaitEvent(post_, follow_ev_, 0);
  return err_;
}

hipError_t PostStream::mark(int slot) {
  if (!on_ || err_ != hipSuccess) return err_;
  err_ = hipEventRecord(slot_ev_[slot & 1], post_);
  if (err_ == hipSuccess) marked_[slot & 1] = true;
  return err_;
}

hipError_t PostStream::wait_slot(int slot) {
  if (!on_ || err_ != hipSuccess || !marked_[slot & 1]) return err_;
  err_ = hipStreamWaitEvent(main_, slot_ev_[slot & 1], 0);
  return err_;
}

hipError_t PostStream::ready(int slot) {
  if (!on_ || err_ != hipSuccess) return err_;
  err_ = hipEventRecord(ready_ev_[slot & 1], post_);
  if (err_ == hipSuccess) readied_[slot & 1] = true;
  return err_;
}

hipError_t PostStream::wait_ready(int slot) {
  if (!on_ || err_ != hipSuccess || !readied_[slot & 1]) return err_;
  err_ = hipStreamWaitEvent(main_, ready_ev_[slot & 1], 0);
  return err_;
}

hipError_t PostStream::wait_slot_on(hipStream_t st, int slot) {
  if (!on_ || err_ != hipSuccess || !marked_[slot & 1]) return err_;
  err_ = hipStreamWaitEvent(st, slot_ev_[slot & 1], 0);
  return err_;
}

hipError_t PostStream::wait_ready_on(hipStream_t st, int slot) {
  if (!on_ || err_ != hipSuccess || !readied_[slot & 1]) return err_;
  err_ = hipStreamWaitEvent(st, ready_ev_[slot & 1], 0);
  return err_;
}

hipError_t PostStream::mark_part(int i) {
  if (!on_ || err_ != hipSuccess || i < 0 || i >= kPostParts) return err_;
  err_ = hipEventRecord(part_ev_[i], post_);
  if (err_ == hipSuccess) part_marked_[i] = true;
  return err_;
}

hipError_t PostStream::wait_part(hipStream_t st, int i) {
  if (!on_ || err_ != hipSuccess || i < 0 || i >= kPostParts || !part_marked_[i]) return err_;
  err_ = hipStreamWaitEvent(st, part_ev_[i], 0);
  return err_;
}

hipError_t PostStream::finish() {
  if (done_) return err_;
  done_ = true;
  if (on_) {
    hipError_t e = hipEventRecord(join_ev_, post_);
    if (e == hipSuccess) e = hipStreamWaitEvent(main_, join_ev_, 0);
    if (e != hipSuccess && err_ == hipSuccess) err_ = e;
  }
  if (lock_.owns_lock()) lock_.unlock();
  return err_;
}

PostStream::~PostStream() { (void)finish(); }

}  // namespace etpc
