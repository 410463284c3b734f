// Concurrent launch lanes (internal).
//
// The per-path traversal launches of one pass are independent of each other (disjoint
// state columns, or separate per-lane copies of what they accumulate).  Launched one
// after another on one stream, every launch ends with a tail in which most compute units
// idle; spread over a few side streams, the next launch fills that tail.  A LaneGroup
// forks n side streams off the caller's stream (event record + wait) and joins them back
// on finish.  The side streams belong to the library (one set per device, default
// priority); groups from different host threads are serialized by a lock held from
// fork to join, which covers only enqueue calls.
#pragma once

#include <mutex>

#include "common.hpp"

namespace etpc {

// Two lanes measured best on MI355X (one launch's tail filled by the next; more lanes
// contend for the four hardware queues of the process).
#ifndef ETPC_LANES
#define ETPC_LANES 2
#endif
constexpr int kLanes = ETPC_LANES;

// Process-wide lane limit in [1, kLanes] (etpc_set_lanes); 1 serializes every launch on
// the caller's stream, e.g. to time kernels one at a time.
int lanes_limit();
void set_lanes_limit(int n);

class LaneGroup {
 public:
  // n lanes (clamped to [1, lanes_limit()]); with n == 1, or if the side streams cannot
  // be created, every lane is the caller's stream itself.
  LaneGroup(hipStream_t main, int n);
  ~LaneGroup();
  LaneGroup(const LaneGroup&) = delete;
  LaneGroup& operator=(const LaneGroup&) = delete;

  int size() const { return n_; }
  hipStream_t lane(int i) const { return forked_ ? side_[i % n_] : main_; }
  // Joins the lanes back into the caller's stream (idempotent).
  hipError_t finish();
  hipError_t status() const { return err_; }

 private:
  hipStream_t main_;
  int n_;
  bool forked_ = false;
  bool done_ = false;
  hipError_t err_ = hipSuccess;
  hipStream_t side_[kLanes] = {};
  hipEvent_t join_[kLanes] = {};
  std::unique_lock<std::mutex> lock_;
};

}  // namespace etpc
