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

class LaneGroup {
 public:
  // n lanes (clamped to [1, kLanes]; callers pass at most their plan's lane count); with
  // n == 1, or if the side streams cannot be created, every lane is the caller's stream.
  LaneGroup(hipStream_t main, int n);
  ~LaneGroup();
  LaneGroup(const LaneGroup&) = delete;
  LaneGroup& operator=(const LaneGroup&) = delete;

  int size() const { return n_; }
  hipStream_t lane(int i) const { return forked_ ? side_[i % n_] : main_; }
  // Stream `target` waits for everything enqueued on the lanes so far; the lanes stay
  // forked, so a pass can keep them across its work items (a no-op when not forked).
  hipError_t signal(hipStream_t target);
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

// A side stream for the node-side GEMMs of a pass (the channel GEMM of a forward output
// group, the x_bar and W_bar GEMMs of a backward input block), so they run while the
// next group's or block's traversals do.  The pass keeps two sets of the buffers those
// GEMMs read and alternates between them; before its traversals write set b again, the
// caller's stream waits for the post work that last read set b (wait_slot).  Disabled
// (every call a no-op, stream() the caller's stream) when `enable` is false (the plan has
// one lane, or the call is too small to gain from it).  Holds a per-device lock from construction to finish; it is taken
// before any LaneGroup lock of the same call, never after.
class PostStream {
 public:
  PostStream(hipStream_t main, bool enable);
  ~PostStream();
  PostStream(const PostStream&) = delete;
  PostStream& operator=(const PostStream&) = delete;

  hipStream_t stream() const { return on_ ? post_ : main_; }
  // The post stream waits for everything enqueued on the caller's stream so far.
  hipError_t follow();
  // Buffer set `slot` is free again once the post work enqueued so far has run.
  hipError_t mark(int slot);
  // The caller's stream waits until buffer set `slot` is free.
  hipError_t wait_slot(int slot);
  // Buffer set `slot` has been filled by the post work enqueued so far...
  hipError_t ready(int slot);
  // ...and the caller's stream waits for that before reading it.
  hipError_t wait_ready(int slot);
  // wait_slot / wait_ready for another stream `st` (a lane kept across work items)
  hipError_t wait_slot_on(hipStream_t st, int slot);
  hipError_t wait_ready_on(hipStream_t st, int slot);
  // Part `i` (< kPostParts) of the post work has been enqueued so far...
  hipError_t mark_part(int i);
  // ...and stream `st` waits for it (a no-op if part `i` was never marked).
  hipError_t wait_part(hipStream_t st, int i);
  // The caller's stream waits for all post work (idempotent).
  hipError_t finish();
  hipError_t status() const { return err_; }
  bool enabled() const { return on_; }

  static constexpr int kPostParts = 16;

 private:
  hipStream_t main_;
  hipStream_t post_ = nullptr;
  bool on_ = false;
  bool done_ = false;
  bool marked_[2] = {false, false};
  bool readied_[2] = {false, false};
  hipEvent_t follow_ev_ = nullptr;
  hipEvent_t slot_ev_[2] = {nullptr, nullptr};
  hipEvent_t ready_ev_[2] = {nullptr, nullptr};
  hipEvent_t join_ev_ = nullptr;
  hipEvent_t part_ev_[kPostParts] = {};
  bool part_marked_[kPostParts] = {};
  hipError_t err_ = hipSuccess;
  std::unique_lock<std::mutex> lock_;
};

}  // namespace etpc
