// Opt-in kernel timing with HIP events on the launch stream (internal).
#pragma once

#include "common.hpp"

namespace etpc {

// Records an event pair around the enclosed launches when profiling is enabled.
class ProfScope {
 public:
  ProfScope(int kind, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

}  // namespace etpc

#define ETPC_LAUNCH(kind, call)              \
  do {                                       \
    ::etpc::ProfScope _etpc_ps((kind), s);   \
    ETPC_HIP(call);                          \
  } while (0)

// The same for a launch on another stream (a concurrent lane) than the call's `s`.
#define ETPC_LAUNCH_ON(kind, stream, call)        \
  do {                                            \
    ::etpc::ProfScope _etpc_ps((kind), (stream)); \
    ETPC_HIP(call);                               \
  } while (0)
