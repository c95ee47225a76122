// Launch bracketing for kvs_trace_* (see trace.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/kvs.h"

namespace kvs {

// Records an event on `st` at construction and another at destruction when
// tracing is on; does nothing otherwise.
class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t st);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  void* a_ = nullptr;
  void* b_ = nullptr;
};

}  // namespace kvs
