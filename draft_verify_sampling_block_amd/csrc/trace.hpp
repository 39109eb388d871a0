// Optional per-kernel timing: when enabled, every launch is bracketed by a
// pair of hipEvents on its stream, and dspark_trace_summary() reports the
// count and mean duration per kernel name.  Off by default; costs nothing
// when off beyond one relaxed flag read per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace dspark {

bool trace_on();
// returns a slot id (>= 0) when tracing, -1 otherwise
int trace_begin(const char* name, hipStream_t stream);
void trace_end(int slot, hipStream_t stream);

struct TraceScope {
  int slot;
  hipStream_t stream;
  // name NULL: this launch is never traced
  TraceScope(const char* name, hipStream_t s)
      : slot(name ? trace_begin(name, s) : -1), stream(s) {}
  ~TraceScope() { trace_end(slot, stream); }
};

}  // namespace dspark
