// Optional per-kernel timing with HIP events recorded on the launch stream.
// Off by default; when on, every kernel launch of the library is bracketed by
// two events and the elapsed times are summed per kernel name on read.
#pragma once
#include <hip/hip_runtime.h>

namespace vl {

bool prof_on();
// Returns a slot to pass to prof_end (or -1 when profiling is off).
int prof_begin(const char* kernel, hipStream_t stream);
void prof_end(int slot, hipStream_t stream);

// RAII bracket around one launch.
struct ProfScope {
  int slot;
  hipStream_t stream;
  ProfScope(const char* kernel, hipStream_t s) : slot(prof_on() ? prof_begin(kernel, s) : -1), stream(s) {}
  ~ProfScope() {
    if (slot >= 0) prof_end(slot, stream);
  }
};

}  // namespace vl
