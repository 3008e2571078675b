// Optional per-kernel timing: while enabled for a kernel name, every launch
// of that kernel is bracketed by hipEvents recorded on its launch stream.
#pragma once

#include <hip/hip_runtime.h>

namespace specdec {

// Returns a non-null token when the named kernel is being timed; pass it to
// prof_end after the launch.
void* prof_begin(const char* kernel, hipStream_t s);
void prof_end(void* token, hipStream_t s);

}  // namespace specdec
