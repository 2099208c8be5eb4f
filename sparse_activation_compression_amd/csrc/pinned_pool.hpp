// pinned_pool.hpp -- reusable pinned host buffers for the small per-call
// arrays of the offload and prefetch pipelines (chunk sizes).
#pragma once

#include <stddef.h>

namespace cdma {

// A pinned, device-accessible host buffer of at least `bytes` bytes, taken
// from a process-wide pool: buffers are allocated on first need and handed
// out again after they are released, so repeated calls do no hipHostMalloc.
// The pool keeps its buffers until the process ends.  Returns nullptr if an
// allocation fails.  Thread safe.
void* pinned_acquire(size_t bytes);

// Return a buffer from pinned_acquire to the pool (nullptr is ignored).  The
// caller must have finished every copy into or out of it.
void pinned_release(void* p);

}  // namespace cdma
