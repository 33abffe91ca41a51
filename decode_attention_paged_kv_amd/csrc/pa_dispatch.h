// pa_dispatch.h -- choice of decode kernel for a call (internal).
#pragma once

#include "pa_launch.h"

namespace pa {

// Runs the fastest kernel that supports the call's shape; the generic kernel
// supports every shape the ABI accepts.
hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st);

}  // namespace pa
