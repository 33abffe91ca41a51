// pa_dispatch.h -- choice of decode kernel for a call (internal).
#pragma once

#include "pa_launch.h"

namespace pa {

// Runs the fastest kernel that supports the call's shape; the generic kernel
// supports every shape the ABI accepts.
hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st);

// Which kernel dispatch_decode runs for a shape, how many workgroups it launches per
// (sequence x shard, partition), and how many fit on one compute unit at once (0 when the
// runtime cannot tell, e.g. without a GPU).
struct KernelChoice {
  int units_per_partition;
  int workgroups_per_cu;
  bool persistent;   // a resident grid deals the units round-robin (else one per workgroup)
};
KernelChoice choose_kernel(const DecodeArgs& a);

}  // namespace pa
