// dispatch.cpp -- decode kernel selection.
#include "pa_dispatch.h"

namespace pa {

hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st) {
  if (gqa_supported(a)) return launch_decode_gqa(a, st);
  if (mla_supported(a)) return launch_decode_mla(a, st);
  return launch_decode_generic(a, st);
}

KernelChoice choose_kernel(const DecodeArgs& a) {
  if (gqa_supported(a)) return {a.hkv * gqa_column_chunks(a), gqa_workgroups_per_cu(a), false};
  if (mla_supported(a))   // one unit per (partition, new token, head group, KV head)
    return {mla_units_per_partition(a), mla_workgroups_per_cu(a.kv_dtype), true};
  return {a.hkv * generic_column_chunks(a), generic_workgroups_per_cu(a.dtype, a.kv_dtype), false};
}

}  // namespace pa
