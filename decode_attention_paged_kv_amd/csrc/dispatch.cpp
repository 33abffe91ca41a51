// dispatch.cpp -- decode kernel selection.
#include "pa_dispatch.h"

namespace pa {

hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st) {
  if (gqa_supported(a)) return launch_decode_gqa(a, st);
  if (mla_supported(a)) return launch_decode_mla(a, st);
  return launch_decode_generic(a, st);
}

KernelChoice choose_kernel(const DecodeArgs& a) {
  const int g = a.hq / a.hkv;
  if (gqa_supported(a)) return {a.hkv * ((g + 15) / 16), gqa_workgroups_per_cu(a.dk, a.kv_dtype), false};
  if (mla_supported(a)) return {a.hkv, mla_workgroups_per_cu(), true};
  return {a.hkv * ((g + 15) / 16), generic_workgroups_per_cu(a.dtype, a.kv_dtype), false};
}

}  // namespace pa
