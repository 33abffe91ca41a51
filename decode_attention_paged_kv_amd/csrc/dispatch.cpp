// dispatch.cpp -- decode kernel selection.
#include "pa_dispatch.h"

namespace pa {

hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st) {
  if (gqa_supported(a)) return launch_decode_gqa(a, st);
  if (mla_supported(a)) return launch_decode_mla(a, st);
  return launch_decode_generic(a, st);
}

}  // namespace pa
