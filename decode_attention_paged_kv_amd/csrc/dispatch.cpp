// dispatch.cpp -- decode kernel selection.
#include "pa_dispatch.h"

namespace pa {

// The decode kernels can store the step's new tokens themselves (fused_append) when each
// (partition, KV head) is read by one workgroup alone and each sequence brings one new
// token; otherwise the append is a launch of its own, ahead of the decode.
static bool append_fusable(const DecodeArgs& a) {
  if (a.query_start != nullptr) return false;
  if (gqa_supported(a)) return gqa_column_chunks(a) == 1;
  if (mla_supported(a)) return mla_units_per_partition(a) == a.hkv;
  return generic_column_chunks(a) == 1;
}

hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.k_new != nullptr && !append_fusable(a)) {
    const hipError_t e = launch_kv_append_routed(
        a.k_new, a.v_new, a.new_dtype, const_cast<void*>(a.k_cache), const_cast<void*>(a.v_cache),
        a.kv_dtype, a.k_scale, a.v_scale, a.n_scales, a.block_table, a.context_lens, a.n_seqs,
        a.n_shards, a.interleave, a.max_blocks, a.hkv, a.dk, a.dv, a.bs, a.n_blocks, a.slots_out,
        a.flag, st);
    if (e != hipSuccess) return e;
    DecodeArgs d = a;
    d.k_new = d.v_new = nullptr;
    d.slots_out = nullptr;
    return dispatch_decode(d, st);
  }
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
