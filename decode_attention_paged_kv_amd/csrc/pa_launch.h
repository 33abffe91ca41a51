// pa_launch.h -- host-side launchers of the kernels (internal to the library).
// The C ABI in pa_api.cpp validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;  // NULL: value = first dv entries of the key row
  const int32_t* block_table;
  const int32_t* context_lens;
  int n_seqs, hq, hkv, dk, dv, bs;
  int64_t n_blocks;
  int max_blocks, n_shards, interleave, part_tokens, max_parts;
  float scale;
  int dtype;
  float* part_out;
  float* part_lse;
  int* flag;
  int kv_dtype;            // cache element type: dtype, or kFP8 (E4M3 codes)
  const float* k_scale;    // kFP8: value = code * scale, per KV head (n_scales ==
  const float* v_scale;    //   hkv) or per tensor (n_scales == 1); NULL otherwise
  int n_scales;
  // several new tokens per sequence: q rows query_start[b] .. query_start[b+1]-1 are
  // sequence b's last tokens, each attending causally; NULL: one row per sequence.
  const int32_t* query_start;
  int max_q;               // grid bound on new tokens per sequence (1 when query_start NULL)
  int n_rows;              // q rows (n_seqs when query_start NULL)
  // The step's append, done by the decode launch (fused_append in pa_append.h): row b of
  // k_new/v_new (element type new_dtype) is sequence b's new token, stored into its slot
  // before it is read; its slot goes to slots_out[b] when that is non-NULL.  k_new NULL:
  // no append.
  const void* k_new;
  const void* v_new;
  int new_dtype;
  int64_t* slots_out;
};

// The library's fixed partials array on the current device (step_static.hip): its device
// address, taken once per device; kStaticScratchBytes is its size.
constexpr size_t kStaticScratchBytes = PA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(char** out);

hipError_t launch_slot_mapping(const int32_t* bt, const int32_t* lens, int n_seqs, int S, int I,
                               int bs, int max_blocks, int64_t n_blocks, int64_t* slots, int* flag,
                               hipStream_t st);
hipError_t launch_slot_mapping_multi(const int32_t* bt, const int32_t* lens, const int32_t* qstart,
                                     int n_seqs, int S, int I, int bs, int max_blocks,
                                     int64_t n_blocks, int n_rows, int64_t* slots, int* flag,
                                     hipStream_t st);
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int64_t* slots, int n_tokens, int hkv, int dk, int dv, int bs,
                            int64_t n_blocks, int dtype, int* flag, hipStream_t st);
hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, int new_dtype,
                                uint8_t* k_cache, uint8_t* v_cache, const float* k_scale,
                                const float* v_scale, int n_scales, const int64_t* slots,
                                int n_tokens, int hkv, int dk, int dv, int bs, int64_t n_blocks,
                                int* flag, hipStream_t st);
// Routing and append in one launch (one new token per sequence); slots_out may be null.
hipError_t launch_kv_append_routed(const void* k_new, const void* v_new, int new_dtype,
                                   void* k_cache, void* v_cache, int cache_dtype,
                                   const float* k_scale, const float* v_scale, int n_scales,
                                   const int32_t* bt, const int32_t* lens, int n_seqs, int S, int I,
                                   int max_blocks, int hkv, int dk, int dv, int bs,
                                   int64_t n_blocks, int64_t* slots_out, int* flag,
                                   hipStream_t st);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int n_pairs,
                              int64_t k_bytes, int64_t v_bytes, int64_t n_blocks, int* flag,
                              hipStream_t st);
hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* bt_row,
                         int L_r, int hkv, int dk, int dv, int bs, int64_t n_blocks,
                         int max_blocks, int dtype, void* k_out, void* v_out, int* flag,
                         hipStream_t st);
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st);
bool gqa_supported(const DecodeArgs& a);
int gqa_column_chunks(const DecodeArgs& a);     // workgroups per (partition, pair, KV head)
int generic_column_chunks(const DecodeArgs& a);
hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st);
bool mla_supported(const DecodeArgs& a);
int mla_units_per_partition(const DecodeArgs& a);   // (new token, head group, KV head) units
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st);
int gqa_workgroups_per_cu(const DecodeArgs& a);
int mla_workgroups_per_cu(int kv_dtype);
int generic_workgroups_per_cu(int dtype, int kv_dtype);
hipError_t launch_merge(const float* part_out, const float* part_lse, int n_seqs, int n_parts,
                        int hq, int dv, void* out, int out_dtype, float* lse, hipStream_t st);

}  // namespace pa
