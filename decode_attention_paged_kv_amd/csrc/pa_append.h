// pa_append.h -- storing a new token's key/value rows into its cache slot (device side).
//
// A decode step stores the new token's key and value rows before the attention reads
// them (qiita.com/systemdesignsimple "KV cache and continuous batching", section "What
// does the KV cache hold?").  The rows are copied bit for bit, or, for an E4M3 cache,
// quantised with the KV head's scale (soroban.highreso.jp, DCP page, the passage that
// sets DCP beside KV-cache quantisation).  Used by the append kernels and by the decode
// kernels, which can perform a step's append themselves (fused_append).
#pragma once

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

// Slot of sequence b's new token, the last of its L context tokens (global position
// L - 1): its shard and local index by the interleave rule, its block through that
// shard's table row.  -1 for an empty sequence or an unusable table entry (flagged).
__device__ inline int64_t new_token_slot(const int32_t* __restrict__ bt, int L, int b, int S, int I,
                                         int bs, int max_blocks, int64_t n_blocks, int* flag) {
  if (L <= 0) return -1;
  const int i = L - 1;
  const int r = shard_of(i, S, I);
  const int t = local_index(i, S, I);
  const int32_t* row = bt + (int64_t(b) * S + r) * max_blocks;
  const int64_t phys = table_block(row, t / bs, max_blocks, n_blocks, flag);
  return phys >= 0 ? phys * bs + t % bs : -1;
}

// Row n, KV head h of the new keys/values into slot `slot` (a valid one), bit for bit.
template <typename RAW>
__device__ inline void append_row(const RAW* __restrict__ k_new, const RAW* __restrict__ v_new,
                                  RAW* __restrict__ k_cache, RAW* __restrict__ v_cache, int n, int h,
                                  int64_t slot, int hkv, int dk, int dv, int bs) {
  const int64_t blk = slot / bs;
  const int off = int(slot % bs);
  const RAW* ks = k_new + (int64_t(n) * hkv + h) * dk;
  RAW* kd = k_cache + key_row(blk, h, hkv, bs, off, dk);
  for (int e = threadIdx.x; e < dk; e += blockDim.x) kd[e] = ks[e];
  if (v_cache != nullptr) {
    const RAW* vs = v_new + (int64_t(n) * hkv + h) * dv;
    RAW* vd = v_cache + value_tile(blk, h, hkv, bs, dv) + off;
    for (int d = threadIdx.x; d < dv; d += blockDim.x) vd[int64_t(d) * bs] = vs[d];
  }
}

// E4M3 cache: each element of the new rows becomes the code of element / scale (the
// scale of its KV head, or the tensor's), rounded as f32_to_e4m3 describes.  The
// division is IEEE (correctly rounded), so the code is a function of the inputs alone.
template <int DT>
__device__ inline void append_row_fp8(const typename Elem<DT>::raw* __restrict__ k_new,
                                      const typename Elem<DT>::raw* __restrict__ v_new,
                                      uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                      const float* __restrict__ k_scale,
                                      const float* __restrict__ v_scale, int n_scales, int n, int h,
                                      int64_t slot, int hkv, int dk, int dv, int bs) {
  using E = Elem<DT>;
  const int64_t blk = slot / bs;
  const int off = int(slot % bs);
  const int si = n_scales > 1 ? h : 0;
  const float ks = k_scale[si];
  const int64_t ksrc = (int64_t(n) * hkv + h) * dk;
  uint8_t* kd = k_cache + key_row(blk, h, hkv, bs, off, dk);
  for (int e = threadIdx.x; e < dk; e += blockDim.x) kd[e] = f32_to_e4m3(__fdiv_rn(E::load(k_new, ksrc + e), ks));
  if (v_cache != nullptr) {
    const float vs = v_scale[si];
    const int64_t vsrc = (int64_t(n) * hkv + h) * dv;
    uint8_t* vd = v_cache + value_tile(blk, h, hkv, bs, dv) + off;
    for (int d = threadIdx.x; d < dv; d += blockDim.x)
      vd[int64_t(d) * bs] = f32_to_e4m3(__fdiv_rn(E::load(v_new, vsrc + d), vs));
  }
}

// The append a decode launch performs itself (DecodeArgs::k_new set, one new token per
// sequence).  Sequence b's new token is its last context token, global position L - 1:
// shard r0 = shard_of(L - 1), local index t.  The workgroup that reads shard r0's
// partition t / part_tokens for KV head h stores the token's rows first, exactly as the
// routed append does, and makes them visible to its own reads (the stores complete,
// then a barrier);
// no other workgroup reads that slot, so none sees it half written.  Requires one
// workgroup per (partition, KV head), which the dispatcher checks.  Called by every thread
// of the workgroup with the same arguments.
__device__ inline void fused_append(const DecodeArgs& a, int b, int r, int p, int h) {
  if (a.k_new == nullptr) return;
  const int L = a.context_lens[b];
  if (L <= 0) {   // no new token: slot -1, recorded once
    if (a.slots_out && p == 0 && r == 0 && h == 0 && threadIdx.x == 0) a.slots_out[b] = -1;
    return;
  }
  const int pos = L - 1;
  if (shard_of(pos, a.n_shards, a.interleave) != r ||
      local_index(pos, a.n_shards, a.interleave) / a.part_tokens != p)
    return;
  // table errors are reported by the decode's own reads of this entry
  const int64_t slot = new_token_slot(a.block_table, L, b, a.n_shards, a.interleave, a.bs,
                                      a.max_blocks, a.n_blocks, nullptr);
  if (a.slots_out && h == 0 && threadIdx.x == 0) a.slots_out[b] = slot;
  if (slot >= 0) {
    if (a.kv_dtype == kFP8) {
      uint8_t* kc = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
      uint8_t* vc = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
      if (a.new_dtype == kF32)
        append_row_fp8<kF32>(static_cast<const uint32_t*>(a.k_new), static_cast<const uint32_t*>(a.v_new),
                             kc, vc, a.k_scale, a.v_scale, a.n_scales, b, h, slot, a.hkv, a.dk, a.dv, a.bs);
      else
        append_row_fp8<kBF16>(static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
                              kc, vc, a.k_scale, a.v_scale, a.n_scales, b, h, slot, a.hkv, a.dk, a.dv, a.bs);
    } else if (a.kv_dtype == kF32) {
      append_row(static_cast<const uint32_t*>(a.k_new), static_cast<const uint32_t*>(a.v_new),
                 static_cast<uint32_t*>(const_cast<void*>(a.k_cache)),
                 static_cast<uint32_t*>(const_cast<void*>(a.v_cache)), b, h, slot, a.hkv, a.dk, a.dv, a.bs);
    } else {
      append_row(static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
                 static_cast<uint16_t*>(const_cast<void*>(a.k_cache)),
                 static_cast<uint16_t*>(const_cast<void*>(a.v_cache)), b, h, slot, a.hkv, a.dk, a.dv, a.bs);
    }
  }
  // Only this workgroup reads the slot, so the stores need no device-scope release or
  // acquire (on this GPU those write back or invalidate the L2): each wave waits until
  // its stores are complete in L2, and the waves meet.  The compute unit's L1 holds no
  // line of the slot (no workgroup has read the block in this launch), so the reads that
  // follow miss it and see the stored rows.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0); expcnt and lgkmcnt not waited for
  __syncthreads();
}

// The same append in two halves, for a decode kernel that issues its own first loads in
// between.  append_fetch reads this thread's share of sequence b's new rows for KV head h
// -- key element threadIdx.x and value element threadIdx.x, so dk and dv must not exceed
// the workgroup size -- before anything is known about the sequence.  append_store then
// does what fused_append does after its reads: it decides from the context length L
// whether this workgroup's partition holds the new token, takes the token's block from
// entry(j), the raw table value of entry j (j < max_blocks), stores the rows (quantised
// for an E4M3 cache), waits for the stores and meets the workgroup.  Both are called by
// every thread of the workgroup with the same arguments.
struct NewRowShare {
  uint32_t k = 0, v = 0;   // raw bits of one key and one value element
};

__device__ inline NewRowShare append_fetch(const DecodeArgs& a, int b, int h) {
  NewRowShare s;
  if (a.k_new == nullptr) return s;
  const int t = threadIdx.x;
  const int nd = a.kv_dtype == kFP8 ? a.new_dtype : a.kv_dtype;   // element type of the new rows
  const int64_t kr = (int64_t(b) * a.hkv + h) * a.dk, vr = (int64_t(b) * a.hkv + h) * a.dv;
  if (nd == kF32) {
    if (t < a.dk) s.k = static_cast<const uint32_t*>(a.k_new)[kr + t];
    if (a.v_cache != nullptr && t < a.dv) s.v = static_cast<const uint32_t*>(a.v_new)[vr + t];
  } else {
    if (t < a.dk) s.k = static_cast<const uint16_t*>(a.k_new)[kr + t];
    if (a.v_cache != nullptr && t < a.dv) s.v = static_cast<const uint16_t*>(a.v_new)[vr + t];
  }
  return s;
}

template <typename Entry>
__device__ inline void append_store(const DecodeArgs& a, const NewRowShare& s, int b, int r, int p,
                                    int h, int L, Entry&& entry) {
  if (a.k_new == nullptr) return;
  if (L <= 0) {   // no new token: slot -1, recorded once
    if (a.slots_out && p == 0 && r == 0 && h == 0 && threadIdx.x == 0) a.slots_out[b] = -1;
    return;
  }
  const int pos = L - 1;
  const int t = local_index(pos, a.n_shards, a.interleave);
  if (shard_of(pos, a.n_shards, a.interleave) != r || t / a.part_tokens != p) return;
  // table errors are reported by the decode's own reads of this entry
  const int j = t / a.bs;
  const int e = j < a.max_blocks ? entry(j) : -1;
  const int64_t slot = (e >= 0 && int64_t(e) < a.n_blocks) ? int64_t(e) * a.bs + t % a.bs : -1;
  if (a.slots_out && h == 0 && threadIdx.x == 0) a.slots_out[b] = slot;
  if (slot >= 0) {
    const int off = t % a.bs, tid = threadIdx.x;
    const bool vals = a.v_cache != nullptr && tid < a.dv;
    if (a.kv_dtype == kFP8) {
      const int si = a.n_scales > 1 ? h : 0;
      auto widen = [&](uint32_t x) { return a.new_dtype == kF32 ? __uint_as_float(x) : bf16_bits_to_f32(uint16_t(x)); };
      uint8_t* kc = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
      uint8_t* vc = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
      if (tid < a.dk) kc[key_row(e, h, a.hkv, a.bs, off, a.dk) + tid] = f32_to_e4m3(__fdiv_rn(widen(s.k), a.k_scale[si]));
      if (vals)
        vc[value_tile(e, h, a.hkv, a.bs, a.dv) + int64_t(tid) * a.bs + off] = f32_to_e4m3(__fdiv_rn(widen(s.v), a.v_scale[si]));
    } else if (a.kv_dtype == kF32) {
      uint32_t* kc = static_cast<uint32_t*>(const_cast<void*>(a.k_cache));
      uint32_t* vc = static_cast<uint32_t*>(const_cast<void*>(a.v_cache));
      if (tid < a.dk) kc[key_row(e, h, a.hkv, a.bs, off, a.dk) + tid] = s.k;
      if (vals) vc[value_tile(e, h, a.hkv, a.bs, a.dv) + int64_t(tid) * a.bs + off] = s.v;
    } else {
      uint16_t* kc = static_cast<uint16_t*>(const_cast<void*>(a.k_cache));
      uint16_t* vc = static_cast<uint16_t*>(const_cast<void*>(a.v_cache));
      if (tid < a.dk) kc[key_row(e, h, a.hkv, a.bs, off, a.dk) + tid] = uint16_t(s.k);
      if (vals) vc[value_tile(e, h, a.hkv, a.bs, a.dv) + int64_t(tid) * a.bs + off] = uint16_t(s.v);
    }
  }
  // as in fused_append: the stores complete in L2, then the waves meet
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0); expcnt and lgkmcnt not waited for
  __syncthreads();
}

}  // namespace pa
