// kv_ops.hip -- slot routing, kv append, block copies and the block-table gather.
//
// kv append: a decode step stores the new token's key and value rows before the
// attention reads them (qiita.com/systemdesignsimple "KV cache and continuous
// batching", section "What does the KV cache hold?").  The copy is of raw bits, so it
// is exact for any element type.
// Slot routing and gather: placement by the DCP interleave rule and block-table
// lookup, as in pa_common.h.
// E4M3 append: the KV cache may be kept in an 8-bit floating type to take fewer bytes
// per token (soroban.highreso.jp, DCP page, the passage that sets DCP beside KV-cache
// quantisation); new rows are quantised with a scale on the way in.
// Block copy: a sequence about to write into a block it shares with others first
// gets a private copy of that block (ai-compass.weeybrid.co.jp, "What is
// PagedAttention?", section "Sharing common blocks and copy-on-write").
#include <algorithm>

#include "pa_append.h"
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

__global__ void slot_mapping_kernel(const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
                                    int n_seqs, int S, int I, int bs, int max_blocks,
                                    int64_t n_blocks, int64_t* __restrict__ slots, int* flag) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_seqs) return;
  slots[b] = new_token_slot(bt, lens[b], b, S, I, bs, max_blocks, n_blocks, flag);
}

// Slots of several new tokens per sequence: new token i of the last n sits at global
// position L - n + i and is placed like any token (rows of the packed query order).
// More new tokens than context tokens: the slots are -1 and the flag is raised; rows
// outside [0, n_rows) are never written (flag raised).
__global__ void slot_mapping_multi_kernel(const int32_t* __restrict__ bt,
                                          const int32_t* __restrict__ lens,
                                          const int32_t* __restrict__ qstart, int n_seqs, int S,
                                          int I, int bs, int max_blocks, int64_t n_blocks,
                                          int n_rows, int64_t* __restrict__ slots, int* flag) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_seqs) return;
  const int L = lens[b];
  const int row0 = qstart[b];
  const int n = qstart[b + 1] - row0;
  if (row0 < 0 || n < 0 || row0 + n > n_rows) {
    raise_flag(flag, kErrCapacity);
    return;
  }
  const bool bad = n > L;
  if (bad) raise_flag(flag, kErrCapacity);
  for (int i = 0; i < n; ++i) {
    int64_t slot = -1;
    if (!bad) {
      const int pos = L - n + i;
      const int r = shard_of(pos, S, I);
      const int t = local_index(pos, S, I);
      const int32_t* row = bt + (int64_t(b) * S + r) * max_blocks;
      const int64_t phys = table_block(row, t / bs, max_blocks, n_blocks, flag);
      if (phys >= 0) slot = phys * bs + t % bs;
    }
    slots[row0 + i] = slot;
  }
}

template <typename RAW>
__global__ void kv_append_kernel(const RAW* __restrict__ k_new, const RAW* __restrict__ v_new,
                                 RAW* __restrict__ k_cache, RAW* __restrict__ v_cache,
                                 const int64_t* __restrict__ slots, int hkv, int dk, int dv, int bs,
                                 int64_t n_blocks, int* flag) {
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = slots[n];
  if (slot < 0) return;
  if (slot >= n_blocks * bs) {
    if (threadIdx.x == 0) raise_flag(flag, kErrSlot);
    return;
  }
  append_row(k_new, v_new, k_cache, v_cache, n, h, slot, hkv, dk, dv, bs);
}

template <int DT>
__global__ void kv_append_fp8_kernel(const void* __restrict__ k_new_, const void* __restrict__ v_new_,
                                     uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                     const float* __restrict__ k_scale,
                                     const float* __restrict__ v_scale, int n_scales,
                                     const int64_t* __restrict__ slots, int hkv, int dk, int dv,
                                     int bs, int64_t n_blocks, int* flag) {
  using raw = typename Elem<DT>::raw;
  const raw* k_new = static_cast<const raw*>(k_new_);
  const raw* v_new = static_cast<const raw*>(v_new_);
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t slot = slots[n];
  if (slot < 0) return;
  if (slot >= n_blocks * bs) {
    if (threadIdx.x == 0) raise_flag(flag, kErrSlot);
    return;
  }
  append_row_fp8<DT>(k_new, v_new, k_cache, v_cache, k_scale, v_scale, n_scales, n, h, slot, hkv,
                     dk, dv, bs);
}

// One launch for a decode step's append: workgroup (b, h) finds sequence b's new-token
// slot as slot_mapping_kernel does (optionally recording it) and writes that token's
// rows of KV head h as kv_append_kernel / kv_append_fp8_kernel do.  F8: an E4M3 cache
// (rows of element type DT quantised); otherwise a plain copy of DT rows.
template <int DT, bool F8>
__global__ void kv_append_routed_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
                                        void* __restrict__ k_cache, void* __restrict__ v_cache,
                                        const float* __restrict__ k_scale,
                                        const float* __restrict__ v_scale, int n_scales,
                                        const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
                                        int S, int I, int max_blocks, int hkv, int dk, int dv, int bs,
                                        int64_t n_blocks, int64_t* __restrict__ slots_out, int* flag) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  __shared__ int64_t slot_s;
  if (threadIdx.x == 0) {
    // every KV head's workgroup resolves the slot; only head 0's reports table errors
    const int64_t slot =
        new_token_slot(bt, lens[b], b, S, I, bs, max_blocks, n_blocks, h == 0 ? flag : nullptr);
    slot_s = slot;
    if (h == 0 && slots_out != nullptr) slots_out[b] = slot;
  }
  __syncthreads();
  const int64_t slot = slot_s;
  if (slot < 0) return;
  using raw = typename Elem<DT>::raw;
  if constexpr (F8)
    append_row_fp8<DT>(static_cast<const raw*>(k_new), static_cast<const raw*>(v_new),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale,
                       v_scale, n_scales, b, h, slot, hkv, dk, dv, bs);
  else
    append_row(static_cast<const raw*>(k_new), static_cast<const raw*>(v_new),
               static_cast<raw*>(k_cache), static_cast<raw*>(v_cache), b, h, slot, hkv, dk, dv, bs);
}

template <typename RAW>
__global__ void gather_kernel(const RAW* __restrict__ k_cache, const RAW* __restrict__ v_cache,
                              const int32_t* __restrict__ row, int hkv, int dk, int dv, int bs,
                              int64_t n_blocks, int max_blocks, RAW* __restrict__ k_out,
                              RAW* __restrict__ v_out, int* flag) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  __shared__ int64_t phys_s;
  if (threadIdx.x == 0) phys_s = table_block(row, t / bs, max_blocks, n_blocks, flag);
  __syncthreads();
  const int64_t phys = phys_s;
  if (phys < 0) return;
  const int off = t % bs;
  const RAW* ks = k_cache + key_row(phys, h, hkv, bs, off, dk);
  RAW* kd = k_out + (int64_t(t) * hkv + h) * dk;
  for (int e = threadIdx.x; e < dk; e += blockDim.x) kd[e] = ks[e];
  RAW* vd = v_out + (int64_t(t) * hkv + h) * dv;
  if (v_cache != nullptr) {
    const RAW* vs = v_cache + value_tile(phys, h, hkv, bs, dv) + off;
    for (int d = threadIdx.x; d < dv; d += blockDim.x) vd[d] = vs[int64_t(d) * bs];
  } else {
    for (int d = threadIdx.x; d < dv; d += blockDim.x) vd[d] = ks[d];
  }
}

// Block copy for copy-on-write: blockIdx.x is the pair, blockIdx.z the tensor (0 = keys,
// 1 = values); the workgroups along y share the block's bytes in W-sized words.  A block
// of one tensor is contiguous (all KV heads of one physical block), so the copy is a
// plain contiguous move with coalesced loads and stores.
template <typename W>
__global__ void copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                   const int64_t* __restrict__ pairs, int64_t k_words,
                                   int64_t v_words, int64_t n_blocks, int* flag) {
  const int64_t i = blockIdx.x;
  const int64_t src = pairs[2 * i];
  const int64_t dst = pairs[2 * i + 1];
  if (src < 0 || src >= n_blocks || dst < 0 || dst >= n_blocks) {
    if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) raise_flag(flag, kErrBlockId);
    return;
  }
  if (src == dst) return;
  const bool values = blockIdx.z != 0;
  const int64_t words = values ? v_words : k_words;
  W* base = reinterpret_cast<W*>(values ? v_cache : k_cache);
  const W* s = base + src * words;
  W* d = base + dst * words;
  const int64_t stride = int64_t(gridDim.y) * blockDim.x;
  for (int64_t e = int64_t(blockIdx.y) * blockDim.x + threadIdx.x; e < words; e += stride)
    d[e] = s[e];
}

}  // namespace

hipError_t launch_kv_append_fp8(const void* k_new, const void* v_new, int new_dtype,
                                uint8_t* k_cache, uint8_t* v_cache, const float* k_scale,
                                const float* v_scale, int n_scales, const int64_t* slots,
                                int n_tokens, int hkv, int dk, int dv, int bs, int64_t n_blocks,
                                int* flag, hipStream_t st) {
  const dim3 grid(n_tokens, hkv);
  if (new_dtype == kF32)
    hipLaunchKernelGGL(kv_append_fp8_kernel<kF32>, grid, dim3(64), 0, st, k_new, v_new, k_cache,
                       v_cache, k_scale, v_scale, n_scales, slots, hkv, dk, dv, bs, n_blocks, flag);
  else
    hipLaunchKernelGGL(kv_append_fp8_kernel<kBF16>, grid, dim3(64), 0, st, k_new, v_new, k_cache,
                       v_cache, k_scale, v_scale, n_scales, slots, hkv, dk, dv, bs, n_blocks, flag);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int n_pairs,
                              int64_t k_bytes, int64_t v_bytes, int64_t n_blocks, int* flag,
                              hipStream_t st) {
  // Widest word that divides both tensors' block sizes and both base addresses.
  uint64_t bits = uint64_t(k_bytes) | uint64_t(reinterpret_cast<uintptr_t>(k_cache));
  if (v_cache != nullptr) bits |= uint64_t(v_bytes) | uint64_t(reinterpret_cast<uintptr_t>(v_cache));
  const int word = (bits % 16 == 0) ? 16 : (bits % 8 == 0) ? 8 : (bits % 4 == 0) ? 4 : (bits % 2 == 0) ? 2 : 1;
  const int threads = 256;
  const int64_t biggest = std::max(k_bytes, v_cache != nullptr ? v_bytes : int64_t(0)) / word;
  const int64_t split = std::min<int64_t>((biggest + threads - 1) / threads, 64);
  const dim3 grid(n_pairs, unsigned(std::max<int64_t>(split, 1)), v_cache != nullptr ? 2 : 1);
  char* k = static_cast<char*>(k_cache);
  char* v = static_cast<char*>(v_cache);
  const int64_t kw = k_bytes / word, vw = v_bytes / word;
  switch (word) {
    case 16: hipLaunchKernelGGL(copy_blocks_kernel<uint4>, grid, dim3(threads), 0, st, k, v, pairs, kw, vw, n_blocks, flag); break;
    case 8: hipLaunchKernelGGL(copy_blocks_kernel<uint2>, grid, dim3(threads), 0, st, k, v, pairs, kw, vw, n_blocks, flag); break;
    case 4: hipLaunchKernelGGL(copy_blocks_kernel<uint32_t>, grid, dim3(threads), 0, st, k, v, pairs, kw, vw, n_blocks, flag); break;
    case 2: hipLaunchKernelGGL(copy_blocks_kernel<uint16_t>, grid, dim3(threads), 0, st, k, v, pairs, kw, vw, n_blocks, flag); break;
    default: hipLaunchKernelGGL(copy_blocks_kernel<uint8_t>, grid, dim3(threads), 0, st, k, v, pairs, kw, vw, n_blocks, flag); break;
  }
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* bt, const int32_t* lens, int n_seqs, int S, int I,
                               int bs, int max_blocks, int64_t n_blocks, int64_t* slots, int* flag,
                               hipStream_t st) {
  const int threads = 256;
  const int blocks = (n_seqs + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, st, bt, lens, n_seqs, S,
                     I, bs, max_blocks, n_blocks, slots, flag);
  return hipGetLastError();
}

hipError_t launch_slot_mapping_multi(const int32_t* bt, const int32_t* lens, const int32_t* qstart,
                                     int n_seqs, int S, int I, int bs, int max_blocks,
                                     int64_t n_blocks, int n_rows, int64_t* slots, int* flag,
                                     hipStream_t st) {
  const int threads = 256;
  const int blocks = (n_seqs + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_multi_kernel, dim3(blocks), dim3(threads), 0, st, bt, lens, qstart,
                     n_seqs, S, I, bs, max_blocks, n_blocks, n_rows, slots, flag);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int64_t* slots, int n_tokens, int hkv, int dk, int dv, int bs,
                            int64_t n_blocks, int dtype, int* flag, hipStream_t st) {
  const dim3 grid(n_tokens, hkv);
  if (dtype == kF32) {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(64), 0, st,
                       (const uint32_t*)k_new, (const uint32_t*)v_new, (uint32_t*)k_cache,
                       (uint32_t*)v_cache, slots, hkv, dk, dv, bs, n_blocks, flag);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(64), 0, st,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, slots, hkv, dk, dv, bs, n_blocks, flag);
  }
  return hipGetLastError();
}

hipError_t launch_kv_append_routed(const void* k_new, const void* v_new, int new_dtype,
                                   void* k_cache, void* v_cache, int cache_dtype,
                                   const float* k_scale, const float* v_scale, int n_scales,
                                   const int32_t* bt, const int32_t* lens, int n_seqs, int S, int I,
                                   int max_blocks, int hkv, int dk, int dv, int bs,
                                   int64_t n_blocks, int64_t* slots_out, int* flag,
                                   hipStream_t st) {
  const dim3 grid(n_seqs, hkv);
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(64), 0, st, k_new, v_new, k_cache, v_cache, k_scale,
                       v_scale, n_scales, bt, lens, S, I, max_blocks, hkv, dk, dv, bs, n_blocks,
                       slots_out, flag);
  };
  if (cache_dtype == kFP8)
    new_dtype == kF32 ? go(kv_append_routed_kernel<kF32, true>) : go(kv_append_routed_kernel<kBF16, true>);
  else
    cache_dtype == kF32 ? go(kv_append_routed_kernel<kF32, false>) : go(kv_append_routed_kernel<kBF16, false>);
  return hipGetLastError();
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, const int32_t* bt_row,
                         int L_r, int hkv, int dk, int dv, int bs, int64_t n_blocks,
                         int max_blocks, int dtype, void* k_out, void* v_out, int* flag,
                         hipStream_t st) {
  const dim3 grid(L_r, hkv);
  if (dtype == kFP8) {
    hipLaunchKernelGGL(gather_kernel<uint8_t>, grid, dim3(64), 0, st, (const uint8_t*)k_cache,
                       (const uint8_t*)v_cache, bt_row, hkv, dk, dv, bs, n_blocks, max_blocks,
                       (uint8_t*)k_out, (uint8_t*)v_out, flag);
  } else if (dtype == kF32) {
    hipLaunchKernelGGL(gather_kernel<uint32_t>, grid, dim3(64), 0, st, (const uint32_t*)k_cache,
                       (const uint32_t*)v_cache, bt_row, hkv, dk, dv, bs, n_blocks, max_blocks,
                       (uint32_t*)k_out, (uint32_t*)v_out, flag);
  } else {
    hipLaunchKernelGGL(gather_kernel<uint16_t>, grid, dim3(64), 0, st, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, bt_row, hkv, dk, dv, bs, n_blocks, max_blocks,
                       (uint16_t*)k_out, (uint16_t*)v_out, flag);
  }
  return hipGetLastError();
}

}  // namespace pa
