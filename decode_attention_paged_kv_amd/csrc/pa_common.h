// pa_common.h -- device/host helpers shared by the paged decode-attention kernels.
//
// Token placement follows the DCP page (soroban.highreso.jp, "Why long-context LLMs
// get slow: distributing the KV cache with Decode Context Parallelism", DCP mechanism
// section): token i goes to shard (i / I) % S, dealt I tokens at a time.  A shard keeps
// its tokens in global order.  Closed forms used here:
//   local index of token i       : (i / (I*S)) * I + i % I
//   tokens on shard r of length L: c*I + clamp(L - c*I*S - r*I, 0, I),  c = L / (I*S)
// Block addressing follows the PagedAttention page (ai-compass.weeybrid.co.jp, "What is
// PagedAttention?", block-table section): local token t of a shard is in the physical
// block listed at entry t / block_size of that shard's table row, at offset
// t % block_size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };  // kFP8: OCP E4M3 cache codes

constexpr int kMaxHeadDim = 576;
constexpr int kMaxBlockSize = 256;

// ---------------------------------------------------------------- placement math
__host__ __device__ inline int shard_len(int L, int S, int I, int r) {
  const int round = I * S;
  const int c = L / round;
  int extra = L - c * round - r * I;
  extra = extra < 0 ? 0 : (extra > I ? I : extra);
  return c * I + extra;
}

__host__ __device__ inline int shard_of(int i, int S, int I) { return (i / I) % S; }

__host__ __device__ inline int local_index(int i, int S, int I) {
  return (i / (I * S)) * I + i % I;
}

// Several new tokens per sequence: the one at global position `pos` attends over
// positions 0..pos (causal among the new tokens), which on shard r are the first
// shard_len(pos + 1) local tokens (a shard keeps global order).
__host__ __device__ inline int visible_on_shard(int pos, int S, int I, int r) {
  return pos >= 0 ? shard_len(pos + 1, S, I, r) : 0;
}

// ---------------------------------------------------------------- error flag
// Device-detected data errors.  Stored with an ordinary vector atomic.
enum : int { kErrBlockId = 1, kErrCapacity = 2, kErrSlot = 4 };

__device__ inline void raise_flag(int* flag, int bits) {
  if (flag) atomicOr(flag, bits);
}

// ---------------------------------------------------------------- block-table addressing
// The one address generator of the library: every kernel that reads or writes cache rows
// through a block table (the decode kernels, the gather, the routed append) resolves an
// entry with table_entry and forms the row's offset with key_row / value_tile.
//
// Entry j of a shard's table row: the physical block holding that shard's local tokens
// j*block_size .. j*block_size+block_size-1, or kPastRow when j lies beyond the row, or
// kBadId when the stored id is outside [0, n_blocks).
enum : int { kBadId = -2, kPastRow = -3 };

__device__ inline int table_entry(const int32_t* row, int j, int max_blocks, int64_t n_blocks) {
  if (j < 0 || j >= max_blocks) return kPastRow;
  const int v = row[j];
  return (v < 0 || int64_t(v) >= n_blocks) ? kBadId : v;
}

// The error-flag bit an entry raises when used: 0 for a valid block id.
__device__ inline int entry_error(int e) {
  return e == kPastRow ? kErrCapacity : (e == kBadId ? kErrBlockId : 0);
}

// Element offset of the key row in slot `off` of physical block `phys`, KV head h, in a
// cache laid out [n_blocks][hkv][bs][d] (a token's row contiguous).
__device__ inline int64_t key_row(int64_t phys, int h, int hkv, int bs, int off, int d) {
  return ((phys * hkv + h) * bs + off) * int64_t(d);
}

// Element offset of the value tile of physical block `phys`, KV head h, in a cache laid
// out [n_blocks][hkv][dv][bs]: element (column c, slot off) sits at + c*bs + off.
__device__ inline int64_t value_tile(int64_t phys, int h, int hkv, int bs, int dv) {
  return (phys * hkv + h) * int64_t(dv) * bs;
}

// Physical block of logical entry j of a table row, or -1 (and the flag raised) when
// the entry lies outside the row or holds an id outside [0, n_blocks).
__device__ inline int64_t table_block(const int32_t* row, int j, int max_blocks, int64_t n_blocks,
                                      int* flag) {
  const int e = table_entry(row, j, max_blocks, n_blocks);
  if (e < 0) {
    raise_flag(flag, entry_error(e));
    return -1;
  }
  return e;
}

// ---------------------------------------------------------------- element types
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN of the same sign.
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  const uint32_t rounded = u + 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(rounded >> 16);
}

// fp32 -> E4M3 code: round to nearest, ties to the even code; magnitudes of 448 and
// above (infinities too) saturate to +-448; NaN gives the NaN code with its sign.
// E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
// subnormals m * 2^-9.
__device__ inline uint8_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return uint8_t(sign | 0x7fu);  // NaN
  if (a >= 0x43e00000u) return uint8_t(sign | 0x7eu); // |y| >= 448
  if (a < 0x3c800000u) {
    // |y| < 2^-6: the nearest multiple of 2^-9 (scaling by 512 is exact); a result of 8
    // is 2^-6, whose code is 0x08 as well
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return uint8_t(sign | uint32_t(m));
  }
  // normal: keep 3 of the 23 fraction bits, round to nearest even (a carry moves into
  // the exponent), then rebias the exponent from 127 to 7
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return uint8_t(sign | (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// E4M3 code -> fp32, exact (the hardware conversion reads the OCP E4M3 format).
__device__ inline float e4m3_to_f32(uint8_t c) { return __builtin_amdgcn_cvt_f32_fp8(int(c), 0); }

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  using raw = uint32_t;
  static __device__ inline float load(const raw* p, int64_t i) { return __uint_as_float(p[i]); }
};
template <>
struct Elem<kBF16> {
  using raw = uint16_t;
  static __device__ inline float load(const raw* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
};
template <>
struct Elem<kFP8> {
  using raw = uint8_t;
  static __device__ inline float load(const raw* p, int64_t i) { return e4m3_to_f32(p[i]); }
};

}  // namespace pa
