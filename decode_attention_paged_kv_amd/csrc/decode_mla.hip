// decode_mla.hip -- paged decode attention over a latent (MLA-style) cache on the matrix
// cores: 128 query heads share one cached 576-wide vector per token whose first 512
// entries are the value (DCP page, soroban.highreso.jp: a latent model caches one
// compressed vector per token and behaves as a single KV head).
//
// What is computed is the same as in decode_generic.hip (softmax attention of each
// partition, output plus LSE; keys and values through the block table).  With 128 heads
// on one KV head both products are real dense contractions (about 240 flops per byte
// read), so both run on the matrix cores.
//
// One workgroup = one (partition, sequence x shard, KV head) with all 128 heads and eight
// waves (two per SIMD).  The partition is walked in 32-token tiles; each tile (32 rows x
// 1152 B, contiguous inside a block) is copied HBM -> LDS with global_load_lds_dwordx4
// (no registers involved) one tile ahead of the one being computed.
//  * Scores: wave w owns heads 16w..16w+15 and keeps their query rows in registers
//    (18 operands of v_mfma_f32_16x16x32_bf16).  S^T[token][head] = K_tile . Q^T with the
//    key operand one 16-byte LDS read per lane per MFMA; each lane ends with 8 tokens of
//    one head, so the row max needs two cross-lane exchanges.
//  * Softmax in base 2 with a lazily moved maximum: the reference max of a head moves
//    only when a score exceeds it by more than 8 (log2 units), so weights stay below 2^8
//    and the output accumulators are rarely rescaled; the final division by the sum makes
//    the result exact for any reference value.  Weights enter the output product rounded
//    to bf16 once; the normaliser (and so the LSE) sums them unrounded in fp32.
//  * Output: wave w owns value columns 64w..64w+63 of all 128 heads, O^T[d][head] +=
//    V^T . P^T on v_mfma_f32_32x32x16_bf16.  The V^T operand (8 tokens of one value
//    column per lane) comes straight from the row-major tile with two ds_read_b64_tr_b16
//    transposing reads; the weights of all heads pass through LDS.
//  * Tokens past the partition end get score -inf and zero value by select.
// LDS rows are padded to 1168 B (73 x 16 B) so the 16 rows read together start in
// different banks.
#include <math.h>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef short s16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int DK = 576, DV = 512, HEADS = 128;
constexpr int NW = 8;                               // waves per workgroup
constexpr int TT = 32;                              // tokens per tile
constexpr int ROW_CHUNKS = DK * 2 / 16;             // 72 chunks of 16 B per key row
constexpr int ROW_SLOTS = ROW_CHUNKS + 1;           // padded LDS row
constexpr int ROW_BYTES = ROW_SLOTS * 16;           // 1168
constexpr int TILE_SLOTS = TT * ROW_SLOTS;          // 2336
constexpr int ROUNDS = (TILE_SLOTS + 64 * NW - 1) / (64 * NW);  // copies per wave per tile
constexpr int BUF_BYTES = ROUNDS * 64 * NW * 16;    // every wave issues ROUNDS copies
constexpr int QH = HEADS / NW;                      // 16 heads per wave for the scores
constexpr int PVC = DV / NW;                        // 64 value columns per wave for the output
constexpr int P_STRIDE = TT + 8;                    // bf16 per weight row (80 B)
constexpr float kLazy = 8.f;                        // log2 headroom before the max moves
constexpr int QL = 8;                               // query k-steps kept in LDS (rest in registers)
constexpr int QR = DK / 32 - QL;                    // query k-steps kept in registers
#ifndef PA_MLA_QG
#define PA_MLA_QG 2
#endif
constexpr int QG = PA_MLA_QG;                       // k-steps of score operands read together
constexpr int TBL = 512;                            // block-table entries staged in LDS

// Workgroup barrier without a memory fence: this wave's LDS reads/writes are drained
// first (lgkmcnt 0); the asynchronous HBM -> LDS copies are waited for separately with
// vmcnt, so a copy still in flight for the next tile does not hold the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), vmcnt/expcnt unchanged
  __builtin_amdgcn_s_barrier();
}

// 16-byte asynchronous copy HBM -> LDS (global_load_lds_dwordx4): each lane copies 16 B
// from its own address; the 64 lanes' data land at consecutive 16-byte slots starting at
// LDS byte address `lds_addr` (wave-uniform, passed in M0).  Issued through asm so the
// compiler does not attach its own conservative waits to later LDS reads; the kernel
// waits for these copies explicitly with vmcnt before the barrier that publishes a tile.
__device__ inline void copy16_to_lds(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

__device__ inline uint32_t lds_address(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

__device__ inline f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(64 * NW) void decode_mla_kernel(DecodeArgs a) {
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);

  __shared__ __attribute__((aligned(16))) char kt0[BUF_BYTES];   // two tile buffers, kept as
  __shared__ __attribute__((aligned(16))) char kt1[BUF_BYTES];   // separate objects
  __shared__ __attribute__((aligned(16))) uint16_t p_s[HEADS * P_STRIDE];
  __shared__ float alpha_s[HEADS];
  __shared__ float m_s[HEADS], l_s[HEADS];
  __shared__ __attribute__((aligned(16))) uint16_t q_s[QL * HEADS * 32];   // [k-step][head][32]
  __shared__ int32_t tbl_s[TBL];   // block-table entries of the partition, TBL at a time

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15, g16 = lane >> 4;   // 16x16x32 operand row/col, k-group
  const int r32 = lane & 31, c32 = lane >> 5;   // 32x32x16 operand row/col, k-group
  const int p = blockIdx.x;
  const int b = blockIdx.y / a.n_shards;
  const int r = blockIdx.y % a.n_shards;
  const int kvh = blockIdx.z;
  const int h0 = kvh * HEADS;
  const int bs = a.bs;

  const int L = a.context_lens[b];
  const int Lr = L > 0 ? shard_len(L, a.n_shards, a.interleave, r) : 0;
  const int T = a.part_tokens;
  if (p == 0 && tid == 0 && (Lr + T - 1) / T > a.max_parts) raise_flag(a.flag, kErrCapacity);
  const int t_begin = p * T;
  const int t_end = min(t_begin + T, Lr);
  const int64_t out_row = ((int64_t(b) * a.n_shards + r) * a.max_parts + p) * a.hq + h0;
  if (t_begin >= t_end) {  // empty partition: lse = -inf, output rows left unwritten
    if (tid < HEADS) a.part_lse[out_row + tid] = -INFINITY;
    return;
  }

  const int32_t* row = a.block_table + (int64_t(b) * a.n_shards + r) * a.max_blocks;
  const int n_tiles = (t_end - t_begin + TT - 1) / TT;

  // Block-table entries of the partition are staged in LDS, TBL at a time, so a tile's
  // block id is an LDS read, not a global load that would wait behind the copies in
  // flight.  Entry e of the row is tbl_s[e - tbl_base]; ids outside [0, n_blocks) or
  // entries past the row read as -1 (flag raised by the tile that uses them).
  const int e_first = t_begin / bs;
  int tbl_base = e_first;
  auto stage_table = [&](int base) {
    for (int j = tid; j < TBL; j += 64 * NW) {
      const int e = base + j;
      int v = -1;
      if (e < a.max_blocks) {
        v = row[e];
        if (v < 0 || v >= a.n_blocks) v = -2;
      } else {
        v = -3;
      }
      tbl_s[j] = v;
    }
  };
  stage_table(tbl_base);

  // physical block of tile i (uniform); -1 if invalid (flag raised, tile skipped)
  auto tile_block = [&](int i) -> int {
    const int e = (t_begin + i * TT) / bs;
    const int v = tbl_s[e - tbl_base];
    if (v < 0) {
      if (tid == 0) raise_flag(a.flag, v == -3 ? kErrCapacity : kErrBlockId);
      return -1;
    }
    return v;
  };

  // HBM -> LDS copy of tile i.  LDS slot s holds tile row s / 73, chunk s % 73 (chunk 72
  // is the row pad, filled from chunk 71).  Each wave instruction writes 64 consecutive
  // slots.  Every wave issues exactly ROUNDS copies with all lanes on -- slots past the
  // tile re-read the tile's last chunk into spare LDS, and a tile with an invalid block
  // re-reads row 0 of block 0 -- so a fixed vmcnt separates one tile's copies from the
  // next one's.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue_tile = [&](int i, char* dst, int phys) {
    const int tok0 = t_begin + i * TT;
    const char* src = phys >= 0
        ? kc + ((int64_t(phys) * a.hkv + kvh) * bs + (tok0 % bs)) * int64_t(DK * 2)
        : kc;
    const uint32_t dst_lds = lds_address(dst);
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
      const int base = (k * NW + wave_u) * 64;
      const int s = base + lane;
      int t = s / ROW_SLOTS;
      int cc = s - t * ROW_SLOTS;
      cc = cc < ROW_CHUNKS ? cc : ROW_CHUNKS - 1;
      uint32_t off = uint32_t(t * (DK * 2) + cc * 16);
      if (s >= TILE_SLOTS) off = uint32_t((TT - 1) * (DK * 2) + (ROW_CHUNKS - 1) * 16);
      if (phys < 0) off = 0;
      copy16_to_lds(src + off, dst_lds + uint32_t(base) * 16);
    }
  };

  // query operand of the scores: lane (head 16w + c16, k-group g16) needs q[head][32ks +
  // 8g16 .. +7] for k-steps ks = 0..17.  The first QL k-steps of all heads sit in LDS
  // ([ks][head][32]), the rest in registers.
  {
    const uint16_t* qb = q + (int64_t(b) * a.hq + h0) * DK;
    for (int i = tid; i < QL * HEADS * 4; i += 64 * NW) {   // 16-byte pieces
      const int ks = i / (HEADS * 4), rem = i % (HEADS * 4), hh = rem / 4, part = rem % 4;
      *reinterpret_cast<uint4*>(q_s + (ks * HEADS + hh) * 32 + 8 * part) =
          *reinterpret_cast<const uint4*>(qb + int64_t(hh) * DK + 32 * ks + 8 * part);
    }
  }
  bf16x8_t qop[QR];
  {
    const uint16_t* qrow = q + (int64_t(b) * a.hq + h0 + QH * wave + c16) * DK + 8 * g16;
#pragma unroll
    for (int j = 0; j < QR; ++j) qop[j] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * (QL + j));
  }
  // settle every global load issued so far here, so that no wait for them is placed
  // inside the tile loop (where it would also wait for the tile copies in flight)
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  const lds_char_t* qlds = (const lds_char_t*)q_s + ((QH * wave + c16) * 32 + 8 * g16) * 2;
  __syncthreads();

  f32x16_t o[2][4];   // [32-column tile][32-head tile]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[mt][nt][e] = 0.f;

  const float c = a.scale * kLog2e;
  const int my_head = QH * wave + c16;
  float m_used = -INFINITY;   // reference max (raw score) of head my_head
  float lsum = 0.f;           // this lane's share of the sum of weights

  // one tile: prefetch tile i+1 into `next`, then compute tile i from `cur`
  auto step = [&](int i, const char* cur, char* next, int phys_cur) -> int {
    int phys_next = -1;
    if (i + 1 < n_tiles) {
      const int e_next = (t_begin + (i + 1) * TT) / bs;
      if (e_next - tbl_base >= TBL) {   // next chunk of the table (rare: T > TBL blocks)
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
        __syncthreads();
        tbl_base = e_next;
        stage_table(tbl_base);
        __syncthreads();
      }
      phys_next = tile_block(i + 1);
      issue_tile(i + 1, next, phys_next);
      __builtin_amdgcn_s_waitcnt((ROUNDS & 15) | (7 << 4) | (15 << 8));  // this tile landed
    } else {
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    }
    lds_barrier();
    const int tok0 = t_begin + i * TT;
    const int valid = phys_cur >= 0 ? min(TT, t_end - tok0) : 0;
    const lds_char_t* tile = (const lds_char_t*)cur;

    // ---- scores of this wave's 16 heads: two 16-token halves of the tile
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (valid > 0) {
      const lds_char_t* krow = tile + c16 * ROW_BYTES + 16 * g16;
      // operands are read in groups of QG k-steps and then consumed, so several LDS
      // reads are in flight together instead of one read, one wait, one MFMA
#pragma unroll
      for (int k0 = 0; k0 < DK / 32; k0 += QG) {
        bf16x8_t kop[QG][2], qk[QG];
#pragma unroll
        for (int j = 0; j < QG; ++j) {
          const int ks = k0 + j;
          qk[j] = ks < QL ? *reinterpret_cast<const lds_bf16x8_t*>(qlds + ks * HEADS * 64)
                          : qop[ks < QL ? 0 : ks - QL];
#pragma unroll
          for (int th = 0; th < 2; ++th)
            kop[j][th] = *reinterpret_cast<const lds_bf16x8_t*>(krow + 16 * th * ROW_BYTES + 64 * ks);
        }
#pragma unroll
        for (int j = 0; j < QG; ++j)
#pragma unroll
          for (int th = 0; th < 2; ++th) acc[th] = mfma16(kop[j][th], qk[j], acc[th]);
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * QG, 0);   // the group's LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * QG, 0);   // then its MFMAs
      }
    }
    float sc[2][4];
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // token 16*th + 4*g16 + e of head my_head
        const int tok = 16 * th + 4 * g16 + e;
        sc[th][e] = tok < valid ? acc[th][e] : -INFINITY;
      }
    float mt = -INFINITY;
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int e = 0; e < 4; ++e) mt = fmaxf(mt, sc[th][e]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    float alpha = 1.f;
    if (mt != -INFINITY && (m_used == -INFINITY || (mt - m_used) * c > kLazy)) {
      alpha = (m_used == -INFINITY) ? 0.f : exp2f((m_used - mt) * c);
      m_used = mt;
    }
    const float mc = (m_used == -INFINITY) ? 0.f : m_used * c;
    float part = 0.f;
    uint32_t pw[2][2];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      uint16_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = exp2f(fmaf(sc[th][e], c, -mc));
        part += pe;
        hb[e] = __builtin_bit_cast(uint16_t, (__bf16)pe);
      }
      pw[th][0] = uint32_t(hb[0]) | (uint32_t(hb[1]) << 16);
      pw[th][1] = uint32_t(hb[2]) | (uint32_t(hb[3]) << 16);
    }
    lsum = fmaf(lsum, alpha, part);
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      uint2 w2;
      w2.x = pw[th][0];
      w2.y = pw[th][1];
      *reinterpret_cast<uint2*>(p_s + my_head * P_STRIDE + 16 * th + 4 * g16) = w2;
    }
    if (g16 == 0) alpha_s[my_head] = alpha;
    lds_barrier();

    // ---- output columns 64w .. 64w+63 of all heads
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float al = alpha_s[32 * nt + r32];
      if (__any(al != 1.f)) {
#pragma unroll
        for (int mt2 = 0; mt2 < 2; ++mt2) o[mt2][nt] *= al;
      }
    }
    if (valid > 0) {
      const int j16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // V^T operand: lane (value column n0 + j16, k-group) holds tokens kb .. kb+7
        const int kb = 16 * ks + 8 * (g16 >> 1);
        bf16x8_t aop[2];
#pragma unroll
        for (int mt2 = 0; mt2 < 2; ++mt2) {
          const int n0 = PVC * wave + 32 * mt2 + 16 * (g16 & 1);
          const lds_char_t* base0 = tile + (kb + (j16 >> 2)) * ROW_BYTES + (n0 + 4 * (j16 & 3)) * 2;
          s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)base0);
          s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base0 + 4 * ROW_BYTES));
          if (valid < TT) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lo[e] = (kb + e < valid) ? lo[e] : short(0);
              hi[e] = (kb + 4 + e < valid) ? hi[e] : short(0);
            }
          }
          const s16x8_t cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          aop[mt2] = __builtin_bit_cast(bf16x8_t, cat);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          // P^T operand: lane (head 32nt + r32, k-group c32) holds tokens 16ks + 8c32 .. +7
          const bf16x8_t bop = *reinterpret_cast<const lds_bf16x8_t*>(
              (const lds_char_t*)p_s + ((32 * nt + r32) * P_STRIDE + 16 * ks + 8 * c32) * 2);
#pragma unroll
          for (int mt2 = 0; mt2 < 2; ++mt2) o[mt2][nt] = mfma32(aop[mt2], bop, o[mt2][nt]);
        }
      }
    }
    lds_barrier();
    return phys_next;
  };

  int phys = tile_block(0);
  issue_tile(0, kt0, phys);
  for (int i = 0; i < n_tiles; i += 2) {
    phys = step(i, kt0, kt1, phys);
    if (i + 1 >= n_tiles) break;
    phys = step(i + 1, kt1, kt0, phys);
  }

  // ---- finish: total weight per head, then o / l
  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  if (g16 == 0) {
    m_s[my_head] = m_used;
    l_s[my_head] = lt;
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int hh = 32 * nt + r32;
    const float inv = 1.f / l_s[hh];
#pragma unroll
    for (int mt2 = 0; mt2 < 2; ++mt2)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = PVC * wave + 32 * mt2 + 8 * jj + 4 * c32;
        float4 v;
        v.x = o[mt2][nt][4 * jj + 0] * inv;
        v.y = o[mt2][nt][4 * jj + 1] * inv;
        v.z = o[mt2][nt][4 * jj + 2] * inv;
        v.w = o[mt2][nt][4 * jj + 3] * inv;
        *reinterpret_cast<float4*>(a.part_out + (out_row + hh) * DV + d) = v;
      }
  }
  if (tid < HEADS) a.part_lse[out_row + tid] = (m_s[tid] * c + log2f(l_s[tid])) * kLn2;
}

}  // namespace

bool mla_supported(const DecodeArgs& a) {
  return a.dtype == kBF16 && a.v_cache == nullptr && a.dk == DK && a.dv == DV &&
         a.hq == HEADS * a.hkv && a.bs % TT == 0;
}

int mla_workgroups_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)decode_mla_kernel, 64 * NW, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.max_parts, a.n_seqs * a.n_shards, a.hkv);
  hipLaunchKernelGGL(decode_mla_kernel, grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
