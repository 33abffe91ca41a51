// decode_mla.hip -- paged decode attention over a latent (MLA-style) cache on the matrix
// cores: 128 query heads share one cached 576-wide vector per token whose first 512
// entries are the value (DCP page, soroban.highreso.jp: a latent model caches one
// compressed vector per token and behaves as a single KV head).
//
// What is computed is the same as in decode_generic.hip (softmax attention of each
// partition, output plus LSE; keys and values through the block table).  With 128 heads
// on one KV head both products are real dense contractions (about 240 flops per byte
// read), so both run on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The grid holds as many workgroups as can be resident at once; each takes every G-th
// unit of work -- a (partition, sequence x shard, new token, group of up to 128 query
// heads, KV head), numbered densely over the non-empty partitions -- with its 128 head
// rows and four waves, one per SIMD.  Wave w owns rows 32w .. 32w+31 from end to end,
// so waves share nothing but the key/value tiles:
//  * Tiles of 32 tokens (32 rows x 1152 B, contiguous inside a block) are copied HBM ->
//    LDS with global_load_lds_dwordx4 (no registers involved) into a ring of three
//    buffers.  Iteration i computes tile i's scores, softmax and output; the copies of
//    tile i+2 issue in the shadow of its score MFMAs, into the buffer tile i-1 has left,
//    so two tiles are in flight while one is computed.  The weights of the value
//    product's first k-step are computed between the two products (with the first value
//    reads in flight), those of the second k-step in the shadow of the first k-step's
//    output MFMAs.  One barrier per tile both publishes a landed tile and frees the
//    buffer of the tile before it.  A single wave per SIMD keeps the matrix core busy
//    only with work placed in the shadow of its own MFMAs, hence this interleaving.
//  * Scores: S^T[token][head] = K_tile . Q^T over 36 k-steps.  33 k-steps of the wave's
//    32 query rows live in registers for the whole partition, 3 in LDS (the score phase's
//    LDS reads are what its time rests on; fewer query reads there measured ~2 % faster
//    than 12 in LDS); the key operand
//    is one 16-byte LDS read per lane per MFMA.
//  * Softmax in base 2 against a reference max per head that is fixed by the first tile
//    holding a valid token of the partition and never moved: later weights may exceed 1
//    (exactly representable growth, up to 2^64), so the output accumulators are never
//    rescaled inside the loop and stay in the AGPR file without a branch over them.  The
//    final division by the sum makes the result exact for any reference value.  If a
//    score ever exceeds the reference by more than 64 (log2 units) the workgroup starts
//    the partition over in two passes: the first finds each head's exact max, the second
//    accumulates with weights <= 1.  Each lane holds 16 tokens of one head, so a tile's
//    row max is one cross-lane exchange; it is taken only on the tile that sets the
//    reference, and a weight above 2^64 shows as the lane's weight sum exceeding 2^64.
//    Weights enter the output product as a bf16 pair -- the weight rounded to bf16 and
//    the rounded remainder, two MFMAs on the same value operand -- which carries ~16
//    significant bits; the normaliser (and so the LSE) sums them unrounded in fp32.
//  * Output: O^T[value column][head] += V^T . P^T, 16 column tiles of 32 x 32.  The
//    score accumulator's layout is exactly the layout of the P^T operand (same token
//    order on both operands), so weights never leave registers; the V^T operand (8
//    tokens of one value column per lane) comes from the row-major tile with two
//    ds_read_b64_tr_b16 transposing reads.
//  * Tokens past the partition end get score -inf; the copy of the last, partial tile
//    fills their rows with the partition's last row, and a tile whose block id is
//    invalid is copied from a zero tile, so every value the weights meet is finite and a
//    masked token adds exactly 0.
// Fewer query heads per KV head (a tensor-parallel share of a latent model's heads) run
// on the same 128-row products: rows past the real head count take a zero query and are
// never written, since the kernel's time is set by its instruction stream, not its rows.
// LDS tiles are unpadded and swizzled at 16-byte granularity: chunk c of token row t sits
// at position c ^ g(t), g(t) = 4*bit1(t) + bits2..3(t), which spreads both the 32 rows of
// a key-operand read and the 4 rows of a transposing read over distinct banks.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "pa_append.h"
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef short s16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Weights a, b as bf16 pairs: hi = (bf16(a), bf16(b)), lo = (bf16(a - hi_a), bf16(b - hi_b)),
// round to nearest even, two weights per conversion; hi + lo carries ~16 significant bits.
struct Bf16Pairs {
  uint32_t hi, lo;
};
__device__ inline Bf16Pairs split_pair(float a, float b) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
  return {h, __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t))};
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int DK = 576, DV = 512, HEADS = 128;
constexpr int NW = 4;                               // waves per workgroup (one per SIMD)
constexpr int HW = HEADS / NW;                      // 32 heads per wave
constexpr int TT = 32;                              // tokens per tile
constexpr int ROW_BYTES = DK * 2;                   // 1152
constexpr int ROW_CHUNKS = ROW_BYTES / 16;          // 72 chunks of 16 B per row
constexpr int TILE_SLOTS = TT * ROW_CHUNKS;         // 2304
constexpr int TILE_BYTES = TILE_SLOTS * 16;         // 36864
constexpr int COPIES = TILE_SLOTS / (64 * NW);      // copies per wave per tile (9)
#ifndef PA_MLA_NBUF
#define PA_MLA_NBUF 3
#endif
constexpr int NBUF = PA_MLA_NBUF;                   // tile buffers
constexpr int KSTEPS = DK / 16;                     // 36 k-steps of the score product
constexpr int MT = DV / 32;                         // 16 value-column tiles
constexpr int TBL = 256;                            // block-table entries staged in LDS
#ifndef PA_MLA_QL
#define PA_MLA_QL 3
#endif
#ifndef PA_MLA_KA
#define PA_MLA_KA 2
#endif
#ifndef PA_MLA_VA
#define PA_MLA_VA 2
#endif
#ifndef PA_MLA_COPY_STRIDE
#define PA_MLA_COPY_STRIDE 4   // MFMA shadows between the tile copies of a wave
#endif
constexpr int QL = PA_MLA_QL;                       // query k-steps kept in LDS (rest in registers)
static_assert(QL >= 0 && QL <= 36 && PA_MLA_KA >= 1 && PA_MLA_VA >= 1, "read-ahead and query split");
// E4M3 cache: the codes are widened to bf16 on their way into the same LDS tile layout,
// by all the workgroup's threads through registers, into two tile buffers; the LDS the
// third buffer frees holds more of the query (fewer query registers).
#ifndef PA_MLA_QL_FP8
#define PA_MLA_QL_FP8 21
#endif
constexpr int NBUF_FP8 = 2;
constexpr int QL_FP8 = PA_MLA_QL_FP8;
constexpr int ROW_BYTES_FP8 = DK;                   // 576 codes per token row
static_assert(QL_FP8 >= 0 && QL_FP8 <= 36 &&
                  NBUF_FP8 * TILE_BYTES + QL_FP8 * 2 * HEADS * 8 * 2 + TBL * 4 + 2 * NW * 4 <= 160 * 1024,
              "E4M3: two tiles, the query part and the table must fit 160 KiB of LDS");
static_assert(TILE_SLOTS % (64 * NW) == 0, "tile copies must split evenly over the waves");
static_assert(ROW_CHUNKS % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");

// Chunk swizzle of token row t (see the header).
__device__ inline int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

// vmcnt(n) with expcnt/lgkmcnt left alone.
#define PA_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier without a memory fence: this wave's LDS reads/writes are drained
// first (lgkmcnt 0); the asynchronous HBM -> LDS copies are waited for separately with
// vmcnt, so copies still in flight for later tiles do not hold the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), vmcnt/expcnt unchanged
  __builtin_amdgcn_s_barrier();
}

// 16-byte asynchronous copy HBM -> LDS (global_load_lds_dwordx4): lane i copies 16 B
// from base + off_i; the 64 lanes' data land at consecutive 16-byte slots starting at
// LDS byte address `lds_addr` (wave-uniform, passed in M0).  The cache is read once per
// step, so the copies use the non-temporal policy (`nt`), which streams random chunks
// from HBM faster on this GPU.  Issued through asm so the
// compiler does not attach its own conservative waits to later LDS reads; the kernel
// waits for these copies explicitly with vmcnt before the barrier that publishes a tile.
__device__ inline void copy16_to_lds(const char* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// The copies take their base address in SGPRs: the value is wave-uniform, and this
// makes it so for the compiler too.
__device__ inline const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// Pins a value at this point of the instruction stream: empty asm statements keep their
// order with the MFMA statements, so work between two pins stays in that MFMA's shadow
// instead of being moved by the compiler's own passes.
template <typename T>
__device__ inline void pin(T& v) {
  asm volatile("" : "+v"(v));
}

__device__ inline uint32_t lds_address(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Both products are written out as asm so that each accumulator stays in one register
// file: the 16 output tiles take the whole AGPR file and the score accumulator lives in
// VGPRs; the compiler's own choice moves them between the two on every tile.  The
// compiler does not see inside these statements, so they carry their wait states: three
// before an MFMA whose operand may just have been written by a VALU instruction or an
// accvgpr write (the first score MFMA of a tile, the first output MFMAs of each k-step),
// none before the others (below), and a drain of 21 after the last score MFMA of a tile
// and 24 after the last output MFMA, before any VALU instruction reads the result.
__device__ inline f32x16_t mfma32_vgpr_first(bf16x8_t a, bf16x8_t b) {
  f32x16_t d;
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
// The score chain's accumulating MFMAs carry no wait states: their operands are LDS
// reads (waited for with lgkmcnt) and query registers loaded before the tile loop, never
// a value a VALU instruction has just written (tests/test_isa_hazards.py checks the
// compiled code for that).
__device__ inline void mfma32_vgpr_acc(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ inline void mfma32_vgpr_last(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
               : "+v"(d) : "v"(a), "v"(b));
}
__device__ inline void mfma32_agpr_acc(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// An output MFMA whose weight operand was formed at least one output MFMA earlier and
// whose value operand is an LDS read: no wait states.
__device__ inline void mfma32_agpr_acc_nowait(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Pins a value of an output tile to the AGPR file (the compiler copies it in), so that
// every definition of the loop-carried output tiles is an AGPR one and the loop keeps
// them there.
__device__ inline f32x16_t to_agpr(f32x16_t v) {
  f32x16_t d;
  asm volatile("" : "=a"(d) : "0"(v));
  return d;
}

// Source of the copy of a tile whose block id is invalid (zero-initialised device memory).
__device__ __attribute__((aligned(16))) char g_zero_tile[TILE_BYTES];

// Progress of the units that share their tiles with a partner (the new tokens of one
// partition, side by side on one XCD): slot u % kProgressSlots holds (u & 0xffff) << 16 |
// tile.  Only a hint: a stale or shared slot makes a unit wait less or not at all, never
// changes a result, and every wait is bounded.
constexpr int kProgressSlots = 4096;
__device__ uint32_t g_progress[kProgressSlots];
constexpr int kSyncEvery = 8;    // tiles between progress checks
constexpr int kSyncDrift = 2;    // tiles a unit may run ahead of its partner
constexpr int kSyncSpins = 80;   // bound of a wait (each spin sleeps ~256 cycles)

// A progress slot read from L2 past the scalar cache (glc), waited for with lgkmcnt so that
// the tile copies in flight (counted by vmcnt) are not waited for.
__device__ inline uint32_t load_progress(const uint32_t* p) {
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

template <bool F8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mla_kernel(DecodeArgs a) {
  constexpr int NB = F8 ? NBUF_FP8 : NBUF;   // tile buffers
  constexpr int QLk = F8 ? QL_FP8 : QL;      // query k-steps in LDS
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);

  __shared__ __attribute__((aligned(16))) char kt[NB * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t q_s[QLk * 2 * HEADS * 8];   // [ks][k-group][head][8]
  __shared__ int32_t tbl_s[TBL];   // block-table entries of the partition, TBL at a time
  static_assert(NB * TILE_BYTES + QLk * 2 * HEADS * 8 * 2 + TBL * 4 + 2 * NW * 4 <= 160 * 1024,
                "the tiles, the query part and the table must fit the compute unit's 160 KiB of LDS");
  __shared__ __attribute__((aligned(16))) int ovf_s[2][NW];   // [tile parity][wave]: overflow seen

  // the zero tile's address, taken once: inside the tile loop its load from the constant
  // table would wait for every LDS read in flight
  const char* zero_tile = g_zero_tile;
  asm volatile("" : "+s"(zero_tile));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, c32 = lane >> 5;   // 32x32x16 operand row/col, k-group
  const int bs = a.bs;
  const int T = a.part_tokens;
  const int Y = a.n_seqs * a.n_shards;   // (sequence, shard) pairs
  // query heads per KV head, taken HEADS at a time (NG groups, each a unit of its own):
  // the products always run on HEADS rows; rows past a group's real count read a zero
  // query and are never written
  const int nh = a.hq / a.hkv;
  const int NG = (nh + HEADS - 1) / HEADS;

  // Units of work are the non-empty (pair y, partition p, KV head) triples, numbered
  // densely in that order (KV head fastest); workgroup g takes units g, g + G, g + 2G, ..
  // (G = the grid), so the work is spread evenly however the lengths fall, and every
  // workgroup stays resident.  Pair y has min(ceil(L_y / T), max_parts) partitions (more
  // is a capacity error, flagged).  Each wave walks the pairs in chunks of 64 with a
  // prefix sum over its lanes; the walk only moves forward, as the units do.
  auto parts_of = [&](int y) -> int {
    if (y >= Y) return 0;
    const int L = a.context_lens[y / a.n_shards];
    const int Lr = L > 0 ? shard_len(L, a.n_shards, a.interleave, y % a.n_shards) : 0;
    const int n = (Lr + T - 1) / T;
    if (n > a.max_parts) raise_flag(a.flag, kErrCapacity);
    return min(n, a.max_parts);
  };
  int w_chunk = 0;   // first pair of the walker's chunk
  int w_base = 0;    // partition slots before it
  int w_cnt = 0, w_incl = 0, w_total = 0;   // lane's count and inclusive prefix; chunk total
  auto load_chunk = [&]() {
    w_cnt = parts_of(w_chunk + lane);
    w_incl = w_cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(w_incl, d);
      if (lane >= d) w_incl += v;
    }
    w_total = __builtin_amdgcn_readfirstlane(__shfl(w_incl, 63));
  };
  load_chunk();
  // Several new tokens per sequence: each (pair, partition) slot holds max_q units per
  // (head group, KV head), one per new token (units past a sequence's own count are
  // skipped).
  const int MQ = a.query_start ? a.max_q : 1;
  const int per_q = a.hkv * NG;

  // Workgroup b runs on XCD b mod 8 (the dispatcher deals workgroups out round-robin);
  // each XCD has an L2 of its own.  Numbering the workgroups XCD by XCD -- first unit
  // (b mod 8) * (G / 8) + b / 8 -- puts units that follow one another on one XCD, at the
  // same time: the new tokens of one partition (consecutive units) then read each tile
  // once from HBM and again from that XCD's L2.  The same units, dealt to other
  // workgroups: the per-workgroup loads are unchanged.
  constexpr int kXcds = 8;
  const int G = gridDim.x;
  const int first = G % kXcds == 0 ? int(blockIdx.x % kXcds) * (G / kXcds) + int(blockIdx.x / kXcds)
                                   : int(blockIdx.x);
  for (int unit = first;; unit += G) {
    // ---- resolve unit -> (pair y, partition p, new token qi, head group grp, KV head
    // kvh); stop past the last pair
    const int slot = unit / (per_q * MQ);
    const int qk = unit - slot * (per_q * MQ);
    const int qi = qk / per_q;
    const int gk = qk - qi * per_q;
    const int grp = gk / a.hkv;
    const int kvh = gk - grp * a.hkv;
    while (slot >= w_base + w_total && w_chunk < Y) {
      w_base += w_total;
      w_chunk += 64;
      load_chunk();
    }
    if (w_chunk >= Y) break;
    const int rel = slot - w_base;
    const uint64_t hit = __ballot(w_incl > rel);
    const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
    const int y = w_chunk + j;
    const int p = rel - (__builtin_amdgcn_readfirstlane(__shfl(w_incl - w_cnt, j)));
    const int b = y / a.n_shards;
    const int r = y - b * a.n_shards;
    const int h0 = kvh * nh + grp * HEADS;   // the unit's first query head
    const int nrow = min(HEADS, nh - grp * HEADS);   // its real rows
    const int L = a.context_lens[b];
    // q row of the unit and how many of the shard's tokens it sees: all of them, or for
    // new token qi of nq (global position L - nq + qi) those at or before its position
    int qr = b;
    int Lq = shard_len(L, a.n_shards, a.interleave, r);
    int partner = -1;   // unit sharing this one's tiles, kept in step with it
    if (a.query_start) {
      const int row0 = a.query_start[b];
      const int nq = a.query_start[b + 1] - row0;
      if (nq > L || nq > a.max_q || row0 < 0 || row0 + nq > a.n_rows) {   // rows left unwritten
        if (tid == 0 && p == 0 && qi == 0 && grp == 0 && kvh == 0) raise_flag(a.flag, kErrCapacity);
        continue;
      }
      if (qi >= nq) continue;
      qr = row0 + qi;
      Lq = visible_on_shard(L - nq + qi, a.n_shards, a.interleave, r);
      // the unit of new token qi ^ 1 reads the same tiles; with the XCD-wise numbering it
      // runs at the same time on the same XCD when it falls in the same block of G / 8
      // units -- then the two keep within a few tiles of each other, so that the second
      // read of each tile is an L2 hit
      const int qp = qi ^ 1;
      if (qp < nq && G % kXcds == 0) {
        const int pu = unit + (qp - qi) * per_q;
        if (pu / (G / kXcds) == unit / (G / kXcds)) partner = pu;
      }
    }
    const int t_begin = p * T;
    const int t_end = min(t_begin + T, Lq);
    const int64_t out_row = ((int64_t(qr) * a.n_shards + r) * a.max_parts + p) * a.hq + h0;
    if (t_end <= t_begin) {   // a new token that sees none of the partition's tokens
      for (int i = tid; i < nrow; i += 64 * NW) a.part_lse[out_row + i] = -INFINITY;
      if (p == 0)
        for (int i = tid; i < nrow * DV; i += 64 * NW) a.part_out[out_row * DV + i] = 0.f;
      continue;
    }
    __syncthreads();   // the previous unit is done with the LDS
    // the step's append, when this launch performs it: before any read of the cache
    if (qi == 0 && grp == 0) fused_append(a, b, r, p, kvh);

  const int32_t* row = a.block_table + (int64_t(b) * a.n_shards + r) * a.max_blocks;
  const int n_tiles = (t_end - t_begin + TT - 1) / TT;

  // Block-table entries of the partition are staged in LDS, TBL at a time, so a tile's
  // block id is an LDS read, not a global load that would wait behind the copies in
  // flight.  Entry e of the row is tbl_s[e - tbl_base], as table_entry reads it: ids
  // outside [0, n_blocks) and entries past the row are negative codes (flag raised by the
  // tile that uses them).
  const int e_first = t_begin / bs;
  int tbl_base = e_first;
  auto stage_table = [&](int base) {
    for (int j = tid; j < TBL; j += 64 * NW) tbl_s[j] = table_entry(row, base + j, a.max_blocks, a.n_blocks);
  };
  stage_table(tbl_base);
  __syncthreads();

  // Block-table entry of tile i as read from LDS (restaging first if the entry lies in
  // another chunk of the table); finish_tile turns it into the wave-uniform block id.
  // Split so that the LDS read can be issued early and its latency hidden.
  auto tile_entry = [&](int i) -> int {
    const int e = (t_begin + i * TT) / bs;
    if (__builtin_expect(e - tbl_base >= TBL || e < tbl_base, 0)) {   // other chunk of the table (long partitions)
      PA_WAIT_VM(0);
      __syncthreads();
      tbl_base = e;
      stage_table(tbl_base);
      __syncthreads();
    }
    return tbl_s[e - tbl_base];
  };

  // Copy of tile i: LDS slot s of the tile holds token row s / 72, chunk (s % 72) ^ g(row).
  // Wave w's k-th copy writes slots (k*NW + w)*64 .. +63.  begin_tile resolves the
  // block; copy_piece(k) issues copy k (the pieces are spread over the score MFMAs).
  // The offsets are recomputed at each copy from an opaque copy of the lane id: hoisted
  // out of the tile loop they would hold nine registers the loop needs.  In the last,
  // partial tile, rows past the partition end repeat its last row.
  const uint32_t kt_lds = lds_address(kt);
  uint32_t bad = 0;   // bit (i % NB): tile i has an invalid block
  struct Copy {
    const char* src;
    uint32_t dst;
    int rows;
  };
  auto finish_tile = [&](int i, int entry) -> Copy {
    int phys = __builtin_amdgcn_readfirstlane(entry);
    if (__builtin_expect(phys < 0, 0)) {   // invalid block id or an entry past the row
      if (tid == 0) raise_flag(a.flag, entry_error(phys));
      phys = -1;
    }
    const int tok0 = t_begin + i * TT;
    const char* src = phys >= 0 ? kc + key_row(phys, kvh, a.hkv, bs, tok0 % bs, ROW_BYTES) : zero_tile;
    const uint32_t slot = uint32_t(i % NB);
    bad = (bad & ~(1u << slot)) | (uint32_t(phys < 0) << slot);
    const int rows = __builtin_amdgcn_readfirstlane(phys < 0 ? TT : min(TT, t_end - tok0));
    return Copy{uniform_ptr(src), kt_lds + slot * TILE_BYTES, rows};
  };
  auto begin_tile = [&](int i) -> Copy { return finish_tile(i, tile_entry(i)); };
  // Slot s = (k NW + w) 64 + lane = s0 + 256 k: with s0 = 72 t0 + x0 and 256 = 3*72 + 40,
  // row t = t0 + 3k + q and chunk x = y - 72 q for y = x0 + 40k, q = floor(y / 72) =
  // (57 y) >> 12 (exact for y < 392; here y <= 71 + 40*8).  Offsets of a full tile are
  // computed once; the last, partial tile recomputes them with its rows clamped.
  const int t0 = (wave * 64 + lane) / ROW_CHUNKS;
  const int x0 = (wave * 64 + lane) % ROW_CHUNKS;
  static_assert(NW * 64 == 3 * ROW_CHUNKS + 40 && COPIES <= 9, "slot stepping above");
  auto slot_offset = [&](int k, int rows) -> uint32_t {
    int t0o = t0, x0o = x0;
    asm volatile("" : "+v"(t0o), "+v"(x0o));
    const uint32_t y = uint32_t(x0o + 40 * k);
    const uint32_t qq = __umul24(y, 57u) >> 12;   // 24-bit multiplies: full rate
    const int t = t0o + 3 * k + int(qq);
    const uint32_t x = y - __umul24(qq, uint32_t(ROW_CHUNKS));
    const uint32_t row_src = uint32_t(min(t, rows - 1));
    return __umul24(row_src, uint32_t(ROW_BYTES)) + ((x ^ uint32_t(swz(t))) << 4);
  };
  uint32_t full_off[COPIES];
  if constexpr (!F8) {
#pragma unroll
    for (int k = 0; k < COPIES; ++k) {
      full_off[k] = slot_offset(k, TT);
      asm volatile("" : "+v"(full_off[k]));
    }
  }
  auto copy_piece = [&](const Copy& cp, int k) {
    // the operands are wave-uniform; reading them from the first lane makes that plain to
    // the compiler wherever the copies are inlined
    const uint32_t dst = __builtin_amdgcn_readfirstlane(cp.dst + uint32_t((k * NW + wave) * 64 * 16));
    const char* src = uniform_ptr(cp.src);
    if (cp.rows == TT) {
      copy16_to_lds(src, full_off[k], dst);
    } else {   // partial tile (a separate asm statement, so the two are not merged)
      const uint32_t off = slot_offset(k, cp.rows);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt ; partial tile"
                   :
                   : "v"(off), "s"(src), "s"(dst)
                   : "memory", "m0");
    }
  };
  auto issue_tile = [&](int i) {
    const Copy cp = begin_tile(i);
#pragma unroll
    for (int k = 0; k < COPIES; ++k) copy_piece(cp, k);
  };
  auto tile_valid = [&](int i) { return (bad >> (i % NB)) & 1 ? 0 : min(TT, t_end - (t_begin + i * TT)); };

  // Query operand (B of the score product): lane (head 32w + r32, k-group c32) needs
  // q[head][16 ks + 8 c32 .. +7] for k-steps ks = 0..35.  The first QL k-steps of all
  // heads sit in LDS as [ks][k-group][head][8] (a wave's read is 1 KB of consecutive
  // 16-byte pieces), the rest in registers for the whole partition.
  bf16x8_t qop[KSTEPS - QLk];
  {
    const uint16_t* qb = q + (int64_t(qr) * a.hq + h0) * DK;
    for (int i = tid; i < QLk * 2 * HEADS; i += 64 * NW) {   // 16-byte pieces
      const int ks = i / (2 * HEADS), g = (i / HEADS) % 2, hh = i % HEADS;
      *reinterpret_cast<uint4*>(q_s + 8 * i) =
          hh < nrow ? *reinterpret_cast<const uint4*>(qb + int64_t(hh) * DK + 16 * ks + 8 * g)
                  : make_uint4(0, 0, 0, 0);
    }
    if (HW * wave + r32 < nrow) {
      const uint16_t* qrow = q + (int64_t(qr) * a.hq + h0 + HW * wave + r32) * DK + 8 * c32;
#pragma unroll
      for (int ks = QLk; ks < KSTEPS; ++ks)
        qop[ks - QLk] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ks);
    } else {
#pragma unroll
      for (int ks = QLk; ks < KSTEPS; ++ks) qop[ks - QLk] = bf16x8_t{};
    }
  }
  const lds_char_t* qlds = (const lds_char_t*)q_s + (c32 * HEADS + HW * wave + r32) * 16;
  // settle every global load issued so far here, so that no wait for them is placed
  // inside the tile loop (where it would also wait for the tile copies in flight)
  PA_WAIT_VM(0);
  __syncthreads();   // q_s written

  // Key operand (A of the score product): lane (token r32, k-group c32) reads chunk
  // 2 ks + c32 of row r32: byte 1152 r32 + 128 (ks / 4) + 16 ((2 (ks % 4) + c32) ^ g).
  uint32_t ka[4];
  {
    const int g = swz(r32);
#pragma unroll
    for (int j = 0; j < 4; ++j) ka[j] = uint32_t(r32 * ROW_BYTES + (((2 * j + c32) ^ g) << 4));
  }
  // Value operand (A of the output product) through ds_read_b64_tr_b16: in 16-lane group
  // G = lane / 16, lane j reads token row 16 kv + 8 h + 4 (G / 2) + j / 4 (h = 0: first
  // read, h = 1: second), bytes 64 mt + 32 (G % 2) + 8 (j % 4) .. +7 of the value.  The
  // chunk is 4 mt + x with x = 2 (G % 2) + (j % 4) / 2; its swizzled position is
  // 4 (mt ^ g2) + (x ^ (g % 4)), so for even mt the byte is base + 64 mt + 64 g2 and for
  // odd mt base + 64 mt - 64 g2.
  uint32_t va[2][2];   // [h][mt parity]
  {
    const int G = lane >> 4, j = lane & 15;
    const int x = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * h + 4 * (G >> 1) + (j >> 2);
      const int g = swz(t);
      const int base = t * ROW_BYTES + ((x ^ (g & 3)) << 4) + 8 * (j & 1);
      va[h][0] = uint32_t(base + 64 * (g >> 2));
      va[h][1] = uint32_t(base - 64 * (g >> 2));
    }
  }

  // E4M3: the tile holds the codes' values; the key scale joins the score multiplier, and
  // (the value being the key's first DV entries) the final division
  float key_scale = 1.f;
  if constexpr (F8) key_scale = a.k_scale[a.n_scales > 1 ? kvh : 0];
  const float c = a.scale * key_scale * kLog2e;
  auto tile_ptr = [&](int i) { return (const lds_char_t*)kt + (i % NB) * TILE_BYTES; };

  // The 36 score MFMAs of the tile at `tile` into s.  Key operands are read KA k-steps
  // ahead of their MFMA; the scheduling fences keep the order as written, so the reads
  // do not all move up front, and filler(ks) -- other work of the wave -- issues in the
  // shadow of MFMA ks.  The per-tile operand bases are opaque so that the compiler keeps
  // the constant parts as instruction offsets instead of one register per read.
  auto scores = [&](const lds_char_t* tile, f32x16_t& s, auto&& filler) {
    const lds_char_t* kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kb[j] = tile + ka[j];
      asm volatile("" : "+v"(kb[j]));
    }
    constexpr int KA = PA_MLA_KA;   // k-steps of read-ahead
    bf16x8_t kop[KA + 1], qlo[KA + 1];
    auto kread = [&](int ks) {
      return *reinterpret_cast<const lds_bf16x8_t*>(kb[ks & 3] + 128 * (ks >> 2));
    };
    auto qread = [&](int ks) {
      return *reinterpret_cast<const lds_bf16x8_t*>(qlds + ks * (2 * HEADS * 16));
    };
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) {
      kop[ks] = kread(ks);
      if (ks < QLk) qlo[ks] = qread(ks);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + KA < KSTEPS) {
        kop[(ks + KA) % (KA + 1)] = kread(ks + KA);
        if (ks + KA < QLk) qlo[(ks + KA) % (KA + 1)] = qread(ks + KA);
      }
      const bf16x8_t kk = kop[ks % (KA + 1)];
      const bf16x8_t qq = ks < QLk ? qlo[ks % (KA + 1)] : qop[ks < QLk ? 0 : ks - QLk];
      if (ks == 0)
        s = mfma32_vgpr_first(kk, qq);
      else if (ks + 1 < KSTEPS)
        mfma32_vgpr_acc(s, kk, qq);
      else
        mfma32_vgpr_last(s, kk, qq);
      __builtin_amdgcn_sched_barrier(0);
      filler(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_filler = [](int) {};

  // Row max of tile i's scores: lane holds head r32, tokens 8 (e / 4) + 4 c32 + e % 4.
  auto masked = [&](const f32x16_t& s, int valid, float (&sc)[16]) {
    const int lim = valid - 4 * c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 8 * (e >> 2) + (e & 3) < lim ? s[e] : -INFINITY;
  };
  auto row_max = [&](const float (&sc)[16]) {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };

  // The output product of one tile: 32 value operands (operand n = kv * MT + m), each
  // taken by two MFMAs (weights rounded to bf16, then their remainders).  Value operands
  // are read VA operands ahead: vstart issues the first VA reads (so their latency can
  // hide under other work), outputs the rest; filler(n) issues in the shadow of operand
  // n's MFMAs.
  constexpr int VA = PA_MLA_VA, NV = 2 * MT;
  struct VBase {
    const lds_char_t* p[2][2];   // [h][mt parity]
  };
  auto vread = [&](const VBase& vb, int n) {
    const int kv = n / MT, m = n % MT;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(vb.p[0][m & 1] + 64 * m + 16 * ROW_BYTES * kv));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(vb.p[1][m & 1] + 64 * m + 16 * ROW_BYTES * kv));
    const s16x8_t cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, cat);
  };
  auto vstart = [&](const lds_char_t* tile, bf16x8_t (&vop)[VA + 1]) -> VBase {
    VBase vb;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        vb.p[h][par] = tile + va[h][par];
        asm volatile("" : "+v"(vb.p[h][par]));
      }
#pragma unroll
    for (int n = 0; n < VA; ++n) vop[n] = vread(vb, n);
    return vb;
  };
  auto outputs = [&](const VBase& vb, bf16x8_t (&vop)[VA + 1], const u32x4_t (&pop)[2],
                     const u32x4_t (&plo)[2], f32x16_t (&o)[MT], auto&& filler) {
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      if (n + VA < NV) vop[(n + VA) % (VA + 1)] = vread(vb, n + VA);
      if (n % MT == 0) {   // first use of a k-step's weights
        mfma32_agpr_acc(o[n % MT], vop[n % (VA + 1)], __builtin_bit_cast(bf16x8_t, pop[n / MT]));
        mfma32_agpr_acc(o[n % MT], vop[n % (VA + 1)], __builtin_bit_cast(bf16x8_t, plo[n / MT]));
      } else {
        mfma32_agpr_acc_nowait(o[n % MT], vop[n % (VA + 1)], __builtin_bit_cast(bf16x8_t, pop[n / MT]));
        mfma32_agpr_acc_nowait(o[n % MT], vop[n % (VA + 1)], __builtin_bit_cast(bf16x8_t, plo[n / MT]));
      }
      __builtin_amdgcn_sched_barrier(0);
      filler(n);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Weights and output product of tile i from its scores s.  Softmax: lane holds head
  // r32, tokens 8 (e / 4) + 4 c32 + e % 4 of the tile; elements 0..7 are the first
  // k-step's weights (computed here, with the first value reads in flight), 8..15 the
  // second's (in the shadow of the first output MFMAs), then the overflow flag: a
  // weight above 2^64 (a score more than 64 log2 units above the reference) makes the
  // lane's sum exceed 2^64.  extra(n) is more of the caller's work for the shadow of
  // operand n's MFMAs.
  auto weigh_and_output = [&](int i, const f32x16_t& s, const VBase& vb, bf16x8_t (&vop)[VA + 1], float mc,
                              f32x16_t (&o)[MT], float& lsum, auto&& extra) {
    float part = 0.f, pe[16];
    u32x4_t pop[2], plo[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c, -mc));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const Bf16Pairs w = split_pair(pe[2 * qq], pe[2 * qq + 1]);
      pop[0][qq] = w.hi;
      plo[0][qq] = w.lo;
    }
    // (the first weights join the sum in the shadow of the output MFMAs too)
    outputs(vb, vop, pop, plo, o, [&](int n) {
      if (n < 4) {
        part += pe[2 * n] + pe[2 * n + 1];
#pragma unroll
        for (int e = 8 + 2 * n; e < 10 + 2 * n; ++e) {
          float v = s[e];
          pin(v);
          pe[e] = __builtin_amdgcn_exp2f(fmaf(v, c, -mc));
          part += pe[e];
          pin(pe[e]);
        }
        pin(part);
      } else if (n < 6) {
#pragma unroll
        for (int qq = 2 * (n - 4); qq < 2 * (n - 4) + 2; ++qq) {
          const Bf16Pairs w = split_pair(pe[8 + 2 * qq], pe[9 + 2 * qq]);
          pop[1][qq] = w.hi;
          plo[1][qq] = w.lo;
        }
        pin(pop[1]);
        pin(plo[1]);
      } else if (n == 6) {
        lsum += part;
        const bool ovf = __any(part > 0x1p64f);
        if (lane == 0) ovf_s[i & 1][wave] = ovf ? 1 : 0;
      }
      extra(n);
    });
  };
  auto zero_tiles = [&](f32x16_t (&o)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f32x16_t z;
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = 0.f;
      o[m] = to_agpr(z);
    }
  };
  auto any_overflow = [&](int parity) {
    const int4 f = *reinterpret_cast<const int4*>(&ovf_s[parity][0]);
    return (f.x | f.y | f.z | f.w) != 0;
  };

  // Accumulating pass.  Iteration i computes tile i's scores, softmax and output.  The
  // copies of tile i+2 issue in the shadow of its score MFMAs, into the buffer tile i-1
  // has left (three buffers: tile i computed, tiles i+1 and i+2 in flight), so each copy
  // has more than an iteration to land.  The weights of the value product's first k-step
  // (tokens 0..15 of the tile) are computed between the two products, with the first
  // value reads in flight; those of the second k-step in the shadow of the first k-step's
  // output MFMAs.  A head whose m_ref is still -inf takes the max of its first tile with a
  // valid token; the pass stops (returns false) as soon as a score exceeds m_ref by more
  // than 64 log2 units (never, when m_ref is already the exact max).
  auto pass_acc = [&](float& m_ref, bool& have_ref, f32x16_t (&o)[MT], float& lsum) -> bool {
    if (tbl_base != e_first) {
      PA_WAIT_VM(0);
      __syncthreads();
      tbl_base = e_first;
      stage_table(tbl_base);
      __syncthreads();
    }
    constexpr int AHEAD = NB - 1;   // tiles copied ahead of the one computed
    for (int i = 0; i < AHEAD && i < n_tiles; ++i) issue_tile(i);
    float mc = have_ref ? m_ref * c : 0.f;
    // copy k of tile i+AHEAD in the shadow of score MFMA 1 + CS k
    constexpr int CS = PA_MLA_COPY_STRIDE;
    static_assert(CS >= 1 && 1 + CS * (COPIES - 1) < KSTEPS, "copy slots");
    auto copy_slot = [](int ks) { return ks >= 1 && (ks - 1) % CS == 0 && (ks - 1) / CS < COPIES; };

    // The common iteration runs straight-line code (a taken branch costs a wave with no
    // other wave on its SIMD tens of cycles): tiles i .. i+AHEAD all full, tile i's block
    // valid, the reference set, and every block of the partition in the staged chunk of
    // the table.  Other iterations (the partition's first and last tiles, invalid blocks,
    // table restaging) take the general path for their first half.  Tile i+AHEAD's block
    // and first row are stepped along instead of divided out.
    const bool table_fits = (t_end - 1) / bs - e_first < TBL;
    auto fast_ok = [&](int i) {
      return have_ref && table_fits && (i + AHEAD + 1) * TT <= t_end - t_begin && !((bad >> (i % NB)) & 1) &&
             (partner < 0 || i % kSyncEvery != 0);
    };
    // Every kSyncEvery tiles of a unit with a partner: publish the tile reached, and let
    // wave 0 wait (the others wait at the barrier that follows) while the partner is more
    // than kSyncDrift tiles behind -- at most kSyncSpins short sleeps, after which the
    // unit stops waiting for it.
    auto pair_wait = [&](int i) {
      if (wave != 0) return;
      if (lane == 0)
        __hip_atomic_store(&g_progress[unit % kProgressSlots], (uint32_t(unit & 0xffff) << 16) | uint32_t(i & 0xffff),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t* slot_p = reinterpret_cast<const uint32_t*>(
          uniform_ptr(reinterpret_cast<const char*>(&g_progress[partner % kProgressSlots])));
      int spins = 0;
#pragma unroll 1
      for (; spins < kSyncSpins; ++spins) {
        const uint32_t v = load_progress(slot_p);
        const int at = (v >> 16) == (uint32_t(partner) & 0xffffu) ? int(v & 0xffffu) : -1;
        if (at >= i - kSyncDrift) break;
        __builtin_amdgcn_s_sleep(4);
      }
      if (spins == kSyncSpins) partner = -1;
    };
    int nblk = (t_begin + AHEAD * TT) / bs;
    int nrow = t_begin + AHEAD * TT - nblk * bs;
    bool ok = true;
    for (int i = 0; i < n_tiles; ++i) {
      f32x16_t s;
      Copy cp{};
      int4 flags;
      if (__builtin_expect(fast_ok(i), 1)) {
        PA_WAIT_VM(COPIES);   // tile i landed, tile i+1's copies may be in flight
        // everyone's copies of tile i are in, everyone is done with tile i-1 (whose buffer
        // tile i+2 takes), and tile i-1's overflow flags are visible
        lds_barrier();
        // LDS reads consumed later, so their latency hides under the MFMAs: tile i-1's
        // overflow flags (checked at the end of the iteration) and tile i+2's table entry
        flags = *reinterpret_cast<const int4*>(&ovf_s[(i + 1) & 1][0]);
        const int entry = tbl_s[nblk - tbl_base];
        scores(tile_ptr(i), s, [&](int ks) {
          if (copy_slot(ks)) {
            const int k = (ks - 1) / CS;
            if (k == 0) {
              int phys = __builtin_amdgcn_readfirstlane(entry);
              if (__builtin_expect(phys < 0, 0)) {   // invalid block id
                if (tid == 0) raise_flag(a.flag, entry_error(phys));
                phys = -1;
              }
              const char* src = phys >= 0 ? kc + key_row(phys, kvh, a.hkv, bs, nrow, ROW_BYTES) : zero_tile;
              const uint32_t slot = uint32_t((i + AHEAD) % NB);
              bad = (bad & ~(1u << slot)) | (uint32_t(phys < 0) << slot);
              cp = Copy{uniform_ptr(src), kt_lds + slot * TILE_BYTES, TT};
            }
            copy16_to_lds(uniform_ptr(cp.src), full_off[k],
                          __builtin_amdgcn_readfirstlane(cp.dst + uint32_t((k * NW + wave) * 64 * 16)));
          }
        });
      } else {
        if (partner >= 0 && i % kSyncEvery == 0) pair_wait(i);
        // tile i landed; the copies of the tiles after it may still be in flight
        const int later = min(AHEAD - 1, n_tiles - 1 - i);
        if (later >= 2) {
          PA_WAIT_VM(2 * COPIES);
        } else if (later == 1) {
          PA_WAIT_VM(COPIES);
        } else {
          PA_WAIT_VM(0);
        }
        lds_barrier();
        flags = *reinterpret_cast<const int4*>(&ovf_s[(i + 1) & 1][0]);
        const bool copy_next = i + AHEAD < n_tiles;
        const int entry = copy_next ? tile_entry(i + AHEAD) : 0;
        scores(tile_ptr(i), s, [&](int ks) {
          if (copy_next && copy_slot(ks)) {
            const int k = (ks - 1) / CS;
            if (k == 0) cp = finish_tile(i + AHEAD, entry);
            copy_piece(cp, k);
          }
        });
        const int valid = tile_valid(i);
        if (valid < TT) {   // the partition's last tile, or an invalid block
          const int lim = valid - 4 * c32;
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = 8 * (e >> 2) + (e & 3) < lim ? s[e] : -INFINITY;
        }
        if (!have_ref && valid > 0) {   // the first tile with a valid token sets the reference
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
          m_ref = fmaxf(mx, __shfl_xor(mx, 32));
          have_ref = true;
          mc = m_ref * c;
        }
      }
      bf16x8_t vop[VA + 1];
      const VBase vb = vstart(tile_ptr(i), vop);
      __builtin_amdgcn_sched_barrier(0);   // the first value reads go out before the weights
      weigh_and_output(i, s, vb, vop, mc, o, lsum, [](int) {});
      if (__builtin_expect(i > 0 && (flags.x | flags.y | flags.z | flags.w) != 0, 0)) {
        ok = false;   // tile i-1 overflowed
        PA_WAIT_VM(0);   // tile i+1's and i+2's copies, before the buffers are reused
        break;
      }
      nrow += TT;
      const bool wrap = nrow == bs;
      nblk += wrap ? 1 : 0;
      nrow = wrap ? 0 : nrow;
    }
    if (ok) {   // the last tile's flags: no later iteration reads them
      lds_barrier();
      ok = !any_overflow((n_tiles - 1) & 1);
    }
    __syncthreads();
    return ok;
  };
  // Scores-only pass: m_ref becomes each head's exact max over the partition.
  auto pass_max = [&](float& m_ref) {
    if (tbl_base != e_first) {
      PA_WAIT_VM(0);
      __syncthreads();
      tbl_base = e_first;
      stage_table(tbl_base);
      __syncthreads();
    }
    for (int i = 0; i < NB - 1 && i < n_tiles; ++i) issue_tile(i);
    for (int i = 0; i < n_tiles; ++i) {
      const int ahead = min(NB - 2, n_tiles - 1 - i);
      if (ahead >= 1) {
        PA_WAIT_VM(COPIES);
      } else {
        PA_WAIT_VM(0);
      }
      lds_barrier();
      if (i + NB - 1 < n_tiles) issue_tile(i + NB - 1);
      f32x16_t s;
      scores(tile_ptr(i), s, no_filler);
      float sc[16];
      masked(s, tile_valid(i), sc);
      m_ref = fmaxf(m_ref, row_max(sc));
    }
    __syncthreads();
  };

  // ---- E4M3 cache: tiles staged through registers (two buffers, no copy in flight
  // across a barrier).  Thread tid fills LDS slots s = tid + 256 k, k < COPIES: slot s is
  // row s / 72, position s % 72 of the tile, which holds source chunk (s % 72) ^ swz(row)
  // -- here 8 codes (8 bytes) of that row, widened to 8 bf16 (16 bytes, exact).  Rows past
  // the partition end repeat its last row; a tile whose block id is invalid reads as
  // zeros.  load_tile_f8 issues the loads (kept in registers), store_tile_f8 widens and
  // writes them once the tile's buffer is free.
  struct RawTile {
    uint2 w[COPIES];
  };
  auto load_tile_f8 = [&](int i, int entry, RawTile& raw) {
    int phys = __builtin_amdgcn_readfirstlane(entry);
    if (phys < 0) {   // invalid block id or an entry past the row
      if (tid == 0) raise_flag(a.flag, entry_error(phys));
      phys = -1;
    }
    const int tok0 = t_begin + i * TT;
    const uint32_t slot = uint32_t(i % NB);
    bad = (bad & ~(1u << slot)) | (uint32_t(phys < 0) << slot);
    const int rows = min(TT, t_end - tok0);
    const char* src = kc + key_row(max(phys, 0), kvh, a.hkv, bs, tok0 % bs, ROW_BYTES_FP8);
#pragma unroll
    for (int k = 0; k < COPIES; ++k) {
      const int s_ = tid + 64 * NW * k;
      const int t = s_ / ROW_CHUNKS, x = s_ % ROW_CHUNKS;
      const int chunk = x ^ swz(t);
      raw.w[k] = phys >= 0
          ? *reinterpret_cast<const uint2*>(src + min(t, rows - 1) * ROW_BYTES_FP8 + 8 * chunk)
          : uint2{0u, 0u};
    }
  };
  // widens piece k of a tile's codes into tile i's buffer (16 bytes per thread)
  auto store_piece_f8 = [&](int i, const RawTile& raw, int k) {
    char* dst = kt + (i % NB) * TILE_BYTES;
    const int s_ = tid + 64 * NW * k;
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w[k].x, 1.0f, false));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w[k].x, 1.0f, true));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w[k].y, 1.0f, false));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.w[k].y, 1.0f, true));
    *reinterpret_cast<uint4*>(dst + 16 * s_) = v;
  };
  auto store_tile_f8 = [&](int i, const RawTile& raw) {
#pragma unroll
    for (int k = 0; k < COPIES; ++k) store_piece_f8(i, raw, k);
  };
  auto restage_first = [&]() {
    if (tbl_base != e_first) {
      __syncthreads();
      tbl_base = e_first;
      stage_table(tbl_base);
      __syncthreads();
    }
  };
  // Accumulating pass: tile i+1's loads are issued before tile i's products, and its codes
  // are widened into the buffer tile i-1 left in the shadow of tile i's later output MFMAs
  // (operands F8_STORE0 ..; in the last iteration that writes unused registers into a
  // buffer nothing reads again); weights and output as in the bf16 path.
  auto pass_acc_f8 = [&](float& m_ref, bool& have_ref, f32x16_t (&o)[MT], float& lsum) -> bool {
    constexpr int F8_STORE0 = 4;
    static_assert(F8_STORE0 + COPIES <= NV, "stores in the output MFMAs' shadow");
    restage_first();
    RawTile raw;
    load_tile_f8(0, tile_entry(0), raw);
    store_tile_f8(0, raw);
    lds_barrier();
    bool ok = true;
    float mc = have_ref ? m_ref * c : 0.f;
    for (int i = 0; i < n_tiles; ++i) {
      if (i + 1 < n_tiles) load_tile_f8(i + 1, tile_entry(i + 1), raw);
      f32x16_t s;
      scores(tile_ptr(i), s, no_filler);
      const int valid = tile_valid(i);
      if (__builtin_expect(valid < TT, 0)) {   // the partition's last tile, or an invalid block
        const int lim = valid - 4 * c32;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 8 * (e >> 2) + (e & 3) < lim ? s[e] : -INFINITY;
      }
      if (__builtin_expect(!have_ref && valid > 0, 0)) {   // the first tile with a valid token sets the reference
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
        m_ref = fmaxf(mx, __shfl_xor(mx, 32));
        have_ref = true;
        mc = m_ref * c;
      }
      bf16x8_t vop[VA + 1];
      const VBase vb = vstart(tile_ptr(i), vop);
      __builtin_amdgcn_sched_barrier(0);   // the first value reads go out before the weights
      weigh_and_output(i, s, vb, vop, mc, o, lsum, [&](int n) {
        if (n >= F8_STORE0 && n < F8_STORE0 + COPIES) store_piece_f8(i + 1, raw, n - F8_STORE0);
      });
      // tile i+1 written by everyone, everyone done with tile i; the overflow flags seen
      lds_barrier();
      if (__builtin_expect(any_overflow(i & 1), 0)) {
        ok = false;
        break;
      }
    }
    __syncthreads();
    return ok;
  };
  // Scores-only pass: m_ref becomes each head's exact max over the partition.
  auto pass_max_f8 = [&](float& m_ref) {
    restage_first();
    RawTile raw;
    load_tile_f8(0, tile_entry(0), raw);
    store_tile_f8(0, raw);
    lds_barrier();
    for (int i = 0; i < n_tiles; ++i) {
      const bool has_next = i + 1 < n_tiles;
      if (has_next) load_tile_f8(i + 1, tile_entry(i + 1), raw);
      f32x16_t s;
      scores(tile_ptr(i), s, no_filler);
      float sc[16];
      masked(s, tile_valid(i), sc);
      m_ref = fmaxf(m_ref, row_max(sc));
      if (has_next) store_tile_f8(i + 1, raw);
      lds_barrier();
    }
    __syncthreads();
  };

  // total weight per head, then o / l (after the last output MFMA drained)
  auto finish = [&](f32x16_t (&o)[MT], float m_ref, float lsum) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                   "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                   "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
    const float lt = lsum + __shfl_xor(lsum, 32);
    const float inv = (F8 ? key_scale : 1.f) / lt;
    const int hh = HW * wave + r32;
    if (hh >= nrow) return;   // a padding row
    float* orow = a.part_out + (out_row + hh) * DV + 4 * c32;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float4 v;
        v.x = o[m][4 * jj + 0] * inv;
        v.y = o[m][4 * jj + 1] * inv;
        v.z = o[m][4 * jj + 2] * inv;
        v.w = o[m][4 * jj + 3] * inv;
        *reinterpret_cast<float4*>(orow + 32 * m + 8 * jj) = v;
        __builtin_amdgcn_sched_barrier(0);
      }
    if (c32 == 0) a.part_lse[out_row + hh] = (m_ref * c + log2f(lt)) * kLn2;
  };

  f32x16_t o[MT];   // O^T tiles: [32-column tile]; lane holds head r32
  float m_ref = -INFINITY;   // reference max (raw score) of head r32 of this wave
  bool have_ref = false;     // set by the first tile with a valid token (every row at once)
  float lsum;                // this lane's share of the sum of weights
  // The accumulating pass runs once, or -- after a score far above the first tile's
  // max -- a second time against each head's exact max, found by a scores-only pass.
  for (;;) {
    zero_tiles(o);
    lsum = 0.f;
    float m_exact = -INFINITY;
    if constexpr (F8) {
      if (pass_acc_f8(m_ref, have_ref, o, lsum)) break;
      pass_max_f8(m_exact);
    } else {
      if (pass_acc(m_ref, have_ref, o, lsum)) break;
      pass_max(m_exact);
    }
    m_ref = m_exact;
    have_ref = true;
  }
  finish(o, m_ref, lsum);
  }

  // partitions past a pair's last one: lse = -inf; their output rows are not written,
  // except in partition 0 of a pair with no tokens, where they are 0 (for every q row of
  // the sequence; none for rows of a sequence whose query_start is invalid)
  for (int y = blockIdx.x; y < Y; y += gridDim.x) {
    const int n = parts_of(y);
    const int b = y / a.n_shards;
    const int r = y - b * a.n_shards;
    int row0 = b, nq = 1;
    if (a.query_start) {
      row0 = a.query_start[b];
      nq = a.query_start[b + 1] - row0;
      if (nq > a.context_lens[b] || nq > a.max_q || row0 < 0 || row0 + nq > a.n_rows) nq = 0;
    }
    // a fused append's slot of a sequence with no tokens (no unit records it)
    if (a.k_new && a.slots_out && r == 0 && tid == 0 && a.context_lens[b] <= 0) a.slots_out[b] = -1;
    for (int qi = 0; qi < nq; ++qi) {
      const int64_t base = (int64_t(row0 + qi) * a.n_shards + r) * a.max_parts;
      for (int p = n; p < a.max_parts; ++p)
        for (int i = tid; i < a.hq; i += 64 * NW) a.part_lse[(base + p) * a.hq + i] = -INFINITY;
      if (n == 0)
        for (int64_t i = tid; i < int64_t(a.hq) * DV; i += 64 * NW) a.part_out[base * a.hq * DV + i] = 0.f;
    }
  }
}

}  // namespace

bool mla_supported(const DecodeArgs& a) {
  return a.dtype == kBF16 && (a.kv_dtype == kBF16 || a.kv_dtype == kFP8) && a.v_cache == nullptr &&
         a.dk == DK && a.dv == DV && a.hkv > 0 && a.hq % a.hkv == 0 && a.bs % TT == 0;
}

int mla_units_per_partition(const DecodeArgs& a) {
  return a.hkv * (a.query_start ? a.max_q : 1) * ((a.hq / a.hkv + HEADS - 1) / HEADS);
}

int mla_workgroups_per_cu(int kv_dtype) {
  int n = 0;
  const void* fn = kv_dtype == kFP8 ? (const void*)decode_mla_kernel<true> : (const void*)decode_mla_kernel<false>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * NW, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

int mla_grid(const DecodeArgs& a) {
  // every workgroup resident: the CUs times the workgroups that fit on one, no more than
  // there can be units
  static std::atomic<int> per_cu[2] = {{0}, {0}};
  std::atomic<int>& slot = per_cu[a.kv_dtype == kFP8 ? 1 : 0];
  int wpc = slot.load(std::memory_order_relaxed);
  if (wpc <= 0) {
    wpc = mla_workgroups_per_cu(a.kv_dtype);
    if (wpc <= 0) wpc = 1;
    slot.store(wpc, std::memory_order_relaxed);
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  const int64_t units = int64_t(a.n_seqs) * a.n_shards * a.max_parts * mla_units_per_partition(a);
  return int(std::max<int64_t>(1, std::min<int64_t>(int64_t(cus) * wpc, units)));
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
  if (a.kv_dtype == kFP8)
    hipLaunchKernelGGL(decode_mla_kernel<true>, dim3(mla_grid(a)), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL(decode_mla_kernel<false>, dim3(mla_grid(a)), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
