// decode_gqa.hip -- paged decode attention on the matrix cores for bf16 GQA/MHA heads
// (head size 64 or 128, block size a multiple of 16, up to 16 query heads per KV head
// per workgroup).
//
// What is computed is the same as in decode_generic.hip: for each partition of a shard's
// local tokens, o = softmax(scale * q.K) V and lse = ln sum exp(scale * q.k), keys and
// values read through the block table (PagedAttention page, ai-compass.weeybrid.co.jp,
// block-table section), outputs and LSEs per partition for the merge (DCP page,
// soroban.highreso.jp, DCP mechanism section).
//
// How it maps onto gfx950:
//  * One workgroup = one (partition, sequence x shard, KV head, 16 columns); a column
//    is a query head of the KV head's group, or, with several new tokens per sequence,
//    a (new token, query head) pair -- then each column also has its own causal end
//    (the new token sees the tokens up to its own position).  Its NW waves split the
//    partition's 16-token sub-tiles into contiguous ranges and merge their (max, sum,
//    output) through LDS at the end.  Each K/V byte is read by exactly one wave, so K/V
//    go straight from HBM into registers (no LDS staging: there is no reuse to stage
//    for).
//  * Scores S^T[token][head] = K (16 x D) . Q^T (D x 16) on v_mfma_f32_16x16x32_bf16:
//    lane (row = lane % 16, group = lane / 16) supplies 8 consecutive head-dim values
//    of key row `row` -- one 16-byte load per MFMA -- and the result leaves scores of
//    tokens 4*group .. 4*group+3 for head lane % 16 in each lane.
//  * Output O^T[d][head] += V^T (16 x 32 tokens) . P^T (32 tokens x 16 heads) on the
//    same instruction.  The value cache stores each block as [d][token]; a lane's
//    operand is 4 tokens of one d row per 16-token sub-tile, and the weights P^T it
//    needs are exactly the scores it already holds (no shuffles for them).  Values are
//    loaded 16 bytes per lane -- whole d rows, 1 KiB per load instruction -- and handed
//    to the lanes whose operand needs them by lane-row swaps (Tile::value_pairs,
//    Tile::value_words); narrower loads streamed measurably slower from HBM.  Value
//    loads take the non-temporal cache policy, key loads the default one.
//  * The softmax weights enter P.V as two bf16 terms, hi = bf16(p) and
//    lo = bf16(p - hi), so they keep ~16 significant bits; K, V and q are used exactly.
//  * Online softmax in base 2: scores stay raw, p = exp2(s*c - m*c) with
//    c = scale * log2(e); the running max is shared by the four lanes of a head with two
//    cross-lane exchanges per 32 tokens; each lane keeps its own partial sum until the
//    end.  The output is rescaled only when some running max moved.
//  * Masked tokens (past the partition end) take score -inf by select and their value
//    entries are zeroed by select, so unused cache slots (whatever they hold) never
//    reach the sums.
//  * E4M3 cache (codes times a per-head or per-tensor scale): keys and values are
//    loaded as codes -- half the bytes -- and widened to bf16 in registers right
//    before their MFMA (every E4M3 value is exact in bf16).  A lane's key bytes for the
//    score MFMAs of a sub-tile are D/4 consecutive bytes (one or two 16-byte loads),
//    dimension grp*D/4 + 8j + e for MFMA j, element e; the query operand is taken in
//    the same order (a dot product does not depend on the order of its terms).  The
//    key scale joins the score multiplier and the value scale the final division.
//  * Block ids: each wave loads 64 consecutive block-table entries with one vector load
//    and reads them back one at a time with readlane.  The next step's keys are loaded
//    into the key registers as soon as the scores have used them, its values into the
//    value registers as soon as the output product has, so each wave keeps a step of
//    loads in flight while it computes, without a second register buffer.
#include <math.h>

#include <type_traits>

#include "pa_append.h"
#include "pa_common.h"
#include "pa_launch.h"

#ifndef PA_GQA_MIN_WAVES_FP8
#define PA_GQA_MIN_WAVES_FP8 2
#endif

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// Value loads use the non-temporal policy (`nt`): the cache is read once per step, and on
// this GPU `nt` streams random 2-16 KiB chunks from HBM ~11 % faster.  It pays only where
// one load instruction covers whole 128-byte lines, as a value load does (d rows x all
// tokens of the sub-tile, contiguous).  A key load covers half of each token's line (the
// other half comes with the next instruction), and under `nt` the long-context decode
// measured 5 % slower with key loads included, 5 % faster without them.
__device__ inline u32x4_t load_nt(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reductions over lanes l, l^16, l^32, l^48 (the four lanes of one column).  A row swap
// (v_permlane16_swap / v_permlane32_swap, both operands the same value) leaves each lane
// holding its own value and its partner's (lane ^ 16, lane ^ 32), so one vector
// instruction and one max/add replace each exchange through the LDS crossbar.
__device__ inline float xor_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// 2^x for the softmax weights (the library call; the transcendental unit's instruction
// alone measured no faster).
__device__ inline float exp2_w(float x) { return exp2f(x); }

__device__ inline float xor_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Keep the bf16 halves of a 32-bit word whose tokens are valid.
__device__ inline uint32_t keep(uint32_t w, bool lo_ok, bool hi_ok) {
  return w & ((lo_ok ? 0x0000ffffu : 0u) | (hi_ok ? 0xffff0000u : 0u));
}

// Two E4M3 codes (bytes 2*hi, 2*hi+1 of w) as two bf16, exactly.
template <bool HI>
__device__ inline uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int D, int SUBS, int KT>
struct Tile {
  static_assert(SUBS % 2 == 0, "the output product takes sub-tiles in pairs");
  static constexpr bool F8 = KT == kFP8;
  static constexpr int KJ = D / 32;  // score MFMAs per sub-tile
  static constexpr int NT = D / 16;  // output tiles of 16 d rows
  // bf16: one 16-byte word per score MFMA; E4M3: the lane's D/4 key bytes
  static constexpr int KW = F8 ? D / 64 : KJ;
  u32x4_t k[SUBS][KW];
  // Values: each lane loads 16 bytes of a d row, so one load instruction reads 1 KiB of
  // whole d rows (contiguous when a block holds 16 tokens); the bytes are then handed to
  // the lanes whose operand needs them (value_pairs, value_words).  bf16: group q covers output tiles 2q, 2q+1; E4M3: tiles 4q .. 4q+3.
  static constexpr int NV = F8 ? NT / 4 : NT / 2;
  u32x4_t v[SUBS][NV];

  // key operand of score MFMA j of sub-tile t
  __device__ inline bf16x8_t key(int t, int j) const {
    if constexpr (F8) {
      const u32x4_t w = k[t][j >> 1];
      const uint32_t d0 = (j & 1) ? w[2] : w[0];
      const uint32_t d1 = (j & 1) ? w[3] : w[1];
      const u32x4_t x = {e4m3x2_to_bf16x2<false>(d0), e4m3x2_to_bf16x2<true>(d0),
                         e4m3x2_to_bf16x2<false>(d1), e4m3x2_to_bf16x2<true>(d1)};
      return __builtin_bit_cast(bf16x8_t, x);
    } else {
      return __builtin_bit_cast(bf16x8_t, k[t][j]);
    }
  }
  // bf16: w[n] = tokens 4 grp .. 4 grp + 3 of d row 16n + col of sub-tile t (the lane's
  // operand words for output tile n).  Lane row 2a + b loaded tokens 8b .. 8b + 7 of d row
  // 16(2q + a) + col.  Lane row g needs, for tile 2q + h, dwords 2(g & 1) and 2(g & 1) + 1
  // of lane row 2h + (g >> 1): the bits (a, b, dword pair) must become (b, pair, h), which
  // a 16-lane swap (row bit b <-> register bit) and then a 32-lane swap (row bit a <->
  // register bit) do for each dword of the pair.
  __device__ inline void value_pairs(int t, uint2 (&w)[NT]) const {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const auto a = __builtin_amdgcn_permlane16_swap(v[t][q][k], v[t][q][2 + k], false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[1], false, false);
        if (k == 0) { w[2 * q].x = b[0]; w[2 * q + 1].x = b[1]; }
        else { w[2 * q].y = b[0]; w[2 * q + 1].y = b[1]; }
      }
    }
  }
  // E4M3: w[n] = the 4 codes (tokens 4 grp .. 4 grp + 3) of d row 16n + col of sub-tile
  // t.  For group q the four 16-lane rows hold a 4 x 4 block of dwords (row h: d row
  // 16(4q + h) + col, dword g: tokens 4g .. 4g + 3); transposing it across the rows, by
  // 32-lane swaps and then 16-lane swaps, leaves row g with dword g of every row.
  __device__ inline void value_words(int t, uint32_t (&w)[NT]) const {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      uint32_t r0 = v[t][q][0], r1 = v[t][q][1], r2 = v[t][q][2], r3 = v[t][q][3];
      const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
      const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
      r0 = a[0], r2 = a[1], r1 = b[0], r3 = b[1];
      const auto c = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
      const auto d = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
      w[4 * q + 0] = c[0], w[4 * q + 1] = c[1], w[4 * q + 2] = d[0], w[4 * q + 3] = d[1];
    }
  }
};

// Where a step's sub-tiles are: local token of the first row (-1: no sub-tile), cache
// offset of its (block, KV head) and row within the block (both 0 when absent).
template <int SUBS>
struct Step {
  int tok0[SUBS];
  int64_t base[SUBS];
  int sub[SUBS];
};

// At least two waves per SIMD (registers capped at 256): each wave's step of loads in
// flight is what hides the HBM latency.
template <int D, int NW, int SUBS, int KT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(KT == kFP8 ? PA_GQA_MIN_WAVES_FP8 : 2))) void decode_gqa_kernel(
    DecodeArgs a) {
  using TileT = Tile<D, SUBS, KT>;
  using raw = typename Elem<KT>::raw;
  constexpr bool F8 = TileT::F8;
  constexpr int KJ = TileT::KJ;
  constexpr int NT = TileT::NT;
  constexpr int KW = TileT::KW;
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const raw* __restrict__ kc = static_cast<const raw*>(a.k_cache);
  const raw* __restrict__ vc = static_cast<const raw*>(a.v_cache);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;   // key row (A operand) / column (B operand, results)
  const int grp = lane >> 4;   // k-slot group
  // grid x = partition + max_parts * (sequence x shard): partition fastest, as a 3-D
  // grid would order them, without a 65535 bound on the (sequence, shard) count
  const int yy = blockIdx.x / a.max_parts;
  const int p = blockIdx.x - yy * a.max_parts;
  const int b = yy / a.n_shards;
  const int r = yy % a.n_shards;
  const int g = a.hq / a.hkv;
  // Columns of the products are (new token, query head of this KV head) pairs, token
  // major; a workgroup takes 16 of them.  One new token per sequence: the heads.
  const int row0 = a.query_start ? a.query_start[b] : b;         // q row of its first new token
  const int nq = a.query_start ? a.query_start[b + 1] - row0 : 1;
  const int chunks = (a.max_q * g + 15) >> 4;
  const int kvh = blockIdx.y / chunks;
  const int c0 = (blockIdx.y % chunks) * 16;
  const int ncol = min(16, nq * g - c0);         // valid columns here
  const int bs = a.bs;
  const int T = a.part_tokens;
  // The step's append, when this launch performs it: the new rows are read first, then
  // the context length and the table window below arrive together with them, and the
  // rows are stored (append_store) before any read of the cache.
  NewRowShare new_rows;
  if (c0 == 0) new_rows = append_fetch(a, b, kvh);
  const int L = a.context_lens[b];
  // Table window: entries tbl_base .. tbl_base + 63 of the shard's row, one per lane,
  // starting at the partition's first block.  Read raw here, so that no wait follows the
  // read, and checked as table_entry checks before the first lookup.
  const int32_t* row = a.block_table + (int64_t(b) * a.n_shards + r) * a.max_blocks;
  auto raw_entry = [&](int j) -> int { return j < a.max_blocks ? row[j] : 0; };
  int tbl_base = p * T / bs;
  int tbl = raw_entry(tbl_base + lane);

  // query operand: lane (column col, group grp) holds q[row][head][32j + 8grp .. +7]
  // (bf16 cache) or [grp*D/4 + 8j .. +7] (E4M3 cache), the order of the key operand.
  // Issued with the reads above, so that the append's wait for its stores also covers
  // them; the rows are inside the array whenever query_start is (checked again below).
  bf16x8_t qop[KJ];
  {
    const bool rows_ok = !a.query_start || (row0 >= 0 && nq >= 0 && row0 + nq <= a.n_rows);
    const int qi = (c0 + col) / g, h = (c0 + col) - qi * g;
    const uint16_t* qrow = q + (int64_t(row0 + qi) * a.hq + kvh * g + h) * D +
                           (F8 ? grp * (D / 4) : 8 * grp);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      if (col < ncol && rows_ok)
        qop[j] = *reinterpret_cast<const bf16x8_t*>(qrow + (F8 ? 8 * j : 32 * j));
      else
        qop[j] = bf16x8_t{};
    }
  }

  if (c0 == 0)
    append_store(a, new_rows, b, r, p, kvh, L, [&](int j) {
      return j >= tbl_base && j - tbl_base < 64 ? __builtin_amdgcn_readlane(tbl, j - tbl_base) : row[j];
    });

  const int Lr = L > 0 ? shard_len(L, a.n_shards, a.interleave, r) : 0;
  // several new tokens: more than the context holds, or rows outside the arrays, is an
  // error (flagged, rows left unwritten); one per sequence: an empty context is allowed
  const bool bad = a.query_start && (nq > L || nq > a.max_q || row0 < 0 || row0 + nq > a.n_rows);
  if (p == 0 && threadIdx.x == 0 && blockIdx.y == 0 && ((Lr + T - 1) / T > a.max_parts || bad))
    raise_flag(a.flag, kErrCapacity);
  if (ncol <= 0 || bad) return;  // no rows here (or bad input)
  const int t_begin = p * T;
  // output row of column cc (< ncol), and how many of the shard's tokens it may see
  auto out_row = [&](int cc) -> int64_t {
    const int qi = (c0 + cc) / g, h = (c0 + cc) - qi * g;
    return ((int64_t(row0 + qi) * a.n_shards + r) * a.max_parts + p) * a.hq + kvh * g + h;
  };
  auto visible = [&](int cc) -> int {
    return visible_on_shard(L - nq + (c0 + cc) / g, a.n_shards, a.interleave, r);
  };
  // the last column sees the most: the workgroup's tokens end there
  const int t_end = min(min(t_begin + T, Lr), visible(ncol - 1));
  if (t_begin >= t_end) {  // empty partition: lse = -inf; output rows 0 in partition 0 only
    if (threadIdx.x < ncol) a.part_lse[out_row(threadIdx.x)] = -INFINITY;
    if (p == 0)
      for (int i = threadIdx.x; i < ncol * D; i += 64 * NW) a.part_out[out_row(i / D) * D + i % D] = 0.f;
    return;
  }
  const int lim = min(t_end, visible(min(col, ncol - 1)));   // this lane's column's end

  // this wave's contiguous range of steps of SUBS 16-token sub-tiles
  const int u0 = t_begin >> 4;                   // first sub-tile (T and bs are multiples of 16)
  const int n_u = (t_end - t_begin + 15) >> 4;   // sub-tiles in the partition
  const int n_steps = (n_u + SUBS - 1) / SUBS;
  const int per = n_steps / NW, extra = n_steps % NW;
  const int s_lo = wave * per + min(wave, extra);
  const int s_hi = s_lo + per + (wave < extra ? 1 : 0);

  const int spb = bs >> 4;  // sub-tiles per block

  tbl = tbl_base + lane >= a.max_blocks ? kPastRow : (tbl < 0 || int64_t(tbl) >= a.n_blocks ? kBadId : tbl);
  auto block_of = [&](int e) -> int {            // e: logical block entry (wave-uniform)
    if (e - tbl_base >= 64 || e < tbl_base) {
      tbl_base = e;
      tbl = table_entry(row, e + lane, a.max_blocks, a.n_blocks);   // errors reported when used
    }
    return __builtin_amdgcn_readlane(tbl, e - tbl_base);
  };

  // Loads are split by operand: the next step's keys go into the key registers as soon as
  // the scores have consumed them, its values into the value registers as soon as the
  // output product has, so every wave keeps a step of loads in flight while it computes.
  using StepT = Step<SUBS>;
  auto locate = [&](StepT& st, int s) {
#pragma unroll
    for (int t = 0; t < SUBS; ++t) {
      const int u_rel = SUBS * s + t;
      st.tok0[t] = -1;
      st.base[t] = 0;
      st.sub[t] = 0;
      if (u_rel < n_u) {
        const int u = u0 + u_rel;
        const int e = u / spb;
        const int phys = block_of(e);
        if (phys >= 0) {
          st.tok0[t] = u << 4;
          st.base[t] = key_row(phys, kvh, a.hkv, bs, 0, D);   // the value tile: the same offset
          st.sub[t] = (u - e * spb) << 4;
        } else if (lane == 0) {
          raise_flag(a.flag, entry_error(phys));
        }
      }
    }
  };
  // Loads are unconditional (an absent sub-tile reads the first rows of block 0, which
  // always exist, and is masked afterwards), so the compiler's waits can count loads
  // exactly instead of waiting for all of them after a branch.
  auto load_k = [&](TileT& tl, const StepT& st) {
#pragma unroll
    for (int t = 0; t < SUBS; ++t) {
      const raw* kp = kc + st.base[t] + int64_t(st.sub[t] + col) * D + (F8 ? grp * (D / 4) : 8 * grp);
#pragma unroll
      for (int w = 0; w < KW; ++w)
        tl.k[t][w] = *reinterpret_cast<const u32x4_t*>(kp + (F8 ? 16 * w : 32 * w));
    }
  };
  auto load_v = [&](TileT& tl, const StepT& st) {
#pragma unroll
    for (int t = 0; t < SUBS; ++t) {
      // 16 bytes per lane rather than the 4 (E4M3) or 8 (bf16) its operand takes: loads
      // of 256 or 512 bytes per instruction measured slower (E4M3: 0.455 vs 0.378 ms on
      // the long-context batch; bf16: 0.744 vs 0.717 ms)
      if constexpr (F8) {
        const raw* vp = vc + st.base[t] + int64_t(16 * grp + col) * bs + st.sub[t];
#pragma unroll
        for (int q = 0; q < TileT::NV; ++q)
          tl.v[t][q] = load_nt(reinterpret_cast<const u32x4_t*>(vp + int64_t(64 * q) * bs));
      } else {
        const raw* vp = vc + st.base[t] + int64_t(16 * (grp >> 1) + col) * bs + st.sub[t] + 8 * (grp & 1);
#pragma unroll
        for (int q = 0; q < TileT::NV; ++q)
          tl.v[t][q] = load_nt(reinterpret_cast<const u32x4_t*>(vp + int64_t(32 * q) * bs));
      }
    }
  };

  float key_scale = 1.f, value_scale = 1.f;
  if constexpr (F8) {
    const int si = a.n_scales > 1 ? kvh : 0;
    key_scale = a.k_scale[si];
    value_scale = a.v_scale[si];
  }
  const float c = a.scale * key_scale * kLog2e;
  float m = -INFINITY;  // running max of raw scores, head col
  float lsum = 0.f;     // this lane's partial sum of weights
  f32x4_t o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one step: scores of the sub-tiles, then after_scores() (the key registers are free),
  // softmax and the output product, then after_output() (the value registers are free)
  auto compute = [&](TileT& tl, const StepT& st, auto&& after_scores, auto&& after_output) {
    // the sub-tiles' score chains are interleaved (k-step outer), so consecutive MFMAs
    // never wait on each other; absent sub-tiles hold whatever block 0 holds and are
    // masked below
    float sc[SUBS][4];
    f32x4_t acc[SUBS];
#pragma unroll
    for (int t = 0; t < SUBS; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j)
#pragma unroll
      for (int t = 0; t < SUBS; ++t) acc[t] = mfma16x16x32(tl.key(t, j), qop[j], acc[t]);
#pragma unroll
    for (int t = 0; t < SUBS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = st.tok0[t] + 4 * grp + i;
        const bool ok = st.tok0[t] >= 0 && tok < lim;
        sc[t][i] = ok ? acc[t][i] : -INFINITY;
      }
    after_scores();
    float mt = m;
#pragma unroll
    for (int t = 0; t < SUBS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[t][i]);
    mt = xor_max(mt);
    const float alpha = (mt == -INFINITY) ? 1.f : exp2_w((m - mt) * c);
    m = mt;
    const float mc = (mt == -INFINITY) ? 0.f : mt * c;   // a column that has seen nothing yet
    float pv[SUBS][4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < SUBS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[t][i] = exp2_w(fmaf(sc[t][i], c, -mc));
        psum += pv[t][i];
      }
    lsum = fmaf(lsum, alpha, psum);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] *= alpha;
    }
    // value operand; tokens that are masked (or sub-tiles not loaded) contribute zeros
    bool ok[SUBS][4];
    bool full = true;
#pragma unroll
    for (int t = 0; t < SUBS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[t][i] = st.tok0[t] >= 0 && st.tok0[t] + 4 * grp + i < t_end;
        full = full && ok[t][i];
      }
#pragma unroll
    for (int t2 = 0; t2 < SUBS; t2 += 2) {   // one MFMA k-step = two sub-tiles (32 tokens)
      bf16x8_t phi, plo;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 h = (__bf16)pv[t2 + t][i];
          phi[4 * t + i] = h;
          plo[4 * t + i] = (__bf16)(pv[t2 + t][i] - (float)h);
        }
      uint32_t wa[NT], wb[NT];
      uint2 pa[NT], pb[NT];
      if constexpr (F8) {
        tl.value_words(t2, wa);
        tl.value_words(t2 + 1, wb);
      } else {
        tl.value_pairs(t2, pa);
        tl.value_pairs(t2 + 1, pb);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        uint2 va, vb;
        if constexpr (F8) {
          va = uint2{e4m3x2_to_bf16x2<false>(wa[n]), e4m3x2_to_bf16x2<true>(wa[n])};
          vb = uint2{e4m3x2_to_bf16x2<false>(wb[n]), e4m3x2_to_bf16x2<true>(wb[n])};
        } else {
          va = pa[n];
          vb = pb[n];
        }
        if (!__all(full)) {
          va.x = keep(va.x, ok[t2][0], ok[t2][1]);
          va.y = keep(va.y, ok[t2][2], ok[t2][3]);
          vb.x = keep(vb.x, ok[t2 + 1][0], ok[t2 + 1][1]);
          vb.y = keep(vb.y, ok[t2 + 1][2], ok[t2 + 1][3]);
        }
        const u32x4_t w = {va.x, va.y, vb.x, vb.y};
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, w);
        o[n] = mfma16x16x32(vop, phi, o[n]);
        o[n] = mfma16x16x32(vop, plo, o[n]);
      }
    }
    after_output();
  };

  if (s_lo < s_hi) {
    TileT A;
    StepT cur, nxt;
    locate(cur, s_lo);
    load_k(A, cur);
    load_v(A, cur);
    for (int s = s_lo; s < s_hi; ++s) {
      // the step after the wave's last is located as absent (block 0, masked): its loads
      // are issued anyway, so no branch sits around a load
      compute(
          A, cur,
          [&] {
            locate(nxt, s + 1 < s_hi ? s + 1 : n_steps);
            load_k(A, nxt);
          },
          [&] { load_v(A, nxt); });
      cur = nxt;
    }
  }

  // ---- merge the waves' partial results through LDS
  __shared__ float m_s[NW][16];
  __shared__ float l_s[NW][16];
  __shared__ float o_s[NW][D][17];
  const float lt = xor_sum(lsum);
  if (grp == 0) {
    m_s[wave][col] = m;
    l_s[wave][col] = lt;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) o_s[wave][16 * n + 4 * grp + i][col] = o[n][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < ncol * D; idx += 64 * NW) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, m_s[w2][hh]);
    float Ls = 0.f, acc = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      const float mw = m_s[w2][hh];
      const float f = (mw == -INFINITY) ? 0.f : exp2f((mw - M) * c);
      Ls = fmaf(f, l_s[w2][hh], Ls);
      acc = fmaf(f, o_s[w2][d][hh], acc);
    }
    const int64_t orow = out_row(hh);
    const bool seen = Ls > 0.f;       // a column may see none of this partition's tokens
    a.part_out[orow * D + d] = seen ? acc / Ls * value_scale : 0.f;
    if (d == 0) a.part_lse[orow] = seen ? (M * c + log2f(Ls)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool gqa_supported(const DecodeArgs& a) {
  return a.dtype == kBF16 && (a.kv_dtype == kBF16 || a.kv_dtype == kFP8) && a.v_cache != nullptr &&
         a.dk == a.dv && (a.dk == 64 || a.dk == 128) && a.bs % 16 == 0;
}

int gqa_column_chunks(const DecodeArgs& a) { return (a.max_q * (a.hq / a.hkv) + 15) / 16; }

#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 8
#endif
#ifndef PA_GQA_SUBS
#define PA_GQA_SUBS 2
#endif
#ifndef PA_GQA_SUBS_FP8
#define PA_GQA_SUBS_FP8 2   // measured: as fast as four sub-tiles and lighter on registers
#endif
#ifndef PA_GQA_WAVES_FP8
#define PA_GQA_WAVES_FP8 4  // measured: the E4M3 kernel runs faster as smaller workgroups
#endif

#ifndef PA_GQA_SHORT_TOKENS
#define PA_GQA_SHORT_TOKENS 512   // partitions this short (or several new tokens) use 4 waves
#endif

namespace {
template <int D, int NW, int KT>
const void* gqa_kernel() {
  constexpr int SUBS = KT == kFP8 ? PA_GQA_SUBS_FP8 : PA_GQA_SUBS;
  return (const void*)decode_gqa_kernel<D, NW, SUBS, KT>;
}

// Waves per workgroup.  Measured: long single-token partitions run best with 8 waves
// (one workgroup per compute unit, each wave a long contiguous range); short partitions
// and several new tokens per sequence (more, shorter workgroups) with 4; the E4M3 cache
// with 4.
int gqa_waves(const DecodeArgs& a) {
  if (a.kv_dtype == kFP8) return PA_GQA_WAVES_FP8;
  return (a.max_q > 1 || a.part_tokens <= PA_GQA_SHORT_TOKENS) ? 4 : PA_GQA_WAVES;
}

const void* gqa_kernel_for(const DecodeArgs& a) {
  const bool d128 = a.dk == 128;
  if (a.kv_dtype == kFP8)
    return d128 ? gqa_kernel<128, PA_GQA_WAVES_FP8, kFP8>() : gqa_kernel<64, PA_GQA_WAVES_FP8, kFP8>();
  if (gqa_waves(a) == 4) return d128 ? gqa_kernel<128, 4, kBF16>() : gqa_kernel<64, 4, kBF16>();
  return d128 ? gqa_kernel<128, PA_GQA_WAVES, kBF16>() : gqa_kernel<64, PA_GQA_WAVES, kBF16>();
}
}  // namespace

int gqa_workgroups_per_cu(const DecodeArgs& a) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_kernel_for(a), 64 * gqa_waves(a), 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.max_parts) * a.n_seqs * a.n_shards), a.hkv * gqa_column_chunks(a));
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  return hipLaunchKernel(gqa_kernel_for(a), grid, dim3(64 * gqa_waves(a)), args, 0, st);
}

}  // namespace pa
