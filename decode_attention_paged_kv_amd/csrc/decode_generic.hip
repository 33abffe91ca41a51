// decode_generic.hip -- paged decode attention for any supported shape (VALU, fp32 math).
//
// One workgroup computes one (partition, sequence x shard, KV head, chunk of up to 16
// columns): a column is a query head of that KV head's group, or, with several new
// tokens per sequence, a (new token, query head) pair with its own causal end.  It walks
// the partition's local tokens in tiles of up to 32: the tile's keys and values are
// copied into LDS (as f32) with all of the tile's loads in flight at once, then come the
// scores of the tile (scale * q.k), an online-softmax update of the running max m, sum l
// and output accumulator, and the weighted values.  At the end it writes
// o = acc / l and lse = m + ln l for the partition (DCP page, soroban.highreso.jp,
// "Why long-context LLMs get slow ...": local attention returns output and LSE, and the
// LSEs of online softmax are what the merge reweights with).  Keys and values are read
// through the block table (PagedAttention page, ai-compass.weeybrid.co.jp, block-table
// section).
//
// This kernel covers every shape and element type the ABI accepts (including fp32,
// tiny head sizes and E4M3 caches); the MFMA kernels take the large bf16 shapes.
// E4M3 cache: a stored value is code * scale (per KV head or per tensor); the key
// scale is folded into the score multiplier and the value scale applied to the output.
#include <math.h>

#include "pa_append.h"
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 16;  // query heads per workgroup
constexpr int kTile = 32;   // tokens per tile
constexpr int kAcc = kHeads * 512 / kThreads;
constexpr int kStage = 8192;  // floats of LDS staging the tile's keys and values
constexpr int kDotLanes = 8;  // lanes per score dot product
static_assert(kTile == 32 && kHeads * 16 == kThreads, "softmax: 16 lanes per head, two tokens each");

template <int QT, int KT>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeArgs a) {
  using EQ = Elem<QT>;
  using E = Elem<KT>;
  using raw = typename E::raw;
  const typename EQ::raw* q = static_cast<const typename EQ::raw*>(a.q);
  const raw* kc = static_cast<const raw*>(a.k_cache);
  const raw* vc = static_cast<const raw*>(a.v_cache);

  // grid x = partition + max_parts * (sequence x shard): partition fastest, as a 3-D
  // grid would order them, without a 65535 bound on the (sequence, shard) count
  const int yy = blockIdx.x / a.max_parts;
  const int p = blockIdx.x - yy * a.max_parts;
  const int b = yy / a.n_shards;
  const int r = yy % a.n_shards;
  const int g = a.hq / a.hkv;
  // columns: (new token, query head of this KV head) pairs, token major; kHeads of them
  // per workgroup (one new token per sequence: the heads)
  const int row0 = a.query_start ? a.query_start[b] : b;
  const int nq = a.query_start ? a.query_start[b + 1] - row0 : 1;
  const int chunks = (a.max_q * g + kHeads - 1) / kHeads;
  const int kvh = blockIdx.y / chunks;
  const int c0 = (blockIdx.y % chunks) * kHeads;
  const int nh = min(kHeads, nq * g - c0);       // valid columns here
  const int tid = threadIdx.x;
  const int dk = a.dk, dv = a.dv, bs = a.bs;
  // the step's append, when this launch performs it: before any read of the cache
  if (c0 == 0) fused_append(a, b, r, p, kvh);

  const int L = a.context_lens[b];
  const int Lr = L > 0 ? shard_len(L, a.n_shards, a.interleave, r) : 0;
  const int T = a.part_tokens;
  // several new tokens: more than the context holds, or rows outside the arrays, is an
  // error (flagged, rows left unwritten); one per sequence: an empty context is allowed
  const bool bad = a.query_start && (nq > L || nq > a.max_q || row0 < 0 || row0 + nq > a.n_rows);
  if (p == 0 && tid == 0 && blockIdx.y == 0 && ((Lr + T - 1) / T > a.max_parts || bad))
    raise_flag(a.flag, kErrCapacity);
  if (nh <= 0 || bad) return;
  const int t_begin = p * T;
  auto col_row = [&](int hh) -> int64_t {   // q row * hq + head of column hh
    const int qi = (c0 + hh) / g;
    return int64_t(row0 + qi) * a.hq + kvh * g + (c0 + hh - qi * g);
  };
  auto out_row = [&](int hh) -> int64_t {
    const int qi = (c0 + hh) / g;
    return ((int64_t(row0 + qi) * a.n_shards + r) * a.max_parts + p) * a.hq + kvh * g + (c0 + hh - qi * g);
  };
  auto visible = [&](int hh) -> int {
    return visible_on_shard(L - nq + (c0 + hh) / g, a.n_shards, a.interleave, r);
  };
  const int t_end = min(min(t_begin + T, Lr), visible(nh - 1));
  if (t_begin >= t_end) {  // empty partition: lse = -inf; output rows 0 in partition 0 only
    if (tid < nh) a.part_lse[out_row(tid)] = -INFINITY;
    if (p == 0)
      for (int i = tid; i < nh * dv; i += blockDim.x) a.part_out[out_row(i / dv) * dv + i % dv] = 0.f;
    return;
  }

  __shared__ float q_s[kHeads * kMaxHeadDim];
  __shared__ float kv_s[kStage];   // the tile's keys, then its values (separate cache)
  __shared__ float s_s[kHeads][kTile];
  __shared__ float m_s[kHeads], l_s[kHeads], alpha_s[kHeads];
  __shared__ int64_t kbase_s[kTile], vbase_s[kTile];
  __shared__ int ok_s[kTile];
  __shared__ int lim_s[kHeads];
  if (tid < kHeads) lim_s[tid] = tid < nh ? min(t_end, visible(tid)) : 0;

  // Tiles of up to kTile tokens whose keys (rows padded by one word) and values (ditto)
  // fit the staging buffer.
  const int kstride = dk + 1, vstride = dv + 1;
  const int tile_n = min(kTile, kStage / (kstride + (vc ? vstride : 0)));
  float* k_s = kv_s;
  float* v_s = kv_s + tile_n * kstride;

  float score_mul = a.scale, out_mul = 1.f;
  if (KT == kFP8) {
    const int si = a.n_scales > 1 ? kvh : 0;
    score_mul = a.scale * a.k_scale[si];
    out_mul = vc ? a.v_scale[si] : a.k_scale[si];
  }
  const int32_t* row = a.block_table + (int64_t(b) * a.n_shards + r) * a.max_blocks;
  // Table entry of token t0 + tid of a tile (threads below its length), read ahead of
  // its use; the entry's checks (those of table_entry) come where it is used, so that
  // the read stays in flight meanwhile.
  auto entry_read = [&](int t0, int n_t) -> int {
    const int j = (t0 + tid) / bs;
    return tid < n_t && j < a.max_blocks ? row[j] : 0;
  };
  auto entry_check = [&](int t0, int v) -> int {
    if ((t0 + tid) / bs >= a.max_blocks) return kPastRow;
    return (v < 0 || int64_t(v) >= a.n_blocks) ? kBadId : v;
  };
  int ent = entry_read(t_begin, min(tile_n, t_end - t_begin));   // in flight with the query loads
#pragma unroll 8
  for (int i = tid; i < nh * dk; i += kThreads) q_s[i] = EQ::load(q, col_row(i / dk) * dk + i % dk);
  if (tid < kHeads) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  // Accumulator k of this thread is element tid + k * kThreads of the (head, column)
  // array: head acc_h0 + ..., column acc_d0 + ..., stepped along (no division per k).
  float acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.f;
  const int acc_h0 = tid / dv, acc_d0 = tid - acc_h0 * dv;
  const int h_step = kThreads / dv, d_step = kThreads - h_step * dv;
  auto next_acc = [&](int& hh, int& d) {
    hh += h_step;
    d += d_step;
    if (d >= dv) {
      d -= dv;
      ++hh;
    }
  };

  for (int t0 = t_begin; t0 < t_end; t0 += tile_n) {
    const int n_t = min(tile_n, t_end - t0);
    if (tid < kTile) {
      int ok = 0;
      int64_t kb = 0, vb = 0;
      if (tid < n_t) {
        ent = entry_check(t0, ent);
        if (ent >= 0) {
          ok = 1;
          const int off = (t0 + tid) % bs;
          kb = key_row(ent, kvh, a.hkv, bs, off, dk);
          vb = vc ? value_tile(ent, kvh, a.hkv, bs, dv) + off : kb;
        } else {
          raise_flag(a.flag, entry_error(ent));
        }
      }
      ok_s[tid] = ok;
      kbase_s[tid] = kb;
      vbase_s[tid] = vb;
    }
    __syncthreads();
    // the next tile's entries, in flight with this tile's loads
    if (t0 + tile_n < t_end) ent = entry_read(t0 + tile_n, min(tile_n, t_end - t0 - tile_n));
    // every load of the tile issued before any is waited for: keys row by row, values
    // token-fastest (a block's tokens are adjacent in the value tile)
#pragma unroll 8
    for (int i = tid; i < n_t * dk; i += kThreads) {
      const int tt = i / dk, d = i - tt * dk;
      k_s[tt * kstride + d] = ok_s[tt] ? E::load(kc, kbase_s[tt] + d) : 0.f;
    }
    if (vc) {
#pragma unroll 8
      for (int i = tid; i < n_t * dv; i += kThreads) {
        const int d = i / n_t, tt = i - d * n_t;
        v_s[tt * vstride + d] = ok_s[tt] ? E::load(vc, vbase_s[tt] + int64_t(d) * bs) : 0.f;
      }
    }
    __syncthreads();
    // scores of the (head, token) pairs of the tile: kDotLanes lanes per pair, each a
    // strided share of the dot product, summed across the lanes
    const int n_pairs = nh * n_t;
    for (int base = 0; base < n_pairs * kDotLanes; base += kThreads) {
      const int pi = (base + tid) / kDotLanes, part = tid % kDotLanes;
      const bool valid = pi < n_pairs;
      const int hh = valid ? pi / n_t : 0, tt = valid ? pi - hh * n_t : 0;
      float dot = 0.f;
      if (valid) {
        const float* kr = k_s + tt * kstride;
        const float* qr = q_s + hh * dk;
        for (int d = part; d < dk; d += kDotLanes) dot = fmaf(qr[d], kr[d], dot);
      }
#pragma unroll
      for (int x = 1; x < kDotLanes; x <<= 1) dot += __shfl_xor(dot, x);
      if (valid && part == 0) s_s[hh][tt] = ok_s[tt] && t0 + tt < lim_s[hh] ? dot * score_mul : -INFINITY;
    }
    __syncthreads();
    // online softmax update: 16 lanes per head, two tokens each
    {
      const int hh = tid >> 4, part = tid & 15;
      const bool hv = hh < nh;
      const float s0 = hv && part < n_t ? s_s[hh][part] : -INFINITY;
      const float s1 = hv && part + 16 < n_t ? s_s[hh][part + 16] : -INFINITY;
      const float m_old = hv ? m_s[hh] : -INFINITY;
      float mt = fmaxf(s0, s1);
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
      mt = fmaxf(mt, m_old);
      const float alpha = (mt == -INFINITY) ? 1.f : expf(m_old - mt);
      const float e0 = s0 != -INFINITY ? expf(s0 - mt) : 0.f;
      const float e1 = s1 != -INFINITY ? expf(s1 - mt) : 0.f;
      float sum = e0 + e1;
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) sum += __shfl_xor(sum, x);
      if (hv) {
        if (part < n_t) s_s[hh][part] = e0;
        if (part + 16 < n_t) s_s[hh][part + 16] = e1;
        if (part == 0) {
          l_s[hh] = l_s[hh] * alpha + sum;
          m_s[hh] = mt;
          alpha_s[hh] = alpha;
        }
      }
    }
    __syncthreads();
    // weighted values (values of a latent cache: the first dv entries of the key rows)
    const float* vt = vc ? v_s : k_s;
    const int vs = vc ? vstride : kstride;
#pragma unroll
    for (int k = 0, hh = acc_h0, d = acc_d0; k < kAcc; ++k) {
      if (hh >= nh) break;
      float v = acc[k] * alpha_s[hh];
#pragma unroll 4
      for (int tt = 0; tt < n_t; ++tt) {
        if (!ok_s[tt]) continue;
        v = fmaf(s_s[hh][tt], vt[tt * vs + d], v);
      }
      acc[k] = v;
      next_acc(hh, d);
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0, hh = acc_h0, d = acc_d0; k < kAcc; ++k) {
    if (hh >= nh) break;
    a.part_out[out_row(hh) * dv + d] = l_s[hh] > 0.f ? acc[k] / l_s[hh] * out_mul : 0.f;
    next_acc(hh, d);
  }
  // a column may see none of this partition's tokens: lse -inf
  if (tid < nh) a.part_lse[out_row(tid)] = l_s[tid] > 0.f ? m_s[tid] + logf(l_s[tid]) : -INFINITY;
}

}  // namespace

int generic_column_chunks(const DecodeArgs& a) {
  return (a.max_q * (a.hq / a.hkv) + kHeads - 1) / kHeads;
}

static const void* generic_kernel(int dtype, int kv_dtype) {
  if (kv_dtype == kFP8)
    return dtype == kF32 ? (const void*)decode_generic_kernel<kF32, kFP8>
                         : (const void*)decode_generic_kernel<kBF16, kFP8>;
  return dtype == kF32 ? (const void*)decode_generic_kernel<kF32, kF32>
                       : (const void*)decode_generic_kernel<kBF16, kBF16>;
}

int generic_workgroups_per_cu(int dtype, int kv_dtype) {
  int n = 0;
  const void* f = generic_kernel(dtype, kv_dtype);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.max_parts) * a.n_seqs * a.n_shards), a.hkv * generic_column_chunks(a));
  if (a.kv_dtype == kFP8) {
    if (a.dtype == kF32)
      hipLaunchKernelGGL((decode_generic_kernel<kF32, kFP8>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((decode_generic_kernel<kBF16, kFP8>), grid, dim3(kThreads), 0, st, a);
  } else if (a.dtype == kF32) {
    hipLaunchKernelGGL((decode_generic_kernel<kF32, kF32>), grid, dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_generic_kernel<kBF16, kBF16>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace pa
