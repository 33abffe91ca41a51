// decode_generic.hip -- paged decode attention for any supported shape (VALU, fp32 math).
//
// One workgroup computes one (partition, sequence x shard, KV head, chunk of up to 16
// columns): a column is a query head of that KV head's group, or, with several new
// tokens per sequence, a (new token, query head) pair with its own causal end.  It walks the partition's local tokens in tiles
// of 32: scores of the tile (scale * q.k), an online-softmax update of the running max m,
// sum l and output accumulator, then the weighted values.  At the end it writes
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
  __shared__ float s_s[kHeads][kTile];
  __shared__ float m_s[kHeads], l_s[kHeads], alpha_s[kHeads];
  __shared__ int64_t kbase_s[kTile], vbase_s[kTile];
  __shared__ int ok_s[kTile];
  __shared__ int lim_s[kHeads];
  if (tid < kHeads) lim_s[tid] = tid < nh ? min(t_end, visible(tid)) : 0;

  float score_mul = a.scale, out_mul = 1.f;
  if (KT == kFP8) {
    const int si = a.n_scales > 1 ? kvh : 0;
    score_mul = a.scale * a.k_scale[si];
    out_mul = vc ? a.v_scale[si] : a.k_scale[si];
  }
  for (int i = tid; i < nh * dk; i += kThreads) q_s[i] = EQ::load(q, col_row(i / dk) * dk + i % dk);
  if (tid < kHeads) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.f;

  const int32_t* row = a.block_table + (int64_t(b) * a.n_shards + r) * a.max_blocks;
  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int n_t = min(kTile, t_end - t0);
    if (tid < kTile) {
      int ok = 0;
      int64_t kb = 0, vb = 0;
      if (tid < n_t) {
        const int t = t0 + tid;
        const int64_t phys = table_block(row, t / bs, a.max_blocks, a.n_blocks, a.flag);
        if (phys >= 0) {
          ok = 1;
          const int off = t % bs;
          kb = key_row(phys, kvh, a.hkv, bs, off, dk);
          vb = vc ? value_tile(phys, kvh, a.hkv, bs, dv) + off : kb;
        }
      }
      ok_s[tid] = ok;
      kbase_s[tid] = kb;
      vbase_s[tid] = vb;
    }
    __syncthreads();
    // scores
    for (int idx = tid; idx < kHeads * kTile; idx += kThreads) {
      const int hh = idx / kTile, tt = idx % kTile;
      float s = -INFINITY;
      if (hh < nh && tt < n_t && ok_s[tt] && t0 + tt < lim_s[hh]) {
        const int64_t kb = kbase_s[tt];
        float dot = 0.f;
        for (int d = 0; d < dk; ++d) dot = fmaf(q_s[hh * dk + d], E::load(kc, kb + d), dot);
        s = dot * score_mul;
      }
      s_s[hh][tt] = s;
    }
    __syncthreads();
    // online softmax update, one thread per head
    if (tid < nh) {
      float mt = m_s[tid];
      for (int tt = 0; tt < n_t; ++tt) mt = fmaxf(mt, s_s[tid][tt]);
      const float alpha = (mt == -INFINITY) ? 1.f : expf(m_s[tid] - mt);
      float sum = 0.f;
      for (int tt = 0; tt < kTile; ++tt) {
        const float e = (tt < n_t && s_s[tid][tt] != -INFINITY) ? expf(s_s[tid][tt] - mt) : 0.f;
        s_s[tid][tt] = e;
        sum += e;
      }
      l_s[tid] = l_s[tid] * alpha + sum;
      m_s[tid] = mt;
      alpha_s[tid] = alpha;
    }
    __syncthreads();
    // weighted values
#pragma unroll
    for (int k = 0; k < kAcc; ++k) {
      const int idx = tid + k * kThreads;
      const int hh = idx / dv, d = idx % dv;
      if (hh < nh) {
        float v = acc[k] * alpha_s[hh];
        for (int tt = 0; tt < n_t; ++tt) {
          if (!ok_s[tt]) continue;
          const float x = vc ? E::load(vc, vbase_s[tt] + int64_t(d) * bs) : E::load(kc, vbase_s[tt] + d);
          v = fmaf(s_s[hh][tt], x, v);
        }
        acc[k] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kAcc; ++k) {
    const int idx = tid + k * kThreads;
    const int hh = idx / dv, d = idx % dv;
    if (hh < nh) a.part_out[out_row(hh) * dv + d] = l_s[hh] > 0.f ? acc[k] / l_s[hh] * out_mul : 0.f;
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
