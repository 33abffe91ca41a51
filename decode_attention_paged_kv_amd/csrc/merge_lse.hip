// merge_lse.hip -- combine per-partition attention results with their LSEs.
//
// The DCP page (soroban.highreso.jp, "Why long-context LLMs get slow ...", DCP mechanism
// section) finishes a decode step by sharing the LSE of every partial result,
// correcting each partial output with its weight and summing.  Written out: with
// lse = M + ln sum_p exp(lse_p - M), M = max_p lse_p, part p has weight exp(lse_p - lse).
// Parts with lse_p = -inf are empty and skipped (no -inf - -inf is ever formed); their
// part_out rows are never read.
//
// One workgroup per (sequence, head) and column block; with at most 64 parts, one wave
// per (sequence, head) and block of columns.
#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;  // parts whose weights are staged in LDS at a time

__device__ inline float block_reduce(float v, float* red, bool is_max) {
  for (int o = 32; o > 0; o >>= 1) {
    const float x = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, x) : v + x;
  }
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

// Each workgroup covers CB consecutive output columns of one (sequence, head).  Parts
// with lse = -inf are empty (their part_out rows are never read); the others are listed
// compactly in LDS.  Threads form a (part group) x (column group) grid: each owns VEC
// consecutive columns and sums every npg-th listed part, so npg parts are read at once
// with no data-dependent branch; the npg partial sums are then added through LDS.
template <int VEC>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ part_out,
                                                         const float* __restrict__ part_lse,
                                                         int n_parts, int hq, int dv, int cb,
                                                         void* out, int out_dtype, float* lse_out) {
  const int b = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  __shared__ float red[kThreads / 64];
  __shared__ float w_s[kChunk];
  __shared__ int idx_s[kChunk];
  __shared__ int cnt_s[kThreads / 64];
  __shared__ float acc_s[kThreads * VEC];
  const float* lse_p = part_lse + int64_t(b) * n_parts * hq + h;       // stride hq
  const float* o_p = part_out + (int64_t(b) * n_parts * hq + h) * dv;  // stride hq*dv

  float m = -INFINITY;
  for (int p = threadIdx.x; p < n_parts; p += kThreads) m = fmaxf(m, lse_p[int64_t(p) * hq]);
  m = block_reduce(m, red, true);
  float total = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.f;
    for (int p = threadIdx.x; p < n_parts; p += kThreads) {
      const float x = lse_p[int64_t(p) * hq];
      if (x != -INFINITY) s += expf(x - m);
    }
    s = block_reduce(s, red, false);
    total = m + logf(s);
  }

  const int col0 = blockIdx.y * cb;
  const int ncols = min(cb, dv - col0);
  const int ncg = ncols / VEC;                 // column groups (VEC divides dv and cb)
  const int npg = kThreads / ncg;              // part groups
  const int cg = threadIdx.x % ncg;
  const int pg = threadIdx.x / ncg;
  const bool active = pg < npg;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  const int64_t stride = int64_t(hq) * dv;
  for (int p0 = 0; p0 < n_parts && total != -INFINITY; p0 += kChunk) {
    const int np = min(kChunk, n_parts - p0);
    // list the non-empty parts of this chunk, in order, with their weights
    int base = 0;
    for (int i0 = 0; i0 < np; i0 += kThreads) {
      __syncthreads();
      const int i = i0 + threadIdx.x;
      float w = 0.f;
      if (i < np) {
        const float x = lse_p[int64_t(p0 + i) * hq];
        if (x != -INFINITY) w = expf(x - total);
      }
      const unsigned long long ball = __ballot(w != 0.f);
      if (lane == 0) cnt_s[wv] = __popcll(ball);
      __syncthreads();
      int before = base;
      for (int j = 0; j < wv; ++j) before += cnt_s[j];
      if (w != 0.f) {
        const int pos = before + __popcll(ball & ((1ull << lane) - 1ull));
        w_s[pos] = w;
        idx_s[pos] = p0 + i;
      }
      for (int j = 0; j < kThreads / 64; ++j) base += cnt_s[j];
    }
    __syncthreads();
    if (active) {
      const float* src = o_p + col0 + cg * VEC;
#pragma unroll 8
      for (int i = pg; i < base; i += npg) {
        const float wi = w_s[i];
        const float* sp = src + int64_t(idx_s[i]) * stride;
        if (VEC == 4) {
          const float4 v = *reinterpret_cast<const float4*>(sp);
          acc[0] = fmaf(wi, v.x, acc[0]);
          acc[1 % VEC] = fmaf(wi, v.y, acc[1 % VEC]);
          acc[2 % VEC] = fmaf(wi, v.z, acc[2 % VEC]);
          acc[3 % VEC] = fmaf(wi, v.w, acc[3 % VEC]);
        } else {
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[k] = fmaf(wi, sp[k], acc[k]);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc_s[threadIdx.x * VEC + k] = active ? acc[k] : 0.f;
  __syncthreads();
  const int64_t orow = (int64_t(b) * hq + h) * dv;
  for (int d = threadIdx.x; d < ncols; d += kThreads) {
    const int c = d / VEC, k = d % VEC;
    float v = 0.f;
    for (int g = 0; g < npg; ++g) v += acc_s[(g * ncg + c) * VEC + k];
    if (out_dtype == kF32)
      static_cast<float*>(out)[orow + col0 + d] = v;
    else
      static_cast<uint16_t*>(out)[orow + col0 + d] = f32_to_bf16_bits(v);
  }
  if (lse_out && threadIdx.x == 0 && blockIdx.y == 0) lse_out[int64_t(b) * hq + h] = total;
}

// Up to 64 parts: one wave per (sequence, head, block of columns), no LDS and no
// barrier, so the dependent steps are one lse load, cross-lane reductions and rounds of
// output loads.  Lane p holds part p's lse; the max and the sum of weights are
// cross-lane reductions.  The lanes then form PG part groups x (64 / PG) column groups of
// VEC columns: in a round, lane (pg, cg) reads parts p0 + pg + PG k, k < 8 (issued
// together) of its columns, so a round covers 8 PG parts; the part groups' sums meet by
// xor exchanges.  PG = 8: one round for up to 64 parts, narrow blocks (many waves when
// rows are few); smaller PG: wider blocks, fewer waves (many rows).
constexpr int kWaveParts = 64;

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int VEC, int PG>
__global__ __launch_bounds__(256) void merge_wave_kernel(const float* __restrict__ part_out,
                                                         const float* __restrict__ part_lse,
                                                         int n_rows, int n_cblk, int n_parts, int hq,
                                                         int dv, void* out, int out_dtype,
                                                         float* lse_out) {
  constexpr int CG = 64 / PG;   // column groups; a block has CG * VEC columns
  const int64_t wid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wid >= int64_t(n_rows) * n_cblk) return;   // the whole wave
  const int row = int(wid / n_cblk), cblk = int(wid - (wid / n_cblk) * n_cblk);
  const int lane = threadIdx.x & 63;
  const int b = row / hq, h = row - (row / hq) * hq;
  const float* lse_p = part_lse + int64_t(b) * n_parts * hq + h;        // stride hq
  const float* o_p = part_out + (int64_t(b) * n_parts * hq + h) * dv;   // stride hq*dv
  const int64_t stride = int64_t(hq) * dv;

  const float x = lane < n_parts ? lse_p[int64_t(lane) * hq] : -INFINITY;
  const float m = wave_max(x);
  float total = -INFINITY, w = 0.f;
  if (m != -INFINITY) {
    total = m + logf(wave_sum(x != -INFINITY ? expf(x - m) : 0.f));
    if (x != -INFINITY) w = expf(x - total);
  }
  const int pg = lane / CG, cg = lane % CG;
  const int c = cblk * CG * VEC + cg * VEC;
  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
  for (int p0 = 0; p0 < n_parts; p0 += 8 * PG) {   // uniform: every lane takes the shuffles
    float wk[8], v[8][VEC];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = p0 + pg + PG * k;
      wk[k] = __shfl(w, p < 64 ? p : 0);
      if (p >= n_parts) wk[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // a part of weight 0 (empty, or past n_parts) is not read
      const bool use = c < dv && wk[k] != 0.f;
      const float* sp = o_p + int64_t(p0 + pg + PG * k) * stride + c;
      if constexpr (VEC == 4) {
        const float4 t = use ? *reinterpret_cast<const float4*>(sp) : float4{0.f, 0.f, 0.f, 0.f};
        v[k][0] = t.x, v[k][1 % VEC] = t.y, v[k][2 % VEC] = t.z, v[k][3 % VEC] = t.w;
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) v[k][j] = use ? sp[j] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < VEC; ++j) acc[j] = fmaf(wk[k], v[k][j], acc[j]);
  }
#pragma unroll
  for (int d = CG; d < 64; d <<= 1)
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] += __shfl_xor(acc[j], d);
  if (pg == 0 && c < dv) {
    const int64_t orow = int64_t(row) * dv + c;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      if (out_dtype == kF32)
        static_cast<float*>(out)[orow + j] = acc[j];
      else
        static_cast<uint16_t*>(out)[orow + j] = f32_to_bf16_bits(acc[j]);
    }
  }
  if (lse_out && lane == 0 && cblk == 0) lse_out[row] = total;
}

template <int VEC, int PG>
void launch_wave(const float* part_out, const float* part_lse, int rows, int n_parts, int hq, int dv,
                 void* out, int out_dtype, float* lse, hipStream_t st) {
  const int n_cblk = (dv + (64 / PG) * VEC - 1) / ((64 / PG) * VEC);
  const dim3 g(unsigned((int64_t(rows) * n_cblk + 3) / 4));
  hipLaunchKernelGGL((merge_wave_kernel<VEC, PG>), g, dim3(256), 0, st, part_out, part_lse, rows,
                     n_cblk, n_parts, hq, dv, out, out_dtype, lse);
}

}  // namespace

hipError_t launch_merge(const float* part_out, const float* part_lse, int n_seqs, int n_parts,
                        int hq, int dv, void* out, int out_dtype, float* lse, hipStream_t st) {
  // Column blocks: narrow (more workgroups, more parts read at once) when there are few
  // (sequence, head) rows to spread over the GPU; otherwise wide (at most 128 column
  // groups per workgroup), so each workgroup has enough work.
  const int vec = dv % 4 == 0 ? 4 : 1;
  if (n_parts <= kWaveParts) {
    // As many part groups (8, 4, 2 or 1; more groups: narrower column blocks, more waves,
    // more parts read at once) as keep the launch within ~16K waves.  Measured, merge
    // alone: latent (4,096 rows, 16 parts) 14.5 / 12.2 / 20.5 / 34.9 us with 1 / 2 / 4 / 8
    // groups; long (256 rows, ~50 parts) 6.8 / 5.0 / 4.0 / 3.5 us.
    const int rows = n_seqs * hq;
    int pg = 8;
    while (pg > 1 && int64_t(rows) * ((dv + (64 / pg) * vec - 1) / ((64 / pg) * vec)) > 16384) pg /= 2;
    auto go = [&](auto v, auto g) {
      launch_wave<decltype(v)::value, decltype(g)::value>(part_out, part_lse, rows, n_parts, hq, dv, out,
                                                          out_dtype, lse, st);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    if (vec == 4) {
      if (pg == 8) go(I4{}, I8{}); else if (pg == 4) go(I4{}, I4{}); else if (pg == 2) go(I4{}, I2{}); else go(I4{}, I1{});
    } else {
      if (pg == 8) go(I1{}, I8{}); else if (pg == 4) go(I1{}, I4{}); else if (pg == 2) go(I1{}, I2{}); else go(I1{}, I1{});
    }
    return hipGetLastError();
  }
  int cb = 128 * vec;
  if (int64_t(n_seqs) * hq < 1024) cb = 8 * vec;
  if (cb > dv) cb = dv;
  const dim3 grid(n_seqs * hq, (dv + cb - 1) / cb);
  if (vec == 4)
    hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(kThreads), 0, st, part_out, part_lse, n_parts,
                       hq, dv, cb, out, out_dtype, lse);
  else
    hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(kThreads), 0, st, part_out, part_lse, n_parts,
                       hq, dv, cb, out, out_dtype, lse);
  return hipGetLastError();
}

}  // namespace pa
