// merge_lse.hip -- combine per-partition attention results with their LSEs.
//
// The DCP page (soroban.highreso.jp, "Why long-context LLMs get slow ...", DCP mechanism
// section) finishes a decode step by sharing the LSE of every partial result,
// correcting each partial output with its weight and summing.  Written out: with
// lse = M + ln sum_p exp(lse_p - M), M = max_p lse_p, part p has weight exp(lse_p - lse).
// Parts with lse_p = -inf are empty and skipped (no -inf - -inf is ever formed).
//
// One workgroup per (sequence, head).
#include <math.h>

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

// Threads form a (part group) x (column group) grid: each thread owns VEC consecutive
// output columns and sums every PG-th part, so PG parts are read at once; the PG
// partial sums are then added through LDS.
template <int VEC>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ part_out,
                                                         const float* __restrict__ part_lse,
                                                         int n_parts, int hq, int dv, void* out,
                                                         int out_dtype, float* lse_out) {
  const int b = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  __shared__ float red[kThreads / 64];
  __shared__ float w_s[kChunk];
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

  // this workgroup's columns: [col0, col0 + ncols), at most 128 column groups
  const int col0 = blockIdx.y * 128 * VEC;
  const int ncols = min(128 * VEC, dv - col0);
  const int ncg = ncols / VEC;                 // column groups (VEC divides dv)
  const int npg = kThreads / ncg;              // part groups (>= 2)
  const int cg = threadIdx.x % ncg;
  const int pg = threadIdx.x / ncg;
  const bool active = pg < npg;
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  for (int p0 = 0; p0 < n_parts && total != -INFINITY; p0 += kChunk) {
    const int np = min(kChunk, n_parts - p0);
    __syncthreads();
    for (int i = threadIdx.x; i < np; i += kThreads) {
      const float x = lse_p[int64_t(p0 + i) * hq];
      w_s[i] = (x != -INFINITY) ? expf(x - total) : 0.f;
    }
    __syncthreads();
    if (active) {
      // no data-dependent branch in the loop, so the loads of several parts are in
      // flight together
      const float* src = o_p + int64_t(p0) * hq * dv + col0 + cg * VEC;
      const int64_t stride = int64_t(hq) * dv;
#pragma unroll 8
      for (int i = pg; i < np; i += npg) {
        const float wi = w_s[i];
        const float* sp = src + i * stride;
        if (VEC == 4) {
          const float4 v = *reinterpret_cast<const float4*>(sp);
          const bool use = wi != 0.f;   // select, not branch: an empty part's values never enter
          acc[0] = use ? fmaf(wi, v.x, acc[0]) : acc[0];
          acc[1 % VEC] = use ? fmaf(wi, v.y, acc[1 % VEC]) : acc[1 % VEC];
          acc[2 % VEC] = use ? fmaf(wi, v.z, acc[2 % VEC]) : acc[2 % VEC];
          acc[3 % VEC] = use ? fmaf(wi, v.w, acc[3 % VEC]) : acc[3 % VEC];
        } else {
          const bool use = wi != 0.f;
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[k] = use ? fmaf(wi, sp[k], acc[k]) : acc[k];
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

}  // namespace

hipError_t launch_merge(const float* part_out, const float* part_lse, int n_seqs, int n_parts,
                        int hq, int dv, void* out, int out_dtype, float* lse, hipStream_t st) {
  if (dv % 4 == 0)
    hipLaunchKernelGGL(merge_kernel<4>, dim3(n_seqs * hq, (dv + 511) / 512), dim3(kThreads), 0,
                       st, part_out, part_lse, n_parts, hq, dv, out, out_dtype, lse);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3(n_seqs * hq, (dv + 127) / 128), dim3(kThreads), 0,
                       st, part_out, part_lse, n_parts, hq, dv, out, out_dtype, lse);
  return hipGetLastError();
}

}  // namespace pa
