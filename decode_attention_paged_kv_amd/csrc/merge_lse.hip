// merge_lse.hip -- combine per-partition attention results with their LSEs.
//
// The DCP page (soroban.highreso.jp, "Why long-context LLMs get slow ...", DCP mechanism
// section) finishes a decode step by sharing the LSE of every partial result,
// correcting each partial output with its weight and summing.  Written out: with
// lse = M + ln sum_p exp(lse_p - M), M = max_p lse_p, part p has weight exp(lse_p - lse).
// Parts with lse_p = -inf are empty and skipped (no -inf - -inf is ever formed).
//
// One workgroup per (sequence, head); threads stride the parts for the two
// reductions, then the output dimension for the weighted sum.
#include <math.h>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kThreads = 128;

__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ inline float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r += red[i];
  return r;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ part_out,
                                                         const float* __restrict__ part_lse,
                                                         int n_parts, int hq, int dv, void* out,
                                                         int out_dtype, float* lse_out) {
  const int b = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  __shared__ float red[kThreads / 64];
  __shared__ float w_s[kThreads];
  const float* lse_p = part_lse + int64_t(b) * n_parts * hq + h;   // stride hq
  const float* o_p = part_out + (int64_t(b) * n_parts * hq + h) * dv;  // stride hq*dv

  float m = -INFINITY;
  for (int p = threadIdx.x; p < n_parts; p += kThreads) m = fmaxf(m, lse_p[int64_t(p) * hq]);
  m = block_max(m, red);
  float total = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.f;
    for (int p = threadIdx.x; p < n_parts; p += kThreads) {
      const float x = lse_p[int64_t(p) * hq];
      if (x != -INFINITY) s += expf(x - m);
    }
    s = block_sum(s, red);
    total = m + logf(s);
  }
  // weighted sum over parts, kThreads parts at a time
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // dv <= 4 * kThreads
  for (int p0 = 0; p0 < n_parts && total != -INFINITY; p0 += kThreads) {
    __syncthreads();
    const int p = p0 + threadIdx.x;
    float w = 0.f;
    if (p < n_parts) {
      const float x = lse_p[int64_t(p) * hq];
      if (x != -INFINITY) w = expf(x - total);
    }
    w_s[threadIdx.x] = w;
    __syncthreads();
    const int np = min(kThreads, n_parts - p0);
    for (int i = 0; i < np; ++i) {
      const float wi = w_s[i];
      if (wi == 0.f) continue;
      const float* src = o_p + int64_t(p0 + i) * hq * dv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = threadIdx.x + k * kThreads;
        if (d < dv) acc[k] = fmaf(wi, src[d], acc[k]);
      }
    }
  }
  const int64_t orow = (int64_t(b) * hq + h) * dv;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = threadIdx.x + k * kThreads;
    if (d < dv) {
      if (out_dtype == kF32)
        static_cast<float*>(out)[orow + d] = acc[k];
      else
        static_cast<uint16_t*>(out)[orow + d] = f32_to_bf16_bits(acc[k]);
    }
  }
  if (lse_out && threadIdx.x == 0) lse_out[int64_t(b) * hq + h] = total;
}

}  // namespace

hipError_t launch_merge(const float* part_out, const float* part_lse, int n_seqs, int n_parts,
                        int hq, int dv, void* out, int out_dtype, float* lse, hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(n_seqs * hq), dim3(kThreads), 0, st, part_out, part_lse,
                     n_parts, hq, dv, out, out_dtype, lse);
  return hipGetLastError();
}

}  // namespace pa
