// Ring attention, the variant the pages set against Ulysses: each GPU keeps
// the queries of its own S/P tokens and passes key/value blocks around a
// ring, computing local attention against the block it holds at each step
// ("Sequence Parallelism for Long-Context AI Training", "Advanced Scaling:
// Ring Attention and Ulysses"; "Ulysses Sequence Parallelism for
// Million-Token Context Training", "Comparing Ulysses and Ring Attention").
//
// One step is attn_fwd of the local queries against one block. Its result
// (o_j, lse_j) is the softmax over that block's keys only; softmax over all
// keys follows from the per-block results exactly:
//   lse = log sum_j exp(lse_j),   o = sum_j exp(lse_j - lse) o_j.
// In the backward pass each step's attn_bwd, given the merged o and lse,
// yields that block's share of dQ (for the local queries) and of dK, dV (for
// the block's owner); the shares add up to the gradient.
//
// Both kernels are elementwise over 16-byte vectors and HBM-bound: one read
// of every part and one write of the result, with nontemporal loads and
// write-through stores (5-9 % faster than plain ones at the 64K ring shapes).
#include <math.h>

#include "uly_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

struct MergeArgs {
  const bf16_t *o[kMaxParts];
  const float *lse[kMaxParts];
  bf16_t *out;
  float *lse_out;
  int n_parts;
  uint32_t total;  // vectors: N * h * (d / 8)
  uint32_t N, h, vpr;
  FastDiv div_vpr, div_h;
  int64_t part_stride, out_stride;  // token strides (elements)
};

__device__ __forceinline__ void acc8(float *acc, const u32x4 &v, float w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = fmaf(w, __uint_as_float(v[e] << 16), acc[2 * e]);
    acc[2 * e + 1] = fmaf(w, __uint_as_float(v[e] & 0xFFFF0000u), acc[2 * e + 1]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float *acc) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
  return r;
}

// One thread per 16-byte vector (8 values of one head of one token).
__global__ void __launch_bounds__(256) lse_merge_kernel(MergeArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t row = a.div_vpr.q(i);  // token * h + head
  const uint32_t c = i - row * a.vpr;
  const uint32_t t = a.div_h.q(row);
  const uint32_t hh = row - t * a.h;
  const int64_t lidx = (int64_t)hh * a.N + t;
  const int64_t col = (int64_t)hh * a.vpr * 8 + (int64_t)c * 8;

  float l[kMaxParts];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxParts; ++j) {
    l[j] = j < a.n_parts ? a.lse[j][lidx] : -INFINITY;
    m = fmaxf(m, l[j]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxParts; ++j) {
      l[j] = expf(l[j] - m);  // 0 for absent parts and -inf rows
      s += l[j];
    }
    const float inv = 1.f / s;
#pragma unroll
    for (int j = 0; j < kMaxParts; ++j)
      if (j < a.n_parts && l[j] > 0.f) {
        const u32x4 v =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.o[j] + (int64_t)t * a.part_stride + col));
        acc8(acc, v, l[j] * inv);
      }
    lse = m + logf(s);
  }
  store_through(a.out + (int64_t)t * a.out_stride + col, pack8(acc));
  if (c == 0) a.lse_out[lidx] = lse;
}

struct SumArgs {
  const bf16_t *p[kMaxParts];
  bf16_t *out;
  int n_parts;
  uint32_t total;  // vectors: rows * (width / 8)
  uint32_t vpr;
  FastDiv div_vpr;
  int64_t part_stride, out_stride;
};

__global__ void __launch_bounds__(256) grad_sum_kernel(SumArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t r = a.div_vpr.q(i);
  const int64_t col = (int64_t)(i - r * a.vpr) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxParts; ++j)
    if (j < a.n_parts)
      acc8(acc, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.p[j] + (int64_t)r * a.part_stride + col)),
           1.f);
  store_through(a.out + (int64_t)r * a.out_stride + col, pack8(acc));
}

}  // namespace

int launch_lse_merge(int n_parts, const bf16_t *const *o, const float *const *lse, bf16_t *out,
                     float *lse_out, int64_t N, int h, int d, int64_t part_stride, int64_t out_stride,
                     hipStream_t stream) {
  MergeArgs a;
  for (int j = 0; j < kMaxParts; ++j) {
    a.o[j] = j < n_parts ? o[j] : nullptr;
    a.lse[j] = j < n_parts ? lse[j] : nullptr;
  }
  a.out = out;
  a.lse_out = lse_out;
  a.n_parts = n_parts;
  a.N = (uint32_t)N;
  a.h = (uint32_t)h;
  a.vpr = (uint32_t)(d / 8);
  a.total = (uint32_t)(N * h * (d / 8));
  a.div_vpr = FastDiv(a.vpr);
  a.div_h = FastDiv(a.h);
  a.part_stride = part_stride;
  a.out_stride = out_stride;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((a.total + 255) / 256), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "lse_merge_kernel");
  return 0;
}

int launch_grad_sum(int n_parts, const bf16_t *const *parts, bf16_t *out, int64_t rows, int width,
                    int64_t part_stride, int64_t out_stride, hipStream_t stream) {
  SumArgs a;
  for (int j = 0; j < kMaxParts; ++j) a.p[j] = j < n_parts ? parts[j] : nullptr;
  a.out = out;
  a.n_parts = n_parts;
  a.vpr = (uint32_t)(width / 8);
  a.total = (uint32_t)(rows * (width / 8));
  a.div_vpr = FastDiv(a.vpr);
  a.part_stride = part_stride;
  a.out_stride = out_stride;
  hipLaunchKernelGGL(grad_sum_kernel, dim3((a.total + 255) / 256), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "grad_sum_kernel");
  return 0;
}

}  // namespace uly
