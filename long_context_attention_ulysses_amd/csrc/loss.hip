// Loss of a sequence-parallel causal-LM step from pre-shifted labels, and its
// weighted aggregation over the SP ranks ("Deepspeed Ulysses/ALST
// integration", opening post, step 2: each rank computes the loss of its own
// token shard from shift_labels, where -100 marks tokens without a loss; the
// per-rank losses are combined as sum_r loss_r * good_r / max(sum_r good_r, 1)
// with good_r the rank's count of labels != -100; "Ulysses sequence
// parallelism", Configure: the Trainer shifts labels and aggregates the loss
// across SP ranks).
//
// Per rank: row r of the logits [n][V] with label y_r gives
//   lse_r = log sum_v exp(logit_rv),  loss_r = lse_r - logit_{r, y_r}
// (cross-entropy), 0 for ignored rows; the rank's loss is the mean over its
// good rows. The gradient of the aggregate with respect to a good row's
// logits is (softmax(row) - onehot(y_r)) / max(G, 1), G = sum_r good_r.
//
// All kernels are HBM-bound row streams: the forward reads the logits once,
// the backward reads them once and writes the gradient once.
#include <math.h>

#include "uly_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kCeThreads = 512;
constexpr int kCeWaves = kCeThreads / 64;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

constexpr float kL2E = 1.4426950408889634f;  // log2(e)
constexpr float kLN2 = 0.6931471805599453f;  // ln(2)

// Adds 8 values (already scaled to log2 units) to a running (max m, sum s of
// 2^(x - m)), rescaling s at most once per 8 values.
__device__ __forceinline__ void online_add8(float &m, float &s, const float *x) {
  float vm = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) vm = fmaxf(vm, x[e]);
  if (vm > m) {
    s *= __builtin_amdgcn_exp2f(m - vm);
    m = vm;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(x[e] - m);
}

// Block-wide merge of per-thread (max, sum) in log2 units: returns the row's
// natural-log log-sum-exp to every thread.
__device__ float block_lse(float m, float s, float *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float wm = wave_max(m);
  s = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f(m - wm);
  s = wave_sum(s);
  if (lane == 0) {
    red[w] = wm;
    red[kCeWaves + w] = s;
  }
  __syncthreads();
  float gm = -INFINITY;
#pragma unroll
  for (int i = 0; i < kCeWaves; ++i) gm = fmaxf(gm, red[i]);
  float gs = 0.f;
#pragma unroll
  for (int i = 0; i < kCeWaves; ++i)
    gs += (red[i] == -INFINITY) ? 0.f : red[kCeWaves + i] * __builtin_amdgcn_exp2f(red[i] - gm);
  return (gm + __builtin_amdgcn_logf(gs)) * kLN2;
}

struct CeArgs {
  const bf16_t *logits;
  int64_t stride;  // elements between rows
  const int32_t *labels;
  uint32_t V, nvec;  // vocabulary, V / 8
  float *row_loss, *row_lse;
};

// One workgroup per row: streams the row once.
__global__ void __launch_bounds__(kCeThreads) ce_fwd_kernel(CeArgs a) {
  __shared__ float red[2 * kCeWaves];
  const int64_t r = blockIdx.x;
  const bf16_t *row = a.logits + r * a.stride;
  float m = -INFINITY, s = 0.f;
  for (uint32_t i = threadIdx.x; i < a.nvec; i += kCeThreads) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + i);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(v[e] << 16) * kL2E;
      x[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u) * kL2E;
    }
    online_add8(m, s, x);
  }
  const float lse = block_lse(m, s, red);
  if (threadIdx.x == 0) {
    const int32_t y = a.labels[r];
    const bool good = y >= 0 && (uint32_t)y < a.V;
    a.row_lse[r] = lse;
    a.row_loss[r] = good ? lse - bf16_to_f32(row[y]) : 0.f;
  }
}

// One workgroup: the rank's loss (mean over good rows, 0 if none) and good
// count, summed in a fixed order (deterministic).
__global__ void __launch_bounds__(kCeThreads) ce_reduce_kernel(const float *row_loss, const int32_t *labels,
                                                              uint32_t n, uint32_t V, float *loss_out,
                                                              int32_t *good_out) {
  __shared__ float rs[kCeThreads];
  __shared__ int rc[kCeThreads];
  float s = 0.f;
  int c = 0;
  for (uint32_t i = threadIdx.x; i < n; i += kCeThreads) {
    const int32_t y = labels[i];
    if (y >= 0 && (uint32_t)y < V) {
      s += row_loss[i];
      ++c;
    }
  }
  rs[threadIdx.x] = s;
  rc[threadIdx.x] = c;
  __syncthreads();
  for (int o = kCeThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      rs[threadIdx.x] += rs[threadIdx.x + o];
      rc[threadIdx.x] += rc[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *good_out = rc[0];
    *loss_out = rc[0] > 0 ? rs[0] / (float)rc[0] : 0.f;
  }
}

struct AggArgs {
  const float *loss[kMaxParts];
  const int32_t *good[kMaxParts];
  int n_ranks;
  float *total, *row_scale;
};

// sum_r loss_r * good_r / max(sum_r good_r, 1), and the per-row gradient
// scale 1 / max(G, 1). One thread.
__global__ void loss_aggregate_kernel(AggArgs a) {
  float t = 0.f;
  int64_t g = 0;
  for (int r = 0; r < a.n_ranks; ++r) {
    t += *a.loss[r] * (float)*a.good[r];
    g += *a.good[r];
  }
  const float den = (float)(g > 1 ? g : 1);
  *a.total = t / den;
  *a.row_scale = 1.f / den;
}

struct CeBwdArgs {
  const bf16_t *logits;
  int64_t stride;
  const int32_t *labels;
  const float *row_lse, *row_scale;
  uint32_t V, nvec;
  bf16_t *grad;
  int64_t gstride;
};

// One workgroup per row: (softmax - onehot) * scale for good rows, zeros for
// ignored rows.
__global__ void __launch_bounds__(kCeThreads) ce_bwd_kernel(CeBwdArgs a) {
  const int64_t r = blockIdx.x;
  const bf16_t *row = a.logits + r * a.stride;
  u32x4 *grow = reinterpret_cast<u32x4 *>(a.grad + r * a.gstride);
  const int32_t y = a.labels[r];
  const bool good = y >= 0 && (uint32_t)y < a.V;
  const float lse2 = a.row_lse[r] * kL2E;
  const float sc = good ? *a.row_scale : 0.f;
  for (uint32_t i = threadIdx.x; i < a.nvec; i += kCeThreads) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + i);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c0 = i * 8 + 2 * e;
      float g0 = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(v[e] << 16), kL2E, -lse2));
      float g1 = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(v[e] & 0xFFFF0000u), kL2E, -lse2));
      if ((int32_t)c0 == y) g0 -= 1.f;
      if ((int32_t)c0 + 1 == y) g1 -= 1.f;
      o[e] = pack_bf16x2(g0 * sc, g1 * sc);
    }
    __builtin_nontemporal_store(o, grow + i);
  }
}

}  // namespace

int launch_ce_fwd(const bf16_t *logits, int64_t stride, const int32_t *labels, int64_t n, int64_t V,
                  float *row_loss, float *row_lse, float *loss_out, int32_t *good_out, hipStream_t stream) {
  CeArgs a{logits, stride, labels, (uint32_t)V, (uint32_t)(V / 8), row_loss, row_lse};
  hipLaunchKernelGGL(ce_fwd_kernel, dim3((unsigned)n), dim3(kCeThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "ce_fwd_kernel");
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(kCeThreads), 0, stream, row_loss, labels, (uint32_t)n,
                     (uint32_t)V, loss_out, good_out);
  e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "ce_reduce_kernel");
  return 0;
}

int launch_loss_aggregate(int n_ranks, const float *const *loss, const int32_t *const *good, float *total,
                          float *row_scale, hipStream_t stream) {
  AggArgs a;
  for (int r = 0; r < kMaxParts; ++r) {
    a.loss[r] = r < n_ranks ? loss[r] : nullptr;
    a.good[r] = r < n_ranks ? good[r] : nullptr;
  }
  a.n_ranks = n_ranks;
  a.total = total;
  a.row_scale = row_scale;
  hipLaunchKernelGGL(loss_aggregate_kernel, dim3(1), dim3(1), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "loss_aggregate_kernel");
  return 0;
}

int launch_ce_bwd(const bf16_t *logits, int64_t stride, const int32_t *labels, const float *row_lse,
                  const float *row_scale, int64_t n, int64_t V, bf16_t *grad, int64_t gstride,
                  hipStream_t stream) {
  CeBwdArgs a{logits, stride, labels, row_lse, row_scale, (uint32_t)V, (uint32_t)(V / 8), grad, gstride};
  hipLaunchKernelGGL(ce_bwd_kernel, dim3((unsigned)n), dim3(kCeThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "ce_bwd_kernel");
  return 0;
}

}  // namespace uly
