// Sequence <-> head layout swap: the local pack/unpack around Ulysses'
// all-to-all ("Ulysses sequence parallelism", HF Transformers docs, intro
// diagram: token split with all heads <-> all tokens with a head block).
//
// The fused token row [H][d] (H = sum of segments, e.g. q|k|v heads) of this
// rank's n tokens is cut into P chunks; chunk p takes, for each segment s,
// the contiguous head block [p*s/P, (p+1)*s/P). Every (chunk p, segment s)
// pair is therefore one contiguous run of (s/P)*d elements per token in both
// the token-split tensor and the chunk tensor, so the swap is a batch of
// strided run copies. It is HBM-bound; each thread moves 16-byte vectors,
// with several loads in flight before its stores.
#include "uly_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kSwapThreads = 256;
constexpr int kSwapVecPerThread = 4;

// One block row (blockIdx.y) per (chunk p, segment s) pair.
struct SwapRun {
  int64_t seq_off;    // element offset of the run inside a token row of x_seq
  int64_t chunk_off;  // element offset of the run inside a token row of chunk p
  int64_t chunk_base; // element offset of chunk p in the chunk tensor (p*n*h*d)
};

struct SwapArgs {
  const u32x4 *src;
  u32x4 *dst;
  uint32_t n;            // tokens
  int64_t seq_row_vec;   // vectors per x_seq token row (H*d/8)
  int64_t chunk_row_vec; // vectors per chunk token row (h*d/8)
  SwapRun run[kMaxSwapRuns];
  uint32_t run_len_vec[kMaxSwapRuns];
  FastDiv run_len_div[kMaxSwapRuns];
};

template <bool kToHead>
__global__ void __launch_bounds__(kSwapThreads) swap_kernel(SwapArgs a) {
  const int r = blockIdx.y;
  const uint32_t len = a.run_len_vec[r];
  const FastDiv ld = a.run_len_div[r];
  const uint32_t total = a.n * len;  // vectors of this run over all tokens
  const int64_t seq_off = a.run[r].seq_off >> 3;
  const int64_t chunk_off = (a.run[r].chunk_base + a.run[r].chunk_off) >> 3;
  const uint32_t stride = gridDim.x * kSwapThreads * kSwapVecPerThread;
  for (uint32_t base = blockIdx.x * kSwapThreads * kSwapVecPerThread + threadIdx.x; base < total;
       base += stride) {
    u32x4 v[kSwapVecPerThread];
    int64_t dst_idx[kSwapVecPerThread];
#pragma unroll
    for (int u = 0; u < kSwapVecPerThread; ++u) {
      const uint32_t i = base + u * kSwapThreads;
      dst_idx[u] = -1;
      if (i < total) {
        const uint32_t t = ld.q(i);
        const uint32_t e = i - t * len;
        const int64_t s_idx = (int64_t)t * a.seq_row_vec + seq_off + e;
        const int64_t c_idx = (int64_t)t * a.chunk_row_vec + chunk_off + e;
        if (kToHead) {
          v[u] = __builtin_nontemporal_load(a.src + s_idx);
          dst_idx[u] = c_idx;
        } else {
          v[u] = __builtin_nontemporal_load(a.src + c_idx);
          dst_idx[u] = s_idx;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSwapVecPerThread; ++u)
      if (dst_idx[u] >= 0) __builtin_nontemporal_store(v[u], a.dst + dst_idx[u]);
  }
}

}  // namespace

int launch_swap(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                const int32_t *seg_heads, int d, hipStream_t stream) {
  int64_t H = 0;
  for (int s = 0; s < nseg; ++s) H += seg_heads[s];
  const int64_t h = H / P;
  const int nruns = P * nseg;
  // Launch rows: at most kMaxSwapRuns (chunk, segment) runs per launch.
  for (int r0 = 0; r0 < nruns; r0 += kMaxSwapRuns) {
    const int nr = (nruns - r0) < kMaxSwapRuns ? (nruns - r0) : kMaxSwapRuns;
    SwapArgs a;
    a.src = reinterpret_cast<const u32x4 *>(src);
    a.dst = reinterpret_cast<u32x4 *>(dst);
    a.n = (uint32_t)n;
    a.seq_row_vec = H * d / 8;
    a.chunk_row_vec = h * d / 8;
    uint32_t max_total = 0;
    for (int j = 0; j < nr; ++j) {
      const int run = r0 + j;
      const int p = run / nseg, s = run % nseg;
      int64_t seg_base = 0, chunk_inner = 0;
      for (int t = 0; t < s; ++t) {
        seg_base += seg_heads[t];
        chunk_inner += seg_heads[t] / P;
      }
      const int64_t local = seg_heads[s] / P;
      a.run[j].seq_off = (seg_base + (int64_t)p * local) * d;
      a.run[j].chunk_off = chunk_inner * d;
      a.run[j].chunk_base = (int64_t)p * n * h * d;
      a.run_len_vec[j] = (uint32_t)(local * d / 8);
      a.run_len_div[j] = FastDiv(a.run_len_vec[j]);
      const uint32_t tot = (uint32_t)(n * a.run_len_vec[j]);
      if (tot > max_total) max_total = tot;
    }
    for (int j = nr; j < kMaxSwapRuns; ++j) {
      a.run[j] = SwapRun{0, 0, 0};
      a.run_len_vec[j] = 0;
      a.run_len_div[j] = FastDiv(1);
    }
    const uint32_t per_block = kSwapThreads * kSwapVecPerThread;
    uint32_t gx = (max_total + per_block - 1) / per_block;
    if (gx > 65535) gx = 65535;
    if (gx == 0) gx = 1;
    dim3 grid(gx, nr);
    if (to_head)
      hipLaunchKernelGGL(swap_kernel<true>, grid, dim3(kSwapThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(swap_kernel<false>, grid, dim3(kSwapThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_hip_error(e, "swap_kernel");
  }
  return 0;
}

}  // namespace uly
