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
//
// Two kernels: the token-major one (used whenever a token row fits its index
// table) reads each token row front to back and scatters its vectors to the
// P chunk runs; the run-major one copies one (chunk, segment) run per block
// row and serves rows too long for the table.
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

// Token-major kernel: a block copies kRowTokens whole token rows. For every
// vector j of a token's chunk-ordered row (chunk p, local vector k) it looks
// up, in two per-block LDS tables, the matching vector of the token-split row
// and the vector's place in the chunk tensor, so both sides are walked in long
// contiguous stretches and the copy loop does no integer division (one
// multiply-shift for the token). Loads and stores are nontemporal: every byte
// is touched once. 512 threads x 4 vectors in flight and 4 tokens per block
// measured best for 8- and 12-KiB rows (8 or 16 tokens per block, or 8
// vectors in flight, were 2-10 % slower). Indexes are 32-bit: the boundary
// rejects tensors of 2^31 vectors or more.
constexpr int kRowThreads = 512;
constexpr int kRowTokens = 4;
constexpr int kRowInFlight = 4;
constexpr int kMaxRowVec = 4096;  // vectors per token row the table can hold

struct RowArgs {
  const u32x4 *src;
  u32x4 *dst;
  uint32_t n;         // tokens
  uint32_t row_vec;   // vectors per token row (H*d/8)
  uint32_t chunk_vec; // vectors per chunk row (h*d/8)
  int nseg;
  uint32_t seg_base_vec[8];   // segment start (vectors) in the token-split row
  uint32_t seg_local_vec[8];  // vectors of one rank's block of the segment
  FastDiv row_div;            // division by row_vec
};

template <bool kToHead>
__global__ void __launch_bounds__(kRowThreads) swap_rows_kernel(RowArgs a) {
  // Vector j of a token's chunk-ordered row (chunk p, vector k of the chunk
  // row): stab[j] = its vector in the token-split row; ctab[j] = its offset
  // in the chunk tensor for token 0 (p * n * chunk_vec + k).
  __shared__ uint32_t stab[kMaxRowVec];
  __shared__ uint32_t ctab[kMaxRowVec];
  for (uint32_t j = threadIdx.x; j < a.row_vec; j += kRowThreads) {
    const uint32_t p = j / a.chunk_vec, k = j - p * a.chunk_vec;
    uint32_t kk = k, src = 0;
    for (int sgi = 0; sgi < a.nseg; ++sgi) {
      const uint32_t L = a.seg_local_vec[sgi];
      if (kk < L) {
        src = a.seg_base_vec[sgi] + p * L + kk;
        break;
      }
      kk -= L;
    }
    stab[j] = src;
    ctab[j] = p * a.n * a.chunk_vec + k;
  }
  __syncthreads();
  const uint32_t t0 = blockIdx.x * kRowTokens;
  const uint32_t nt = (a.n - t0) < (uint32_t)kRowTokens ? (a.n - t0) : (uint32_t)kRowTokens;
  const uint32_t total = nt * a.row_vec;
  const u32x4 *src = a.src;
  u32x4 *dst = a.dst;
  constexpr int U = kRowInFlight;
  for (uint32_t base = threadIdx.x; base < total; base += kRowThreads * U) {
    u32x4 v[U];
    uint32_t di[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kRowThreads;
      ok[u] = i < total;
      if (ok[u]) {
        const uint32_t tl = a.row_div.q(i);  // token within the block
        const uint32_t j = i - tl * a.row_vec;
        const uint32_t t = t0 + tl;
        const uint32_t c_idx = t * a.chunk_vec + ctab[j];
        const uint32_t s_idx = t * a.row_vec + stab[j];
        if (kToHead) {
          v[u] = __builtin_nontemporal_load(src + s_idx);
          di[u] = c_idx;
        } else {
          v[u] = __builtin_nontemporal_load(src + c_idx);
          di[u] = s_idx;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) __builtin_nontemporal_store(v[u], dst + di[u]);
  }
}

}  // namespace

static int launch_swap_rows(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                     const int32_t *seg_heads, int d, hipStream_t stream) {
  RowArgs a;
  a.src = reinterpret_cast<const u32x4 *>(src);
  a.dst = reinterpret_cast<u32x4 *>(dst);
  a.n = (uint32_t)n;
  int64_t H = 0;
  for (int s = 0; s < nseg; ++s) H += seg_heads[s];
  a.row_vec = (uint32_t)(H * d / 8);
  a.chunk_vec = (uint32_t)(H / P * d / 8);
  a.row_div = FastDiv(a.row_vec);
  a.nseg = nseg;
  uint32_t base = 0;
  for (int s = 0; s < 8; ++s) {
    a.seg_base_vec[s] = s < nseg ? base : 0;
    a.seg_local_vec[s] = s < nseg ? (uint32_t)(seg_heads[s] / P * d / 8) : 0;
    if (s < nseg) base += (uint32_t)(seg_heads[s] * d / 8);
  }
  const unsigned blocks = (unsigned)((n + kRowTokens - 1) / kRowTokens);
  if (to_head)
    hipLaunchKernelGGL(swap_rows_kernel<true>, dim3(blocks), dim3(kRowThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(swap_rows_kernel<false>, dim3(blocks), dim3(kRowThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "swap_rows_kernel");
  return 0;
}

int launch_swap(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                const int32_t *seg_heads, int d, hipStream_t stream) {
  int64_t H = 0;
  for (int s = 0; s < nseg; ++s) H += seg_heads[s];
  if (H * d / 8 <= kMaxRowVec) return launch_swap_rows(to_head, src, dst, n, P, nseg, seg_heads, d, stream);
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
