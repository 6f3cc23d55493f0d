// Sequence <-> head layout swap: the local pack/unpack around Ulysses'
// all-to-all ("Ulysses sequence parallelism", HF Transformers docs, intro
// diagram: token split with all heads <-> all tokens with a head block).
//
// The fused token row [H][d] (H = sum of segments, e.g. q|k|v heads) of this
// rank's n tokens is cut into P chunks; chunk p takes, for each segment s,
// the contiguous head block [p*s/P, (p+1)*s/P). Every (chunk p, segment s)
// pair is therefore one contiguous run of (s/P)*d elements per token in both
// the token-split tensor and the chunk tensor, so the swap is a batch of
// strided run copies. It is HBM-bound.
//
// One kernel, one 16-byte vector per thread: thread i moves vector i of the
// token rows taken in chunk order (token t, then chunk p, then the vector k of
// rank p's chunk row). Consecutive threads therefore read consecutive vectors
// of a segment run of the token-split row and write consecutive vectors of a
// chunk row. The token, the chunk and k come from two multiply-shift
// divisions and the source vector from a walk over the (at most 8) segments,
// so no index table is built and nothing but registers limits how many
// blocks a CU holds. Every byte is touched once, so loads are nontemporal and
// stores are nontemporal at agent scope (sc1): they write through the XCD's L2
// instead of leaving dirty lines there to be evicted later, which measured 4
// to 14 % faster than nontemporal stores alone on a cold L2; the load's scope
// bits made no difference. One vector per thread with 256-thread blocks
// measured faster than 2 or 4 vectors in flight per thread, than per-block
// LDS index tables, than a walk in chunk-tensor order and than skewing the
// chunks' tokens against each other. Indexes are 32-bit: the boundary rejects tensors of 2^31
// vectors or more.
#include "uly_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kSwapThreads = 256;

struct SwapArgs {
  const u32x4 *src;
  u32x4 *dst;
  uint32_t n;          // tokens
  uint32_t row_vec;    // vectors per token row (H*d/8)
  uint32_t chunk_vec;  // vectors per chunk row (H/P*d/8)
  uint32_t total;      // n * row_vec
  int nseg;
  uint32_t seg_base_vec[8];   // segment start (vectors) in the token-split row
  uint32_t seg_local_vec[8];  // vectors of one rank's block of the segment
  FastDiv row_div, chunk_div;
};

template <bool kToHead>
__global__ void __launch_bounds__(kSwapThreads) swap_kernel(SwapArgs a) {
  const uint32_t i = blockIdx.x * kSwapThreads + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t t = a.row_div.q(i);
  const uint32_t j = i - t * a.row_vec;  // chunk-ordered vector of token t
  const uint32_t p = a.chunk_div.q(j);
  const uint32_t k = j - p * a.chunk_vec;
  // Segment of k and its place in the token-split row.
  uint32_t kk = k, off = 0;
  bool found = false;
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    if (!found && sg < a.nseg) {
      const uint32_t L = a.seg_local_vec[sg];
      if (kk < L) {
        off = a.seg_base_vec[sg] + p * L + kk;
        found = true;
      } else {
        kk -= L;
      }
    }
  }
  const uint32_t c_idx = (p * a.n + t) * a.chunk_vec + k;
  const uint32_t s_idx = t * a.row_vec + off;
  if (kToHead)
    store_through(a.dst + c_idx, __builtin_nontemporal_load(a.src + s_idx));
  else
    store_through(a.dst + s_idx, __builtin_nontemporal_load(a.src + c_idx));
}

}  // namespace

int launch_swap(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                const int32_t *seg_heads, int d, hipStream_t stream) {
  SwapArgs a;
  a.src = reinterpret_cast<const u32x4 *>(src);
  a.dst = reinterpret_cast<u32x4 *>(dst);
  a.n = (uint32_t)n;
  int64_t H = 0;
  for (int s = 0; s < nseg; ++s) H += seg_heads[s];
  a.row_vec = (uint32_t)(H * d / 8);
  a.chunk_vec = (uint32_t)(H / P * d / 8);
  a.total = (uint32_t)(n * a.row_vec);
  a.row_div = FastDiv(a.row_vec);
  a.chunk_div = FastDiv(a.chunk_vec);
  a.nseg = nseg;
  uint32_t base = 0;
  for (int s = 0; s < 8; ++s) {
    a.seg_base_vec[s] = s < nseg ? base : 0;
    a.seg_local_vec[s] = s < nseg ? (uint32_t)(seg_heads[s] / P * d / 8) : 0;
    if (s < nseg) base += (uint32_t)(seg_heads[s] * d / 8);
  }
  const unsigned blocks = (unsigned)((a.total + kSwapThreads - 1) / kSwapThreads);
  if (to_head)
    hipLaunchKernelGGL(swap_kernel<true>, dim3(blocks), dim3(kSwapThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(swap_kernel<false>, dim3(blocks), dim3(kSwapThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "swap_kernel");
  return 0;
}

}  // namespace uly
