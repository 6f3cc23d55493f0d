// Workgroup schedules of the attention kernels over packed documents.
//
// Under a plain causal mask the kernels issue their blocks in a fixed order
// that is heaviest-first (last query blocks first, first key blocks first).
// Over packed documents ("Ulysses sequence parallelism", Configure: samples
// packed into one sequence must not attend across their boundaries) a
// block's work depends on where it sits in its document, so that order is
// heaviest-first only within one document and the longest blocks can start
// last. This pass sorts the blocks by decreasing work instead, one
// workgroup per order: the work of a block of bs rows is the number of
// 64-row tiles its range spans (the kernels' own ranges): key ranges for
// query blocks, query ranges for key blocks. Keys (work, id) are sorted with
// a bitonic network in LDS, so equal work keeps id order. More than
// kMaxOrder blocks keep the id order.
#include "attn_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kOrderThreads = 1024;
constexpr int kMaxOrder = 16384;

struct OrderArgs {
  const int32_t *cu;
  int n_seqs;
  int64_t N;
  int causal;
  int bs[2];         // rows per block: [0] query blocks, [1] key blocks
  int nb[2];         // blocks
  int32_t *order[2]; // outputs (nullptr: not wanted)
};

__global__ void __launch_bounds__(kOrderThreads) block_order_kernel(OrderArgs a) {
  __shared__ uint64_t keys[kMaxOrder];
  const int which = blockIdx.x;  // 0: query blocks by key ranges, 1: key blocks by query ranges
  int32_t *order = a.order[which];
  if (!order) return;
  const int nb = a.nb[which], bs = a.bs[which];
  const int tid = threadIdx.x;
  if (nb > kMaxOrder) {
    for (int i = tid; i < nb; i += kOrderThreads) order[i] = i;
    return;
  }
  int p2 = 1;
  while (p2 < nb) p2 <<= 1;
  for (int i = tid; i < p2; i += kOrderThreads) {
    uint64_t key = ~0ull;
    if (i < nb) {
      const int64_t b0 = (int64_t)i * bs;
      const int64_t b1 = (b0 + bs < a.N ? b0 + bs : a.N) - 1;
      const KeyRange r0 = which ? query_range(a.cu, a.n_seqs, a.N, a.causal, b0)
                                : key_range(a.cu, a.n_seqs, a.N, a.causal, b0);
      const KeyRange r1 = which ? query_range(a.cu, a.n_seqs, a.N, a.causal, b1)
                                : key_range(a.cu, a.n_seqs, a.N, a.causal, b1);
      const uint32_t work = (uint32_t)((r1.hi + 63) / 64 - r0.lo / 64);
      key = ((uint64_t)(0xFFFFFFFFu - work) << 32) | (uint32_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < p2; i += kOrderThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = keys[i], y = keys[l];
          if ((x > y) == ((i & k) == 0)) {
            keys[i] = y;
            keys[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < nb; i += kOrderThreads) order[i] = (int32_t)(uint32_t)keys[i];
}

}  // namespace

int launch_block_orders(const int32_t *cu, int n_seqs, int64_t N, int causal, int q_bs, int32_t *q_order,
                        int k_bs, int32_t *k_order, hipStream_t stream) {
  OrderArgs a;
  a.cu = cu;
  a.n_seqs = n_seqs;
  a.N = N;
  a.causal = causal;
  a.bs[0] = q_bs;
  a.bs[1] = k_bs;
  a.nb[0] = q_order ? (int)((N + q_bs - 1) / q_bs) : 0;
  a.nb[1] = k_order ? (int)((N + k_bs - 1) / k_bs) : 0;
  a.order[0] = q_order;
  a.order[1] = k_order;
  hipLaunchKernelGGL(block_order_kernel, dim3(2), dim3(kOrderThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "block_order_kernel");
  return 0;
}

}  // namespace uly
