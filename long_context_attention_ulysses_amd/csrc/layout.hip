// Transposed, contraction-ordered copies of Q, K, V or dO for the attention
// kernels.
//
// An MFMA operand whose contraction index is the token (V in O = P V, K in
// dQ = dS K, Q and dO in dK = dS^T Q and dV = P^T dO) needs the tokens of one
// d value contiguous. This pass writes, for each head, a [D][Np] copy:
//   xt[h][d][t*64 + key_pos(j)] = x[t*64 + j][h][d]   (zero for tokens >= N)
// with Np = N rounded up to 64, so the attention kernels can stream 64-token
// tiles of it straight into LDS and read operands with 16-byte loads. It is
// HBM-bound and costs about one read and one write of the tensor.
#include "attn_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

template <int D>
__global__ void __launch_bounds__(256) to_trans_kernel(const bf16_t *__restrict__ x, int64_t xs,
                                                       int64_t N, int64_t Np, bf16_t *__restrict__ xt) {
  constexpr int ROW = D + 8;  // padded LDS row (elements)
  __shared__ __align__(16) bf16_t tile[64 * ROW];
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)t * 64;
  const bf16_t *src = x + (int64_t)h * D;

  constexpr int VECS = 64 * D / 8;
#pragma unroll
  for (int i = threadIdx.x; i < VECS; i += 256) {
    const int r = i / (D / 8), c = i % (D / 8);
    u32x4 v = {0, 0, 0, 0};
    if (t0 + r < N) v = *reinterpret_cast<const u32x4 *>(src + (t0 + r) * xs + c * 8);
    *reinterpret_cast<u32x4 *>(tile + r * ROW + c * 8) = v;
  }
  __syncthreads();

  bf16_t *dst = xt + (int64_t)h * D * Np + t0;
#pragma unroll
  for (int i = threadIdx.x; i < VECS; i += 256) {
    const int d = i / 8, c = i % 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = key_pos(c * 8 + 2 * e), j1 = key_pos(c * 8 + 2 * e + 1);
      w[e] = (uint32_t)tile[j0 * ROW + d] | ((uint32_t)tile[j1 * ROW + d] << 16);
    }
    u32x4 v = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4 *>(dst + (int64_t)d * Np + c * 8) = v;
  }
}

}  // namespace

int launch_to_trans(const bf16_t *x, int64_t xs, int heads, int d, int64_t N, bf16_t *xt,
                    hipStream_t stream) {
  const int64_t Np = pad64(N);
  dim3 grid((unsigned)(Np / 64), (unsigned)heads);
  if (d == 128)
    hipLaunchKernelGGL(to_trans_kernel<128>, grid, dim3(256), 0, stream, x, xs, N, Np, xt);
  else
    hipLaunchKernelGGL(to_trans_kernel<64>, grid, dim3(256), 0, stream, x, xs, N, Np, xt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "to_trans_kernel");
  return 0;
}

}  // namespace uly
