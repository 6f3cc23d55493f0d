// TiledMLP: the SwiGLU MLP of the model run over the sequence in token tiles,
// so that only one tile's intermediate activations ([tile][2I] gate|up and
// [tile][I] activation) ever exist; the backward pass recomputes them tile
// by tile. The pages name it as the second memory component of ALST next to
// Ulysses ("Ulysses sequence parallelism", intro note on ALST; "Ulysses
// Sequence Parallelism for Million-Token Context Training", Additional
// Kernels) without describing it; this is the plainest reading: per token,
//   gu = x W_gu^T (gate | up, [2I]),  a = silu(gate) * up,  y = a W_down^T,
// with the token dimension processed tile by tile. The result does not depend
// on the tile size (every token is independent), only the peak memory does.
//
// The three GEMMs per tile are plain bf16 GEMMs with float32 accumulation and
// go to hipBLASLt; the SwiGLU forward and backward are HIP kernels. Weight
// gradients accumulate in float32 across tiles.
#include <hipblaslt/hipblaslt.h>
#include <math.h>

#include <mutex>

#include "uly_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

// ------------------------------------------------------------ SwiGLU ----

struct GluArgs {
  const bf16_t *gu;  // [T][2I]: gate | up
  const bf16_t *da;  // [T][I] upstream gradient of the activation (bwd)
  bf16_t *act;       // [T][I]
  bf16_t *dgu;       // [T][2I] (bwd)
  uint32_t vpr;      // 16-byte vectors per activation row (I / 8)
  uint32_t total;    // T * vpr
  FastDiv div_vpr;
  uint32_t I;
};

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

// act = silu(gate) * up, 8 values per thread.
__global__ void __launch_bounds__(256) swiglu_fwd_kernel(GluArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t r = a.div_vpr.q(i);
  const uint32_t c = (i - r * a.vpr) * 8;
  const int64_t row2 = (int64_t)r * 2 * a.I;
  const u32x4 g = *reinterpret_cast<const u32x4 *>(a.gu + row2 + c);
  const u32x4 u = *reinterpret_cast<const u32x4 *>(a.gu + row2 + a.I + c);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float g0 = __uint_as_float(g[e] << 16), g1 = __uint_as_float(g[e] & 0xFFFF0000u);
    const float u0 = __uint_as_float(u[e] << 16), u1 = __uint_as_float(u[e] & 0xFFFF0000u);
    o[e] = pack_bf16x2(g0 * sigmoidf_(g0) * u0, g1 * sigmoidf_(g1) * u1);
  }
  *reinterpret_cast<u32x4 *>(a.act + (int64_t)r * a.I + c) = o;
}

// From gate, up and dA: dgate = dA * up * s * (1 + g (1 - s)) with
// s = sigmoid(g), dup = dA * silu(g); also recomputes act for dW_down.
__global__ void __launch_bounds__(256) swiglu_bwd_kernel(GluArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t r = a.div_vpr.q(i);
  const uint32_t c = (i - r * a.vpr) * 8;
  const int64_t row2 = (int64_t)r * 2 * a.I, row1 = (int64_t)r * a.I;
  const u32x4 g = *reinterpret_cast<const u32x4 *>(a.gu + row2 + c);
  const u32x4 u = *reinterpret_cast<const u32x4 *>(a.gu + row2 + a.I + c);
  const u32x4 d = *reinterpret_cast<const u32x4 *>(a.da + row1 + c);
  u32x4 og, ou, oa;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float gv[2] = {__uint_as_float(g[e] << 16), __uint_as_float(g[e] & 0xFFFF0000u)};
    float uv[2] = {__uint_as_float(u[e] << 16), __uint_as_float(u[e] & 0xFFFF0000u)};
    float dv[2] = {__uint_as_float(d[e] << 16), __uint_as_float(d[e] & 0xFFFF0000u)};
    float dg[2], du[2], av[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float s = sigmoidf_(gv[k]);
      const float silu = gv[k] * s;
      av[k] = silu * uv[k];
      du[k] = dv[k] * silu;
      dg[k] = dv[k] * uv[k] * s * (1.f + gv[k] * (1.f - s));
    }
    og[e] = pack_bf16x2(dg[0], dg[1]);
    ou[e] = pack_bf16x2(du[0], du[1]);
    oa[e] = pack_bf16x2(av[0], av[1]);
  }
  *reinterpret_cast<u32x4 *>(a.dgu + row2 + c) = og;
  *reinterpret_cast<u32x4 *>(a.dgu + row2 + a.I + c) = ou;
  *reinterpret_cast<u32x4 *>(a.act + row1 + c) = oa;
}

int launch_glu(bool bwd, const bf16_t *gu, const bf16_t *da, bf16_t *act, bf16_t *dgu, int64_t T, int I,
               hipStream_t stream) {
  GluArgs a;
  a.gu = gu;
  a.da = da;
  a.act = act;
  a.dgu = dgu;
  a.I = (uint32_t)I;
  a.vpr = (uint32_t)(I / 8);
  a.total = (uint32_t)(T * (I / 8));
  a.div_vpr = FastDiv(a.vpr);
  const dim3 grid((a.total + 255) / 256);
  if (bwd)
    hipLaunchKernelGGL(swiglu_bwd_kernel, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(swiglu_fwd_kernel, grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, bwd ? "swiglu_bwd_kernel" : "swiglu_fwd_kernel");
  return 0;
}

// ------------------------------------------------------------- GEMMs ----

// One hipBLASLt handle per device, created on first use and kept until the
// process ends (the library's only state beyond the error message).
constexpr int kMaxDevices = 64;
hipblasLtHandle_t g_lt[kMaxDevices];
std::mutex g_lt_mu;

int blas_error(hipblasStatus_t st, const char *where) {
  char msg[160];
  snprintf(msg, sizeof(msg), "%s: hipBLASLt status %d", where, (int)st);
  return set_error_text(msg);
}

int lt_handle(hipblasLtHandle_t *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_error_text("device index out of range for hipBLASLt handles");
  std::lock_guard<std::mutex> lock(g_lt_mu);
  if (!g_lt[dev]) {
    hipblasStatus_t st = hipblasLtCreate(&g_lt[dev]);
    if (st != HIPBLAS_STATUS_SUCCESS) {
      g_lt[dev] = nullptr;
      return blas_error(st, "hipblasLtCreate");
    }
  }
  *out = g_lt[dev];
  return 0;
}

// Column-major D (m x n, leading dimension ldd) = op(A) op(B) + beta D, with
// A, B bf16 (lda, ldb), D bf16 or float32, float32 accumulation.
int gemm(hipblasLtHandle_t h, bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void *A, int64_t lda,
         const void *B, int64_t ldb, void *D, int64_t ldd, bool d_f32, float beta, void *ws, size_t ws_bytes,
         hipStream_t stream) {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  int rc = 0;
  hipblasStatus_t st;
  const hipblasOperation_t opa = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipDataType dt = d_f32 ? HIP_R_32F : HIP_R_16BF;
  const uint64_t wsb = ws_bytes;
  hipblasLtMatmulHeuristicResult_t heur[1];
  int found = 0;
  const float alpha = 1.f;
#define ULY_LT(call, name)                   \
  do {                                       \
    st = (call);                             \
    if (st != HIPBLAS_STATUS_SUCCESS) {      \
      rc = blas_error(st, name);             \
      goto done;                             \
    }                                        \
  } while (0)
  ULY_LT(hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F), "hipblasLtMatmulDescCreate");
  ULY_LT(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)), "TRANSA");
  ULY_LT(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)), "TRANSB");
  ULY_LT(hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, ta ? k : m, ta ? m : k, lda), "layout A");
  ULY_LT(hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, tb ? n : k, tb ? k : n, ldb), "layout B");
  ULY_LT(hipblasLtMatrixLayoutCreate(&ld, dt, m, n, ldd), "layout D");
  ULY_LT(hipblasLtMatmulPreferenceCreate(&pref), "hipblasLtMatmulPreferenceCreate");
  ULY_LT(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb)),
         "workspace preference");
  ULY_LT(hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, 1, heur, &found), "heuristic");
  if (found < 1) {
    rc = set_error_text("hipBLASLt found no algorithm for a TiledMLP GEMM");
    goto done;
  }
  ULY_LT(hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &heur[0].algo, ws, ws_bytes, stream),
         "hipblasLtMatmul");
#undef ULY_LT
done:
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return rc;
}

}  // namespace

// Row-major tensors: x, y, dy, dx [n][H]; w_gu [2I][H]; w_down [H][I];
// dw_gu [2I][H], dw_down [H][I] float32. A row-major [r][c] matrix is a
// column-major (c x r) matrix with leading dimension c.
int launch_mlp(bool bwd, const MlpPtrs &p, int64_t n, int H, int I, int64_t tile, bool accumulate,
               hipStream_t stream) {
  hipblasLtHandle_t h;
  int rc = lt_handle(&h);
  if (rc) return rc;
  const MlpWs L = mlp_ws_layout(tile, H, I);
  bf16_t *gu = reinterpret_cast<bf16_t *>(p.ws + L.gu);
  bf16_t *act = reinterpret_cast<bf16_t *>(p.ws + L.act);
  bf16_t *dact = reinterpret_cast<bf16_t *>(p.ws + L.dact);
  bf16_t *dgu = reinterpret_cast<bf16_t *>(p.ws + L.dgu);
  void *bws = p.ws + L.blas;
  const size_t bwsb = L.total - L.blas;
  for (int64_t t0 = 0; t0 < n; t0 += tile) {
    const int64_t T = (n - t0) < tile ? (n - t0) : tile;
    const bf16_t *xt = p.x + t0 * H;
    // gu^T (2I x T) = W_gu (2I x H) . x_t^T (H x T)
    if ((rc = gemm(h, true, false, 2 * I, T, H, p.w_gu, H, xt, H, gu, 2 * I, false, 0.f, bws, bwsb, stream)))
      return rc;
    if (!bwd) {
      if ((rc = launch_glu(false, gu, nullptr, act, nullptr, T, I, stream))) return rc;
      // y_t^T (H x T) = W_down (H x I) . a^T (I x T)
      if ((rc = gemm(h, true, false, H, T, I, p.w_down, I, act, I, p.y + t0 * H, H, false, 0.f, bws, bwsb,
                     stream)))
        return rc;
      continue;
    }
    const bf16_t *dyt = p.dy + t0 * H;
    // dA^T (I x T) = W_down^T (I x H) . dy_t^T (H x T)
    if ((rc = gemm(h, false, false, I, T, H, p.w_down, I, dyt, H, dact, I, false, 0.f, bws, bwsb, stream)))
      return rc;
    if ((rc = launch_glu(true, gu, dact, act, dgu, T, I, stream))) return rc;
    // dx_t^T (H x T) = W_gu^T (H x 2I) . dgu^T (2I x T)
    if ((rc = gemm(h, false, false, H, T, 2 * I, p.w_gu, H, dgu, 2 * I, p.dx + t0 * H, H, false, 0.f, bws, bwsb,
                   stream)))
      return rc;
    const float beta = (accumulate || t0 > 0) ? 1.f : 0.f;
    // dW_gu^T (H x 2I) += x_t^T (H x T) . dgu (T x 2I)
    if ((rc = gemm(h, false, true, H, 2 * I, T, xt, H, dgu, 2 * I, p.dw_gu, H, true, beta, bws, bwsb, stream)))
      return rc;
    // dW_down^T (I x H) += a^T (I x T) . dy_t (T x H)
    if ((rc = gemm(h, false, true, I, H, T, act, I, dyt, H, p.dw_down, I, true, beta, bws, bwsb, stream)))
      return rc;
  }
  return 0;
}

}  // namespace uly
