// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uly_common.h"

namespace uly {

// Records a HIP error message for uly_last_error() and returns ULY_E_HIP.
int set_hip_error(hipError_t e, const char *where);

// Records a message for uly_last_error() and returns ULY_E_HIP (failures of
// library calls other than HIP's own).
int set_error_text(const char *msg);

// Packs (to_head) or unpacks the token-split tensor; arguments validated.
int launch_swap(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                const int32_t *seg_heads, int d, hipStream_t stream);

__host__ __device__ inline int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Over packed documents: q_order (if not null) receives the ids of the
// blocks of q_bs queries by decreasing number of 64-key tiles in their key
// ranges, k_order (if not null) those of the blocks of k_bs keys by
// decreasing number of 64-query tiles in their query ranges.
int launch_block_orders(const int32_t *cu, int n_seqs, int64_t N, int causal, int q_bs, int32_t *q_order,
                        int k_bs, int32_t *k_order, hipStream_t stream);

// Writes xt[h][d][pad64(N)]: the contraction-ordered, transposed copy of the
// `heads` heads of x (token stride xs), zero beyond N.
int launch_to_trans(const bf16_t *x, int64_t xs, int heads, int d, int64_t N, bf16_t *xt,
                    hipStream_t stream);

// Forward workspace: V^T [hkv][d][pad64(N)].
// Number of workgroups the forward splits each (query block of 256 / hpw
// rows, group of hpw query heads) pair's key range over: 1 when there are at
// least 512 pairs (two per CU), else enough to reach 512, at most 4; hpw is
// the largest of 4, 2, 1 dividing the GQA group size. With a split the
// kernel writes float32 partial softmax states (unnormalised O, running max,
// sum) and a second pass merges them. The dq kernel uses the same blocks.
inline int fwd_ksplit(int64_t N, int hq, int hkv) {
  const int G = hq / hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int64_t bm = 256 / hpw;
  const int64_t pairs = (N + bm - 1) / bm * (hq / hpw);
  if (pairs >= 512) return 1;
  const int64_t s = (512 + pairs - 1) / pairs;
  return s < 4 ? (int)s : 4;
}

// Forward workspace: V^T [hkv][d][pad64(N)] bf16, then, when the forward
// splits its key ranges, float32 partials: O [s][N][hq][d], max [s][hq][N],
// sum [s][hq][N], then the int32 order of the query blocks for packed
// documents (pad64(N) / 64 entries).
inline size_t fwd_ws_part(int64_t N, int hkv, int d) {
  return align256((size_t)hkv * d * pad64(N) * sizeof(bf16_t));
}
inline size_t fwd_ws_order(int64_t N, int hq, int hkv, int d) {
  const int s = fwd_ksplit(N, hq, hkv);
  return fwd_ws_part(N, hkv, d) + (s > 1 ? align256((size_t)s * N * hq * (d + 2) * 4) : 0);
}
inline size_t fwd_ws_bytes(int64_t N, int hq, int hkv, int d) {
  return fwd_ws_order(N, hq, hkv, d) + align256((size_t)pad64(N) / 64 * 4);
}

// Number of workgroups the dK/dV kernel splits each (128-key block, KV head)
// pair's query range over: 1 when there are at least 512 pairs (two per CU
// of the MI355X), else enough to reach 512, at most 4. With a split the
// kernel writes float32 partial dK/dV and a second pass sums them.
inline int dkdv_ksplit(int64_t N, int hkv) {
  const int64_t pairs = (N + 127) / 128 * hkv;
  if (pairs >= 512) return 1;
  const int64_t s = (512 + pairs - 1) / pairs;
  return s < 4 ? (int)s : 4;
}

// The dq kernel splits its key ranges by the same rule as the forward
// (same blocks); with a split it writes float32 partial dQ and a second
// pass sums them.
inline int dq_ksplit(int64_t N, int hq, int hkv) { return fwd_ksplit(N, hq, hkv); }

// Backward workspace regions (byte offsets): -D and LSE*log2(e) as float
// [hq][pad64(N)], then K^T, Q^T, dO^T as contraction-ordered bf16 copies,
// then the int32 orders of the dK/dV kernel's key blocks and of the dq
// kernel's query blocks for packed documents (pad64(N) / 64 entries each),
// then, when the dK/dV kernel splits its
// query ranges, the float32 partials [ksplit][N][hkv][dK, dV][d], and when
// the dq kernel splits its key ranges, the float32 partials [s][N][hq][d].
struct BwdWs {
  size_t delta, lse2, kt, qt, dot, korder, qorder, part, qpart, total;
};

inline BwdWs bwd_ws_layout(int64_t N, int hq, int hkv, int d) {
  const size_t np = (size_t)pad64(N);
  BwdWs w;
  w.delta = 0;
  w.lse2 = w.delta + align256((size_t)hq * np * 4);
  w.kt = w.lse2 + align256((size_t)hq * np * 4);
  w.qt = w.kt + align256((size_t)hkv * d * np * 2);
  w.dot = w.qt + align256((size_t)hq * d * np * 2);
  w.korder = w.dot + align256((size_t)hq * d * np * 2);
  w.qorder = w.korder + align256(np / 64 * 4);
  w.part = w.qorder + align256(np / 64 * 4);
  const int ks = dkdv_ksplit(N, hkv);
  w.qpart = w.part + (ks > 1 ? align256((size_t)ks * N * hkv * 2 * d * 4) : 0);
  const int qs = dq_ksplit(N, hq, hkv);
  w.total = w.qpart + (qs > 1 ? align256((size_t)qs * N * hq * d * 4) : 0);
  return w;
}

// Attention problem description shared by the forward and backward launches.
struct AttnShape {
  int64_t N;
  int hq, hkv, d;
  int64_t q_stride, k_stride, v_stride, o_stride;
  float scale;
  int causal;
  const int32_t *cu;  // device cu_seqlens or nullptr
  int n_seqs;
};

// ws: fwd_ws_bytes(N, hq, hkv, d) bytes, 256-byte aligned.
int launch_attn_fwd(const AttnShape &s, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                    bf16_t *o, float *lse, void *ws, hipStream_t stream);

struct AttnBwdPtrs {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;
  bf16_t *dq, *dk, *dv;
  int64_t do_stride, dq_stride, dk_stride, dv_stride;
  char *ws;  // workspace laid out by bwd_ws_layout
};

// parts: 1 = D and dQ, 2 = dK and dV (reads D), 3 = both in that order.
int launch_attn_bwd(const AttnShape &s, const AttnBwdPtrs &p, int parts, hipStream_t stream);

// Most per-block results one merge or gradient-sum launch takes.
constexpr int kMaxParts = 16;

// out, lse_out = merge of n_parts (o, lse) results over disjoint key blocks;
// arguments validated.
int launch_lse_merge(int n_parts, const bf16_t *const *o, const float *const *lse, bf16_t *out,
                     float *lse_out, int64_t N, int h, int d, int64_t part_stride, int64_t out_stride,
                     hipStream_t stream);

// out = sum of n_parts bf16 [rows][width] views (float accumulation).
int launch_grad_sum(int n_parts, const bf16_t *const *parts, bf16_t *out, int64_t rows, int width,
                    int64_t part_stride, int64_t out_stride, hipStream_t stream);

// Shifted-label cross-entropy of one rank: per-row loss and log-sum-exp,
// then the rank's mean loss over good rows and its good count.
int launch_ce_fwd(const bf16_t *logits, int64_t stride, const int32_t *labels, int64_t n, int64_t V,
                  float *row_loss, float *row_lse, float *loss_out, int32_t *good_out, hipStream_t stream);

// Weighted aggregation over ranks and the per-row gradient scale.
int launch_loss_aggregate(int n_ranks, const float *const *loss, const int32_t *const *good, float *total,
                          float *row_scale, hipStream_t stream);

// Gradient of the aggregate loss with respect to one rank's logits.
int launch_ce_bwd(const bf16_t *logits, int64_t stride, const int32_t *labels, const float *row_lse,
                  const float *row_scale, int64_t n, int64_t V, bf16_t *grad, int64_t gstride,
                  hipStream_t stream);

// TiledMLP workspace regions (byte offsets) for tiles of `tile` tokens:
// gate|up [tile][2I], activation and its gradient [tile][I], gate|up
// gradient [tile][2I] (bf16), then the GEMM library's workspace.
constexpr size_t kMlpBlasWs = (size_t)64 << 20;
struct MlpWs {
  size_t gu, act, dact, dgu, blas, total;
};
inline MlpWs mlp_ws_layout(int64_t tile, int H, int I) {
  (void)H;
  MlpWs w;
  w.gu = 0;
  w.act = w.gu + align256((size_t)tile * 2 * I * 2);
  w.dact = w.act + align256((size_t)tile * I * 2);
  w.dgu = w.dact + align256((size_t)tile * I * 2);
  w.blas = w.dgu + align256((size_t)tile * 2 * I * 2);
  w.total = w.blas + kMlpBlasWs;
  return w;
}

struct MlpPtrs {
  const bf16_t *x, *w_gu, *w_down, *dy;
  bf16_t *y, *dx;
  float *dw_gu, *dw_down;
  char *ws;
};

// Forward (y) or backward (dx, dw_gu, dw_down; added to when accumulate)
// of the SwiGLU MLP over token tiles; arguments validated.
int launch_mlp(bool bwd, const MlpPtrs &p, int64_t n, int H, int I, int64_t tile, bool accumulate,
               hipStream_t stream);

}  // namespace uly
