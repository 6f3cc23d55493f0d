// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uly_common.h"

namespace uly {

// (chunk, segment) runs handled by one swap launch (grid.y).
constexpr int kMaxSwapRuns = 32;

// Records a HIP error message for uly_last_error() and returns ULY_E_HIP.
int set_hip_error(hipError_t e, const char *where);

// Packs (to_head) or unpacks the token-split tensor; arguments validated.
int launch_swap(bool to_head, const bf16_t *src, bf16_t *dst, int64_t n, int P, int nseg,
                const int32_t *seg_heads, int d, hipStream_t stream);

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

int launch_attn_fwd(const AttnShape &s, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                    bf16_t *o, float *lse, hipStream_t stream);

struct AttnBwdPtrs {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;
  bf16_t *dq, *dk, *dv;
  int64_t do_stride, dq_stride, dk_stride, dv_stride;
  float *delta;  // workspace: D = rowsum(dO * O), [hq][N] float32
};

// parts: 1 = D and dQ, 2 = dK and dV (reads D), 3 = both in that order.
int launch_attn_bwd(const AttnShape &s, const AttnBwdPtrs &p, int parts, hipStream_t stream);

}  // namespace uly
