// Pieces shared by the attention forward and backward kernels (gfx950).
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16, wave64; lane l, slot i):
//   A (32 x 16, M x K): lane l holds A[l % 32][(l / 32) * 8 + i], i = 0..7
//   B (16 x 32, K x N): lane l holds B[(l / 32) * 8 + i][l % 32]
//   C (32 x 32):        lane l, reg i holds C[(i / 4) * 8 + (l / 32) * 4 + i % 4][l % 32]
// Scores are computed transposed, S^T = K Q^T (M = keys, N = queries), so a
// lane owns one query and the softmax reductions over keys stay inside the
// lane except for one exchange with lane l ^ 32.
//
// Feeding S^T's C registers straight back as the B operand of the next
// product (key index as the contraction index) visits the 16 keys of a step
// in the order given by swapping bits 2 and 3 of the key index; the other
// operand is stored in LDS in that order, see key_pos().
#pragma once

#include "uly_common.h"

namespace uly {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Position of key `j` (within a 16-aligned group) in the MFMA-contraction
// order described above: bits 2 and 3 swapped.
__host__ __device__ __forceinline__ int key_pos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// Eight fp32 values -> eight bf16 (round to nearest even) as an MFMA operand.
__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  u32x4 r;
  r[0] = pack_bf16x2(a0, a1);
  r[1] = pack_bf16x2(a2, a3);
  r[2] = pack_bf16x2(a4, a5);
  r[3] = pack_bf16x2(a6, a7);
  return as_bf16x8(r);
}

// Element offset of (row r, position p) in a transposed LDS tile whose rows
// hold 64 positions (keys or queries, in MFMA-contraction order). The eight
// 16-byte chunks of a row are XOR-swizzled with bits 1..3 of the row so that
// sixteen consecutive rows read at one chunk position hit distinct banks.
__device__ __forceinline__ int tr_off(int r, int p) {
  const int chunk = (p >> 3) ^ ((r >> 1) & 7);
  return r * 64 + (chunk << 3) + (p & 7);
}

// Value of lane l ^ 32.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Document containing token t: largest b with cu[b] <= t (cu strictly increasing).
__device__ __forceinline__ int doc_of(const int32_t *cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Keys visible to query i: [lo, hi).
struct KeyRange {
  int64_t lo, hi;
};

__device__ __forceinline__ KeyRange key_range(const int32_t *cu, int n_seqs, int64_t N, int causal,
                                              int64_t i) {
  KeyRange r;
  if (cu) {
    int b = doc_of(cu, n_seqs, i);
    r.lo = cu[b];
    r.hi = cu[b + 1];
  } else {
    r.lo = 0;
    r.hi = N;
  }
  if (causal) r.hi = i + 1;
  return r;
}

// Queries that see key j: [lo, hi).
__device__ __forceinline__ KeyRange query_range(const int32_t *cu, int n_seqs, int64_t N,
                                                int causal, int64_t j) {
  KeyRange r;
  if (cu) {
    int b = doc_of(cu, n_seqs, j);
    r.lo = cu[b];
    r.hi = cu[b + 1];
  } else {
    r.lo = 0;
    r.hi = N;
  }
  if (causal) r.lo = j;
  return r;
}

}  // namespace uly
