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

#define ULY_LDS __attribute__((address_space(3)))

// ---- LDS tiles -------------------------------------------------------------
// Two tile shapes, both 64 rows/positions deep and filled by direct-to-LDS
// copies (buffer_load_dwordx4 ... lds: lane i's 16 bytes land at base + 16 i, so
// any permutation of 16-byte chunks inside a 1 KiB block is free to build):
//
//   row tile   [64 rows][D]: a token's d values in one row; the 16-byte
//              chunks of row r are XOR-swizzled so that 16 consecutive rows
//              read at one chunk position hit 16 distinct bank groups.
//   trans tile [D rows][64 positions]: one row per d, positions in MFMA
//              contraction order; chunks XOR-swizzled with bits 1..3 of the
//              row for the same reason (a row is half the 256-byte bank width).
// Both are read with ds_read_b128 only (a row tile as the [row][k] operand,
// a trans tile as the [d][position] operand).

// Swizzle of row tile row r (chunk index space of D/8 chunks).
template <int D>
__device__ __forceinline__ int row_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Element offset of logical 16-byte chunk c of row r in a row tile.
template <int D>
__device__ __forceinline__ int rt_off(int r, int c) {
  return r * D + ((c ^ row_swz<D>(r)) << 3);
}

// Element offset of logical 16-byte chunk c (positions 8c..8c+7) of row r in
// a trans tile.
__device__ __forceinline__ int tr_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// ---- Row tiles read both ways (d = 128) ------------------------------------
// A [64 rows][128] row tile that is read both as the [row][k] operand (16
// consecutive rows at one 16-byte chunk, as above) and, transposed, as the
// [d][row] operand of a product that contracts over its rows. The
// transposed operand comes from ds_read_b64_tr_b16: in each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces that lanes
// i / 4 + 4 j (j = 0..3) point at. With lane s of the group pointing at row
// base + s / 4, elements 4 (s % 4) .. +3 of a 16-column block, lane i
// receives column i of rows base .. base + 3: four consecutive rows of one
// column, as the MFMA operand needs. Two such reads give the eight rows of
// one 16-position contraction step, in the contraction order of the score
// registers (positions 8 h + e hold rows 16 c + 8 (e / 4) + 4 h + e % 4).
// The swizzle swaps the two 2-bit halves of the row's low 4 bits, so that
// both the 16 rows of a row read and the 4 rows x 4 chunks of the 32 lanes
// of a transposing read land on distinct banks.
__device__ __forceinline__ int rt2_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Element offset of logical 16-byte chunk c of row r.
__device__ __forceinline__ int rt2_off(int r, int c) { return r * 128 + ((c ^ rt2_swz(r)) << 3); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One transposing 8-byte LDS read at LDS byte address `addr`.
__device__ __forceinline__ u32x2 ds_read_tr(uint32_t addr) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane byte offsets, inside a row tile, of the two transposing reads
// (r = 0, 1) that make the [32 d][16 rows] operand for d block db and the
// first 16-row step; step c adds 4096 c bytes.
struct TrOffsets {
  uint32_t off[2][4];
};

__device__ __forceinline__ TrOffsets tr_offsets(int lane) {
  const int hi = lane >> 5, y = (lane & 15) >> 2, x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1), h = lane & 1;
  TrOffsets t;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int m = (y << 2) ^ (2 * r + hi) ^ x;  // chunk 4 db + x of row 8 r + 4 hi + y, swizzled
#pragma unroll
    for (int db = 0; db < 4; ++db)
      t.off[r][db] = (uint32_t)(((8 * r + 4 * hi + y) * 128 + (((4 * db) ^ m) << 3) + 4 * h) * 2);
  }
  return t;
}

// The transposed operand (A[m = d][k = row]) for d block db and 16-row step
// c of the row tile at LDS byte address `tile`.
__device__ __forceinline__ bf16x8 tr_frag(uint32_t tile, const TrOffsets &t, int db, int c) {
  const u32x2 lo = ds_read_tr(tile + t.off[0][db] + 4096 * c);
  const u32x2 hi = ds_read_tr(tile + t.off[1][db] + 4096 * c);
  u32x4 v;
  v[0] = lo[0];
  v[1] = lo[1];
  v[2] = hi[0];
  v[3] = hi[1];
  return as_bf16x8(v);
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// 16-byte LDS reads at LDS byte address `addr` (16-byte aligned).
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) { return *(const lds_u32x4 *)(uintptr_t)addr; }
__device__ __forceinline__ f32x4 lds_read16f(uint32_t addr) { return *(const lds_f32x4 *)(uintptr_t)addr; }

// Buffer resource (four SGPRs) over the `bytes` bytes at `base`: buffer
// loads at byte offsets >= bytes return zeros (raw buffer, stride 0).
typedef uint32_t BufRes __attribute__((ext_vector_type(4)));
__device__ __forceinline__ BufRes make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  BufRes r;
  r[0] = (uint32_t)b;
  r[1] = (uint32_t)(b >> 32) & 0xFFFFu;
  r[2] = bytes;
  r[3] = 0x00020000u;
  return r;
}

// LDS byte address of a (generic) pointer into a __shared__ array, made
// wave-uniform: the low 32 bits of a flat address in the LDS aperture (taking
// them needs no null check, unlike a cast to the LDS address space).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// The resource words as SGPR values: the asm operands below must be SGPRs,
// and the compiler does not move a value it takes for divergent into them by
// itself (free where the value is already uniform).
__device__ __forceinline__ BufRes uniform(BufRes r) {
  BufRes u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// Wave-wide direct-to-LDS copy of 16 bytes per lane from buffer `r` at byte
// offset voff + soff (voff per lane, soff wave-uniform): lane i's bytes land
// at lds + 16 i (`lds` points into a __shared__ array, wave-uniform).
// Range checking uses voff only.
//
// Written as inline asm so that the compiler keeps no record of the copy:
// it cannot tell which LDS bytes an in-flight copy writes and would
// otherwise wait for every copy still in flight before each LDS read, which
// drains the prefetch ring. The caller orders the copy against its readers
// with wait_vmcnt and barrier (both also compiler memory fences), and keeps
// voff in a loop-invariant register (move the tile's start into the resource
// base instead), so that no copy waits for a register it reads. The leading
// s_nop 4 gives the five wait states a VMEM instruction needs after a VALU
// write of an SGPR it reads (a resource word restored by v_readlane) and
// covers the one after the M0 write: the compiler's hazard check does not
// look into inline asm.
__device__ __forceinline__ void dma16(BufRes r, uint32_t voff, uint32_t soff, const void *lds) {
  const uint32_t m0 = lds_addr(lds);
  r = uniform(r);
  soff = __builtin_amdgcn_readfirstlane(soff);
  __asm__ volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                   :
                   : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
                   : "memory");
}

// Same with 4 bytes per lane (lane i -> lds + 4 i).
__device__ __forceinline__ void dma4(BufRes r, uint32_t voff, uint32_t soff, const void *lds) {
  const uint32_t m0 = lds_addr(lds);
  r = uniform(r);
  soff = __builtin_amdgcn_readfirstlane(soff);
  __asm__ volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
                   :
                   : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
                   : "memory");
}

// Bytes from the start of a head's first row to the end of its row N-1 in a
// [N][heads][d] bf16 tensor with token stride `stride` (elements): the
// buffer range of one head's rows, so rows >= N read as zeros.
__host__ __device__ __forceinline__ uint32_t head_rows_bytes(int64_t N, int64_t stride, int d) {
  return (uint32_t)(((N - 1) * stride + d) * 2);
}


// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N); the other counters are left unconstrained). The empty
// asm statements keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier without a memory fence: LDS tiles written by
// direct-to-LDS copies are covered by the explicit vmcnt waits before it.
// The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier after this wave's own LDS stores (s_waitcnt lgkmcnt(0),
// then s_barrier), without waiting for direct-to-LDS copies still in flight.
// The empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Scheduling hint for the basic block it ends: LA LDS reads first, then
// one MFMA and one LDS read alternately, then the last LA MFMAs, so that
// each MFMA's operand was requested LA reads earlier (group masks: 0x100
// LDS reads, 0x008 MFMA).
template <int NR, int LA = 4>
__device__ __forceinline__ void pipeline_reads_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
  for (int i = 0; i < NR - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// The same for blocks whose MFMAs take RPM LDS reads each: LA MFMAs'
// worth of reads first, then one MFMA and its next RPM reads alternately.
template <int NM, int RPM, int LA = 4>
__device__ __forceinline__ void pipeline_reads_mfma_n() {
  __builtin_amdgcn_sched_group_barrier(0x100, LA * RPM, 0);
#pragma unroll
  for (int i = 0; i < NM - LA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// A lane's token range [lo, hi) relative to a 64-token tile at t0, for
// masking the tile's elements: element offset E (0..63) is inside iff
// lo <= E - lane_off < hi. The offsets are clamped to [-1, 65] first, which
// keeps every comparison with E in 0..63, so they fit in 32 bits.
struct RelRange {
  int lo, hi;
};
__host__ __device__ __forceinline__ RelRange rel_range(int64_t lo, int64_t hi, int64_t t0, int lane_off) {
  int64_t l = lo - t0, h = hi - t0;
  l = l < -1 ? -1 : (l > 65 ? 65 : l);
  h = h < -1 ? -1 : (h > 65 ? 65 : h);
  return RelRange{(int)l - lane_off, (int)h - lane_off};
}

// Value of lane l ^ 32.
// Max and sum of x over lanes l and l ^ 32, in every lane of the wave.
// v_permlane32_swap trades the upper 32 lanes of its first operand for the
// lower 32 of its second; with x in both, each lane ends up holding x of
// both halves (its own and its partner's) in registers, where a shuffle
// goes through LDS and waits for every LDS access in flight. max and +
// commute, so both lanes of a pair get the same bits.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Document containing token t: largest b with cu[b] <= t (cu strictly increasing).
__host__ __device__ __forceinline__ int doc_of(const int32_t *cu, int n_seqs, int64_t t) {
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

// A range cut to [0, N) with lo <= hi. For a valid cu_seqlens table this
// changes nothing; for a table the host did not check (entries past N,
// negative or unsorted) it keeps every tile index the kernels derive from
// the range inside the tensors, so such a table gives wrong values rather
// than out-of-range addresses.
__host__ __device__ __forceinline__ KeyRange clamp_range(KeyRange r, int64_t N) {
  if (r.hi > N) r.hi = N;
  if (r.lo < 0) r.lo = 0;
  if (r.lo > r.hi) r.lo = r.hi;
  return r;
}

__host__ __device__ __forceinline__ KeyRange key_range(const int32_t *cu, int n_seqs, int64_t N, int causal,
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
  return clamp_range(r, N);
}

// Queries that see key j: [lo, hi).
__host__ __device__ __forceinline__ KeyRange query_range(const int32_t *cu, int n_seqs, int64_t N,
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
  return clamp_range(r, N);
}

// The same ranges for a token i when the document b of a token at or
// before i is known (b = doc_start(t0) with t0 <= i): the document of i is
// found by scanning forward from b, since the rows of one block cross few
// document boundaries, instead of by a binary search per token. For a valid
// table the ranges equal key_range / query_range; for any table b stays in
// [b, n_seqs - 1], so the table reads and the clamped range stay in bounds.
__host__ __device__ __forceinline__ int doc_start(const int32_t *cu, int n_seqs, int64_t t0) {
  return cu ? doc_of(cu, n_seqs, t0) : 0;
}

__host__ __device__ __forceinline__ int doc_after(const int32_t *cu, int n_seqs, int b, int64_t t) {
  while (b + 1 < n_seqs && (int64_t)cu[b + 1] <= t) ++b;
  return b;
}

__host__ __device__ __forceinline__ KeyRange key_range_from(const int32_t *cu, int n_seqs, int64_t N, int causal,
                                                            int b, int64_t i) {
  KeyRange r;
  if (cu) {
    b = doc_after(cu, n_seqs, b, i);
    r.lo = cu[b];
    r.hi = cu[b + 1];
  } else {
    r.lo = 0;
    r.hi = N;
  }
  if (causal) r.hi = i + 1;
  return clamp_range(r, N);
}

__host__ __device__ __forceinline__ KeyRange query_range_from(const int32_t *cu, int n_seqs, int64_t N, int causal,
                                                              int b, int64_t j) {
  KeyRange r;
  if (cu) {
    b = doc_after(cu, n_seqs, b, j);
    r.lo = cu[b];
    r.hi = cu[b + 1];
  } else {
    r.lo = 0;
    r.hi = N;
  }
  if (causal) r.lo = j;
  return clamp_range(r, N);
}

}  // namespace uly
