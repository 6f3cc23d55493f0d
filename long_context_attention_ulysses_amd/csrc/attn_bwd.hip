// Attention backward for the local heads of one Ulysses rank: gradients of
// the exact softmax attention computed by attn_fwd, recomputing the scores
// tile by tile from the saved log-sum-exp instead of storing an N x N matrix
// ("The Challenge of Long Sequence Training": O(n) memory for O(n^2) work).
//
// With p_ij = exp(s_ij - LSE_i), s = scale * q.k, loss L = sum dO * O:
//   D_i   = sum_e dO_ie O_ie
//   dp_ij = dO_i . v_j,  ds_ij = p_ij (dp_ij - D_i)
//   dQ_i  = scale * sum_j ds_ij k_j
//   dK_j  = scale * sum_{heads of the group} sum_i ds_ij q_i
//   dV_j  = sum_{heads of the group} sum_i p_ij dO_i
//
// Two kernels, no atomics (the result is deterministic). Operands whose
// contraction index is the token come from contraction-ordered transposed
// copies (K^T, Q^T, dO^T, written once per call into the workspace); all
// tiles stream into LDS with direct-to-LDS copies and are read with 16-byte
// loads only.
//   1. dq kernel, parallel over (query block, head): D and LSE*log2(e) for
//      its rows (-D and LSE*log2(e) to the workspace), then per 64-key tile
//      (3-stage ring):
//      S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, dQ^T += K^T dS^T
//      (Q and dO stay in registers as B operands; a lane owns one query).
//   2. dkdv kernel, parallel over (key block, KV head): loops over its
//      64-query tiles from the last one down, the group's heads innermost
//      (3-stage rings at d = 128; concurrent workgroups walk the same tiles
//      in step):
//      S = Q K^T, dP = dO V^T (K, V in registers; a lane owns one key),
//      P, dS, dV^T += dO^T P, dK^T += Q^T dS.
// Small problems (fewer than 512 blocks of either kernel) split each block's
// tiles over up to 4 workgroups that write float32 partials, summed in split
// order by a second pass (still deterministic); over packed documents both
// kernels take their blocks in order of decreasing work.
#include <type_traits>

#include "attn_common.h"
#include "uly_internal.h"

// MFMAs' worth of transposing reads the dK and dV updates keep in flight.
#ifndef ULY_TR_LA
#define ULY_TR_LA 4
#endif
// 16-query steps of the deferred dK update done in phase 1 (the rest in phase 2).
#ifndef ULY_DK_P1
#define ULY_DK_P1 4
#endif

namespace uly {

namespace {

struct BwdArgs {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;
  bf16_t *dq, *dk, *dv;
  float *delta, *lse2;             // workspace [hq][Np]
  const bf16_t *kt, *qt, *dot;     // workspace: contraction-ordered transposes
  int64_t N, Np;
  int64_t q_stride, k_stride, v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride;
  int hq, hkv, G;
  int nblk, nhg;  // blocks along the sequence, head groups
  float c;        // scale * log2(e)
  float scale;
  int causal;
  const int32_t *cu;
  int n_seqs;
  const int32_t *korder;  // packed documents: key blocks by decreasing work
  const int32_t *qorder;  // packed documents: dq query blocks by decreasing work
  int ksplit;             // dK/dV: workgroups per (key block, KV head)
  float *dkv_part;        // dK/dV partials [ksplit][N][hkv][2][d] when ksplit > 1
  int qsplit;             // dq: workgroups per (query block, head group)
  float *dq_part;         // dQ partials [qsplit][N][hq][d] when qsplit > 1
};

// ------------------------------------------------------------ dq kernel ----

// kTr (d = 128): the K^T operand of dQ^T += K^T dS^T is read transposed
// from the K row tile (rt2 layout, as in the dK/dV kernel) instead of being
// copied from the transposed copy of K, so each key tile copies K and V rows
// only.
template <int D, int HPW, int RB>
struct DqCfg {
  static constexpr int NW = HPW * RB;
  static constexpr int NT = NW * 64;
  static constexpr int BN = 64;
  static constexpr int BM = 32 * RB;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int JS = BN / 16;
  static constexpr int TILE = BN * D;
  static constexpr int NI = TILE / 512;    // 1 KiB copies per tile and tensor
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  static constexpr bool kTr = D == 128;
  static constexpr int NLW = (kTr ? 2 : 3) * NI / NW;  // copies per wave per tile (K, V[, K^T])
};

template <int D, int HPW, int RB, bool kSplit>
__global__ void __launch_bounds__(HPW * RB * 64, 1) attn_bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D, HPW, RB>;
  constexpr bool kTr = C::kTr;
  constexpr int TT = kTr ? 8 : C::TILE;  // trans tiles (unused with kTr)
  __shared__ __align__(16) bf16_t k0[C::TILE], k1[C::TILE], k2[C::TILE];
  __shared__ __align__(16) bf16_t v0[C::TILE], v1[C::TILE], v2[C::TILE];
  __shared__ __align__(16) bf16_t t0_[TT], t1_[TT], t2_[TT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;

  // With a split the pieces of one query block are consecutive ids.
  const int item = blockIdx.x;
  const int hg = item % a.nhg;
  const int qbi = kSplit ? item / a.nhg / a.qsplit : item / a.nhg;
  const int qb = a.qorder ? a.qorder[qbi] : a.nblk - 1 - qbi;
  const int split = kSplit ? item / a.nhg % a.qsplit : 0;
  const int64_t q0 = (int64_t)qb * C::BM;
  const int h = hg * HPW + w / RB;
  const int g = (hg * HPW) / a.G;
  const int64_t r0 = q0 + (int64_t)(w % RB) * 32;

  const int64_t q_last = (q0 + C::BM < a.N ? q0 + C::BM : a.N) - 1;
  const int b0 = doc_start(a.cu, a.n_seqs, q0);  // documents found from the block's first row on
  const int64_t kv_lo = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, q0).lo;
  const int64_t kv_hi = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, q_last).hi;
  const bool wave_valid = r0 < a.N;
  const int64_t w_last = (r0 + 32 < a.N ? r0 + 32 : a.N) - 1;
  const KeyRange wr0 = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? r0 : q0);
  const KeyRange wr1 = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? w_last : q0);
  const int64_t w_lo = wr0.lo, w_hi = wr1.hi;
  const int64_t w_lo_max = wr1.lo, w_hi_min = wr0.hi;

  const int64_t row = r0 + l32;
  const bool row_ok = row < a.N;
  int64_t rlo = 0, rhi = 0;
  if (row_ok) {
    const KeyRange kr = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, row);
    rlo = kr.lo;
    rhi = kr.hi;
  }

  // Q and dO fragments (B operands), D = rowsum(dO * O), LSE in log2 units.
  bf16x8 qf[C::KS], dof[C::KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 vq = {0, 0, 0, 0}, vd = {0, 0, 0, 0}, vo = {0, 0, 0, 0};
    if (row_ok) {
      const int64_t col = (int64_t)h * D + ks * 16 + hi32 * 8;
      vq = *reinterpret_cast<const u32x4 *>(a.q + row * a.q_stride + col);
      vd = *reinterpret_cast<const u32x4 *>(a.dout + row * a.do_stride + col);
      vo = *reinterpret_cast<const u32x4 *>(a.o + row * a.o_stride + col);
    }
    qf[ks] = as_bf16x8(vq);
    dof[ks] = as_bf16x8(vd);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart = fmaf(__uint_as_float(vd[e] << 16), __uint_as_float(vo[e] << 16), dpart);
      dpart = fmaf(__uint_as_float(vd[e] & 0xFFFF0000u), __uint_as_float(vo[e] & 0xFFFF0000u), dpart);
    }
  }
  const float delta = sum_halves(dpart);
  const float lse2 = row_ok ? a.lse[(int64_t)h * a.N + row] * kLog2e : 0.f;
  if (row_ok && hi32 == 0 && split == 0) {
    a.delta[(int64_t)h * a.Np + row] = -delta;  // the dK/dV kernel starts its dP accumulators at -D
    a.lse2[(int64_t)h * a.Np + row] = lse2;
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  f32x16 negd;  // starting value of the dP^T accumulators
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -delta;

  // Key tiles of the block, and this workgroup's share of them [kt0, kt1).
  const int kta = (int)(kv_lo / C::BN);
  const int ktb = (int)((kv_hi + C::BN - 1) / C::BN);
  const int kt0 = kSplit ? kta + (int)((int64_t)(ktb - kta) * split / a.qsplit) : kta;
  const int kt1 = kSplit ? kta + (int)((int64_t)(ktb - kta) * (split + 1) / a.qsplit) : ktb;
  // Buffer views: K and V rows of KV head g (rows >= N read as zeros; their
  // scores are masked) and K^T of head g.
  const uint32_t ksb = (uint32_t)(a.k_stride * 2), vsb = (uint32_t)(a.v_stride * 2);
  const bf16_t *kbase = a.k + (int64_t)g * D, *vbase = a.v + (int64_t)g * D;
  const uint32_t kbytes = head_rows_bytes(a.N, a.k_stride, D), vbytes = head_rows_bytes(a.N, a.v_stride, D);
  const BufRes trs = make_rsrc(a.kt + (int64_t)g * D * a.Np, (uint32_t)(D * a.Np * 2));
  // Row-tile layout of the K and V tiles (rt2 with kTr: K is also read transposed).
  auto roff = [](int r, int c) __attribute__((always_inline)) {
    if constexpr (kTr) return rt2_off(r, c);
    else return rt_off<D>(r, c);
  };
  auto rswz = [](int r) __attribute__((always_inline)) {
    if constexpr (kTr) return rt2_swz(r);
    else return row_swz<D>(r);
  };
  uint32_t koff[C::NI / C::NW], voff[C::NI / C::NW], toff[C::NI / C::NW];
#pragma unroll
  for (int i = 0; i < C::NI / C::NW; ++i) {
    const int s = (w + i * C::NW) * 64 + lane;
    const int r = s / (D / 8);
    const uint32_t cb = ((s % (D / 8)) ^ rswz(r)) << 4;
    koff[i] = r * ksb + cb;
    voff[i] = r * vsb + cb;
    const int d = s >> 3;
    toff[i] = (uint32_t)(d * a.Np * 2) + (((s & 7) ^ ((d >> 1) & 7)) << 4);
  }
  [[maybe_unused]] const TrOffsets tro = kTr ? tr_offsets(lane) : TrOffsets{};

  // K and V rows from tile row t0 on (resources from row t0 to the end of
  // row N-1).
  auto issue = [&](int kt, bf16_t *ks_, bf16_t *vs_, bf16_t *ts_) {
    const uint32_t t0 = (uint32_t)kt * C::BN;
    const BufRes krs = make_rsrc(kbase + (int64_t)t0 * a.k_stride, kbytes - t0 * ksb);
    const BufRes vrs = make_rsrc(vbase + (int64_t)t0 * a.v_stride, vbytes - t0 * vsb);
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i) {
      const int u = w + i * C::NW;
      dma16(krs, koff[i], 0, ks_ + u * 512);
      dma16(vrs, voff[i], 0, vs_ + u * 512);
      if constexpr (!kTr) dma16(trs, toff[i], t0 * 2, ts_ + u * 512);
    }
  };

  // One 64-key tile, as two 32-key halves in turn (keeps one half's S^T and
  // dP^T in registers at a time).
  auto compute = [&](int kt, const bf16_t *ks_, const bf16_t *vs_, const bf16_t *ts_) {
    const int64_t t0 = (int64_t)kt * C::BN;
    if (!(wave_valid && t0 < w_hi && t0 + C::BN > w_lo)) return;
    const bool need_mask = (t0 < w_lo_max) || (t0 + C::BN > w_hi_min);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // dP^T accumulates onto -D of the lane's row, leaving dP^T - D.
      f32x16 s, dp = negd;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int off = roff(kb * 32 + l32, ks * 2 + hi32);
        const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4 *>(ks_ + off));
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(vs_ + off));
        s = mfma32(ak, qf[ks], s);
        dp = mfma32(av, dof[ks], dp);
      }
      // Reads issued ahead of their MFMAs (with all 256 registers in use the
      // compiler otherwise waits for every read right after issuing it;
      // asking for more than 2 reads ahead makes it give up entirely).
      pipeline_reads_mfma<2 * C::KS, 2>();
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = t0 + kb * 32 + (i >> 2) * 8 + hi32 * 4 + (i & 3);
          if (key < rlo || key >= rhi) s[i] = -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.c, -lse2));
        s[i] = p * dp[i];  // dS^T
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = kb * 2 + jj;
        const int b = jj * 8;
        const bf16x8 dsf = cvt8(s[b + 0], s[b + 1], s[b + 2], s[b + 3], s[b + 4], s[b + 5], s[b + 6], s[b + 7]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          bf16x8 ak;
          if constexpr (kTr) ak = tr_frag(lds_addr(ks_), tro, db, j);
          else ak = as_bf16x8(*reinterpret_cast<const u32x4 *>(ts_ + tr_off(db * 32 + l32, 2 * j + hi32)));
          acc[db] = mfma32(ak, dsf, acc[db]);
        }
      }
      if constexpr (kTr) pipeline_reads_mfma_n<2 * C::DB, 2, 2>();
    }
  };

  auto step = [&](int t, const bf16_t *ks_, const bf16_t *vs_, const bf16_t *ts_, bf16_t *kn,
                  bf16_t *vn, bf16_t *tn) {
    if (t + 1 < kt1) wait_vmcnt<C::NLW>();
    else wait_vmcnt<0>();
    barrier();
    if (t + 2 < kt1) issue(t + 2, kn, vn, tn);
    compute(t, ks_, vs_, ts_);
  };

  wait_vmcnt<0>();  // Q, dO fragments loaded: only tile copies are counted below
  if (kt0 < kt1) issue(kt0, k0, v0, t0_);
  if (kt0 + 1 < kt1) issue(kt0 + 1, k1, v1, t1_);
  for (int kt = kt0; kt < kt1; kt += 3) {
    step(kt, k0, v0, t0_, k2, v2, t2_);
    if (kt + 1 < kt1) step(kt + 1, k1, v1, t1_, k0, v0, t0_);
    if (kt + 2 < kt1) step(kt + 2, k2, v2, t2_, k1, v1, t1_);
  }

  if (row_ok) {
    if constexpr (!kSplit) {
      bf16_t *out = a.dq + row * a.dq_stride + (int64_t)h * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + gq * 8 + hi32 * 4;
          u32x2 pk;
          pk[0] = pack_bf16x2(acc[db][gq * 4 + 0] * a.scale, acc[db][gq * 4 + 1] * a.scale);
          pk[1] = pack_bf16x2(acc[db][gq * 4 + 2] * a.scale, acc[db][gq * 4 + 3] * a.scale);
          *reinterpret_cast<u32x2 *>(out + d0) = pk;
        }
    } else {
      float *out = a.dq_part + (((int64_t)split * a.N + row) * a.hq + h) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + gq * 8 + hi32 * 4;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[db][gq * 4 + e] * a.scale;
          *reinterpret_cast<f32x4 *>(out + d0) = v;
        }
    }
  }
}

// Sum of the dq kernel's float32 partials over its key-range split, in split
// order (deterministic), rounded to bf16 into dq: one thread per 8 values.
struct DqSumArgs {
  const float *part;  // [ks][N][hq][d]
  bf16_t *dq;
  int64_t N, dq_stride;
  int hq, d, ks;
  uint32_t total;     // N * hq * d / 8
};

__global__ void __launch_bounds__(256) dq_part_sum_kernel(DqSumArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t cpr = (uint32_t)a.d / 8;  // chunks of 8 per (row, head)
  const uint32_t rh = i / cpr, c = i - rh * cpr;
  const int64_t row = rh / a.hq;
  const int h = (int)(rh - row * a.hq);
  const size_t split_stride = (size_t)a.N * a.hq * a.d;
  const float *p = a.part + (size_t)rh * a.d + c * 8;
  f32x4 s0 = *reinterpret_cast<const f32x4 *>(p), s1 = *reinterpret_cast<const f32x4 *>(p + 4);
  for (int s = 1; s < a.ks; ++s) {
    s0 += *reinterpret_cast<const f32x4 *>(p + s * split_stride);
    s1 += *reinterpret_cast<const f32x4 *>(p + s * split_stride + 4);
  }
  u32x4 o;
  o[0] = pack_bf16x2(s0[0], s0[1]);
  o[1] = pack_bf16x2(s0[2], s0[3]);
  o[2] = pack_bf16x2(s1[0], s1[1]);
  o[3] = pack_bf16x2(s1[2], s1[3]);
  *reinterpret_cast<u32x4 *>(a.dq + row * a.dq_stride + (int64_t)h * a.d + c * 8) = o;
}

// ---------------------------------------------------------- dkdv kernel ----

template <int D>
struct DkvCfg {
  static constexpr int NKB = 4;         // 32-key blocks per workgroup
  static constexpr int NW = 2 * NKB;    // two waves per key block
  static constexpr int NT = NW * 64;
  static constexpr int BNK = 32 * NKB;  // keys per workgroup
  static constexpr int BQ = 64;         // queries per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BQ * D;
  static constexpr int NI = TILE / 512;  // 1 KiB copies per tile and tensor
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
};

// Waves w and w + NKB share key block w % NKB and split the work of a tile:
//   wave w       (S role):  S = Q K^T, P = exp(S - LSE), dV^T += dO^T P
//   wave w + NKB (dP role): dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS
// The S-role wave hands P (bf16, in MFMA operand order) to its partner
// through LDS; dS is formed from that same rounded P, which is the P the
// dV product uses. Each wave then holds one of K or V and one of the dK or
// dV accumulators, so a wave fits in 256 registers and two waves share each
// SIMD: one's MFMAs run while the other computes exponentials or dS.
//
// kTr (d = 128): the dO^T and Q^T operands of the dV and dK products are
// read from the Q and dO row tiles with transposing LDS reads (rt2 layout)
// instead of being copied in from the transposed copies, which halves the
// bytes copied into LDS per tile (Q and dO rows only). Q rows then need a
// 3-stage ring, since the deferred dK update reads tile t-1's while tile
// t+1's arrive; dO rows and LSE/D get three stages too, so that the tile
// loop unrolls over the stages. Without kTr all four operands are copied
// (2-stage rings).
template <int D, bool kSplit, bool kTr>
__global__ void __launch_bounds__(DkvCfg<D>::NT, 1) attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvCfg<D>;
  static_assert(!kTr || D == 128, "the transposing-read layout is for d = 128");
  // With kTr the copies of tile t + 1 are issued at tile t and every ring
  // has three stages: Q rows stay one tile longer than dO rows (deferred dK
  // update), and with equal rings the tile loop unrolls over the stages.
  constexpr int PF = 1;
  constexpr int QST = kTr ? 3 : 2;  // stages of the Q row ring
  constexpr int DST = kTr ? 3 : 2;  // stages of the dO row and LSE/D rings
  constexpr int TT = kTr ? 8 : C::TILE;       // trans tiles (unused with kTr)
  __shared__ __align__(16) bf16_t qrow[QST][C::TILE];   // Q row tiles
  __shared__ __align__(16) bf16_t drow[DST][C::TILE];   // dO row tiles
  __shared__ __align__(16) bf16_t qtt[2][TT];           // Q^T trans tiles
  __shared__ __align__(16) bf16_t dtt[2][TT];           // dO^T trans tiles
  __shared__ __align__(16) float lsb[DST][2 * C::BQ];   // LSE*log2e, D
  __shared__ __align__(16) bf16_t xp[C::NKB * 4 * 512];  // P hand-over

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;
  const int kbw = w % C::NKB;        // this wave's 32-key block
  const bool srole = w < C::NKB;     // S role (else dP role)

  // Heaviest key blocks (earliest keys under the causal mask) first;
  // consecutive ids alternate KV heads.
  // With a split the pieces of one key block are consecutive ids.
  const int item = blockIdx.x;
  const int g = item % a.hkv;
  const int kbi = kSplit ? item / a.hkv / a.ksplit : item / a.hkv;
  const int split = kSplit ? item / a.hkv % a.ksplit : 0;
  const int kb = a.korder ? a.korder[kbi] : kbi;
  const int64_t k0 = (int64_t)kb * C::BNK;
  const int64_t k_last = (k0 + C::BNK < a.N ? k0 + C::BNK : a.N) - 1;
  const int64_t kw0 = k0 + (int64_t)kbw * 32;
  const bool wave_valid = kw0 < a.N;
  const int64_t kw_last = (kw0 + 32 < a.N ? kw0 + 32 : a.N) - 1;

  const int b0 = doc_start(a.cu, a.n_seqs, k0);  // documents found from the block's first key on
  const int64_t qr_lo = query_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, k0).lo;
  const int64_t qr_hi = query_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, k_last).hi;
  const KeyRange wq0 = query_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? kw0 : k0);
  const KeyRange wq1 = query_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? kw_last : k0);
  const int64_t w_lo = wq0.lo, w_hi = wq1.hi;
  const int64_t w_lo_max = wq1.lo, w_hi_min = wq0.hi;

  const int64_t key = kw0 + l32;
  const bool key_ok = key < a.N;
  int64_t qlo = 0, qhi = 0;
  if (key_ok) {
    const KeyRange qr = query_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, key);
    qlo = qr.lo;
    qhi = qr.hi;
  }

  // K (S role) or V (dP role) row of this lane's key as B operand (B[k = d][n = key]).
  const bf16_t *kv = srole ? a.k : a.v;
  const int64_t kv_stride = srole ? a.k_stride : a.v_stride;
  bf16x8 xf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 x = {0, 0, 0, 0};
    if (key_ok) x = *reinterpret_cast<const u32x4 *>(kv + key * kv_stride + (int64_t)g * D + ks * 16 + hi32 * 8);
    xf[ks] = as_bf16x8(x);
  }

  f32x16 acc[C::DB];  // dV^T (S role) or dK^T (dP role), [d][key]
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int qt0_ = (int)(qr_lo / C::BQ);
  const int qt1_ = (int)((qr_hi + C::BQ - 1) / C::BQ);
  const int ntq = qt1_ - qt0_;
  const int ntiles = ntq * a.G;  // (head of the group, query tile) pairs
  // This workgroup's share of them: tiles [tb, te).
  const int tb = kSplit ? (int)((int64_t)ntiles * split / a.ksplit) : 0;
  const int te = kSplit ? (int)((int64_t)ntiles * (split + 1) / a.ksplit) : ntiles;

  // Row-tile element offset of logical chunk c of row r, in the layout the
  // Q and dO row tiles use.
  auto roff = [](int r, int c) __attribute__((always_inline)) {
    if constexpr (kTr) return rt2_off(r, c);
    else return rt_off<D>(r, c);
  };
  auto rswz = [](int r) __attribute__((always_inline)) {
    if constexpr (kTr) return rt2_swz(r);
    else return row_swz<D>(r);
  };

  // Per-lane byte offsets of this wave's 16-byte slots inside a tile: row
  // tiles of Q and dO (token stride), trans tiles of Q^T and dO^T.
  const uint32_t qsb = (uint32_t)(a.q_stride * 2), dsb = (uint32_t)(a.do_stride * 2);
  uint32_t qoff[C::NI / C::NW], doff[C::NI / C::NW], toff[C::NI / C::NW];
#pragma unroll
  for (int i = 0; i < C::NI / C::NW; ++i) {
    const int s = (w + i * C::NW) * 64 + lane;
    const int r = s / (D / 8);
    const uint32_t cb = ((s % (D / 8)) ^ rswz(r)) << 4;
    qoff[i] = r * qsb + cb;
    doff[i] = r * dsb + cb;
    const int d = s >> 3;
    toff[i] = (uint32_t)(d * a.Np * 2) + (((s & 7) ^ ((d >> 1) & 7)) << 4);
  }
  [[maybe_unused]] const TrOffsets tro = kTr ? tr_offsets(lane) : TrOffsets{};
  // Byte offsets of this lane's 16-byte operand slots in a row tile, one per
  // 16-wide d step (the second 32-row half adds 32 rows).
  uint32_t rlo[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) rlo[ks] = (uint32_t)roff(l32, ks * 2 + hi32) * 2;

  // Tile t: query tiles from the last one down (every workgroup of a wave of
  // launches starts on the same tiles and walks them in step, so they are
  // shared through L2), the group's heads innermost. A cursor holds tile t's
  // head within the group and query tile (counted from the last one); the
  // next tile's comes from a compare and two selects (dividing t by G, known
  // only at run time, costs about 15 scalar instructions per tile).
  struct TileCur {
    int hh, qi;
  };
  auto cur_at = [&](int t) { return TileCur{t % a.G, t / a.G}; };
  auto next_cur = [&](TileCur c) {
    const bool wrap = c.hh + 1 == a.G;
    return TileCur{wrap ? 0 : c.hh + 1, wrap ? c.qi + 1 : c.qi};
  };
  auto tile_head = [&](TileCur c) { return g * a.G + c.hh; };
  auto tile_u0 = [&](TileCur c) { return (uint32_t)(qt1_ - 1 - c.qi) * C::BQ; };

  // Copies of tile t: Q and dO row tiles, the dO^T trans tile (without kTr)
  // and the tile's LSE*log2e and D (issue_rows); the Q^T trans tile
  // (issue_qt, without kTr), which is needed one tile later than the others
  // (see the schedule below).
  auto issue_rows = [&](TileCur t, bf16_t *qs, bf16_t *ds, bf16_t *dts, float *ls) {
    const int h = tile_head(t);
    const uint32_t u0 = tile_u0(t);
    // Q and dO rows of head h from row u0 to the end of row N-1 (rows >= N
    // read as zeros; they are masked).
    const BufRes qrs = make_rsrc(a.q + (int64_t)u0 * a.q_stride + (int64_t)h * D,
                                 head_rows_bytes(a.N, a.q_stride, D) - u0 * qsb);
    const BufRes drs = make_rsrc(a.dout + (int64_t)u0 * a.do_stride + (int64_t)h * D,
                                 head_rows_bytes(a.N, a.do_stride, D) - u0 * dsb);
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i) {
      const int u = w + i * C::NW;
      dma16(qrs, qoff[i], 0, qs + u * 512);
      dma16(drs, doff[i], 0, ds + u * 512);
    }
    if constexpr (!kTr) {
      const BufRes dtr = make_rsrc(a.dot + (int64_t)h * D * a.Np, (uint32_t)(D * a.Np * 2));
#pragma unroll
      for (int i = 0; i < C::NI / C::NW; ++i) {
        const int u = w + i * C::NW;
        dma16(dtr, toff[i], u0 * 2, dts + u * 512);
      }
    }
    if (w < 2) {  // wave 0: LSE*log2e of the 64 rows, wave 1: D; rows >= N read as zeros
      const float *src = (w == 0 ? a.lse2 : a.delta) + (int64_t)h * a.Np;
      dma4(make_rsrc(src + u0, (uint32_t)((a.N - u0) * 4)), lane * 4, 0, ls + w * C::BQ);
    }
  };
  auto issue_qt = [&](TileCur t, bf16_t *qts) {
    const int h = tile_head(t);
    const uint32_t u0 = tile_u0(t);
    const BufRes qtr = make_rsrc(a.qt + (int64_t)h * D * a.Np, (uint32_t)(D * a.Np * 2));
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i) dma16(qtr, toff[i], u0 * 2, qts + (w + i * C::NW) * 512);
  };
  auto active = [&](TileCur t) {
    const int64_t u0 = tile_u0(t);
    return wave_valid && u0 < w_hi && u0 + C::BQ > w_lo;
  };

  // Schedule of tile t (stage t % 3 of every ring with kTr, t % 2 without;
  // B = ring barrier, X = P hand-over barrier):
  //   wait for tile t's copies (without kTr: all but Q^T(t)), B, issue_rows(t + 1)
  //   phase 1  S role:  S(t), P(t), P -> LDS
  //            dP role: dK += Q^T(t-1) dS(t-1), dP(t)
  //   X, without kTr: issue_qt(t + 1) (its stage held Q^T(t-1), last read in phase 1)
  //   phase 2  S role:  dV += dO^T(t) P(t)
  //            dP role: P(t) <- LDS, dS(t) (kept in registers for tile t+1)
  // Each phase pairs one wave's exponentials or dS arithmetic with its
  // partner's MFMAs on the same SIMD.
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool S = decltype(role)::value;
    bf16_t *xw = xp + kbw * 4 * 512 + lane * 8;  // this lane's 4 fragments, 1 KiB apart
    bf16x8 sf[4];                                 // dP role: dS of the previous tile
    bool pend = false;                            // dP role: sf holds a tile not yet applied

    // dK^T += Q^T(t-1) dS(t-1): Q^T from its trans tile, or (kTr) read
    // transposed from tile t-1's Q rows.
    // Query steps [C0, C1) of the update.
    auto dk_update = [&](const bf16_t *qts, auto c0, auto c1) __attribute__((always_inline)) {
      constexpr int C0 = decltype(c0)::value, C1 = decltype(c1)::value;
      [[maybe_unused]] const uint32_t qa = lds_addr(qts);
#pragma unroll
      for (int c = C0; c < C1; ++c)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          bf16x8 aqt;
          if constexpr (kTr) aqt = tr_frag(qa, tro, db, c);
          else aqt = as_bf16x8(*reinterpret_cast<const u32x4 *>(qts + tr_off(db * 32 + l32, c * 2 + hi32)));
          acc[db] = mfma32(aqt, sf[c], acc[db]);
        }
      if constexpr (kTr) pipeline_reads_mfma_n<(C1 - C0) * C::DB, 2, ULY_TR_LA>();
      else pipeline_reads_mfma<(C1 - C0) * C::DB>();
    };
    using IC0 = std::integral_constant<int, 0>;
    using ICP1 = std::integral_constant<int, kTr ? ULY_DK_P1 : 4>;
    using IC4 = std::integral_constant<int, 4>;

    // qs_prev: Q^T(t-1) trans tile, or (kTr) tile t-1's Q rows.
    // qs_n, ds_n, ls_n: stages for tile t + PF's copies.
    // tc, tn: cursors of tiles t and t + 1.
    auto tile = [&](int t, TileCur tc, TileCur tn, const bf16_t *qs, const bf16_t *ds, const bf16_t *dts, const float *ls,
                    const bf16_t *qs_prev, bf16_t *qs_n, bf16_t *ds_n, bf16_t *dts_n, float *ls_n,
                    bf16_t *qts_n) __attribute__((always_inline)) {
      if constexpr (kTr) {
        // tile t's copies done; those of tiles t+1 .. t+PF-1 may be in flight
        constexpr int per = 2 * (C::NI / C::NW);
        if (t + PF - 1 < te) {
          if (w < 2) wait_vmcnt<(PF - 1) * (per + 1)>();
          else wait_vmcnt<(PF - 1) * per>();
        } else {
          wait_vmcnt<0>();
        }
      } else {
        wait_vmcnt<C::NI / C::NW>();
      }
      barrier();
      if (t + PF < te) issue_rows(tn, qs_n, ds_n, dts_n, ls_n);
      const int64_t u0 = tile_u0(tc);
      const bool act = active(tc);
      f32x16 x[2];
      bf16x8 pf[4];
      if constexpr (!S) {
        // The dP accumulators start at -D of their query rows (the workspace
        // holds -D), so the product leaves dP - D; read before the deferred
        // dK update so that the reads complete under it.
        if (act) {
          const uint32_t la = lds_addr(ls) + (C::BQ + hi32 * 4) * 4;
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x4 d4 = lds_read16f(la + (q * 32 + gq * 8) * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) x[q][gq * 4 + e] = d4[e];
            }
        }
        if (pend) dk_update(qs_prev, IC0{}, ICP1{});
      }
      if (act) {
        if constexpr (S) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 16; ++i) x[q][i] = 0.f;
        }
        const uint32_t rb = lds_addr(S ? qs : ds);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const bf16x8 ar = as_bf16x8(lds_read16(rb + rlo[ks] + q * 32 * D * 2));
            x[q] = mfma32(ar, xf[ks], x[q]);
          }
        pipeline_reads_mfma<2 * C::KS>();
        if constexpr (S) {
          if ((u0 < w_lo_max) || (u0 + C::BQ > w_hi_min)) {
            const RelRange rr = rel_range(qlo, qhi, u0, hi32 * 4);
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int e = q * 32 + (i >> 2) * 8 + (i & 3);
                if (e < rr.lo || e >= rr.hi) x[q][i] = -INFINITY;
              }
          }
          const uint32_t la = lds_addr(ls) + hi32 * 16;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x4 l4 = lds_read16f(la + (q * 32 + gq * 8) * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                x[q][gq * 4 + e] = __builtin_amdgcn_exp2f(fmaf(x[q][gq * 4 + e], a.c, -l4[e]));
            }
#pragma unroll
            for (int jq = 0; jq < 2; ++jq) {
              const int b = jq * 8;
              pf[q * 2 + jq] = cvt8(x[q][b + 0], x[q][b + 1], x[q][b + 2], x[q][b + 3], x[q][b + 4],
                                    x[q][b + 5], x[q][b + 6], x[q][b + 7]);
              *reinterpret_cast<bf16x8 *>(xw + (q * 2 + jq) * 512) = pf[q * 2 + jq];
            }
          }
        }
      }
      lds_barrier();
      if constexpr (!kTr) {
        if (t + 1 < te) issue_qt(tn, qts_n);
      }
      if constexpr (S) {
        if (act) {
          [[maybe_unused]] const uint32_t da = lds_addr(ds);
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              bf16x8 adt;
              if constexpr (kTr) adt = tr_frag(da, tro, db, c);
              else adt = as_bf16x8(*reinterpret_cast<const u32x4 *>(dts + tr_off(db * 32 + l32, c * 2 + hi32)));
              acc[db] = mfma32(adt, pf[c], acc[db]);
            }
          if constexpr (kTr) pipeline_reads_mfma_n<4 * C::DB, 2, ULY_TR_LA>();
          else pipeline_reads_mfma<4 * C::DB>();
        }
      } else {
        if constexpr (ICP1::value < 4) {
          if (pend) dk_update(qs_prev, ICP1{}, IC4{});
        }
        pend = act;
        if (act) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int jq = 0; jq < 2; ++jq) {
              const u32x4 pw = *reinterpret_cast<const u32x4 *>(xw + (q * 2 + jq) * 512);
              float dsv[8];
#pragma unroll
              for (int gq2 = 0; gq2 < 2; ++gq2) {
                const int gq = jq * 2 + gq2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int k = gq2 * 4 + e;  // fragment element
                  const uint32_t wd = pw[k >> 1];
                  const float p = __uint_as_float((k & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                  dsv[k] = p * x[q][gq * 4 + e];  // x holds dP - D
                }
              }
              sf[q * 2 + jq] = cvt8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
            }
        }
      }
    };

    wait_vmcnt<0>();  // K or V fragments loaded: only tile copies are counted below
    if constexpr (kTr) {
      // Unrolled over the three stages, so that every LDS address in a tile
      // is a constant plus a lane offset (the constant goes into the read's
      // offset field; a stage picked at run time costs one VALU add per read).
      static_assert(PF == 1 && QST == 3 && DST == 3, "the unrolled loop assumes 3-stage rings");
      TileCur c0 = cur_at(tb);
      if (tb < te) issue_rows(c0, qrow[0], drow[0], nullptr, lsb[0]);
      for (int t = tb; t < te; t += 3) {
        const TileCur c1 = next_cur(c0), c2 = next_cur(c1), c3 = next_cur(c2);
        tile(t, c0, c1, qrow[0], drow[0], nullptr, lsb[0], qrow[2], qrow[1], drow[1], nullptr, lsb[1], nullptr);
        if (t + 1 < te)
          tile(t + 1, c1, c2, qrow[1], drow[1], nullptr, lsb[1], qrow[0], qrow[2], drow[2], nullptr, lsb[2], nullptr);
        if (t + 2 < te)
          tile(t + 2, c2, c3, qrow[2], drow[2], nullptr, lsb[2], qrow[1], qrow[0], drow[0], nullptr, lsb[0], nullptr);
        c0 = c3;
      }
      // The last tile's dK update (its Q rows stay in place: nothing more is copied).
      if constexpr (!S) {
        if (pend) dk_update(qrow[(te - 1 - tb) % QST], IC0{}, IC4{});
      }
    } else {
      TileCur c0 = cur_at(tb);
      if (tb < te) {
        issue_rows(c0, qrow[0], drow[0], dtt[0], lsb[0]);
        issue_qt(c0, qtt[0]);
      }
      for (int t = tb; t < te; t += 2) {
        const TileCur c1 = next_cur(c0), c2 = next_cur(c1);
        tile(t, c0, c1, qrow[0], drow[0], dtt[0], lsb[0], qtt[1], qrow[1], drow[1], dtt[1], lsb[1], qtt[1]);
        if (t + 1 < te)
          tile(t + 1, c1, c2, qrow[1], drow[1], dtt[1], lsb[1], qtt[0], qrow[0], drow[0], dtt[0], lsb[0], qtt[0]);
        c0 = c2;
      }
      // The last tile's dK update: its Q^T copy is complete once every wave
      // has waited for its own part of it.
      wait_vmcnt<0>();
      barrier();
      if constexpr (!S) {
        if (pend) dk_update((te - 1 - tb) % 2 == 0 ? qtt[0] : qtt[1], IC0{}, IC4{});
      }
    }
  };
  if (srole)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (key_ok) {
    const float f = srole ? 1.f : a.scale;
    if constexpr (!kSplit) {
      bf16_t *out = srole ? a.dv + key * a.dv_stride + (int64_t)g * D : a.dk + key * a.dk_stride + (int64_t)g * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + gq * 8 + hi32 * 4;
          u32x2 pk;
          pk[0] = pack_bf16x2(acc[db][gq * 4 + 0] * f, acc[db][gq * 4 + 1] * f);
          pk[1] = pack_bf16x2(acc[db][gq * 4 + 2] * f, acc[db][gq * 4 + 3] * f);
          *reinterpret_cast<u32x2 *>(out + d0) = pk;
        }
    } else {
      float *out = a.dkv_part + (((int64_t)split * a.N + key) * a.hkv + g) * 2 * D + (srole ? D : 0);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + gq * 8 + hi32 * 4;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[db][gq * 4 + e] * f;
          *reinterpret_cast<f32x4 *>(out + d0) = v;
        }
    }
  }
}

// Sum of the dK/dV kernel's float32 partials over its query-range split, in
// split order (deterministic), rounded to bf16 into dk and dv: one thread per
// 8 values.
struct PartSumArgs {
  const float *part;  // [ks][N][hkv][2][d]
  bf16_t *dk, *dv;
  int64_t N, dk_stride, dv_stride;
  int hkv, d, ks;
  uint32_t total;     // N * hkv * 2 * d / 8
};

__global__ void __launch_bounds__(256) dkdv_part_sum_kernel(PartSumArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t cpr = (uint32_t)a.d / 8;       // chunks of 8 per (key, head, which) row
  const uint32_t row = i / cpr, c = i - row * cpr;
  const int which = (int)(row % 2);             // 0: dK, 1: dV
  const int64_t kg = row / 2;                   // key * hkv + g
  const int64_t key = kg / a.hkv;
  const int g = (int)(kg - key * a.hkv);
  const size_t split_stride = (size_t)a.N * a.hkv * 2 * a.d;
  const float *p = a.part + (size_t)row * a.d + c * 8;
  f32x4 s0 = *reinterpret_cast<const f32x4 *>(p), s1 = *reinterpret_cast<const f32x4 *>(p + 4);
  for (int s = 1; s < a.ks; ++s) {
    const f32x4 t0 = *reinterpret_cast<const f32x4 *>(p + s * split_stride);
    const f32x4 t1 = *reinterpret_cast<const f32x4 *>(p + s * split_stride + 4);
    s0 += t0;
    s1 += t1;
  }
  u32x4 o;
  o[0] = pack_bf16x2(s0[0], s0[1]);
  o[1] = pack_bf16x2(s0[2], s0[3]);
  o[2] = pack_bf16x2(s1[0], s1[1]);
  o[3] = pack_bf16x2(s1[2], s1[3]);
  bf16_t *dst = which ? a.dv + key * a.dv_stride : a.dk + key * a.dk_stride;
  *reinterpret_cast<u32x4 *>(dst + (int64_t)g * a.d + c * 8) = o;
}

template <int D, int HPW, int RB>
int launch_dq_cfg(BwdArgs a, hipStream_t stream) {
  using C = DqCfg<D, HPW, RB>;
  a.nblk = (int)((a.N + C::BM - 1) / C::BM);
  a.nhg = a.hq / HPW;
  a.qsplit = dq_ksplit(a.N, a.hq, a.hkv);
  if (a.qsplit > 1)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, RB, true>),
                       dim3((unsigned)((int64_t)a.nblk * a.nhg * a.qsplit)), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, RB, false>), dim3((unsigned)((int64_t)a.nblk * a.nhg)),
                       dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dq_kernel");
  if (a.qsplit > 1) {
    DqSumArgs ps;
    ps.part = a.dq_part;
    ps.dq = a.dq;
    ps.N = a.N;
    ps.dq_stride = a.dq_stride;
    ps.hq = a.hq;
    ps.d = D;
    ps.ks = a.qsplit;
    ps.total = (uint32_t)(a.N * a.hq * D / 8);
    hipLaunchKernelGGL(dq_part_sum_kernel, dim3((ps.total + 255) / 256), dim3(256), 0, stream, ps);
    e = hipGetLastError();
    if (e != hipSuccess) return set_hip_error(e, "dq_part_sum_kernel");
  }
  return 0;
}

template <int D>
int launch_dkdv_cfg(BwdArgs a, hipStream_t stream) {
  using C = DkvCfg<D>;
  a.nblk = (int)((a.N + C::BNK - 1) / C::BNK);
  a.ksplit = dkdv_ksplit(a.N, a.hkv);
  constexpr bool kTr = D == 128;
  const unsigned grid = (unsigned)((int64_t)a.nblk * a.hkv * a.ksplit);
  if (a.ksplit > 1) {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, kTr>), dim3(grid), dim3(C::NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, kTr>), dim3(grid), dim3(C::NT), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dkdv_kernel");
  if (a.ksplit > 1) {
    PartSumArgs ps;
    ps.part = a.dkv_part;
    ps.dk = a.dk;
    ps.dv = a.dv;
    ps.N = a.N;
    ps.dk_stride = a.dk_stride;
    ps.dv_stride = a.dv_stride;
    ps.hkv = a.hkv;
    ps.d = D;
    ps.ks = a.ksplit;
    ps.total = (uint32_t)(a.N * a.hkv * 2 * D / 8);
    hipLaunchKernelGGL(dkdv_part_sum_kernel, dim3((ps.total + 255) / 256), dim3(256), 0, stream, ps);
    e = hipGetLastError();
    if (e != hipSuccess) return set_hip_error(e, "dkdv_part_sum_kernel");
  }
  return 0;
}

}  // namespace

int launch_attn_bwd(const AttnShape &s, const AttnBwdPtrs &p, int parts, hipStream_t stream) {
  const BwdWs L = bwd_ws_layout(s.N, s.hq, s.hkv, s.d);
  BwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.dout = p.dout;
  a.lse = p.lse;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.delta = reinterpret_cast<float *>(p.ws + L.delta);
  a.lse2 = reinterpret_cast<float *>(p.ws + L.lse2);
  a.kt = reinterpret_cast<const bf16_t *>(p.ws + L.kt);
  a.qt = reinterpret_cast<const bf16_t *>(p.ws + L.qt);
  a.dot = reinterpret_cast<const bf16_t *>(p.ws + L.dot);
  a.N = s.N;
  a.Np = pad64(s.N);
  a.q_stride = s.q_stride;
  a.k_stride = s.k_stride;
  a.v_stride = s.v_stride;
  a.o_stride = s.o_stride;
  a.do_stride = p.do_stride;
  a.dq_stride = p.dq_stride;
  a.dk_stride = p.dk_stride;
  a.dv_stride = p.dv_stride;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.G = s.hq / s.hkv;
  a.nblk = a.nhg = 0;
  a.c = s.scale * kLog2e;
  a.scale = s.scale;
  a.causal = s.causal;
  a.cu = s.cu;
  a.n_seqs = s.n_seqs;
  a.korder = s.cu ? reinterpret_cast<const int32_t *>(p.ws + L.korder) : nullptr;
  a.qorder = s.cu ? reinterpret_cast<const int32_t *>(p.ws + L.qorder) : nullptr;
  a.ksplit = 1;
  a.dkv_part = reinterpret_cast<float *>(p.ws + L.part);
  a.qsplit = 1;
  a.dq_part = reinterpret_cast<float *>(p.ws + L.qpart);
  const int hpw = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
  int rc = 0;
  if (parts & 1) {
    // Transposed copies for both kernels: K^T for this one, Q^T and dO^T for
    // the dK/dV kernel (made here so that kernel runs alone).
    bf16_t *ws_kt = reinterpret_cast<bf16_t *>(p.ws + L.kt);
    bf16_t *ws_qt = reinterpret_cast<bf16_t *>(p.ws + L.qt);
    bf16_t *ws_dot = reinterpret_cast<bf16_t *>(p.ws + L.dot);
    if (s.d != 128) {  // at d = 128 both kernels read the row tiles transposed in LDS
      if ((rc = launch_to_trans(p.k, s.k_stride, s.hkv, s.d, s.N, ws_kt, stream))) return rc;
      if ((rc = launch_to_trans(p.q, s.q_stride, s.hq, s.d, s.N, ws_qt, stream))) return rc;
      if ((rc = launch_to_trans(p.dout, p.do_stride, s.hq, s.d, s.N, ws_dot, stream))) return rc;
    }
    // Over packed documents, the block orders of both kernels (the dK/dV
    // kernel, run alone, reads its order from the workspace as left here).
    if (s.cu) {
      const int q_bs = s.d == 128 ? (hpw == 4 ? DqCfg<128, 4, 2>::BM : hpw == 2 ? DqCfg<128, 2, 4>::BM
                                                                              : DqCfg<128, 1, 8>::BM)
                                  : (hpw == 4 ? DqCfg<64, 4, 2>::BM : hpw == 2 ? DqCfg<64, 2, 4>::BM
                                                                             : DqCfg<64, 1, 8>::BM);
      const int k_bs = s.d == 128 ? DkvCfg<128>::BNK : DkvCfg<64>::BNK;
      if ((rc = launch_block_orders(s.cu, s.n_seqs, s.N, s.causal, q_bs, reinterpret_cast<int32_t *>(p.ws + L.qorder),
                                    k_bs, reinterpret_cast<int32_t *>(p.ws + L.korder), stream)))
        return rc;
    }
    if (s.d == 128)
      rc = hpw == 4 ? launch_dq_cfg<128, 4, 2>(a, stream)
           : hpw == 2 ? launch_dq_cfg<128, 2, 4>(a, stream)
                      : launch_dq_cfg<128, 1, 8>(a, stream);
    else
      rc = hpw == 4 ? launch_dq_cfg<64, 4, 2>(a, stream)
           : hpw == 2 ? launch_dq_cfg<64, 2, 4>(a, stream)
                      : launch_dq_cfg<64, 1, 8>(a, stream);
    if (rc) return rc;
  }
  if (parts & 2) rc = s.d == 128 ? launch_dkdv_cfg<128>(a, stream) : launch_dkdv_cfg<64>(a, stream);
  return rc;
}

}  // namespace uly
