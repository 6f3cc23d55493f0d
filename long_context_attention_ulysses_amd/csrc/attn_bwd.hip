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
//      its rows (to the workspace), then per 64-key tile (3-stage ring):
//      S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, dQ^T += K^T dS^T
//      (Q and dO stay in registers as B operands; a lane owns one query).
//   2. dkdv kernel, parallel over (key block, KV head): loops over its
//      64-query tiles from the last one down, the group's heads innermost
//      (2-stage ring; concurrent workgroups walk the same tiles in step):
//      S = Q K^T, dP = dO V^T (K, V in registers; a lane owns one key),
//      P, dS, dV^T += dO^T P, dK^T += Q^T dS.
#include "attn_common.h"
#include "uly_internal.h"

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
};

// ------------------------------------------------------------ dq kernel ----

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
  static constexpr int NLW = 3 * NI / NW;  // copies per wave per tile (K, V, K^T)
};

template <int D, int HPW, int RB>
__global__ void __launch_bounds__(HPW * RB * 64, 1) attn_bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D, HPW, RB>;
  __shared__ __align__(16) bf16_t k0[C::TILE], k1[C::TILE], k2[C::TILE];
  __shared__ __align__(16) bf16_t v0[C::TILE], v1[C::TILE], v2[C::TILE];
  __shared__ __align__(16) bf16_t t0_[C::TILE], t1_[C::TILE], t2_[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;

  const int item = blockIdx.x;
  const int hg = item % a.nhg;
  const int qb = a.nblk - 1 - item / a.nhg;
  const int64_t q0 = (int64_t)qb * C::BM;
  const int h = hg * HPW + w / RB;
  const int g = (hg * HPW) / a.G;
  const int64_t r0 = q0 + (int64_t)(w % RB) * 32;

  const int64_t q_last = (q0 + C::BM < a.N ? q0 + C::BM : a.N) - 1;
  const int64_t kv_lo = key_range(a.cu, a.n_seqs, a.N, a.causal, q0).lo;
  const int64_t kv_hi = key_range(a.cu, a.n_seqs, a.N, a.causal, q_last).hi;
  const bool wave_valid = r0 < a.N;
  const int64_t w_last = (r0 + 32 < a.N ? r0 + 32 : a.N) - 1;
  const KeyRange wr0 = key_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? r0 : 0);
  const KeyRange wr1 = key_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? w_last : 0);
  const int64_t w_lo = wr0.lo, w_hi = wr1.hi;
  const int64_t w_lo_max = wr1.lo, w_hi_min = wr0.hi;

  const int64_t row = r0 + l32;
  const bool row_ok = row < a.N;
  int64_t rlo = 0, rhi = 0;
  if (row_ok) {
    const KeyRange kr = key_range(a.cu, a.n_seqs, a.N, a.causal, row);
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
  const float delta = dpart + xor32(dpart);
  const float lse2 = row_ok ? a.lse[(int64_t)h * a.N + row] * kLog2e : 0.f;
  if (row_ok && hi32 == 0) {
    a.delta[(int64_t)h * a.Np + row] = delta;
    a.lse2[(int64_t)h * a.Np + row] = lse2;
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int kt0 = (int)(kv_lo / C::BN);
  const int kt1 = (int)((kv_hi + C::BN - 1) / C::BN);
  // Buffer views: K and V rows of KV head g (rows >= N read as zeros; their
  // scores are masked) and K^T of head g.
  const uint32_t ksb = (uint32_t)(a.k_stride * 2), vsb = (uint32_t)(a.v_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + (int64_t)g * D, head_rows_bytes(a.N, a.k_stride, D));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + (int64_t)g * D, head_rows_bytes(a.N, a.v_stride, D));
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(a.kt + (int64_t)g * D * a.Np, (uint32_t)(D * a.Np * 2));
  uint32_t koff[C::NI / C::NW], voff[C::NI / C::NW], toff[C::NI / C::NW];
#pragma unroll
  for (int i = 0; i < C::NI / C::NW; ++i) {
    const int s = (w + i * C::NW) * 64 + lane;
    const int r = s / (D / 8);
    const uint32_t cb = ((s % (D / 8)) ^ row_swz<D>(r)) << 4;
    koff[i] = r * ksb + cb;
    voff[i] = r * vsb + cb;
    const int d = s >> 3;
    toff[i] = (uint32_t)(d * a.Np * 2) + (((s & 7) ^ ((d >> 1) & 7)) << 4);
  }

  auto issue = [&](int kt, bf16_t *ks_, bf16_t *vs_, bf16_t *ts_) {
    const uint32_t t0 = (uint32_t)kt * C::BN;
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i) {
      const int u = w + i * C::NW;
      dma16(krs, koff[i] + t0 * ksb, 0, lds_ptr(ks_ + u * 512));
      dma16(vrs, voff[i] + t0 * vsb, 0, lds_ptr(vs_ + u * 512));
      dma16(trs, toff[i], t0 * 2, lds_ptr(ts_ + u * 512));
    }
  };

  auto compute = [&](int kt, const bf16_t *ks_, const bf16_t *vs_, const bf16_t *ts_) {
    const int64_t t0 = (int64_t)kt * C::BN;
    if (!(wave_valid && t0 < w_hi && t0 + C::BN > w_lo)) return;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = 0.f;
        dp[kb][i] = 0.f;
      }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int off = rt_off<D>(kb * 32 + l32, ks * 2 + hi32);
        const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4 *>(ks_ + off));
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(vs_ + off));
        s[kb] = mfma32(ak, qf[ks], s[kb]);
        dp[kb] = mfma32(av, dof[ks], dp[kb]);
      }
    }
    if ((t0 < w_lo_max) || (t0 + C::BN > w_hi_min)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = t0 + kb * 32 + (i >> 2) * 8 + hi32 * 4 + (i & 3);
          if (key < rlo || key >= rhi) s[kb][i] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c, -lse2));
        s[kb][i] = p * (dp[kb][i] - delta);  // dS^T
      }
#pragma unroll
    for (int j = 0; j < C::JS; ++j) {
      const f32x16 &sv = s[j >> 1];
      const int b = (j & 1) * 8;
      const bf16x8 dsf =
          cvt8(sv[b + 0], sv[b + 1], sv[b + 2], sv[b + 3], sv[b + 4], sv[b + 5], sv[b + 6], sv[b + 7]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 ak =
            as_bf16x8(*reinterpret_cast<const u32x4 *>(ts_ + tr_off(db * 32 + l32, 2 * j + hi32)));
        acc[db] = mfma32(ak, dsf, acc[db]);
      }
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

  if (kt0 < kt1) issue(kt0, k0, v0, t0_);
  if (kt0 + 1 < kt1) issue(kt0 + 1, k1, v1, t1_);
  for (int kt = kt0; kt < kt1; kt += 3) {
    step(kt, k0, v0, t0_, k2, v2, t2_);
    if (kt + 1 < kt1) step(kt + 1, k1, v1, t1_, k0, v0, t0_);
    if (kt + 2 < kt1) step(kt + 2, k2, v2, t2_, k1, v1, t1_);
  }

  if (row_ok) {
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
  }
}

// ---------------------------------------------------------- dkdv kernel ----

template <int D, int NWK>
struct DkvCfg {
  static constexpr int NT = NWK * 64;
  static constexpr int BNK = 32 * NWK;  // keys per workgroup
  static constexpr int BQ = 64;         // queries per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BQ * D;
  static constexpr int NI = TILE / 512;  // 1 KiB copies per tile and tensor
  static_assert(NI % NWK == 0, "copies must split evenly over the waves");
};

template <int D, int NWK>
__global__ void __launch_bounds__(NWK * 64, 1) attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvCfg<D, NWK>;
  __shared__ __align__(16) bf16_t q0s[C::TILE], q1s[C::TILE];    // Q row tiles
  __shared__ __align__(16) bf16_t d0s[C::TILE], d1s[C::TILE];    // dO row tiles
  __shared__ __align__(16) bf16_t qt0[C::TILE], qt1[C::TILE];    // Q^T trans tiles
  __shared__ __align__(16) bf16_t dt0[C::TILE], dt1[C::TILE];    // dO^T trans tiles
  __shared__ __align__(16) float ls0[2 * C::BQ], ls1[2 * C::BQ];  // LSE*log2e, D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;

  // Heaviest key blocks (earliest keys under the causal mask) first;
  // consecutive ids alternate KV heads.
  const int item = blockIdx.x;
  const int g = item % a.hkv;
  const int kb = item / a.hkv;
  const int64_t k0 = (int64_t)kb * C::BNK;
  const int64_t k_last = (k0 + C::BNK < a.N ? k0 + C::BNK : a.N) - 1;
  const int64_t kw0 = k0 + (int64_t)w * 32;
  const bool wave_valid = kw0 < a.N;
  const int64_t kw_last = (kw0 + 32 < a.N ? kw0 + 32 : a.N) - 1;

  const int64_t qr_lo = query_range(a.cu, a.n_seqs, a.N, a.causal, k0).lo;
  const int64_t qr_hi = query_range(a.cu, a.n_seqs, a.N, a.causal, k_last).hi;
  const KeyRange wq0 = query_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? kw0 : 0);
  const KeyRange wq1 = query_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? kw_last : 0);
  const int64_t w_lo = wq0.lo, w_hi = wq1.hi;
  const int64_t w_lo_max = wq1.lo, w_hi_min = wq0.hi;

  const int64_t key = kw0 + l32;
  const bool key_ok = key < a.N;
  int64_t qlo = 0, qhi = 0;
  if (key_ok) {
    const KeyRange qr = query_range(a.cu, a.n_seqs, a.N, a.causal, key);
    qlo = qr.lo;
    qhi = qr.hi;
  }

  // K and V rows of this lane's key as B operands (B[k = d][n = key]).
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 vk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (key_ok) {
      const int64_t col = (int64_t)g * D + ks * 16 + hi32 * 8;
      vk = *reinterpret_cast<const u32x4 *>(a.k + key * a.k_stride + col);
      vv = *reinterpret_cast<const u32x4 *>(a.v + key * a.v_stride + col);
    }
    kf[ks] = as_bf16x8(vk);
    vf[ks] = as_bf16x8(vv);
  }

  f32x16 acc_dk[C::DB], acc_dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc_dk[db][i] = 0.f;
      acc_dv[db][i] = 0.f;
    }

  const int qt0_ = (int)(qr_lo / C::BQ);
  const int qt1_ = (int)((qr_hi + C::BQ - 1) / C::BQ);
  const int ntq = qt1_ - qt0_;
  const int ntiles = ntq * a.G;  // (head of the group, query tile) pairs

  // Per-lane byte offsets of this wave's 16-byte slots inside a tile: row
  // tiles of Q and dO (token stride), trans tiles of Q^T and dO^T.
  const uint32_t qsb = (uint32_t)(a.q_stride * 2), dsb = (uint32_t)(a.do_stride * 2);
  uint32_t qoff[C::NI / NWK], doff[C::NI / NWK], toff[C::NI / NWK];
#pragma unroll
  for (int i = 0; i < C::NI / NWK; ++i) {
    const int s = (w + i * NWK) * 64 + lane;
    const int r = s / (D / 8);
    const uint32_t cb = ((s % (D / 8)) ^ row_swz<D>(r)) << 4;
    qoff[i] = r * qsb + cb;
    doff[i] = r * dsb + cb;
    const int d = s >> 3;
    toff[i] = (uint32_t)(d * a.Np * 2) + (((s & 7) ^ ((d >> 1) & 7)) << 4);
  }

  // Tile t: query tiles from the last one down (every workgroup of a wave of
  // launches starts on the same tiles and walks them in step, so they are
  // shared through L2), the group's heads innermost.
  auto tile_head = [&](int t) { return g * a.G + t % a.G; };
  auto tile_u0 = [&](int t) { return (uint32_t)(qt1_ - 1 - t / a.G) * C::BQ; };

  auto issue = [&](int t, bf16_t *qs, bf16_t *ds, bf16_t *qts, bf16_t *dts, float *ls) {
    const int h = tile_head(t);
    const uint32_t u0 = tile_u0(t);
    // Q and dO rows of head h (rows >= N read as zeros; they are masked).
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q + (int64_t)h * D, head_rows_bytes(a.N, a.q_stride, D));
    const __amdgpu_buffer_rsrc_t drs =
        make_rsrc(a.dout + (int64_t)h * D, head_rows_bytes(a.N, a.do_stride, D));
    const __amdgpu_buffer_rsrc_t qtr = make_rsrc(a.qt + (int64_t)h * D * a.Np, (uint32_t)(D * a.Np * 2));
    const __amdgpu_buffer_rsrc_t dtr = make_rsrc(a.dot + (int64_t)h * D * a.Np, (uint32_t)(D * a.Np * 2));
#pragma unroll
    for (int i = 0; i < C::NI / NWK; ++i) {
      const int u = w + i * NWK;
      dma16(qrs, qoff[i] + u0 * qsb, 0, lds_ptr(qs + u * 512));
      dma16(drs, doff[i] + u0 * dsb, 0, lds_ptr(ds + u * 512));
      dma16(qtr, toff[i], u0 * 2, lds_ptr(qts + u * 512));
      dma16(dtr, toff[i], u0 * 2, lds_ptr(dts + u * 512));
    }
    if (w < 2) {  // wave 0: LSE*log2e of the 64 rows, wave 1: D (padded rows, masked)
      const float *src = (w == 0 ? a.lse2 : a.delta) + (int64_t)h * a.Np;
      dma4(make_rsrc(src, (uint32_t)(a.Np * 4)), lane * 4, u0 * 4, lds_ptr(ls + w * C::BQ));
    }
  };

  auto compute = [&](int t, const bf16_t *qs, const bf16_t *ds, const bf16_t *qts, const bf16_t *dts,
                     const float *ls) {
    const int64_t u0 = tile_u0(t);
    if (!(wave_valid && u0 < w_hi && u0 + C::BQ > w_lo)) return;
    const bool need_mask = (u0 < w_lo_max) || (u0 + C::BQ > w_hi_min);
    {
      constexpr int QB0 = 0, QBN = 2;  // both 32-query halves of the tile at once
      f32x16 s[QBN], dp[QBN];
#pragma unroll
    for (int qi_ = 0; qi_ < QBN; ++qi_)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[qi_][i] = 0.f;
        dp[qi_][i] = 0.f;
      }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int qi_ = 0; qi_ < QBN; ++qi_) {
        const int qb2 = QB0 + qi_;
        const int off = rt_off<D>(qb2 * 32 + l32, ks * 2 + hi32);
        const bf16x8 aq = as_bf16x8(*reinterpret_cast<const u32x4 *>(qs + off));
        const bf16x8 ad = as_bf16x8(*reinterpret_cast<const u32x4 *>(ds + off));
        s[qi_] = mfma32(aq, kf[ks], s[qi_]);
        dp[qi_] = mfma32(ad, vf[ks], dp[qi_]);
      }
    }
#pragma unroll
    for (int qi_ = 0; qi_ < QBN; ++qi_) {
      const int qb2 = QB0 + qi_;
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t qi = u0 + qb2 * 32 + (i >> 2) * 8 + hi32 * 4 + (i & 3);
          if (qi < qlo || qi >= qhi) s[qi_][i] = -INFINITY;
        }
      }
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int qo = qb2 * 32 + gq * 8 + hi32 * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(ls + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(ls + C::BQ + qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = gq * 4 + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(s[qi_][i], a.c, -l4[e]));
          s[qi_][i] = p;
          dp[qi_][i] = p * (dp[qi_][i] - d4[e]);  // dS
        }
      }
    }
#pragma unroll
    for (int qi_ = 0; qi_ < QBN; ++qi_) {
      const int qb2 = QB0 + qi_;
#pragma unroll
      for (int jq = 0; jq < 2; ++jq) {
        const int b = jq * 8;
        const f32x16 &pv = s[qi_];
        const f32x16 &sv = dp[qi_];
        const bf16x8 pf = cvt8(pv[b + 0], pv[b + 1], pv[b + 2], pv[b + 3], pv[b + 4], pv[b + 5], pv[b + 6],
                               pv[b + 7]);
        const bf16x8 sf = cvt8(sv[b + 0], sv[b + 1], sv[b + 2], sv[b + 3], sv[b + 4], sv[b + 5], sv[b + 6],
                               sv[b + 7]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int off = tr_off(db * 32 + l32, qb2 * 4 + jq * 2 + hi32);
          const bf16x8 adt = as_bf16x8(*reinterpret_cast<const u32x4 *>(dts + off));
          const bf16x8 aqt = as_bf16x8(*reinterpret_cast<const u32x4 *>(qts + off));
          acc_dv[db] = mfma32(adt, pf, acc_dv[db]);
          acc_dk[db] = mfma32(aqt, sf, acc_dk[db]);
        }
      }
    }
    }
  };

  // Two stages: wait for tile t, barrier (tile t complete, the other stage
  // free), prefetch t+1 into the other stage, compute t.
  if (ntiles > 0) issue(0, q0s, d0s, qt0, dt0, ls0);
  for (int t = 0; t < ntiles; t += 2) {
    wait_vmcnt<0>();
    barrier();
    if (t + 1 < ntiles) issue(t + 1, q1s, d1s, qt1, dt1, ls1);
    compute(t, q0s, d0s, qt0, dt0, ls0);
    if (t + 1 < ntiles) {
      wait_vmcnt<0>();
      barrier();
      if (t + 2 < ntiles) issue(t + 2, q0s, d0s, qt0, dt0, ls0);
      compute(t + 1, q1s, d1s, qt1, dt1, ls1);
    }
  }

  if (key_ok) {
    bf16_t *dko = a.dk + key * a.dk_stride + (int64_t)g * D;
    bf16_t *dvo = a.dv + key * a.dv_stride + (int64_t)g * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + gq * 8 + hi32 * 4;
        u32x2 pk, pv2;
        pk[0] = pack_bf16x2(acc_dk[db][gq * 4 + 0] * a.scale, acc_dk[db][gq * 4 + 1] * a.scale);
        pk[1] = pack_bf16x2(acc_dk[db][gq * 4 + 2] * a.scale, acc_dk[db][gq * 4 + 3] * a.scale);
        pv2[0] = pack_bf16x2(acc_dv[db][gq * 4 + 0], acc_dv[db][gq * 4 + 1]);
        pv2[1] = pack_bf16x2(acc_dv[db][gq * 4 + 2], acc_dv[db][gq * 4 + 3]);
        *reinterpret_cast<u32x2 *>(dko + d0) = pk;
        *reinterpret_cast<u32x2 *>(dvo + d0) = pv2;
      }
  }
}

template <int D, int HPW, int RB>
int launch_dq_cfg(BwdArgs a, hipStream_t stream) {
  using C = DqCfg<D, HPW, RB>;
  a.nblk = (int)((a.N + C::BM - 1) / C::BM);
  a.nhg = a.hq / HPW;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, RB>), dim3((unsigned)((int64_t)a.nblk * a.nhg)),
                     dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dq_kernel");
  return 0;
}

template <int D, int NWK>
int launch_dkdv_cfg(BwdArgs a, hipStream_t stream) {
  using C = DkvCfg<D, NWK>;
  a.nblk = (int)((a.N + C::BNK - 1) / C::BNK);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NWK>), dim3((unsigned)((int64_t)a.nblk * a.hkv)),
                     dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dkdv_kernel");
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
  const int hpw = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
  int rc = 0;
  if (parts & 1) {
    // Transposed copies for both kernels: K^T for this one, Q^T and dO^T for
    // the dK/dV kernel (made here so that kernel runs alone).
    bf16_t *ws_kt = reinterpret_cast<bf16_t *>(p.ws + L.kt);
    bf16_t *ws_qt = reinterpret_cast<bf16_t *>(p.ws + L.qt);
    bf16_t *ws_dot = reinterpret_cast<bf16_t *>(p.ws + L.dot);
    if ((rc = launch_to_trans(p.k, s.k_stride, s.hkv, s.d, s.N, ws_kt, stream))) return rc;
    if ((rc = launch_to_trans(p.q, s.q_stride, s.hq, s.d, s.N, ws_qt, stream))) return rc;
    if ((rc = launch_to_trans(p.dout, p.do_stride, s.hq, s.d, s.N, ws_dot, stream))) return rc;
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
  if (parts & 2) rc = s.d == 128 ? launch_dkdv_cfg<128, 4>(a, stream) : launch_dkdv_cfg<64, 4>(a, stream);
  return rc;
}

}  // namespace uly
