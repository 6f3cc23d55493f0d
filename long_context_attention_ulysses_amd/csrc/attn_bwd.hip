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
// Two kernels, no atomics (the result is deterministic):
//   1. dq kernel, parallel over (query block, head): computes D for its rows
//      (written to the workspace), then loops over key tiles:
//      S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//      K and V tiles are staged in LDS row-major, plus K^T in contraction
//      order; Q and dO stay in registers as MFMA B operands.
//   2. dkdv kernel, parallel over (key block, KV head): loops over the query
//      heads of the group and their query tiles:
//      S = Q K^T, dP = dO V^T (K, V in registers), P, dS,
//      dV^T += dO^T P, dK^T += Q^T dS. Q, dO tiles are staged in LDS both
//      row-major and transposed, with the rows' LSE and D.
// Orientation: in kernel 1 a lane owns one query (scores transposed), in
// kernel 2 a lane owns one key, so the per-row quantities (LSE, D, mask
// bounds) are always a lane scalar or a short LDS read.
#include "attn_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

struct BwdArgs {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;
  bf16_t *dq, *dk, *dv;
  float *delta;
  int64_t N;
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
  static constexpr int KROW = D + 8;
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = BN * KROW;
  static constexpr int KT_ELEMS = D * BN;
  static constexpr int STAGE = K_ELEMS + V_ELEMS + KT_ELEMS;
  static constexpr int K_UNITS = (BN / 2) * (D / 8);  // (key pair, d chunk)
  static constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static constexpr int V_VECS = BN * D / 8;
  static constexpr int V_PER_T = (V_VECS + NT - 1) / NT;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(bf16_t);
};

template <int D, int HPW, int RB>
__global__ void __launch_bounds__(HPW * RB * 64, 1) attn_bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D, HPW, RB>;
  extern __shared__ __align__(16) bf16_t smem[];

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
  if (row_ok && hi32 == 0) a.delta[(int64_t)h * a.N + row] = delta;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int kt0 = (int)(kv_lo / C::BN);
  const int kt1 = (int)((kv_hi + C::BN - 1) / C::BN);
  const bf16_t *kbase = a.k + (int64_t)g * D;
  const bf16_t *vbase = a.v + (int64_t)g * D;

  u32x4 kreg[C::K_PER_T][2];
  u32x4 vreg[C::V_PER_T];

  auto load_tile = [&](int kt) {
    const int64_t t0 = (int64_t)kt * C::BN;
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      const int kp = idx / (D / 8);
      const int dc = idx % (D / 8);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        u32x4 v = {0, 0, 0, 0};
        const int64_t key = t0 + 2 * kp + r;
        if (idx < C::K_UNITS && key < a.N)
          v = *reinterpret_cast<const u32x4 *>(kbase + key * a.k_stride + dc * 8);
        kreg[u][r] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      const int key = idx / (D / 8);
      const int dc = idx % (D / 8);
      u32x4 v = {0, 0, 0, 0};
      if (idx < C::V_VECS && t0 + key < a.N)
        v = *reinterpret_cast<const u32x4 *>(vbase + (t0 + key) * a.v_stride + dc * 8);
      vreg[u] = v;
    }
  };

  auto store_tile = [&](int stage) {
    bf16_t *ks_ = smem + stage * C::STAGE;
    bf16_t *vs_ = ks_ + C::K_ELEMS;
    bf16_t *kt_ = vs_ + C::V_ELEMS;
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (idx < C::K_UNITS) {
        const int kp = idx / (D / 8);
        const int dc = idx % (D / 8);
        *reinterpret_cast<u32x4 *>(ks_ + (2 * kp) * C::KROW + dc * 8) = kreg[u][0];
        *reinterpret_cast<u32x4 *>(ks_ + (2 * kp + 1) * C::KROW + dc * 8) = kreg[u][1];
        const int p = key_pos(2 * kp);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (kreg[u][0][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          const uint32_t hi = (kreg[u][1][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          *reinterpret_cast<uint32_t *>(kt_ + tr_off(dc * 8 + e, p)) = lo | (hi << 16);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (idx < C::V_VECS) {
        const int key = idx / (D / 8);
        const int dc = idx % (D / 8);
        *reinterpret_cast<u32x4 *>(vs_ + key * C::KROW + dc * 8) = vreg[u];
      }
    }
  };

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    if (kt + 1 < kt1) load_tile(kt + 1);
    const int64_t t0 = (int64_t)kt * C::BN;
    if (wave_valid && t0 < w_hi && t0 + C::BN > w_lo) {
      const bf16_t *ks_ = smem + stage * C::STAGE;
      const bf16_t *vs_ = ks_ + C::K_ELEMS;
      const bf16_t *kt_ = vs_ + C::V_ELEMS;
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
          const int off = (kb * 32 + l32) * C::KROW + ks * 16 + hi32 * 8;
          const bf16x8 ak = as_bf16x8(*reinterpret_cast<const u32x4 *>(ks_ + off));
          const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(vs_ + off));
          s[kb] = mfma32(ak, qf[ks], s[kb]);
          dp[kb] = mfma32(av, dof[ks], dp[kb]);
        }
      }
      const bool need_mask = (t0 < w_lo_max) || (t0 + C::BN > w_hi_min);
      if (need_mask) {
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
      bf16x8 dsf[C::JS];
#pragma unroll
      for (int j = 0; j < C::JS; ++j) {
        const f32x16 &sv = s[j >> 1];
        const int b = (j & 1) * 8;
        dsf[j] = cvt8(sv[b + 0], sv[b + 1], sv[b + 2], sv[b + 3], sv[b + 4], sv[b + 5], sv[b + 6],
                      sv[b + 7]);
      }
#pragma unroll
      for (int j = 0; j < C::JS; ++j) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 ak = as_bf16x8(
              *reinterpret_cast<const u32x4 *>(kt_ + tr_off(db * 32 + l32, j * 16 + hi32 * 8)));
          acc[db] = mfma32(ak, dsf[j], acc[db]);
        }
      }
    }
    if (kt + 1 < kt1) store_tile(stage ^ 1);
    __syncthreads();
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
  static constexpr int KROW = D + 8;
  static constexpr int Q_ELEMS = BQ * KROW;
  static constexpr int QT_ELEMS = D * BQ;
  // stage: Q, dO (row-major), Q^T, dO^T (transposed), then lse2[BQ], delta[BQ] floats
  static constexpr int STAGE = 2 * Q_ELEMS + 2 * QT_ELEMS + 2 * BQ * 2;
  static constexpr int UNITS = (BQ / 2) * (D / 8);  // (query pair, d chunk)
  static constexpr int U_PER_T = (UNITS + NT - 1) / NT;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(bf16_t);
};

template <int D, int NWK>
__global__ void __launch_bounds__(NWK * 64, 1) attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = DkvCfg<D, NWK>;
  extern __shared__ __align__(16) bf16_t smem[];

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

  const int qt0 = (int)(qr_lo / C::BQ);
  const int qt1 = (int)((qr_hi + C::BQ - 1) / C::BQ);
  const int ntq = qt1 - qt0;
  const int ntiles = ntq * a.G;  // (head of the group, query tile) pairs

  u32x4 qreg[C::U_PER_T][2], dreg[C::U_PER_T][2];
  float lreg = 0.f;

  auto load_tile = [&](int t) {
    const int hh = t / ntq;
    const int h = g * a.G + hh;
    const int64_t u0 = (int64_t)(qt0 + t % ntq) * C::BQ;
#pragma unroll
    for (int u = 0; u < C::U_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      const int qp = idx / (D / 8);
      const int dc = idx % (D / 8);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        u32x4 vq = {0, 0, 0, 0}, vd = {0, 0, 0, 0};
        const int64_t qi = u0 + 2 * qp + r;
        if (idx < C::UNITS && qi < a.N) {
          const int64_t col = (int64_t)h * D + dc * 8;
          vq = *reinterpret_cast<const u32x4 *>(a.q + qi * a.q_stride + col);
          vd = *reinterpret_cast<const u32x4 *>(a.dout + qi * a.do_stride + col);
        }
        qreg[u][r] = vq;
        dreg[u][r] = vd;
      }
    }
    lreg = 0.f;
    if (tid < 2 * C::BQ) {
      const int64_t qi = u0 + (tid % C::BQ);
      if (qi < a.N)
        lreg = (tid < C::BQ) ? a.lse[(int64_t)h * a.N + qi] * kLog2e : a.delta[(int64_t)h * a.N + qi];
    }
  };

  auto store_tile = [&](int stage) {
    bf16_t *qs = smem + stage * C::STAGE;
    bf16_t *ds = qs + C::Q_ELEMS;
    bf16_t *qts = ds + C::Q_ELEMS;
    bf16_t *dts = qts + C::QT_ELEMS;
    float *ls = reinterpret_cast<float *>(dts + C::QT_ELEMS);
#pragma unroll
    for (int u = 0; u < C::U_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (idx < C::UNITS) {
        const int qp = idx / (D / 8);
        const int dc = idx % (D / 8);
        *reinterpret_cast<u32x4 *>(qs + (2 * qp) * C::KROW + dc * 8) = qreg[u][0];
        *reinterpret_cast<u32x4 *>(qs + (2 * qp + 1) * C::KROW + dc * 8) = qreg[u][1];
        *reinterpret_cast<u32x4 *>(ds + (2 * qp) * C::KROW + dc * 8) = dreg[u][0];
        *reinterpret_cast<u32x4 *>(ds + (2 * qp + 1) * C::KROW + dc * 8) = dreg[u][1];
        const int p = key_pos(2 * qp);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t q0v = (qreg[u][0][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t q1v = (qreg[u][1][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t d0v = (dreg[u][0][e >> 1] >> sh) & 0xFFFFu;
          const uint32_t d1v = (dreg[u][1][e >> 1] >> sh) & 0xFFFFu;
          *reinterpret_cast<uint32_t *>(qts + tr_off(dc * 8 + e, p)) = q0v | (q1v << 16);
          *reinterpret_cast<uint32_t *>(dts + tr_off(dc * 8 + e, p)) = d0v | (d1v << 16);
        }
      }
    }
    if (tid < 2 * C::BQ) ls[tid] = lreg;
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int64_t u0 = (int64_t)(qt0 + t % ntq) * C::BQ;
    if (wave_valid && u0 < w_hi && u0 + C::BQ > w_lo) {
      const bf16_t *qs = smem + stage * C::STAGE;
      const bf16_t *ds = qs + C::Q_ELEMS;
      const bf16_t *qts = ds + C::Q_ELEMS;
      const bf16_t *dts = qts + C::QT_ELEMS;
      const float *ls = reinterpret_cast<const float *>(dts + C::QT_ELEMS);
      const bool need_mask = (u0 < w_lo_max) || (u0 + C::BQ > w_hi_min);
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = 0.f;
          dp[i] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const int off = (qb2 * 32 + l32) * C::KROW + ks * 16 + hi32 * 8;
          const bf16x8 aq = as_bf16x8(*reinterpret_cast<const u32x4 *>(qs + off));
          const bf16x8 ad = as_bf16x8(*reinterpret_cast<const u32x4 *>(ds + off));
          s = mfma32(aq, kf[ks], s);
          dp = mfma32(ad, vf[ks], dp);
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t qi = u0 + qb2 * 32 + (i >> 2) * 8 + hi32 * 4 + (i & 3);
            if (qi < qlo || qi >= qhi) s[i] = -INFINITY;
          }
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int qo = qb2 * 32 + gq * 8 + hi32 * 4;
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(ls + qo);
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(ls + C::BQ + qo);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = gq * 4 + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], a.c, -l4[e]));
            pv[i] = p;
            dsv[i] = p * (dp[i] - d4[e]);
          }
        }
#pragma unroll
        for (int jq = 0; jq < 2; ++jq) {
          const int b = jq * 8;
          const bf16x8 pf = cvt8(pv[b + 0], pv[b + 1], pv[b + 2], pv[b + 3], pv[b + 4], pv[b + 5],
                                 pv[b + 6], pv[b + 7]);
          const bf16x8 sf = cvt8(dsv[b + 0], dsv[b + 1], dsv[b + 2], dsv[b + 3], dsv[b + 4],
                                 dsv[b + 5], dsv[b + 6], dsv[b + 7]);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int off = tr_off(db * 32 + l32, qb2 * 32 + jq * 16 + hi32 * 8);
            const bf16x8 adt = as_bf16x8(*reinterpret_cast<const u32x4 *>(dts + off));
            const bf16x8 aqt = as_bf16x8(*reinterpret_cast<const u32x4 *>(qts + off));
            acc_dv[db] = mfma32(adt, pf, acc_dv[db]);
            acc_dk[db] = mfma32(aqt, sf, acc_dk[db]);
          }
        }
      }
    }
    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
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
  hipError_t e = hipFuncSetAttribute((const void *)attn_bwd_dq_kernel<D, HPW, RB>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd dq: hipFuncSetAttribute");
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, RB>), dim3((unsigned)((int64_t)a.nblk * a.nhg)),
                     dim3(C::NT), C::LDS_BYTES, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dq_kernel");
  return 0;
}

template <int D, int NWK>
int launch_dkdv_cfg(BwdArgs a, hipStream_t stream) {
  using C = DkvCfg<D, NWK>;
  a.nblk = (int)((a.N + C::BNK - 1) / C::BNK);
  hipError_t e = hipFuncSetAttribute((const void *)attn_bwd_dkdv_kernel<D, NWK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd dkdv: hipFuncSetAttribute");
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NWK>), dim3((unsigned)((int64_t)a.nblk * a.hkv)),
                     dim3(C::NT), C::LDS_BYTES, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_bwd_dkdv_kernel");
  return 0;
}

}  // namespace

int launch_attn_bwd(const AttnShape &s, const AttnBwdPtrs &p, int parts, hipStream_t stream) {
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
  a.delta = p.delta;
  a.N = s.N;
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
  if (s.d == 128) {
    if (parts & 1)
      rc = hpw == 4 ? launch_dq_cfg<128, 4, 1>(a, stream)
           : hpw == 2 ? launch_dq_cfg<128, 2, 2>(a, stream)
                      : launch_dq_cfg<128, 1, 4>(a, stream);
    if (rc) return rc;
    return (parts & 2) ? launch_dkdv_cfg<128, 4>(a, stream) : 0;
  }
  if (parts & 1)
    rc = hpw == 4 ? launch_dq_cfg<64, 4, 2>(a, stream)
         : hpw == 2 ? launch_dq_cfg<64, 2, 4>(a, stream)
                    : launch_dq_cfg<64, 1, 8>(a, stream);
  if (rc) return rc;
  return (parts & 2) ? launch_dkdv_cfg<64, 4>(a, stream) : 0;
}

}  // namespace uly
