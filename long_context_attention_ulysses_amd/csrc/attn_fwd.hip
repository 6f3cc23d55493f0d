// Attention forward over the full sequence for the local heads of one
// Ulysses rank ("Ulysses Sequence Parallelism for Million-Token Context
// Training", "How Ulysses Sequence Parallelism Works", step 4: local attention
// over all tokens of the rank's heads).
//
// Exact softmax attention computed tile by tile with a running max and sum
// (online softmax), so memory stays O(N) ("The Challenge of Long Sequence
// Training": FlashAttention-style tiling keeps the O(n^2) compute, not the
// O(n^2) memory).
//
// Work decomposition (one workgroup):
//   * HPW query heads of one GQA group x RB row blocks of QW = 32*NQB rows;
//     wave w takes head (w / RB) and row block (w % RB). All waves share the
//     K/V tiles (BN = 64 keys) staged in LDS, double-buffered: tile t+1 is
//     fetched into registers while tile t is computed, then written to the
//     other LDS stage.
//   * K is kept in LDS as [key][d] (rows padded by 16 bytes); V is stored
//     transposed, [d][key], with keys in MFMA-contraction order (key_pos) and
//     16-byte chunks XOR-swizzled by row so the operand reads hit distinct
//     banks.
//   * Per tile and wave: S^T = K Q^T with bf16 MFMA (Q stays in registers as
//     the B operand), mask where the tile crosses the diagonal or a document
//     edge, running max in the log2 domain, p = exp2(s*scale*log2e - m),
//     O^T += V^T P^T with P^T taken straight from the score registers.
//   * Workgroups are issued heaviest-first (last query blocks first under the
//     causal mask), and consecutive workgroup ids alternate GQA groups, so
//     the round-robin assignment of ids to the 8 XCDs keeps one KV head per
//     XCD L2 whenever the number of groups divides 8.
#include "attn_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

struct FwdArgs {
  const bf16_t *q, *k, *v;
  bf16_t *o;
  float *lse;
  int64_t N;
  int64_t q_stride, k_stride, v_stride, o_stride;
  int hq, G;       // query heads, GQA group size
  int nqb, nhg;    // query blocks, head groups (hq / HPW)
  float c;         // scale * log2(e)
  int causal;
  const int32_t *cu;
  int n_seqs;
};

// Headroom (log2 units) the running max may lag the true max by; see the
// softmax step of the kernel.
constexpr float kMaxSlack = 8.f;

template <int D, int NQB, int HPW, int RB>
struct FwdCfg {
  static constexpr int NW = HPW * RB;
  static constexpr int NT = NW * 64;
  static constexpr int BN = 64;
  static constexpr int QW = 32 * NQB;
  static constexpr int BM = QW * RB;
  static constexpr int KS = D / 16;         // 16-wide k-steps over d
  static constexpr int DB = D / 32;         // 32-row blocks of O^T
  static constexpr int JS = BN / 16;        // 16-key steps of P V
  static constexpr int KROW = D + 8;        // K stage row stride (elements)
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = D * BN;    // V^T stage, rows of BN keys
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int K_VECS = BN * D / 8;          // 16-byte vectors per K tile
  static constexpr int K_PER_T = (K_VECS + NT - 1) / NT;
  static constexpr int V_UNITS = (BN / 2) * (D / 8); // (key pair, 8-wide d chunk)
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(bf16_t);
};

template <int D, int NQB, int HPW, int RB>
__global__ void __launch_bounds__(HPW * RB * 64, 1) attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D, NQB, HPW, RB>;
  extern __shared__ __align__(16) bf16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;

  // Heaviest query blocks first; consecutive ids alternate head groups.
  const int item = blockIdx.x;
  const int hg = item % a.nhg;
  const int qb = a.nqb - 1 - item / a.nhg;
  const int64_t q0 = (int64_t)qb * C::BM;
  const int h = hg * HPW + w / RB;
  const int g = (hg * HPW) / a.G;
  const int64_t r0 = q0 + (int64_t)(w % RB) * C::QW;

  // Key range of the workgroup and of this wave.
  const int64_t q_last = (q0 + C::BM < a.N ? q0 + C::BM : a.N) - 1;
  const int64_t kv_lo = key_range(a.cu, a.n_seqs, a.N, a.causal, q0).lo;
  const int64_t kv_hi = key_range(a.cu, a.n_seqs, a.N, a.causal, q_last).hi;
  const bool wave_valid = r0 < a.N;
  const int64_t w_last = (r0 + C::QW < a.N ? r0 + C::QW : a.N) - 1;
  KeyRange wr0 = key_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? r0 : 0);
  KeyRange wr1 = key_range(a.cu, a.n_seqs, a.N, a.causal, wave_valid ? w_last : 0);
  const int64_t w_lo = wr0.lo, w_hi = wr1.hi;       // union of the rows' ranges
  const int64_t w_lo_max = wr1.lo, w_hi_min = wr0.hi; // intersection

  // Per-lane query rows and their key ranges.
  int64_t row[NQB];
  int64_t rlo[NQB], rhi[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    row[nb] = r0 + nb * 32 + l32;
    if (row[nb] < a.N) {
      KeyRange kr = key_range(a.cu, a.n_seqs, a.N, a.causal, row[nb]);
      rlo[nb] = kr.lo;
      rhi[nb] = kr.hi;
    } else {
      rlo[nb] = 0;
      rhi[nb] = 0;
    }
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds q[row][ks*16 + hi32*8 .. +8].
  bf16x8 qf[NQB][C::KS];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (row[nb] < a.N)
        v = *reinterpret_cast<const u32x4 *>(a.q + row[nb] * a.q_stride + (int64_t)h * D + ks * 16 +
                                             hi32 * 8);
      qf[nb][ks] = as_bf16x8(v);
    }
  }

  f32x16 acc_o[NQB][C::DB];
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[nb][db][i] = 0.f;
  }

  const int kt0 = (int)(kv_lo / C::BN);
  const int kt1 = (int)((kv_hi + C::BN - 1) / C::BN);

  const bf16_t *kbase = a.k + (int64_t)g * D;
  const bf16_t *vbase = a.v + (int64_t)g * D;

  // Register staging for the next tile.
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][2];

  auto load_tile = [&](int kt) {
    const int64_t t0 = (int64_t)kt * C::BN;
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      const int key = idx / (D / 8);
      const int dc = idx % (D / 8);
      u32x4 v = {0, 0, 0, 0};
      if (idx < C::K_VECS && t0 + key < a.N)
        v = *reinterpret_cast<const u32x4 *>(kbase + (t0 + key) * a.k_stride + dc * 8);
      kreg[u] = v;
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      const int kp = idx / (D / 8);
      const int dc = idx % (D / 8);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        u32x4 v = {0, 0, 0, 0};
        const int64_t key = t0 + 2 * kp + r;
        if (idx < C::V_UNITS && key < a.N)
          v = *reinterpret_cast<const u32x4 *>(vbase + key * a.v_stride + dc * 8);
        vreg[u][r] = v;
      }
    }
  };

  auto store_tile = [&](int stage) {
    bf16_t *ks_ = smem + stage * C::STAGE;
    bf16_t *vs_ = ks_ + C::K_ELEMS;
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (idx < C::K_VECS) {
        const int key = idx / (D / 8);
        const int dc = idx % (D / 8);
        *reinterpret_cast<u32x4 *>(ks_ + key * C::KROW + dc * 8) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (idx < C::V_UNITS) {
        const int kp = idx / (D / 8);
        const int dc = idx % (D / 8);
        const int p = key_pos(2 * kp);  // 2kp and 2kp+1 stay adjacent
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (vreg[u][0][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          const uint32_t hi = (vreg[u][1][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          *reinterpret_cast<uint32_t *>(vs_ + tr_off(dc * 8 + e, p)) = lo | (hi << 16);
        }
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

      // S^T = K Q^T
      f32x16 s[NQB][2];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[nb][kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 af = as_bf16x8(
              *reinterpret_cast<const u32x4 *>(ks_ + (kb * 32 + l32) * C::KROW + ks * 16 + hi32 * 8));
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) s[nb][kb] = mfma32(af, qf[nb][ks], s[nb][kb]);
        }
      }

      const bool need_mask = (t0 < w_lo_max) || (t0 + C::BN > w_hi_min);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int64_t key = t0 + kb * 32 + (i >> 2) * 8 + hi32 * 4 + (i & 3);
              if (key < rlo[nb] || key >= rhi[nb]) s[nb][kb][i] = -INFINITY;
            }
      }

      bf16x8 pf[NQB][C::JS];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][kb][i]);
        mx = fmaxf(mx, xor32(mx));
        // The running max m only moves when this tile's max exceeds it by
        // more than kMaxSlack (log2 units), so p = exp2(s*c - m) stays below
        // 2^kMaxSlack; O and l are rescaled only when some lane of the wave
        // moves its max. The result is exact either way (O / l and
        // m + log2 l do not depend on which m was used).
        const float m_cand = mx * a.c;
        const bool grow = m_cand > m_run[nb] + kMaxSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[nb] - m_cand) : 1.f;
          m_run[nb] = grow ? m_cand : m_run[nb];
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_o[nb][db][i] *= alpha;
        }
        const float m_use = (m_run[nb] == -INFINITY) ? 0.f : m_run[nb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[nb][kb][i], a.c, -m_use));
            s[nb][kb][i] = p;
            rs += p;
          }
        l_run[nb] += rs;
#pragma unroll
        for (int j = 0; j < C::JS; ++j) {
          const f32x16 &sv = s[nb][j >> 1];
          const int b = (j & 1) * 8;
          pf[nb][j] = cvt8(sv[b + 0], sv[b + 1], sv[b + 2], sv[b + 3], sv[b + 4], sv[b + 5],
                           sv[b + 6], sv[b + 7]);
        }
      }

      // O^T += V^T P^T
#pragma unroll
      for (int j = 0; j < C::JS; ++j) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 af = as_bf16x8(
              *reinterpret_cast<const u32x4 *>(vs_ + tr_off(db * 32 + l32, j * 16 + hi32 * 8)));
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) acc_o[nb][db] = mfma32(af, pf[nb][j], acc_o[nb][db]);
        }
      }
    }

    if (kt + 1 < kt1) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2.
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const float l_tot = l_run[nb] + xor32(l_run[nb]);
    if (!(row[nb] < a.N)) continue;
    const float inv = 1.f / l_tot;
    bf16_t *orow = a.o + row[nb] * a.o_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + gq * 8 + hi32 * 4;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc_o[nb][db][gq * 4 + 0] * inv, acc_o[nb][db][gq * 4 + 1] * inv);
        pk[1] = pack_bf16x2(acc_o[nb][db][gq * 4 + 2] * inv, acc_o[nb][db][gq * 4 + 3] * inv);
        *reinterpret_cast<u32x2 *>(orow + d0) = pk;
      }
    if (hi32 == 0) a.lse[(int64_t)h * a.N + row[nb]] = (m_run[nb] + log2f(l_tot)) * kLn2;
  }
}

template <int D, int NQB, int HPW, int RB>
int launch_fwd_cfg(const FwdArgs &args0, hipStream_t stream) {
  using C = FwdCfg<D, NQB, HPW, RB>;
  FwdArgs a = args0;
  a.nqb = (int)((a.N + C::BM - 1) / C::BM);
  a.nhg = a.hq / HPW;
  const int64_t blocks = (int64_t)a.nqb * a.nhg;
  hipError_t ea = hipFuncSetAttribute((const void *)attn_fwd_kernel<D, NQB, HPW, RB>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (ea != hipSuccess) return set_hip_error(ea, "attn_fwd: hipFuncSetAttribute");
  hipLaunchKernelGGL((attn_fwd_kernel<D, NQB, HPW, RB>), dim3((unsigned)blocks), dim3(C::NT),
                     C::LDS_BYTES, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_fwd_kernel");
  return 0;
}

}  // namespace

int launch_attn_fwd(const AttnShape &s, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                    bf16_t *o, float *lse, hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = s.N;
  a.q_stride = s.q_stride;
  a.k_stride = s.k_stride;
  a.v_stride = s.v_stride;
  a.o_stride = s.o_stride;
  a.hq = s.hq;
  a.G = s.hq / s.hkv;
  a.c = s.scale * kLog2e;
  a.causal = s.causal;
  a.cu = s.cu;
  a.n_seqs = s.n_seqs;
  a.nqb = a.nhg = 0;
  // Heads per workgroup: the largest of 4, 2, 1 dividing the group size, so
  // every workgroup reads a single KV head; 8 waves per workgroup.
  const int hpw = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
  if (s.d == 128) {
    if (hpw == 4) return launch_fwd_cfg<128, 1, 4, 2>(a, stream);
    if (hpw == 2) return launch_fwd_cfg<128, 1, 2, 4>(a, stream);
    return launch_fwd_cfg<128, 1, 1, 8>(a, stream);
  }
  if (hpw == 4) return launch_fwd_cfg<64, 1, 4, 2>(a, stream);
  if (hpw == 2) return launch_fwd_cfg<64, 1, 2, 4>(a, stream);
  return launch_fwd_cfg<64, 1, 1, 8>(a, stream);
}

}  // namespace uly
