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
// Work decomposition (one workgroup of HPW x RB waves):
//   * HPW query heads of one GQA group x RB row blocks of 32 rows; wave w
//     takes head w / RB and row block w % RB, so every K/V tile staged in LDS
//     serves HPW * RB * 32 query rows.
//   * K/V tiles of 64 keys stream through a 3-stage LDS ring with
//     direct-to-LDS copies (no register staging): K as a row tile, V from its
//     contraction-ordered transposed copy as a trans tile. One barrier per
//     tile; tile t+2 is in flight while tile t is computed.
//   * Per tile and wave: S^T = K Q^T with bf16 MFMA 32x32x16 (Q stays in
//     registers as the B operand, so a lane owns one query), mask only where
//     the tile crosses the diagonal or a document edge, running max in the
//     log2 domain, p = exp2(s*scale*log2e - m), O^T += V^T P^T with P^T taken
//     straight from the score registers.
//   * Workgroups are issued heaviest-first (last query blocks first under the
//     causal mask; over packed documents in the order a small sorting pass
//     writes into the workspace), and consecutive workgroup ids alternate GQA
//     groups, so the round-robin assignment of ids to the 8 XCDs keeps one KV
//     head per XCD L2 whenever the number of groups divides 8.
//   * With fewer than 512 (query block, head group) pairs, each pair's key
//     tiles are split over up to 4 workgroups that write their float32
//     softmax states (unnormalised O, running max, sum); a merge pass combines
//     them (exact: the states are rescaled to a common max).
#include "attn_common.h"
#include "uly_internal.h"

namespace uly {

namespace {

struct FwdArgs {
  const bf16_t *q, *k;
  const bf16_t *vt;  // V^T [hkv][D][Np], contraction-ordered
  bf16_t *o;
  float *lse;
  int64_t N, Np;
  int64_t q_stride, k_stride, o_stride;
  int hq, G;     // query heads, GQA group size
  int nqb, nhg;  // query blocks, head groups (hq / HPW)
  float c;       // scale * log2(e)
  int causal;
  const int32_t *cu;
  int n_seqs;
  int32_t *qorder;               // packed documents: query blocks by decreasing work
  int qsplit;                    // workgroups per (query block, head group)
  float *opart, *mpart, *lpart;  // partials when qsplit > 1: O [s][N][hq][D], max and sum [s][hq][N]
};

// Headroom (log2 units) the running max may lag the true max by; see the
// softmax step of the kernel.
constexpr float kMaxSlack = 8.f;

template <int D, int HPW, int RB>
struct FwdCfg {
  static constexpr int NW = HPW * RB;
  static constexpr int NT = NW * 64;
  static constexpr int BN = 64;
  static constexpr int BM = 32 * RB;
  static constexpr int KS = D / 16;     // 16-wide k-steps over d
  static constexpr int DB = D / 32;     // 32-row blocks of O^T
  static constexpr int JS = BN / 16;    // 16-key steps of P V
  static constexpr int TILE = BN * D;   // elements of one K (or V^T) tile
  static constexpr int NI = TILE / 512; // 1 KiB direct-to-LDS copies per tile
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  static constexpr int NLW = 2 * NI / NW;  // copies per wave per tile (K and V^T)
};

template <int D, int HPW, int RB, bool kSplit>
__global__ void __launch_bounds__(HPW * RB * 64, 1) attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D, HPW, RB>;
  __shared__ __align__(16) bf16_t k0[C::TILE], k1[C::TILE], k2[C::TILE];
  __shared__ __align__(16) bf16_t v0[C::TILE], v1[C::TILE], v2[C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hi32 = lane >> 5;

  // Heaviest query blocks first (the last ones under a causal mask, the
  // sorted order over packed documents); consecutive ids alternate head
  // groups, and with a split the pieces of one query block are consecutive.
  const int item = blockIdx.x;
  const int hg = item % a.nhg;
  const int qbi = kSplit ? item / a.nhg / a.qsplit : item / a.nhg;
  const int qb = a.qorder ? a.qorder[qbi] : a.nqb - 1 - qbi;
  const int split = kSplit ? item / a.nhg % a.qsplit : 0;
  const int64_t q0 = (int64_t)qb * C::BM;
  const int h = hg * HPW + w / RB;
  const int g = (hg * HPW) / a.G;
  const int64_t r0 = q0 + (int64_t)(w % RB) * 32;

  // Key range of the workgroup and of this wave (documents found from the
  // block's first row on).
  const int64_t q_last = (q0 + C::BM < a.N ? q0 + C::BM : a.N) - 1;
  const int b0 = doc_start(a.cu, a.n_seqs, q0);
  const int64_t kv_lo = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, q0).lo;
  const int64_t kv_hi = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, q_last).hi;
  const bool wave_valid = r0 < a.N;
  const int64_t w_last = (r0 + 32 < a.N ? r0 + 32 : a.N) - 1;
  const KeyRange wr0 = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? r0 : q0);
  const KeyRange wr1 = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, wave_valid ? w_last : q0);
  const int64_t w_lo = wr0.lo, w_hi = wr1.hi;          // union of the rows' ranges
  const int64_t w_lo_max = wr1.lo, w_hi_min = wr0.hi;  // intersection

  // This lane's query row and its key range.
  const int64_t row = r0 + l32;
  const bool row_ok = row < a.N;
  int64_t rlo = 0, rhi = 0;
  if (row_ok) {
    const KeyRange kr = key_range_from(a.cu, a.n_seqs, a.N, a.causal, b0, row);
    rlo = kr.lo;
    rhi = kr.hi;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds q[row][ks*16 + hi32*8 .. +8].
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 v = {0, 0, 0, 0};
    if (row_ok)
      v = *reinterpret_cast<const u32x4 *>(a.q + row * a.q_stride + (int64_t)h * D + ks * 16 + hi32 * 8);
    qf[ks] = as_bf16x8(v);
  }

  f32x16 acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Key tiles of the block, and this workgroup's share of them [kt0, kt1).
  const int kta = (int)(kv_lo / C::BN);
  const int ktb = (int)((kv_hi + C::BN - 1) / C::BN);
  const int kt0 = kSplit ? kta + (int)((int64_t)(ktb - kta) * split / a.qsplit) : kta;
  const int kt1 = kSplit ? kta + (int)((int64_t)(ktb - kta) * (split + 1) / a.qsplit) : ktb;
  // Buffer views: K rows of KV head g (rows >= N read as zeros, and their
  // scores are masked) and V^T of head g.
  const uint32_t kstride_b = (uint32_t)(a.k_stride * 2);
  const bf16_t *kbase = a.k + (int64_t)g * D;
  const uint32_t kbytes = head_rows_bytes(a.N, a.k_stride, D);
  const BufRes vrs = make_rsrc(a.vt + (int64_t)g * D * a.Np, (uint32_t)(D * a.Np * 2));
  // Per-lane byte offsets of this wave's 16-byte slots inside a tile.
  uint32_t koff[C::NI / C::NW], voff[C::NI / C::NW];
#pragma unroll
  for (int i = 0; i < C::NI / C::NW; ++i) {
    const int s = (w + i * C::NW) * 64 + lane;
    const int r = s / (D / 8);
    koff[i] = r * kstride_b + (((s % (D / 8)) ^ row_swz<D>(r)) << 4);
    const int d = s >> 3;
    voff[i] = (uint32_t)(d * a.Np * 2) + (((s & 7) ^ ((d >> 1) & 7)) << 4);
  }

  // Direct-to-LDS copies of tile kt: this wave's share of the 1 KiB blocks.
  // K rows from tile row t0 on: the resource starts at row t0 and still ends
  // after row N-1.
  auto issue = [&](int kt, bf16_t *ks_, bf16_t *vs_) {
    const uint32_t t0 = (uint32_t)kt * C::BN;
    const BufRes krs = make_rsrc(kbase + (int64_t)t0 * a.k_stride, kbytes - t0 * kstride_b);
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i)
      dma16(krs, koff[i], 0, ks_ + (w + i * C::NW) * 512);
#pragma unroll
    for (int i = 0; i < C::NI / C::NW; ++i)
      dma16(vrs, voff[i], t0 * 2, vs_ + (w + i * C::NW) * 512);
  };

  auto compute = [&](int kt, const bf16_t *ks_, const bf16_t *vs_) {
    const int64_t t0 = (int64_t)kt * C::BN;
    if (!(wave_valid && t0 < w_hi && t0 + C::BN > w_lo)) return;
    // S^T = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 af = as_bf16x8(
            *reinterpret_cast<const u32x4 *>(ks_ + rt_off<D>(kb * 32 + l32, ks * 2 + hi32)));
        s[kb] = mfma32(af, qf[ks], s[kb]);
      }
    }
    pipeline_reads_mfma<2 * C::KS>();
    if ((t0 < w_lo_max) || (t0 + C::BN > w_hi_min)) {
      const RelRange rr = rel_range(rlo, rhi, t0, hi32 * 4);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = kb * 32 + (i >> 2) * 8 + (i & 3);
          if (e < rr.lo || e >= rr.hi) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_halves(mx);
    // The running max m only moves when this tile's max exceeds it by more
    // than kMaxSlack (log2 units), so p = exp2(s*c - m) stays below
    // 2^kMaxSlack; O and l are rescaled only when some lane of the wave moves
    // its max. The result is exact either way (O / l and m + log2 l do not
    // depend on which m was used).
    const float m_cand = mx * a.c;
    const bool grow = m_cand > m_run + kMaxSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_cand) : 1.f;
      m_run = grow ? m_cand : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = -0.f;  // -0 + p is p exactly, so the first add folds away
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c, -m_use));
        s[kb][i] = p;
        rs += p;
      }
    l_run += rs;
    bf16x8 pf[C::JS];
#pragma unroll
    for (int j = 0; j < C::JS; ++j) {
      const f32x16 &sv = s[j >> 1];
      const int b = (j & 1) * 8;
      pf[j] = cvt8(sv[b + 0], sv[b + 1], sv[b + 2], sv[b + 3], sv[b + 4], sv[b + 5], sv[b + 6], sv[b + 7]);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int j = 0; j < C::JS; ++j) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 af =
            as_bf16x8(*reinterpret_cast<const u32x4 *>(vs_ + tr_off(db * 32 + l32, 2 * j + hi32)));
        acc_o[db] = mfma32(af, pf[j], acc_o[db]);
      }
    }
    pipeline_reads_mfma<C::JS * C::DB>();
  };

  // Tile t lives in stage (t - kt0) % 3; at step t: wait for tile t, barrier
  // (tile t complete in LDS, stage of tile t-1 free), prefetch t+2, compute t.
  auto step = [&](int t, const bf16_t *ks_, const bf16_t *vs_, bf16_t *kn, bf16_t *vn) {
    if (t + 1 < kt1) wait_vmcnt<C::NLW>();
    else wait_vmcnt<0>();
    barrier();
    if (t + 2 < kt1) issue(t + 2, kn, vn);
    compute(t, ks_, vs_);
  };

  wait_vmcnt<0>();  // Q fragments loaded: only tile copies are counted below
  if (kt0 < kt1) issue(kt0, k0, v0);
  if (kt0 + 1 < kt1) issue(kt0 + 1, k1, v1);
  for (int kt = kt0; kt < kt1; kt += 3) {
    step(kt, k0, v0, k2, v2);
    if (kt + 1 < kt1) step(kt + 1, k1, v1, k0, v0);
    if (kt + 2 < kt1) step(kt + 2, k2, v2, k1, v1);
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2; with a split, the
  // unnormalised O^T, m and l of this share of the keys.
  const float l_tot = sum_halves(l_run);
  if constexpr (kSplit) {
    if (row_ok) {
      float *orow = a.opart + (((int64_t)split * a.N + row) * a.hq + h) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + gq * 8 + hi32 * 4;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc_o[db][gq * 4 + e];
          *reinterpret_cast<f32x4 *>(orow + d0) = v;
        }
      if (hi32 == 0) {
        const int64_t ml = ((int64_t)split * a.hq + h) * a.N + row;
        a.mpart[ml] = m_run;
        a.lpart[ml] = l_tot;
      }
    }
    return;
  }
  if (row_ok) {
    const float inv = 1.f / l_tot;
    bf16_t *orow = a.o + row * a.o_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + gq * 8 + hi32 * 4;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc_o[db][gq * 4 + 0] * inv, acc_o[db][gq * 4 + 1] * inv);
        pk[1] = pack_bf16x2(acc_o[db][gq * 4 + 2] * inv, acc_o[db][gq * 4 + 3] * inv);
        *reinterpret_cast<u32x2 *>(orow + d0) = pk;
      }
    if (hi32 == 0) a.lse[(int64_t)h * a.N + row] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// Merge of the forward's partial softmax states over its key-range split:
// with M = max_s m_s and w_s = 2^(m_s - M), O = sum_s w_s O_s / sum_s w_s l_s
// and LSE = (M + log2 sum_s w_s l_s) ln 2 (m in log2 units), the same result
// the unsplit kernel forms from one running state. One thread per 8 values.
struct FwdMergeArgs {
  const float *opart, *mpart, *lpart;
  bf16_t *o;
  float *lse;
  int64_t N, o_stride;
  int hq, d, ks;
  uint32_t total;  // N * hq * d / 8
};

__global__ void __launch_bounds__(256) fwd_merge_kernel(FwdMergeArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t cpr = (uint32_t)a.d / 8;
  const uint32_t rh = i / cpr, c = i - rh * cpr;
  const int64_t row = rh / a.hq;
  const int h = (int)(rh - row * a.hq);
  float M = -INFINITY;
  for (int s = 0; s < a.ks; ++s) M = fmaxf(M, a.mpart[((int64_t)s * a.hq + h) * a.N + row]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float l = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.ks; ++s) {
    const int64_t ml = ((int64_t)s * a.hq + h) * a.N + row;
    const float ms = a.mpart[ml];
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - Mu);
    l += wgt * a.lpart[ml];
    const float *p = a.opart + (((int64_t)s * a.N + row) * a.hq + h) * a.d + c * 8;
    o0 += wgt * *reinterpret_cast<const f32x4 *>(p);
    o1 += wgt * *reinterpret_cast<const f32x4 *>(p + 4);
  }
  const float inv = 1.f / l;
  u32x4 pk;
  pk[0] = pack_bf16x2(o0[0] * inv, o0[1] * inv);
  pk[1] = pack_bf16x2(o0[2] * inv, o0[3] * inv);
  pk[2] = pack_bf16x2(o1[0] * inv, o1[1] * inv);
  pk[3] = pack_bf16x2(o1[2] * inv, o1[3] * inv);
  *reinterpret_cast<u32x4 *>(a.o + row * a.o_stride + (int64_t)h * a.d + c * 8) = pk;
  if (c == 0) a.lse[(int64_t)h * a.N + row] = (M + log2f(l)) * kLn2;
}

template <int D, int HPW, int RB>
int launch_fwd_cfg(FwdArgs a, hipStream_t stream) {
  using C = FwdCfg<D, HPW, RB>;
  a.nqb = (int)((a.N + C::BM - 1) / C::BM);
  a.nhg = a.hq / HPW;
  a.qsplit = fwd_ksplit(a.N, a.hq, a.hq / a.G);
  if (a.qorder) {
    const int rc = launch_block_orders(a.cu, a.n_seqs, a.N, a.causal, C::BM, a.qorder, 0, nullptr, stream);
    if (rc) return rc;
  }
  const int64_t blocks = (int64_t)a.nqb * a.nhg * a.qsplit;
  if (a.qsplit > 1)
    hipLaunchKernelGGL((attn_fwd_kernel<D, HPW, RB, true>), dim3((unsigned)blocks), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, HPW, RB, false>), dim3((unsigned)blocks), dim3(C::NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "attn_fwd_kernel");
  if (a.qsplit > 1) {
    FwdMergeArgs m;
    m.opart = a.opart;
    m.mpart = a.mpart;
    m.lpart = a.lpart;
    m.o = a.o;
    m.lse = a.lse;
    m.N = a.N;
    m.o_stride = a.o_stride;
    m.hq = a.hq;
    m.d = D;
    m.ks = a.qsplit;
    m.total = (uint32_t)(a.N * a.hq * D / 8);
    hipLaunchKernelGGL(fwd_merge_kernel, dim3((m.total + 255) / 256), dim3(256), 0, stream, m);
    e = hipGetLastError();
    if (e != hipSuccess) return set_hip_error(e, "fwd_merge_kernel");
  }
  return 0;
}

}  // namespace

int launch_attn_fwd(const AttnShape &s, const bf16_t *q, const bf16_t *k, const bf16_t *v,
                    bf16_t *o, float *lse, void *ws, hipStream_t stream) {
  bf16_t *vt = static_cast<bf16_t *>(ws);
  int rc = launch_to_trans(v, s.v_stride, s.hkv, s.d, s.N, vt, stream);
  if (rc) return rc;
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.N = s.N;
  a.Np = pad64(s.N);
  a.q_stride = s.q_stride;
  a.k_stride = s.k_stride;
  a.o_stride = s.o_stride;
  a.hq = s.hq;
  a.G = s.hq / s.hkv;
  a.c = s.scale * kLog2e;
  a.causal = s.causal;
  a.cu = s.cu;
  a.n_seqs = s.n_seqs;
  a.qorder = s.cu ? reinterpret_cast<int32_t *>(static_cast<char *>(ws) + fwd_ws_order(s.N, s.hq, s.hkv, s.d))
                  : nullptr;
  a.nqb = a.nhg = 0;
  {
    const int ks = fwd_ksplit(s.N, s.hq, s.hkv);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + fwd_ws_part(s.N, s.hkv, s.d));
    a.qsplit = 1;
    a.opart = part;
    a.mpart = part + (size_t)ks * s.N * s.hq * s.d;
    a.lpart = a.mpart + (size_t)ks * s.hq * s.N;
  }
  // Heads per workgroup: the largest of 4, 2, 1 dividing the group size, so
  // every workgroup reads a single KV head; 8 waves per workgroup.
  const int hpw = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
  if (s.d == 128) {
    if (hpw == 4) return launch_fwd_cfg<128, 4, 2>(a, stream);
    if (hpw == 2) return launch_fwd_cfg<128, 2, 4>(a, stream);
    return launch_fwd_cfg<128, 1, 8>(a, stream);
  }
  if (hpw == 4) return launch_fwd_cfg<64, 4, 2>(a, stream);
  if (hpw == 2) return launch_fwd_cfg<64, 2, 4>(a, stream);
  return launch_fwd_cfg<64, 1, 8>(a, stream);
}

}  // namespace uly
