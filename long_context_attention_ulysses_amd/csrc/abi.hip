// C-ABI of libulysses: argument validation (host only, before any launch),
// status strings, and dispatch to the kernels. Declarations and the contract
// of every call are in include/ulysses.h.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "ulysses.h"
#include "uly_internal.h"

// Workspace of attn_fwd_noalloc, for callers that cannot allocate: one
// static buffer per GPU, created when the library's code is loaded on that
// GPU and held until the process ends. Host code never passes `scratch`
// itself to a kernel (on the host it is only a stand-in for the symbol); it
// passes the device address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[ULY_NOALLOC_SCRATCH_BYTES];

namespace uly {

static thread_local char g_last_error[256] = "";

int set_hip_error(hipError_t e, const char *where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return ULY_E_HIP;
}

int set_error_text(const char *msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return ULY_E_HIP;
}

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// N rows of `stride` elements stay below 2 GiB of bf16 (byte offsets fit 31 bits).
bool fits_rows(int64_t N, int64_t stride) { return N * stride < ((int64_t)1 << 30); }

// [a, a + na) and [b, b + nb) overlap (byte ranges).
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Bytes spanned by a strided [rows][width] bf16 view.
size_t span_bytes(int64_t rows, int64_t stride, int64_t width) {
  if (rows <= 0) return 0;
  return (size_t)(((rows - 1) * stride + width) * 2);
}

int check_swap(const void *src, const void *dst, int64_t n, int32_t P, int32_t nseg,
               const int32_t *seg, int32_t d) {
  if (!src || !dst || !seg) return ULY_E_NULL;
  if (n <= 0 || P <= 0 || nseg <= 0 || nseg > 8 || d <= 0) return ULY_E_SHAPE;
  if (d % 8 != 0) return ULY_E_ALIGN;
  int64_t H = 0;
  for (int s = 0; s < nseg; ++s) {
    if (seg[s] <= 0) return ULY_E_SHAPE;
    if (seg[s] % P != 0) return ULY_E_DIV_P;
    H += seg[s];
  }
  // every 16-byte vector index of the tensor must fit the kernels' 32-bit indexes
  if (n * H * d / 8 >= (int64_t)1 << 31) return ULY_E_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return ULY_E_ALIGN;
  const size_t bytes = (size_t)(n * H * d * 2);
  if (overlaps(src, bytes, dst, bytes)) return ULY_E_ALIAS;
  return ULY_OK;
}

int check_attn_common(const void *q, const void *k, const void *v, int64_t N, int32_t hq,
                      int32_t hkv, int32_t d, int64_t qs, int64_t ks, int64_t vs, float scale) {
  if (!q || !k || !v) return ULY_E_NULL;
  if (N <= 0 || hq <= 0 || hkv <= 0) return ULY_E_SHAPE;
  if (N >= (int64_t)1 << 31) return ULY_E_SHAPE;  // tile indices are 32-bit
  if (!(scale > 0.f) || scale > 3.4e38f) return ULY_E_SHAPE;
  if (hq % hkv != 0) return ULY_E_GQA;
  if (d != 64 && d != 128) return ULY_E_HEADDIM;
  if (qs < (int64_t)hq * d || ks < (int64_t)hkv * d || vs < (int64_t)hkv * d) return ULY_E_STRIDE;
  if (qs % 8 || ks % 8 || vs % 8) return ULY_E_ALIGN;
  // the kernels address one head's rows with 32-bit byte offsets
  if (!fits_rows(N, qs) || !fits_rows(N, ks) || !fits_rows(N, vs) || !fits_rows(pad64(N), d))
    return ULY_E_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ULY_E_ALIGN;
  return ULY_OK;
}

int check_out(const void *out, int64_t N, int64_t stride, int64_t width) {
  if (!out) return ULY_E_NULL;
  if (stride < width) return ULY_E_STRIDE;
  if (stride % 8) return ULY_E_ALIGN;
  if (!aligned16(out)) return ULY_E_ALIGN;
  (void)N;
  return ULY_OK;
}

int check_varlen_args(const int32_t *cu, int32_t n_seqs, int32_t max_seqlen, int64_t N) {
  if (!cu) return ULY_E_NULL;
  if (n_seqs <= 0 || n_seqs > N) return ULY_E_SHAPE;
  if (max_seqlen <= 0 || max_seqlen > N) return ULY_E_SHAPE;
  return ULY_OK;
}

// Device address of `scratch` on device `dev`, looked up once per device
// with that device current (each GPU holds its own copy at its own address).
constexpr int kMaxScratchDevices = 64;

int scratch_address(int dev, void **out) {
  static std::once_flag once[kMaxScratchDevices];
  static void *addr[kMaxScratchDevices];
  static hipError_t err[kMaxScratchDevices];
  if (dev < 0 || dev >= kMaxScratchDevices) return set_error_text("attn_fwd_noalloc: device index out of range");
  std::call_once(once[dev], [dev] {
    int prev = 0;
    err[dev] = hipGetDevice(&prev);
    if (err[dev] == hipSuccess && prev != dev) err[dev] = hipSetDevice(dev);
    if (err[dev] == hipSuccess) err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
  });
  if (err[dev] != hipSuccess) return set_hip_error(err[dev], "attn_fwd_noalloc: hipGetSymbolAddress(scratch)");
  *out = addr[dev];
  return ULY_OK;
}

// ws == nullptr with use_scratch: the forward's workspace is the static
// scratch buffer of the stream's device (attn_fwd_noalloc).
int attn_fwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o,
                  float *lse, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t qs,
                  int64_t ks, int64_t vs, int64_t os, float scale, int32_t causal,
                  const int32_t *cu, int32_t n_seqs, void *ws, size_t ws_bytes,
                  hipStream_t stream, bool use_scratch = false) {
  int rc = check_attn_common(q, k, v, N, hq, hkv, d, qs, ks, vs, scale);
  if (rc) return rc;
  if ((rc = check_out(o, N, os, (int64_t)hq * d))) return rc;
  if (!lse) return ULY_E_NULL;
  const size_t ob = span_bytes(N, os, (int64_t)hq * d);
  if (overlaps(o, ob, q, span_bytes(N, qs, (int64_t)hq * d)) ||
      overlaps(o, ob, k, span_bytes(N, ks, (int64_t)hkv * d)) ||
      overlaps(o, ob, v, span_bytes(N, vs, (int64_t)hkv * d)) ||
      overlaps(lse, (size_t)N * hq * 4, o, ob))
    return ULY_E_ALIAS;
  const size_t wb = fwd_ws_bytes(N, hq, hkv, d);
  if (use_scratch) {
    if (wb > (size_t)ULY_NOALLOC_SCRATCH_BYTES) return ULY_E_SCRATCH;
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return set_hip_error(e, "attn_fwd_noalloc: device of the stream");
    if ((rc = scratch_address(dev, &ws))) return rc;
  } else {
    if (!ws || ws_bytes < wb || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ULY_E_WORKSPACE;
    if (overlaps(ws, wb, o, ob) || overlaps(ws, wb, lse, (size_t)N * hq * 4) ||
        overlaps(ws, wb, q, span_bytes(N, qs, (int64_t)hq * d)) ||
        overlaps(ws, wb, k, span_bytes(N, ks, (int64_t)hkv * d)) ||
        overlaps(ws, wb, v, span_bytes(N, vs, (int64_t)hkv * d)))
      return ULY_E_ALIAS;
  }
  AttnShape s;
  s.N = N;
  s.hq = hq;
  s.hkv = hkv;
  s.d = d;
  s.q_stride = qs;
  s.k_stride = ks;
  s.v_stride = vs;
  s.o_stride = os;
  s.scale = scale;
  s.causal = causal ? 1 : 0;
  s.cu = cu;
  s.n_seqs = n_seqs;
  return launch_attn_fwd(s, q, k, v, o, lse, ws, stream);
}

int attn_bwd_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
                  const float *lse, const uint16_t *dout, uint16_t *dq, uint16_t *dk,
                  uint16_t *dv, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t qs,
                  int64_t ks, int64_t vs, int64_t os, int64_t dos, int64_t dqs, int64_t dks,
                  int64_t dvs, float scale, int32_t causal, const int32_t *cu, int32_t n_seqs,
                  void *ws, size_t ws_bytes, int parts, hipStream_t stream) {
  int rc = check_attn_common(q, k, v, N, hq, hkv, d, qs, ks, vs, scale);
  if (rc) return rc;
  const bool want_dq = parts & 1, want_dkv = parts & 2;
  if (!lse || !dout || (want_dq && !o)) return ULY_E_NULL;
  const int64_t wq = (int64_t)hq * d, wk = (int64_t)hkv * d;
  if (dos < wq || (want_dq && os < wq)) return ULY_E_STRIDE;
  if (!fits_rows(N, dos)) return ULY_E_SHAPE;
  if (dos % 8 || (want_dq && os % 8)) return ULY_E_ALIGN;
  if (!aligned16(dout) || (want_dq && !aligned16(o))) return ULY_E_ALIGN;
  if (want_dq && (rc = check_out(dq, N, dqs, wq))) return rc;
  if (want_dkv && (rc = check_out(dk, N, dks, wk))) return rc;
  if (want_dkv && (rc = check_out(dv, N, dvs, wk))) return rc;
  if (!ws) return ULY_E_WORKSPACE;
  const size_t wb = bwd_ws_layout(N, hq, hkv, d).total;
  if (ws_bytes < wb) return ULY_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return ULY_E_WORKSPACE;
  // outputs must not overlap any input or the workspace (they may interleave
  // with each other, as views into one fused buffer)
  struct R {
    const void *p;
    size_t n;
  };
  const R ins[] = {{q, span_bytes(N, qs, wq)},
                   {k, span_bytes(N, ks, wk)},
                   {v, span_bytes(N, vs, wk)},
                   {o, want_dq ? span_bytes(N, os, wq) : 0},
                   {dout, span_bytes(N, dos, wq)},
                   {lse, (size_t)N * hq * 4},
                   {ws, wb}};
  const R outs[] = {{dq, want_dq ? span_bytes(N, dqs, wq) : 0},
                    {dk, want_dkv ? span_bytes(N, dks, wk) : 0},
                    {dv, want_dkv ? span_bytes(N, dvs, wk) : 0}};
  for (const R &x : outs)
    for (const R &y : ins)
      if (x.n && y.n && overlaps(x.p, x.n, y.p, y.n)) return ULY_E_ALIAS;
  AttnShape s;
  s.N = N;
  s.hq = hq;
  s.hkv = hkv;
  s.d = d;
  s.q_stride = qs;
  s.k_stride = ks;
  s.v_stride = vs;
  s.o_stride = os;
  s.scale = scale;
  s.causal = causal ? 1 : 0;
  s.cu = cu;
  s.n_seqs = cu ? n_seqs : 0;
  AttnBwdPtrs p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.do_stride = dos;
  p.dq_stride = dqs;
  p.dk_stride = dks;
  p.dv_stride = dvs;
  p.ws = static_cast<char *>(ws);
  return launch_attn_bwd(s, p, parts, stream);
}

}  // namespace
}  // namespace uly

using namespace uly;

extern "C" {

const char *uly_status_string(int status) {
  switch (status) {
    case ULY_OK: return "ok";
    case ULY_E_NULL: return "null pointer";
    case ULY_E_SHAPE: return "size out of range";
    case ULY_E_DIV_P: return "not divisible by the sequence-parallel degree";
    case ULY_E_GQA: return "query heads not a multiple of KV heads";
    case ULY_E_HEADDIM: return "unsupported head dim (64 or 128)";
    case ULY_E_STRIDE: return "token stride smaller than the row";
    case ULY_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case ULY_E_ALIAS: return "output overlaps an input";
    case ULY_E_HIP: return "HIP error";
    case ULY_E_SEQLENS: return "invalid cu_seqlens";
    case ULY_E_ALIGN: return "pointer or stride not 16-byte aligned";
    case ULY_E_SCRATCH: return "problem needs more than the static scratch buffer (ULY_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

const char *uly_last_error(void) { return g_last_error; }

int ulysses_shard_len(int64_t N, int32_t P, int64_t *n_local) {
  if (!n_local) return ULY_E_NULL;
  if (N <= 0 || P <= 0) return ULY_E_SHAPE;
  if (N % P != 0) return ULY_E_DIV_P;
  *n_local = N / P;
  return ULY_OK;
}

int ulysses_check_cu_seqlens(const int32_t *cu, int32_t n_seqs, int64_t N) {
  if (!cu) return ULY_E_NULL;
  if (n_seqs <= 0 || N <= 0) return ULY_E_SHAPE;
  if (cu[0] != 0 || (int64_t)cu[n_seqs] != N) return ULY_E_SEQLENS;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (cu[i + 1] <= cu[i]) return ULY_E_SEQLENS;
  return ULY_OK;
}

int ulysses_seq_to_head(const uint16_t *x_seq, uint16_t *x_send, int64_t n_local, int32_t P,
                        int32_t n_seg, const int32_t *seg_heads, int32_t d, hipStream_t stream) {
  int rc = check_swap(x_seq, x_send, n_local, P, n_seg, seg_heads, d);
  if (rc) return rc;
  return launch_swap(true, x_seq, x_send, n_local, P, n_seg, seg_heads, d, stream);
}

int ulysses_head_to_seq(const uint16_t *x_recv, uint16_t *x_seq, int64_t n_local, int32_t P,
                        int32_t n_seg, const int32_t *seg_heads, int32_t d, hipStream_t stream) {
  int rc = check_swap(x_recv, x_seq, n_local, P, n_seg, seg_heads, d);
  if (rc) return rc;
  return launch_swap(false, x_recv, x_seq, n_local, P, n_seg, seg_heads, d, stream);
}

size_t attn_fwd_workspace_bytes(int64_t N, int32_t hq, int32_t hkv, int32_t d) {
  (void)hq;
  if (N <= 0 || hkv <= 0 || d <= 0) return 0;
  return fwd_ws_bytes(N, hq, hkv, d);
}

int attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o, float *lse,
             int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride,
             int64_t v_stride, int64_t o_stride, float scale, int32_t causal, void *ws,
             size_t ws_bytes, hipStream_t stream) {
  return attn_fwd_impl(q, k, v, o, lse, N, hq, hkv, d, q_stride, k_stride, v_stride, o_stride,
                       scale, causal, nullptr, 0, ws, ws_bytes, stream);
}

int attn_fwd_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o,
                     float *lse, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride,
                     int64_t k_stride, int64_t v_stride, int64_t o_stride, float scale,
                     int32_t causal, hipStream_t stream) {
  return attn_fwd_impl(q, k, v, o, lse, N, hq, hkv, d, q_stride, k_stride, v_stride, o_stride,
                       scale, causal, nullptr, 0, nullptr, 0, stream, true);
}

int attn_fwd_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o,
                    float *lse, int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride,
                    int64_t k_stride, int64_t v_stride, int64_t o_stride, float scale,
                    int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs,
                    int32_t max_seqlen, void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_varlen_args(cu_seqlens, n_seqs, max_seqlen, N);
  if (rc) return rc;
  return attn_fwd_impl(q, k, v, o, lse, N, hq, hkv, d, q_stride, k_stride, v_stride, o_stride,
                       scale, causal, cu_seqlens, n_seqs, ws, ws_bytes, stream);
}

size_t attn_bwd_workspace_bytes(int64_t N, int32_t hq, int32_t hkv, int32_t d, int32_t n_seqs) {
  (void)n_seqs;
  if (N <= 0 || hq <= 0 || hkv <= 0 || d <= 0) return 0;
  return bwd_ws_layout(N, hq, hkv, d).total;
}

int attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
             const float *lse, const uint16_t *dout, uint16_t *dq, uint16_t *dk, uint16_t *dv,
             int64_t N, int32_t hq, int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride,
             int64_t v_stride, int64_t o_stride, int64_t do_stride, int64_t dq_stride,
             int64_t dk_stride, int64_t dv_stride, float scale, int32_t causal, void *ws,
             size_t ws_bytes, hipStream_t stream) {
  return attn_bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, N, hq, hkv, d, q_stride, k_stride,
                       v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale,
                       causal, nullptr, 0, ws, ws_bytes, 3, stream);
}

int attn_bwd_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
                    const float *lse, const uint16_t *dout, uint16_t *dq, uint16_t *dk,
                    uint16_t *dv, int64_t N, int32_t hq, int32_t hkv, int32_t d,
                    int64_t q_stride, int64_t k_stride, int64_t v_stride, int64_t o_stride,
                    int64_t do_stride, int64_t dq_stride, int64_t dk_stride, int64_t dv_stride,
                    float scale, int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs,
                    int32_t max_seqlen, void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_varlen_args(cu_seqlens, n_seqs, max_seqlen, N);
  if (rc) return rc;
  return attn_bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, N, hq, hkv, d, q_stride, k_stride,
                       v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale,
                       causal, cu_seqlens, n_seqs, ws, ws_bytes, 3, stream);
}

int attn_bwd_dq(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *o,
                const float *lse, const uint16_t *dout, uint16_t *dq, int64_t N, int32_t hq,
                int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                int64_t o_stride, int64_t do_stride, int64_t dq_stride, float scale,
                int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs, void *ws,
                size_t ws_bytes, hipStream_t stream) {
  if (cu_seqlens && (n_seqs <= 0 || n_seqs > N)) return ULY_E_SHAPE;
  return attn_bwd_impl(q, k, v, o, lse, dout, dq, nullptr, nullptr, N, hq, hkv, d, q_stride,
                       k_stride, v_stride, o_stride, do_stride, dq_stride, 0, 0, scale, causal,
                       cu_seqlens, n_seqs, ws, ws_bytes, 1, stream);
}

int attn_bwd_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *lse,
                  const uint16_t *dout, uint16_t *dk, uint16_t *dv, int64_t N, int32_t hq,
                  int32_t hkv, int32_t d, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                  int64_t do_stride, int64_t dk_stride, int64_t dv_stride, float scale,
                  int32_t causal, const int32_t *cu_seqlens, int32_t n_seqs, void *ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (cu_seqlens && (n_seqs <= 0 || n_seqs > N)) return ULY_E_SHAPE;
  return attn_bwd_impl(q, k, v, nullptr, lse, dout, nullptr, dk, dv, N, hq, hkv, d, q_stride,
                       k_stride, v_stride, 0, do_stride, 0, dk_stride, dv_stride, scale, causal,
                       cu_seqlens, n_seqs, ws, ws_bytes, 2, stream);
}

}  // extern "C"

namespace uly {
namespace {

int check_parts(int32_t n_parts, const void *const *parts, int64_t rows, int64_t width,
                int64_t part_stride) {
  if (!parts) return ULY_E_NULL;
  if (n_parts < 1 || n_parts > uly::kMaxParts) return ULY_E_SHAPE;
  if (rows <= 0 || width <= 0) return ULY_E_SHAPE;
  if (width % 8) return ULY_E_ALIGN;
  if (rows * (width / 8) >= (int64_t)1 << 31) return ULY_E_SHAPE;  // 32-bit vector index
  if (part_stride < width) return ULY_E_STRIDE;
  if (part_stride % 8) return ULY_E_ALIGN;
  for (int j = 0; j < n_parts; ++j) {
    if (!parts[j]) return ULY_E_NULL;
    if (!aligned16(parts[j])) return ULY_E_ALIGN;
  }
  return ULY_OK;
}

}  // namespace
}  // namespace uly

extern "C" int attn_lse_merge(int32_t n_parts, const uint16_t *const *o_parts,
                              const float *const *lse_parts, uint16_t *o_out, float *lse_out,
                              int64_t N, int32_t h, int32_t d, int64_t part_stride,
                              int64_t out_stride, hipStream_t stream) {
  using namespace uly;
  if (!lse_parts || !o_out || !lse_out) return ULY_E_NULL;
  if (h <= 0 || d <= 0) return ULY_E_SHAPE;
  const int64_t width = (int64_t)h * d;
  int rc = check_parts(n_parts, reinterpret_cast<const void *const *>(o_parts), N, width, part_stride);
  if (rc) return rc;
  if ((rc = check_out(o_out, N, out_stride, width))) return rc;
  if (reinterpret_cast<uintptr_t>(lse_out) & 3u) return ULY_E_ALIGN;
  const size_t ob = span_bytes(N, out_stride, width), lb = (size_t)N * h * 4;
  if (overlaps(o_out, ob, lse_out, lb)) return ULY_E_ALIAS;
  for (int j = 0; j < n_parts; ++j) {
    if (!lse_parts[j]) return ULY_E_NULL;
    if (reinterpret_cast<uintptr_t>(lse_parts[j]) & 3u) return ULY_E_ALIGN;
    const size_t pb = span_bytes(N, part_stride, width);
    if (overlaps(o_out, ob, o_parts[j], pb) || overlaps(o_out, ob, lse_parts[j], lb) ||
        overlaps(lse_out, lb, o_parts[j], pb) || overlaps(lse_out, lb, lse_parts[j], lb))
      return ULY_E_ALIAS;
  }
  return uly::launch_lse_merge(n_parts, o_parts, lse_parts, o_out, lse_out, N, h, d, part_stride,
                               out_stride, stream);
}

extern "C" int ring_grad_sum(int32_t n_parts, const uint16_t *const *parts, uint16_t *out,
                             int64_t rows, int32_t width, int64_t part_stride, int64_t out_stride,
                             hipStream_t stream) {
  using namespace uly;
  if (!out) return ULY_E_NULL;
  int rc = check_parts(n_parts, reinterpret_cast<const void *const *>(parts), rows, width, part_stride);
  if (rc) return rc;
  if ((rc = check_out(out, rows, out_stride, width))) return rc;
  const size_t ob = span_bytes(rows, out_stride, width);
  for (int j = 0; j < n_parts; ++j)
    if (overlaps(out, ob, parts[j], span_bytes(rows, part_stride, width))) return ULY_E_ALIAS;
  return uly::launch_grad_sum(n_parts, parts, out, rows, width, part_stride, out_stride, stream);
}

namespace uly {
namespace {

int check_logits(const void *logits, int64_t n, int64_t V, int64_t stride) {
  if (!logits) return ULY_E_NULL;
  if (n <= 0 || n >= ((int64_t)1 << 31) || V < 8 || V >= ((int64_t)1 << 31)) return ULY_E_SHAPE;
  if (V % 8) return ULY_E_ALIGN;
  if (stride < V) return ULY_E_STRIDE;
  if (stride % 8 || !aligned16(logits)) return ULY_E_ALIGN;
  return ULY_OK;
}

}  // namespace
}  // namespace uly

extern "C" int shifted_ce_fwd(const uint16_t *logits, const int32_t *labels, int64_t n, int64_t V,
                              int64_t stride, float *row_loss, float *row_lse, float *loss_out,
                              int32_t *good_out, hipStream_t stream) {
  using namespace uly;
  int rc = check_logits(logits, n, V, stride);
  if (rc) return rc;
  if (!labels || !row_loss || !row_lse || !loss_out || !good_out) return ULY_E_NULL;
  const size_t lb = span_bytes(n, stride, V), rb = (size_t)n * 4;
  if (overlaps(row_loss, rb, row_lse, rb) || overlaps(row_loss, rb, logits, lb) ||
      overlaps(row_lse, rb, logits, lb) || overlaps(row_loss, rb, labels, rb) || overlaps(row_lse, rb, labels, rb))
    return ULY_E_ALIAS;
  return launch_ce_fwd(logits, stride, labels, n, V, row_loss, row_lse, loss_out, good_out, stream);
}

extern "C" int sp_loss_aggregate(int32_t n_ranks, const float *const *rank_loss,
                                 const int32_t *const *rank_good, float *total_out,
                                 float *row_grad_scale_out, hipStream_t stream) {
  using namespace uly;
  if (!rank_loss || !rank_good || !total_out || !row_grad_scale_out) return ULY_E_NULL;
  if (n_ranks < 1 || n_ranks > kMaxParts) return ULY_E_SHAPE;
  for (int r = 0; r < n_ranks; ++r)
    if (!rank_loss[r] || !rank_good[r]) return ULY_E_NULL;
  if (total_out == row_grad_scale_out) return ULY_E_ALIAS;
  return launch_loss_aggregate(n_ranks, rank_loss, rank_good, total_out, row_grad_scale_out, stream);
}

extern "C" int shifted_ce_bwd(const uint16_t *logits, const int32_t *labels, const float *row_lse,
                              const float *row_grad_scale, int64_t n, int64_t V, int64_t stride,
                              uint16_t *dlogits, int64_t dstride, hipStream_t stream) {
  using namespace uly;
  int rc = check_logits(logits, n, V, stride);
  if (rc) return rc;
  if ((rc = check_logits(dlogits, n, V, dstride))) return rc;
  if (!labels || !row_lse || !row_grad_scale) return ULY_E_NULL;
  const bool in_place = (const void *)dlogits == (const void *)logits && dstride == stride;
  if (!in_place && overlaps(dlogits, span_bytes(n, dstride, V), logits, span_bytes(n, stride, V)))
    return ULY_E_ALIAS;
  return launch_ce_bwd(logits, stride, labels, row_lse, row_grad_scale, n, V, dlogits, dstride, stream);
}

extern "C" size_t tiled_mlp_workspace_bytes(int64_t tile, int32_t H, int32_t I) {
  if (tile <= 0 || H <= 0 || I <= 0) return 0;
  return uly::mlp_ws_layout(tile, H, I).total;
}

namespace uly {
namespace {

int check_mlp(const void *x, const void *w_gu, const void *w_down, int64_t n, int32_t H, int32_t I,
              int64_t tile, const void *ws, size_t ws_bytes) {
  if (!x || !w_gu || !w_down) return ULY_E_NULL;
  if (n <= 0 || H <= 0 || I <= 0 || tile <= 0) return ULY_E_SHAPE;
  if (H % 8 || I % 8) return ULY_E_ALIGN;
  if (n * H >= ((int64_t)1 << 40) || tile * I * 2 >= ((int64_t)1 << 31)) return ULY_E_SHAPE;
  if (!aligned16(x) || !aligned16(w_gu) || !aligned16(w_down)) return ULY_E_ALIGN;
  if (!ws || ws_bytes < mlp_ws_layout(tile, H, I).total || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return ULY_E_WORKSPACE;
  return ULY_OK;
}

}  // namespace
}  // namespace uly

extern "C" int tiled_mlp_fwd(const uint16_t *x, const uint16_t *w_gu, const uint16_t *w_down, uint16_t *y,
                             int64_t n, int32_t H, int32_t I, int64_t tile, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  using namespace uly;
  int rc = check_mlp(x, w_gu, w_down, n, H, I, tile, ws, ws_bytes);
  if (rc) return rc;
  if (!y) return ULY_E_NULL;
  if (!aligned16(y)) return ULY_E_ALIGN;
  const size_t xb = (size_t)n * H * 2, wgb = (size_t)2 * I * H * 2, wdb = (size_t)H * I * 2;
  const size_t wsb = mlp_ws_layout(tile, H, I).total;
  if (overlaps(y, xb, x, xb) || overlaps(y, xb, w_gu, wgb) || overlaps(y, xb, w_down, wdb) || overlaps(ws, wsb, y, xb) ||
      overlaps(ws, wsb, x, xb) || overlaps(ws, wsb, w_gu, wgb) || overlaps(ws, wsb, w_down, wdb))
    return ULY_E_ALIAS;
  MlpPtrs p{reinterpret_cast<const bf16_t *>(x), reinterpret_cast<const bf16_t *>(w_gu),
            reinterpret_cast<const bf16_t *>(w_down), nullptr, reinterpret_cast<bf16_t *>(y), nullptr, nullptr,
            nullptr, static_cast<char *>(ws)};
  return launch_mlp(false, p, n, H, I, tile, false, stream);
}

extern "C" int tiled_mlp_bwd(const uint16_t *x, const uint16_t *w_gu, const uint16_t *w_down, const uint16_t *dy,
                             uint16_t *dx, float *dw_gu, float *dw_down, int64_t n, int32_t H, int32_t I,
                             int64_t tile, int32_t accumulate, void *ws, size_t ws_bytes, hipStream_t stream) {
  using namespace uly;
  int rc = check_mlp(x, w_gu, w_down, n, H, I, tile, ws, ws_bytes);
  if (rc) return rc;
  if (!dy || !dx || !dw_gu || !dw_down) return ULY_E_NULL;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(dw_gu) || !aligned16(dw_down)) return ULY_E_ALIGN;
  const size_t xb = (size_t)n * H * 2, wgb = (size_t)2 * I * H * 2, wdb = (size_t)H * I * 2;
  const size_t gwg = (size_t)2 * I * H * 4, gwd = (size_t)H * I * 4;
  const size_t wsb = mlp_ws_layout(tile, H, I).total;
  const void *ins[4] = {x, w_gu, w_down, dy};
  const size_t inb[4] = {xb, wgb, wdb, xb};
  const void *outs[4] = {dx, dw_gu, dw_down, ws};
  const size_t outb[4] = {xb, gwg, gwd, wsb};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], outb[o], ins[i], inb[i])) return ULY_E_ALIAS;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o], outb[o], outs[o2], outb[o2])) return ULY_E_ALIAS;
  }
  MlpPtrs p{reinterpret_cast<const bf16_t *>(x), reinterpret_cast<const bf16_t *>(w_gu),
            reinterpret_cast<const bf16_t *>(w_down), reinterpret_cast<const bf16_t *>(dy), nullptr,
            reinterpret_cast<bf16_t *>(dx), dw_gu, dw_down, static_cast<char *>(ws)};
  return launch_mlp(true, p, n, H, I, tile, accumulate != 0, stream);
}
