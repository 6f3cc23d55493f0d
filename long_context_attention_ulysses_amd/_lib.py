"""ctypes binding of libulysses.so (C-ABI in include/ulysses.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch device tensors used as plain memory (data_ptr, strides);
the stream is torch's current HIP stream unless one is given. If the library
is not built this module raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libulysses.so")

ULY_OK = 0
STATUS = {
    -1: "ULY_E_NULL", -2: "ULY_E_SHAPE", -3: "ULY_E_DIV_P", -4: "ULY_E_GQA", -5: "ULY_E_HEADDIM",
    -6: "ULY_E_STRIDE", -7: "ULY_E_WORKSPACE", -8: "ULY_E_ALIAS", -9: "ULY_E_HIP",
    -10: "ULY_E_SEQLENS", -11: "ULY_E_ALIGN", -12: "ULY_E_SCRATCH",
}
CODE = {v: k for k, v in STATUS.items()}

if not os.path.exists(LIB_PATH):
    raise ImportError("libulysses.so is not built (run `python long_context_attention_ulysses_amd/build.py`"
                      " or __graft_entry__.build())")

# torch ships its own HIP runtime with the same soname as /opt/rocm's. Load it
# first so libulysses binds to that one runtime: device pointers and streams
# handed in from torch must belong to the runtime that launches the kernels.
import torch  # noqa: E402,F401

_L = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_SIGS = {
    "uly_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "uly_last_error": ([], ctypes.c_char_p),
    "ulysses_shard_len": ([_i64, _i32, ctypes.POINTER(_i64)], ctypes.c_int),
    "ulysses_check_cu_seqlens": ([ctypes.POINTER(_i32), _i32, _i64], ctypes.c_int),
    "ulysses_seq_to_head": ([_p, _p, _i64, _i32, _i32, ctypes.POINTER(_i32), _i32, _p], ctypes.c_int),
    "ulysses_head_to_seq": ([_p, _p, _i64, _i32, _i32, ctypes.POINTER(_i32), _i32, _p], ctypes.c_int),
    "attn_fwd": ([_p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _f32, _i32, _p, _sz,
                  _p], ctypes.c_int),
    "attn_fwd_varlen": ([_p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _f32, _i32,
                         _p, _i32, _i32, _p, _sz, _p], ctypes.c_int),
    "attn_fwd_noalloc": ([_p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _f32, _i32, _p],
                         ctypes.c_int),
    "attn_fwd_workspace_bytes": ([_i64, _i32, _i32, _i32], _sz),
    "attn_bwd_workspace_bytes": ([_i64, _i32, _i32, _i32, _i32], _sz),
    "attn_bwd": ([_p] * 9 + [_i64, _i32, _i32, _i32] + [_i64] * 8 + [_f32, _i32, _p, _sz, _p], ctypes.c_int),
    "attn_bwd_varlen": ([_p] * 9 + [_i64, _i32, _i32, _i32] + [_i64] * 8 + [_f32, _i32, _p, _i32, _i32, _p, _sz,
                                                                          _p], ctypes.c_int),
    "attn_bwd_dq": ([_p] * 7 + [_i64, _i32, _i32, _i32] + [_i64] * 6 + [_f32, _i32, _p, _i32, _p, _sz, _p],
                    ctypes.c_int),
    "attn_bwd_dkdv": ([_p] * 7 + [_i64, _i32, _i32, _i32] + [_i64] * 6 + [_f32, _i32, _p, _i32, _p, _sz, _p],
                      ctypes.c_int),
    "attn_lse_merge": ([_i32, ctypes.POINTER(_p), ctypes.POINTER(_p), _p, _p, _i64, _i32, _i32, _i64, _i64, _p],
                       ctypes.c_int),
    "ring_grad_sum": ([_i32, ctypes.POINTER(_p), _p, _i64, _i32, _i64, _i64, _p], ctypes.c_int),
    "shifted_ce_fwd": ([_p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p], ctypes.c_int),
    "sp_loss_aggregate": ([_i32, ctypes.POINTER(_p), ctypes.POINTER(_p), _p, _p, _p], ctypes.c_int),
    "shifted_ce_bwd": ([_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "tiled_mlp_workspace_bytes": ([_i64, _i32, _i32], _sz),
    "tiled_mlp_fwd": ([_p, _p, _p, _p, _i64, _i32, _i32, _i64, _p, _sz, _p], ctypes.c_int),
    "tiled_mlp_bwd": ([_p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i64, _i32, _p, _sz, _p], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_L, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class UlyssesError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        detail = _L.uly_status_string(status).decode()
        if status == CODE["ULY_E_HIP"]:
            detail += ": " + _L.uly_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, self.name, detail))


def raw():
    """The ctypes library handle (C names, C argument order)."""
    return _L


def _check(rc: int, where: str):
    if rc != ULY_OK:
        raise UlyssesError(rc, where)


def _stream(stream, device) -> int:
    """The given stream (a raw HIP stream handle or a torch stream), else
    torch's current stream on the tensors' device."""
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


_BITS16 = "bf16 bits (any 2-byte dtype)"


class _Args:
    """Checks the tensor arguments of one call for what the C interface
    cannot see: every tensor is on the same GPU (a host pointer handed to a
    kernel faults the device), has the element type the call reads, and,
    where the call takes no strides, the shape and contiguity it assumes.
    All checks run before the library is called."""

    def __init__(self, where: str):
        self.where = where
        self.device = None

    def __call__(self, t, name: str, kind=_BITS16, shape=None, contiguous: bool = False,
                 min_numel: int = 0) -> int:
        w = "%s: %s" % (self.where, name)
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % w)
        if not t.is_cuda:
            raise ValueError("%s must be on a GPU" % w)
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            raise ValueError("%s is on %s, the call's other tensors on %s" % (w, t.device, self.device))
        if kind is _BITS16:
            if t.element_size() != 2:
                raise ValueError("%s must hold %s, got %s" % (w, _BITS16, t.dtype))
        elif kind is not None and t.dtype != kind:
            raise ValueError("%s must be %s, got %s" % (w, kind, t.dtype))
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (w, tuple(shape), tuple(t.shape)))
        if contiguous and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % w)
        if t.numel() < min_numel:
            raise ValueError("%s needs at least %d elements" % (w, min_numel))
        return t.data_ptr()

    def opt(self, t, name: str, **kw) -> Optional[int]:
        return None if t is None else self(t, name, **kw)

    def rows(self, t, name: str, N: int, heads: int, d: int) -> int:
        """A [N, heads, d] view with unit element stride and head stride d
        (any token stride): its token stride."""
        self(t, name, shape=(N, heads, d))
        return _tok_stride(t, heads, d)

    def ws(self, t, name: str = "ws") -> int:
        if t is None:
            raise ValueError("%s: %s (device workspace) is required" % (self.where, name))
        self(t, name, kind=None, contiguous=True)
        return t.numel() * t.element_size()

    def cu(self, t, N: int) -> int:
        """cu_seqlens: contiguous int32 [n_seqs + 1] on the device; its values
        are not read here (ulysses_check_cu_seqlens checks a host copy)."""
        self(t, "cu_seqlens", kind=torch.int32, contiguous=True)
        if t.dim() != 1 or t.numel() < 2 or t.numel() - 1 > N:
            raise ValueError("%s: cu_seqlens must be 1-D with 2 to N + 1 entries" % self.where)
        return t.numel() - 1

    def stream(self, stream) -> int:
        return _stream(stream, self.device)


def status_string(status: int) -> str:
    return _L.uly_status_string(status).decode()


def ulysses_shard_len(N: int, P: int) -> int:
    out = _i64(0)
    _check(_L.ulysses_shard_len(N, P, ctypes.byref(out)), "ulysses_shard_len")
    return out.value


def ulysses_check_cu_seqlens(cu: Sequence[int], N: int) -> None:
    arr = (_i32 * len(cu))(*[int(x) for x in cu])
    _check(_L.ulysses_check_cu_seqlens(arr, len(cu) - 1, N), "ulysses_check_cu_seqlens")


def _seg(seg_heads):
    return (_i32 * len(seg_heads))(*[int(s) for s in seg_heads])


def _swap_shapes(where, x_seq, seg_heads):
    if x_seq.dim() != 3:
        raise ValueError("%s: the sequence-split tensor must be [n, H, d]" % where)
    n, H, d = x_seq.shape
    if sum(int(h) for h in seg_heads) != H:
        raise ValueError("%s: segments %s do not add up to H = %d" % (where, list(seg_heads), H))
    return n, H, d


def ulysses_seq_to_head(x_seq, x_send, P: int, seg_heads: Sequence[int], stream=None) -> None:
    """x_seq [n, H, d] -> x_send [P, n, H/P, d] (contiguous 16-bit tensors)."""
    a = _Args("ulysses_seq_to_head")
    n, H, d = _swap_shapes(a.where, x_seq, seg_heads)
    src = a(x_seq, "x_seq", contiguous=True)
    dst = a(x_send, "x_send", contiguous=True)
    if x_send.numel() != P * n * (H // P) * d:
        raise ValueError("ulysses_seq_to_head: x_send must hold P * n * (H/P) * d elements")
    _check(_L.ulysses_seq_to_head(src, dst, n, P, len(seg_heads), _seg(seg_heads), d, a.stream(stream)),
           "ulysses_seq_to_head")


def ulysses_head_to_seq(x_recv, x_seq, P: int, seg_heads: Sequence[int], stream=None) -> None:
    """x_recv [P, n, H/P, d] -> x_seq [n, H, d] (contiguous 16-bit tensors)."""
    a = _Args("ulysses_head_to_seq")
    n, H, d = _swap_shapes(a.where, x_seq, seg_heads)
    src = a(x_recv, "x_recv", contiguous=True)
    dst = a(x_seq, "x_seq", contiguous=True)
    if x_recv.numel() != P * n * (H // P) * d:
        raise ValueError("ulysses_head_to_seq: x_recv must hold P * n * (H/P) * d elements")
    _check(_L.ulysses_head_to_seq(src, dst, n, P, len(seg_heads), _seg(seg_heads), d, a.stream(stream)),
           "ulysses_head_to_seq")


def _tok_stride(t, heads, d):
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != d or t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError("expected a [N, heads, d] view with unit element stride and head stride d")
    return t.stride(0)


def attn_fwd_workspace_bytes(N: int, hq: int, hkv: int, d: int) -> int:
    return int(_L.attn_fwd_workspace_bytes(N, hq, hkv, d))


def _allocation_stream(handle: int, device):
    """Context under which torch's caching allocator hands out memory for
    work on stream `handle`: that stream itself. A block taken on another
    stream and freed when the call returns could go to that stream's next
    allocation while the kernels launched here still use it; a block taken
    on the stream the kernels run on is only reused by later work on the
    same stream, which runs after them."""
    if handle == torch.cuda.current_stream(device).cuda_stream:
        return contextlib.nullcontext()
    return torch.cuda.stream(torch.cuda.ExternalStream(handle, device=device))


def _workspace(nbytes: int, like, stream_handle: int):
    """Device memory for a workspace (torch's allocator; 256-byte aligned),
    allocated on the stream the call launches on."""
    with _allocation_stream(stream_handle, like.device):
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


def _qkv_dims(q, k):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [N, hq, d] and k, v [N, hkv, d]")
    N, hq, d = q.shape
    return N, hq, k.shape[1], d


def attn_fwd(q, k, v, o, lse, scale: float, causal: bool = True, cu_seqlens=None,
             max_seqlen: Optional[int] = None, ws=None, stream=None) -> None:
    """q [N, hq, d], k/v [N, hkv, d], o [N, hq, d] (views with any token stride);
    lse [hq, N] float32. cu_seqlens: int32 device tensor [n_seqs + 1] or None.
    ws: device buffer of at least attn_fwd_workspace_bytes(...) bytes (one is
    allocated when None)."""
    a = _Args("attn_fwd" if cu_seqlens is None else "attn_fwd_varlen")
    N, hq, hkv, d = _qkv_dims(q, k)
    strides = (a.rows(q, "q", N, hq, d), a.rows(k, "k", N, hkv, d), a.rows(v, "v", N, hkv, d),
               a.rows(o, "o", N, hq, d))
    a(lse, "lse", kind=torch.float32, shape=(hq, N), contiguous=True)
    n_seqs = a.cu(cu_seqlens, N) if cu_seqlens is not None else 0
    sh = a.stream(stream)
    if ws is None:
        ws = _workspace(attn_fwd_workspace_bytes(N, hq, hkv, d), q, sh)
    wsb = a.ws(ws)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), N, hq, hkv, d) + strides + (float(scale),
                                                                                        int(bool(causal)))
    if cu_seqlens is None:
        _check(_L.attn_fwd(*args, _ptr(ws), wsb, sh), "attn_fwd")
    else:
        _check(_L.attn_fwd_varlen(*args, _ptr(cu_seqlens), n_seqs, int(max_seqlen or N), _ptr(ws), wsb, sh),
               "attn_fwd_varlen")


# Bytes of the static scratch buffer attn_fwd_noalloc works in.
NOALLOC_SCRATCH_BYTES = 80 << 20


def attn_fwd_noalloc(q, k, v, o, lse, scale: float, causal: bool = True, stream=None) -> None:
    """attn_fwd in the library's static per-GPU scratch buffer: no workspace
    argument and no allocation (for callers that cannot allocate). Calls that
    may overlap on one GPU race on that buffer."""
    a = _Args("attn_fwd_noalloc")
    N, hq, hkv, d = _qkv_dims(q, k)
    strides = (a.rows(q, "q", N, hq, d), a.rows(k, "k", N, hkv, d), a.rows(v, "v", N, hkv, d),
               a.rows(o, "o", N, hq, d))
    a(lse, "lse", kind=torch.float32, shape=(hq, N), contiguous=True)
    _check(_L.attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), N, hq, hkv, d, *strides,
                               float(scale), int(bool(causal)), a.stream(stream)), "attn_fwd_noalloc")


def attn_bwd_workspace_bytes(N: int, hq: int, hkv: int, d: int, n_seqs: int = 1) -> int:
    return int(_L.attn_bwd_workspace_bytes(N, hq, hkv, d, n_seqs))


def _bwd_args(a, q, k, v, o, lse, dout, N, hq, hkv, d):
    """Pointers and token strides of the inputs every backward call reads."""
    st = (a.rows(q, "q", N, hq, d), a.rows(k, "k", N, hkv, d), a.rows(v, "v", N, hkv, d))
    st_o = a.rows(o, "o", N, hq, d) if o is not None else None
    st_do = a.rows(dout, "dout", N, hq, d)
    a(lse, "lse", kind=torch.float32, shape=(hq, N), contiguous=True)
    return st, st_o, st_do


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale: float, causal: bool = True, ws=None,
             cu_seqlens=None, max_seqlen: Optional[int] = None, stream=None) -> None:
    """Gradients for attn_fwd with the same q, k, v, scale, mask. ws: device
    buffer of at least attn_bwd_workspace_bytes(...) bytes, 256-byte aligned."""
    a = _Args("attn_bwd" if cu_seqlens is None else "attn_bwd_varlen")
    N, hq, hkv, d = _qkv_dims(q, k)
    st, st_o, st_do = _bwd_args(a, q, k, v, o, lse, dout, N, hq, hkv, d)
    st_g = (a.rows(dq, "dq", N, hq, d), a.rows(dk, "dk", N, hkv, d), a.rows(dv, "dv", N, hkv, d))
    n_seqs = a.cu(cu_seqlens, N) if cu_seqlens is not None else 1
    sh = a.stream(stream)
    if ws is None:
        ws = _workspace(attn_bwd_workspace_bytes(N, hq, hkv, d, n_seqs), q, sh)
    ws_bytes = a.ws(ws)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            N, hq, hkv, d) + st + (st_o, st_do) + st_g + (float(scale), int(bool(causal)))
    if cu_seqlens is None:
        _check(_L.attn_bwd(*args, _ptr(ws), ws_bytes, sh), "attn_bwd")
    else:
        _check(_L.attn_bwd_varlen(*args, _ptr(cu_seqlens), n_seqs, int(max_seqlen or N), _ptr(ws), ws_bytes, sh),
               "attn_bwd_varlen")


def attn_bwd_dq(q, k, v, o, lse, dout, dq, scale: float, causal: bool = True, ws=None, cu_seqlens=None,
                stream=None) -> None:
    """First step of attn_bwd: -D, D = rowsum(dout * o), and LSE*log2(e) into ws
    (with, at d = 64, the transposed copies and, over packed documents, both
    steps' block orders), and dq."""
    a = _Args("attn_bwd_dq")
    N, hq, hkv, d = _qkv_dims(q, k)
    st, st_o, st_do = _bwd_args(a, q, k, v, o, lse, dout, N, hq, hkv, d)
    st_dq = a.rows(dq, "dq", N, hq, d)
    n_seqs = a.cu(cu_seqlens, N) if cu_seqlens is not None else 0
    ws_bytes = a.ws(ws)
    _check(_L.attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), N, hq, hkv, d,
                          *st, st_o, st_do, st_dq, float(scale), int(bool(causal)), _ptr(cu_seqlens), n_seqs,
                          _ptr(ws), ws_bytes, a.stream(stream)), "attn_bwd_dq")


def attn_bwd_dkdv(q, k, v, lse, dout, dk, dv, scale: float, causal: bool = True, ws=None, cu_seqlens=None,
                  stream=None) -> None:
    """Second step of attn_bwd: dk and dv, reading -D, LSE, the transposed
    copies and the key-block order from ws (left there by attn_bwd_dq) and
    overwriting ws's dK/dV partial region (so concurrent calls need their own
    ws)."""
    a = _Args("attn_bwd_dkdv")
    N, hq, hkv, d = _qkv_dims(q, k)
    st, _, st_do = _bwd_args(a, q, k, v, None, lse, dout, N, hq, hkv, d)
    st_kv = (a.rows(dk, "dk", N, hkv, d), a.rows(dv, "dv", N, hkv, d))
    n_seqs = a.cu(cu_seqlens, N) if cu_seqlens is not None else 0
    ws_bytes = a.ws(ws)
    _check(_L.attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dk), _ptr(dv), N, hq, hkv, d,
                            *st, st_do, *st_kv, float(scale), int(bool(causal)), _ptr(cu_seqlens), n_seqs,
                            _ptr(ws), ws_bytes, a.stream(stream)), "attn_bwd_dkdv")


def _ptr_array(ptrs):
    return (_p * len(ptrs))(*ptrs)


def attn_lse_merge(o_parts, lse_parts, o_out, lse_out, stream=None) -> None:
    """Merge per-block attention results (ring attention): o_parts are
    [N, h, d] views with one common token stride, lse_parts [h, N] float32;
    o_out [N, h, d], lse_out [h, N]."""
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("need as many lse parts as o parts, at least one")
    a = _Args("attn_lse_merge")
    if o_out.dim() != 3:
        raise ValueError("attn_lse_merge: o_out must be [N, h, d]")
    N, h, d = o_out.shape
    strides = {a.rows(t, "o_parts[%d]" % i, N, h, d) for i, t in enumerate(o_parts)}
    if len(strides) != 1:
        raise ValueError("o parts must share one token stride")
    lp = [a(t, "lse_parts[%d]" % i, kind=torch.float32, shape=(h, N), contiguous=True)
          for i, t in enumerate(lse_parts)]
    op = [t.data_ptr() for t in o_parts]
    out_stride = a.rows(o_out, "o_out", N, h, d)
    a(lse_out, "lse_out", kind=torch.float32, shape=(h, N), contiguous=True)
    _check(_L.attn_lse_merge(len(o_parts), _ptr_array(op), _ptr_array(lp), _ptr(o_out), _ptr(lse_out), N, h, d,
                             strides.pop(), out_stride, a.stream(stream)), "attn_lse_merge")


def ring_grad_sum(parts, out, stream=None) -> None:
    """out = sum of parts (bf16 [rows, heads, d] views with one common token
    stride), accumulated in float32."""
    if not parts:
        raise ValueError("need at least one part")
    a = _Args("ring_grad_sum")
    if out.dim() != 3:
        raise ValueError("ring_grad_sum: out must be [rows, heads, d]")
    rows, heads, d = out.shape
    strides = {a.rows(t, "parts[%d]" % i, rows, heads, d) for i, t in enumerate(parts)}
    if len(strides) != 1:
        raise ValueError("parts must share one token stride")
    out_stride = a.rows(out, "out", rows, heads, d)
    _check(_L.ring_grad_sum(len(parts), _ptr_array([t.data_ptr() for t in parts]), _ptr(out), rows, heads * d,
                            strides.pop(), out_stride, a.stream(stream)), "ring_grad_sum")


def _row_stride(t, V):
    if t.dim() != 2 or t.shape[1] != V or t.stride(1) != 1:
        raise ValueError("expected an [n, V] view with unit element stride")
    return t.stride(0)


def shifted_ce_fwd(logits, labels, row_loss, row_lse, loss_out, good_out, stream=None) -> None:
    """Per-rank loss from pre-shifted labels: logits [n, V] bf16 bits,
    labels [n] int32 (-100 = no loss); outputs row_loss, row_lse [n] float32,
    loss_out [1] float32 (mean over good rows), good_out [1] int32."""
    a = _Args("shifted_ce_fwd")
    if logits.dim() != 2:
        raise ValueError("shifted_ce_fwd: logits must be [n, V]")
    n, V = logits.shape
    a(logits, "logits")
    a(labels, "labels", kind=torch.int32, shape=(n,), contiguous=True)
    a(row_loss, "row_loss", kind=torch.float32, shape=(n,), contiguous=True)
    a(row_lse, "row_lse", kind=torch.float32, shape=(n,), contiguous=True)
    a(loss_out, "loss_out", kind=torch.float32, min_numel=1)
    a(good_out, "good_out", kind=torch.int32, min_numel=1)
    _check(_L.shifted_ce_fwd(_ptr(logits), _ptr(labels), n, V, _row_stride(logits, V), _ptr(row_loss),
                             _ptr(row_lse), _ptr(loss_out), _ptr(good_out), a.stream(stream)), "shifted_ce_fwd")


def sp_loss_aggregate(rank_losses, rank_goods, total_out, row_grad_scale_out, stream=None) -> None:
    """sum_r loss_r * good_r / max(sum_r good_r, 1) over the ranks' device
    scalars, and the per-row gradient scale 1 / max(sum_r good_r, 1)."""
    if len(rank_losses) != len(rank_goods) or not rank_losses:
        raise ValueError("need one good count per rank loss, at least one rank")
    a = _Args("sp_loss_aggregate")
    lp = [a(t, "rank_losses[%d]" % i, kind=torch.float32, min_numel=1) for i, t in enumerate(rank_losses)]
    gp = [a(t, "rank_goods[%d]" % i, kind=torch.int32, min_numel=1) for i, t in enumerate(rank_goods)]
    a(total_out, "total_out", kind=torch.float32, min_numel=1)
    a(row_grad_scale_out, "row_grad_scale_out", kind=torch.float32, min_numel=1)
    _check(_L.sp_loss_aggregate(len(rank_losses), _ptr_array(lp), _ptr_array(gp), _ptr(total_out),
                                _ptr(row_grad_scale_out), a.stream(stream)), "sp_loss_aggregate")


def shifted_ce_bwd(logits, labels, row_lse, row_grad_scale, dlogits, stream=None) -> None:
    """Gradient of the aggregate loss with respect to one rank's logits
    (dlogits may be logits itself)."""
    a = _Args("shifted_ce_bwd")
    if logits.dim() != 2:
        raise ValueError("shifted_ce_bwd: logits must be [n, V]")
    n, V = logits.shape
    a(logits, "logits")
    a(labels, "labels", kind=torch.int32, shape=(n,), contiguous=True)
    a(row_lse, "row_lse", kind=torch.float32, shape=(n,), contiguous=True)
    a(row_grad_scale, "row_grad_scale", kind=torch.float32, min_numel=1)
    a(dlogits, "dlogits", shape=(n, V))
    _check(_L.shifted_ce_bwd(_ptr(logits), _ptr(labels), _ptr(row_lse), _ptr(row_grad_scale), n, V,
                             _row_stride(logits, V), _ptr(dlogits), _row_stride(dlogits, V), a.stream(stream)),
           "shifted_ce_bwd")


def tiled_mlp_workspace_bytes(tile: int, H: int, I: int) -> int:
    return int(_L.tiled_mlp_workspace_bytes(tile, H, I))


def tiled_mlp_fwd(x, w_gu, w_down, y, tile: int, ws=None, stream=None) -> None:
    """y [n, H] = SwiGLU MLP of x [n, H] with w_gu [2I, H], w_down [H, I]
    (bf16 bits), over token tiles of `tile`."""
    a = _Args("tiled_mlp_fwd")
    if x.dim() != 2 or w_down.dim() != 2:
        raise ValueError("tiled_mlp_fwd: x must be [n, H] and w_down [H, I]")
    n, H = x.shape
    I = w_down.shape[1]
    for t, nm, sh in ((x, "x", (n, H)), (w_gu, "w_gu", (2 * I, H)), (w_down, "w_down", (H, I)), (y, "y", (n, H))):
        a(t, nm, shape=sh, contiguous=True)
    sh = a.stream(stream)
    if ws is None:
        ws = _workspace(tiled_mlp_workspace_bytes(tile, H, I), x, sh)
    wsb = a.ws(ws)
    _check(_L.tiled_mlp_fwd(_ptr(x), _ptr(w_gu), _ptr(w_down), _ptr(y), n, H, I, tile, _ptr(ws), wsb, sh),
           "tiled_mlp_fwd")


def tiled_mlp_bwd(x, w_gu, w_down, dy, dx, dw_gu, dw_down, tile: int, accumulate: bool = False, ws=None,
                  stream=None) -> None:
    """dx [n, H] (bf16) and the float32 weight gradients dw_gu [2I, H],
    dw_down [H, I] of the SwiGLU MLP, recomputing each tile's activations."""
    a = _Args("tiled_mlp_bwd")
    if x.dim() != 2 or w_down.dim() != 2:
        raise ValueError("tiled_mlp_bwd: x must be [n, H] and w_down [H, I]")
    n, H = x.shape
    I = w_down.shape[1]
    for t, nm, sh in ((x, "x", (n, H)), (w_gu, "w_gu", (2 * I, H)), (w_down, "w_down", (H, I)), (dy, "dy", (n, H)),
                      (dx, "dx", (n, H))):
        a(t, nm, shape=sh, contiguous=True)
    a(dw_gu, "dw_gu", kind=torch.float32, shape=(2 * I, H), contiguous=True)
    a(dw_down, "dw_down", kind=torch.float32, shape=(H, I), contiguous=True)
    sh = a.stream(stream)
    if ws is None:
        ws = _workspace(tiled_mlp_workspace_bytes(tile, H, I), x, sh)
    wsb = a.ws(ws)
    _check(_L.tiled_mlp_bwd(_ptr(x), _ptr(w_gu), _ptr(w_down), _ptr(dy), _ptr(dx), _ptr(dw_gu), _ptr(dw_down), n,
                            H, I, tile, int(bool(accumulate)), _ptr(ws), wsb, sh), "tiled_mlp_bwd")
