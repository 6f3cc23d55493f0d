"""fp64 CPU oracle for one rank's share of Ulysses sequence parallelism.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path never imports it. It shares no
code with the HIP library (it compiles its own C source, ``oracle.c``, with
gcc + OpenMP into ``liboracle.so`` next to this file).

Functions (each a plain restatement of what the pages describe; the C file
carries the citations):
  seq_to_head / head_to_seq   the local pack/unpack around the all-to-all
  exchange                    the all-to-all itself, as buffer re-indexing
  attn_fwd                    softmax attention, causal and/or packed docs
  attn_bwd                    its textbook gradient
  lse_merge                   ring attention: softmax over the union of
                              disjoint key blocks from per-block results
  shift_labels / shifted_ce / sp_loss_aggregate / shifted_ce_grad
                              the per-rank loss from pre-shifted labels and
                              its weighted aggregation over the SP ranks
  swiglu_mlp / swiglu_mlp_bwd the MLP that TiledMLP runs over token tiles
                              (here untiled: tiling changes memory, not
                              the result)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        for name in ("orc_seq_to_head", "orc_head_to_seq"):
            f = getattr(L, name)
            f.argtypes = [u16p, u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p, ctypes.c_int32]
            f.restype = None
        L.orc_attn_fwd.argtypes = [f64p, f64p, f64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_double, ctypes.c_int32, i32p, ctypes.c_int32,
                                   i64p, ctypes.c_int64, f64p, f64p]
        L.orc_attn_fwd.restype = ctypes.c_int
        L.orc_attn_bwd.argtypes = [f64p, f64p, f64p, f64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_double, ctypes.c_int32, i32p, ctypes.c_int32,
                                   i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, f64p, f64p, f64p]
        L.orc_attn_bwd.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.POINTER(ctype)()
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns: the 16 bits are the top half of an
    IEEE binary32 whose low half is zero."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return np.ascontiguousarray(a, dtype=np.float64)


# ------------------------------------------------------------------ O1 ----

def seq_to_head(x_seq: np.ndarray, P: int, seg_heads: Sequence[int]) -> np.ndarray:
    """x_seq [n, H, d] (uint16 bits) -> send [P, n, H/P, d]."""
    x = np.ascontiguousarray(x_seq, dtype=np.uint16)
    n, H, d = x.shape
    assert H == sum(seg_heads) and all(s % P == 0 for s in seg_heads)
    out = np.empty((P, n, H // P, d), dtype=np.uint16)
    seg = np.asarray(seg_heads, dtype=np.int32)
    lib().orc_seq_to_head(_ptr(x, ctypes.c_uint16), _ptr(out, ctypes.c_uint16), n, P, len(seg),
                          _ptr(seg, ctypes.c_int32), d)
    return out


def head_to_seq(recv: np.ndarray, P: int, seg_heads: Sequence[int]) -> np.ndarray:
    """recv [P, n, H/P, d] (uint16 bits) -> x_seq [n, H, d]."""
    x = np.ascontiguousarray(recv, dtype=np.uint16)
    P_, n, h, d = x.shape
    assert P_ == P and h * P == sum(seg_heads)
    out = np.empty((n, h * P, d), dtype=np.uint16)
    seg = np.asarray(seg_heads, dtype=np.int32)
    lib().orc_head_to_seq(_ptr(x, ctypes.c_uint16), _ptr(out, ctypes.c_uint16), n, P, len(seg),
                          _ptr(seg, ctypes.c_int32), d)
    return out


def exchange(sends: Sequence[np.ndarray]) -> list:
    """The all-to-all as re-indexing: recv_r[s] = send_s[r] for P ranks.
    sends[s] is rank s's [P, n, h, d] send buffer; returns the P receive
    buffers, each [P, n, h, d] with source ranks in token order."""
    P = len(sends)
    return [np.stack([sends[s][r] for s in range(P)]) for r in range(P)]


# ------------------------------------------------------------- O2 / O3 ----

def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = True,
             cu: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None
             ) -> Tuple[np.ndarray, np.ndarray]:
    """q [N, hq, d], k/v [N, hkv, d] (bf16 bits or floats) -> (o [R, hq, d], lse [hq, R])
    for the query rows ``rows`` (all N if None), in fp64."""
    qd, kd, vd = _as_f64(q), _as_f64(k), _as_f64(v)
    N, hq, d = qd.shape
    hkv = kd.shape[1]
    cu_a = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = N if rows_a is None else len(rows_a)
    o = np.empty((R, hq, d), dtype=np.float64)
    lse = np.empty((hq, R), dtype=np.float64)
    rc = lib().orc_attn_fwd(_ptr(qd, ctypes.c_double), _ptr(kd, ctypes.c_double), _ptr(vd, ctypes.c_double),
                            N, hq, hkv, d, float(scale), int(bool(causal)), _ptr(cu_a, ctypes.c_int32),
                            0 if cu_a is None else len(cu_a) - 1, _ptr(rows_a, ctypes.c_int64), R,
                            _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("orc_attn_fwd failed: %d" % rc)
    return o, lse


def attn_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float,
             causal: bool = True, cu: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None,
             key_lo: int = 0, key_hi: Optional[int] = None, want_dq: bool = True, want_dkv: bool = True
             ) -> Tuple[Optional[np.ndarray], Optional[np.ndarray], Optional[np.ndarray]]:
    """Gradients of L = sum(dout * O): dq [R, hq, d] for ``rows``; dk, dv
    [key_hi - key_lo, hkv, d] for keys [key_lo, key_hi). fp64."""
    qd, kd, vd, dod = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    N, hq, d = qd.shape
    hkv = kd.shape[1]
    key_hi = N if key_hi is None else key_hi
    cu_a = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = N if rows_a is None else len(rows_a)
    dq = np.empty((R, hq, d), dtype=np.float64) if want_dq else None
    dk = np.empty((key_hi - key_lo, hkv, d), dtype=np.float64) if want_dkv else None
    dv = np.empty((key_hi - key_lo, hkv, d), dtype=np.float64) if want_dkv else None
    rc = lib().orc_attn_bwd(_ptr(qd, ctypes.c_double), _ptr(kd, ctypes.c_double), _ptr(vd, ctypes.c_double),
                            _ptr(dod, ctypes.c_double), N, hq, hkv, d, float(scale), int(bool(causal)),
                            _ptr(cu_a, ctypes.c_int32), 0 if cu_a is None else len(cu_a) - 1,
                            _ptr(rows_a, ctypes.c_int64), R, key_lo, key_hi,
                            _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("orc_attn_bwd failed: %d" % rc)
    return dq, dk, dv


# ------------------------------------------------------------------ O4 ----

def lse_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Ring attention ("Sequence Parallelism for Long-Context AI Training",
    "Advanced Scaling: Ring Attention and Ulysses": each GPU attends its own
    queries to one key/value block at a time as the blocks travel a ring).
    Part j is attention over block j's keys only: o_j [N, h, d] and natural
    log lse_j [h, N]. With the key blocks disjoint, the softmax over all of
    them is, by the definition of softmax:
        lse = log sum_j exp(lse_j)
        o   = sum_j exp(lse_j - lse) o_j
    (the max is taken out of the sum so that nothing overflows). A row that is
    -inf in every part has no keys: o = 0, lse = -inf. fp64."""
    L = [np.asarray(l, dtype=np.float64) for l in lse_parts]
    O = [np.asarray(o, dtype=np.float64) for o in o_parts]
    m = L[0].copy()
    for l in L[1:]:
        m = np.maximum(m, l)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    total = np.zeros_like(m)
    for l in L:
        total += np.exp(l - m_safe)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    o = np.zeros_like(O[0])
    for l, oj in zip(L, O):
        w = np.where(empty, 0.0, np.exp(l - np.where(empty, 0.0, lse)))  # [h, N]
        o += w.T[:, :, None] * oj
    return o, lse


# ------------------------------------------------------------------ O5 ----
# "Deepspeed Ulysses/ALST integration", opening post, step 2: each rank
# computes the loss of its token shard from shift_labels (-100 = no loss);
# the ranks' losses are combined as sum_r loss_r * good_r / max(sum_r good_r,
# 1), good_r = the rank's count of labels != -100. "Ulysses sequence
# parallelism", Configure: labels are shifted before sharding.

IGNORE = -100


def shift_labels(labels: np.ndarray) -> np.ndarray:
    """Pre-shifted labels of a whole sequence: position i is trained to
    predict token i+1, so its label is labels[i+1]; the last position has
    none (-100)."""
    lab = np.asarray(labels, dtype=np.int64)
    out = np.full(lab.shape, IGNORE, dtype=np.int64)
    out[:-1] = lab[1:]
    return out


def shifted_ce(logits: np.ndarray, labels: np.ndarray) -> Tuple[np.ndarray, np.ndarray, float, int]:
    """One rank: logits [n, V] (bf16 bits or floats), labels [n].
    Returns (row_loss [n], row_lse [n], rank mean loss, good count), fp64.
    Row loss = log sum_v exp(logit_v) - logit_y for labels in [0, V), 0 for
    the others; the rank's loss is the mean over good rows (0 if none)."""
    x = _as_f64(logits)
    lab = np.asarray(labels, dtype=np.int64)
    n, V = x.shape
    row_lse = np.empty(n)
    row_loss = np.zeros(n)
    good = 0
    for r in range(n):
        m = np.max(x[r])
        row_lse[r] = m + np.log(np.sum(np.exp(x[r] - m)))
        if 0 <= lab[r] < V:
            row_loss[r] = row_lse[r] - x[r, lab[r]]
            good += 1
    loss = float(np.sum(row_loss) / good) if good else 0.0
    return row_loss, row_lse, loss, good


def sp_loss_aggregate(rank_losses: Sequence[float], rank_goods: Sequence[int]) -> float:
    """sum_r loss_r * good_r / max(sum_r good_r, 1)."""
    total = 0.0
    for l, g in zip(rank_losses, rank_goods):
        total += float(l) * int(g)
    return total / max(int(sum(int(g) for g in rank_goods)), 1)


def shifted_ce_grad(logits: np.ndarray, labels: np.ndarray, total_good: int) -> np.ndarray:
    """Gradient of the aggregate with respect to one rank's logits:
    (softmax(row) - onehot(y)) / max(G, 1) for good rows, 0 otherwise."""
    x = _as_f64(logits)
    lab = np.asarray(labels, dtype=np.int64)
    n, V = x.shape
    g = np.zeros_like(x)
    for r in range(n):
        if 0 <= lab[r] < V:
            p = np.exp(x[r] - np.max(x[r]))
            p /= np.sum(p)
            p[lab[r]] -= 1.0
            g[r] = p / max(int(total_good), 1)
    return g


# ------------------------------------------------------------------ O6 ----
# TiledMLP ("Ulysses sequence parallelism", intro note on ALST; "Ulysses
# Sequence Parallelism for Million-Token Context Training", Additional
# Kernels: named only). The plainest reading: the model's SwiGLU MLP, applied
# to every token; processing the tokens in tiles only bounds the memory of
# the intermediates. Weights in nn.Linear layout [out][in]; w_gu stacks the
# gate rows over the up rows.

def _silu_parts(g: np.ndarray):
    s = 1.0 / (1.0 + np.exp(-g))
    return s, g * s


def swiglu_mlp(x: np.ndarray, w_gu: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T, fp64. x [n, H], w_gu [2I, H], w_down [H, I]."""
    xd, wgu, wd = _as_f64(x), _as_f64(w_gu), _as_f64(w_down)
    I = wd.shape[1]
    g = xd @ wgu[:I].T
    u = xd @ wgu[I:].T
    _, silu = _silu_parts(g)
    return (silu * u) @ wd.T


def swiglu_mlp_bwd(x: np.ndarray, w_gu: np.ndarray, w_down: np.ndarray, dy: np.ndarray):
    """Gradients of sum(dy * y): (dx [n, H], dw_gu [2I, H], dw_down [H, I]), fp64.
    With s = sigmoid(g): da = dy Wd; dWd = dy^T a; du = da silu(g);
    dg = da u s (1 + g (1 - s)); dx = [dg | du] W_gu; dW_gu = [dg | du]^T x."""
    xd, wgu, wd, dyd = _as_f64(x), _as_f64(w_gu), _as_f64(w_down), _as_f64(dy)
    I = wd.shape[1]
    g = xd @ wgu[:I].T
    u = xd @ wgu[I:].T
    s, silu = _silu_parts(g)
    a = silu * u
    da = dyd @ wd
    dw_down = dyd.T @ a
    du = da * silu
    dg = da * u * s * (1.0 + g * (1.0 - s))
    dgu = np.concatenate([dg, du], axis=1)
    return dgu @ wgu, dgu.T @ xd, dw_down
