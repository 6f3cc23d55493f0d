"""GPU parity of attention forward/backward against the fp64 oracle, plus
invariants checked on the GPU results themselves (determinism, causality,
head-shard concatenation, single-document varlen == dense)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import uniform_scores
from tests._gpu import (FWD_MAX_ABS, FWD_REL, GRAD_MAX_ABS, GRAD_REL, LSE_MAX_ABS, assert_close, dev,
                        f64, host, sentinel)

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")


# Keys at the end of the sequence whose dK/dV the sampled tests compare with
# the oracle (only the query rows in that tail see them).
TAIL_KEYS = 512


class Run:
    """One attention problem on the GPU with q|k|v fused along the head axis
    ([N, hq + 2 hkv, d], the head shard the all-to-all delivers) and
    dq|dk|dv written into one fused gradient buffer."""

    def __init__(self, qkv_bits, hq, hkv, scale, causal=True, cu=None):
        self.N, ht, self.d = qkv_bits.shape
        assert ht == hq + 2 * hkv
        self.hq, self.hkv, self.scale, self.causal = hq, hkv, scale, causal
        self.cu = cu
        self.qkv = dev(qkv_bits)
        self.q = self.qkv[:, :hq]
        self.k = self.qkv[:, hq:hq + hkv]
        self.v = self.qkv[:, hq + hkv:]
        self.cu_dev = None if cu is None else torch.tensor(np.asarray(cu, dtype=np.int32), device="cuda")
        self.max_seqlen = None if cu is None else int(np.max(np.diff(cu)))

    def fwd(self):
        self.o = sentinel((self.N, self.hq, self.d))
        self.lse = torch.full((self.hq, self.N), float("nan"), dtype=torch.float32, device="cuda")
        uly.attn_fwd(self.q, self.k, self.v, self.o, self.lse, self.scale, self.causal, self.cu_dev,
                     self.max_seqlen)
        torch.cuda.synchronize()
        return host(self.o), self.lse.cpu().numpy()

    def bwd(self, dy_bits):
        self.dy = dev(dy_bits)
        dqkv = sentinel((self.N, self.hq + 2 * self.hkv, self.d))
        dq, dk, dv = dqkv[:, :self.hq], dqkv[:, self.hq:self.hq + self.hkv], dqkv[:, self.hq + self.hkv:]
        nb = uly.attn_bwd_workspace_bytes(self.N, self.hq, self.hkv, self.d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        uly.attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.dy, dq, dk, dv, self.scale, self.causal, ws,
                     self.cu_dev, self.max_seqlen)
        torch.cuda.synchronize()
        b = host(dqkv)
        return b[:, :self.hq], b[:, self.hq:self.hq + self.hkv], b[:, self.hq + self.hkv:]


def _split(qkv_bits, hq, hkv):
    return qkv_bits[:, :hq], qkv_bits[:, hq:hq + hkv], qkv_bits[:, hq + hkv:]


def _check_full(qkv, dy, hq, hkv, scale, causal, cu, tag):
    r = Run(qkv, hq, hkv, scale, causal, cu)
    o, lse = r.fwd()
    q, k, v = _split(qkv, hq, hkv)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, causal, cu)
    assert_close(tag + " O", oracle.bf16_to_f64(o), o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close(tag + " LSE", lse.astype(np.float64), lse_ref, LSE_MAX_ABS, 1.0)
    dq, dk, dv = r.bwd(dy)
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dy, scale, causal, cu)
    assert_close(tag + " dQ", oracle.bf16_to_f64(dq), dq_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close(tag + " dK", oracle.bf16_to_f64(dk), dk_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close(tag + " dV", oracle.bf16_to_f64(dv), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    return r


SMALL = [
    # N, hq, hkv, d, causal, cu, sigma
    (256, 2, 1, 64, True, None, 1.0),
    (1, 2, 1, 64, True, None, 1.0),
    (33, 4, 2, 128, True, None, 0.5),
    (300, 4, 2, 128, True, None, 0.5),
    (1000, 8, 2, 128, True, None, 0.5),
    (517, 4, 4, 64, False, None, 1.0),
    (777, 3, 1, 128, True, None, 0.5),
    (640, 4, 2, 128, True, [0, 1, 2, 100, 101, 350, 640], 0.5),
    (700, 2, 1, 64, False, [0, 64, 65, 300, 700], 1.0),
    (1536, 8, 2, 128, True, None, 0.5),
    (64, 2, 2, 128, True, None, 0.5),                               # exactly one tile, G = 1
    (65, 8, 1, 128, True, None, 0.5),                               # one row past a tile, G = 8
    (129, 6, 2, 64, True, None, 1.0),                               # G = 3, d = 64
    (200, 4, 1, 128, True, [0, 1, 2, 3, 67, 130, 131, 200], 0.5),  # one-token documents
    (300, 4, 1, 128, False, None, 0.5),                             # non-causal, d = 128, G = 4
    (384, 8, 2, 128, False, [0, 100, 101, 384], 0.5),               # non-causal documents, d = 128
]


@pytest.mark.parametrize("N,hq,hkv,d,causal,cu,sigma", SMALL)
def test_attention_small_full_oracle(N, hq, hkv, d, causal, cu, sigma):
    print("attn N=%d hq=%d hkv=%d d=%d causal=%d docs=%s" % (N, hq, hkv, d, causal, cu), flush=True)
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=N * 7 + hq, sigma=sigma)
    dy = workloads.normal_bf16((N, hq, d), seed=N * 11 + d)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    _check_full(qkv, dy, hq, hkv, 1.0 / np.sqrt(d), causal, cu_a, "N=%d" % N)


def test_tiny_workload_full_ulysses_layer():
    """The whole tiny layer on the GPU: seq->head pack on both simulated ranks,
    exchange, attention fwd/bwd per rank, head->seq unpack; compared with the
    oracle's full-head attention in sequence layout."""
    w = workloads.WORKLOADS["tiny"]
    X = workloads.gen_x(w, range(w.Ht))
    dY = workloads.gen_dy(w, range(w.Hq))
    Q, K, V = X[:, :w.Hq], X[:, w.Hq:w.Hq + w.Hkv], X[:, w.Hq + w.Hkv:]
    o_ref, lse_ref = oracle.attn_fwd(Q, K, V, w.scale, True)
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(Q, K, V, dY, w.scale, True)

    sends, dsends = [], []
    for s in range(w.P):
        xs = dev(X[s * w.n:(s + 1) * w.n])
        out = sentinel((w.P, w.n, w.ht, w.d))
        uly.ulysses_seq_to_head(xs, out, w.P, w.segments)
        sends.append(out)
        ds = dev(dY[s * w.n:(s + 1) * w.n])
        dout = sentinel((w.P, w.n, w.hq, w.d))
        uly.ulysses_seq_to_head(ds, dout, w.P, [w.Hq])
        dsends.append(dout)
    o_chunks, g_chunks = [], []
    for r in range(w.P):
        recv = torch.stack([sends[s][r] for s in range(w.P)]).reshape(w.N, w.ht, w.d)
        drecv = torch.stack([dsends[s][r] for s in range(w.P)]).reshape(w.N, w.hq, w.d)
        q, k, v = recv[:, :w.hq], recv[:, w.hq:w.hq + w.hkv], recv[:, w.hq + w.hkv:]
        o = sentinel((w.N, w.hq, w.d))
        lse = torch.empty((w.hq, w.N), dtype=torch.float32, device="cuda")
        uly.attn_fwd(q, k, v, o, lse, w.scale, True)
        assert_close("tiny rank%d LSE" % r, lse.cpu().numpy().astype(np.float64),
                     lse_ref[r * w.hq:(r + 1) * w.hq], LSE_MAX_ABS, 1.0)
        dqkv = sentinel((w.N, w.ht, w.d))
        ws = torch.empty(uly.attn_bwd_workspace_bytes(w.N, w.hq, w.hkv, w.d), dtype=torch.uint8, device="cuda")
        uly.attn_bwd(q, k, v, o, lse, drecv, dqkv[:, :w.hq], dqkv[:, w.hq:w.hq + w.hkv], dqkv[:, w.hq + w.hkv:],
                     w.scale, True, ws)
        o_chunks.append(o.reshape(w.P, w.n, w.hq, w.d))
        g_chunks.append(dqkv.reshape(w.P, w.n, w.ht, w.d))
    o_seq, g_seq = [], []
    for s in range(w.P):
        o_recv = torch.stack([o_chunks[r][s] for r in range(w.P)])     # chunk r from rank r
        g_recv = torch.stack([g_chunks[r][s] for r in range(w.P)])
        o_out = sentinel((w.n, w.Hq, w.d))
        uly.ulysses_head_to_seq(o_recv.contiguous(), o_out, w.P, [w.Hq])
        g_out = sentinel((w.n, w.Ht, w.d))
        uly.ulysses_head_to_seq(g_recv.contiguous(), g_out, w.P, w.segments)
        o_seq.append(f64(o_out))
        g_seq.append(f64(g_out))
    O = np.concatenate(o_seq)
    G = np.concatenate(g_seq)
    assert_close("tiny layer O", O, o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close("tiny layer dQ", G[:, :w.Hq], dq_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close("tiny layer dK", G[:, w.Hq:w.Hq + w.Hkv], dk_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close("tiny layer dV", G[:, w.Hq + w.Hkv:], dv_ref, GRAD_MAX_ABS, GRAD_REL)


def _sample_rows(N, n_local, count, seed):
    rng = np.random.default_rng(seed)
    must = [0, 1, 63, 64, N - 1, N - 2]
    for s in range(1, N // n_local):
        must += [s * n_local - 1, s * n_local, s * n_local + 1]
    rows = set(x for x in must if 0 <= x < N)
    rows.update(int(x) for x in rng.integers(0, N, size=count))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["8k", "64k", "varlen", "256k"])
def test_workload_head_shard_sampled(name):
    """Rank 0's head shard at the workload's full size, in the launch shape the
    benchmark times; oracle on sampled query rows (O, LSE, dQ), on the last
    512 keys (dK, dV) and, where the oracle is fast enough, on the first 128;
    the Q = 0 / K = 0 closed forms check every key at 64K and 256K."""
    w = workloads.WORKLOADS[name]
    print("workload %s N=%d hq=%d hkv=%d" % (name, w.N, w.hq, w.hkv), flush=True)
    qkv = workloads.gen_head_shard(w, 0)
    dy = workloads.gen_dy_head_shard(w, 0)
    cu = workloads.cu_seqlens(w) if w.varlen else None
    r = Run(qkv, w.hq, w.hkv, w.scale, True, cu)
    o, lse = r.fwd()
    dq, dk, dv = r.bwd(dy)
    q, k, v = _split(qkv, w.hq, w.hkv)
    rows = _sample_rows(w.N, w.n, 96 if name == "256k" else 160, seed=len(name))
    if cu is not None:
        rows = np.unique(np.concatenate([rows, cu[:-1], cu[1:] - 1]))
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.scale, True, cu, rows=rows)
    assert_close(name + " O[rows]", oracle.bf16_to_f64(o[rows]), o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close(name + " LSE[rows]", lse[:, rows].astype(np.float64), lse_ref, LSE_MAX_ABS, 1.0)
    klo = w.N - TAIL_KEYS
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dy, w.scale, True, cu, rows=rows, key_lo=klo)
    assert_close(name + " dQ[rows]", oracle.bf16_to_f64(dq[rows]), dq_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close(name + " dK[tail]", oracle.bf16_to_f64(dk[klo:]), dk_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close(name + " dV[tail]", oracle.bf16_to_f64(dv[klo:]), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    if name in ("8k", "varlen"):
        # The first key block sees every query tile of its document(s), the
        # longest walk through the dK/dV kernel's rings (the oracle needs a
        # few seconds for it at these sizes).
        _, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dy, w.scale, True, cu, rows=rows[:1], key_lo=0,
                                            key_hi=128, want_dq=False)
        assert_close(name + " dK[head]", oracle.bf16_to_f64(dk[:128]), dk_ref, GRAD_MAX_ABS, GRAD_REL)
        assert_close(name + " dV[head]", oracle.bf16_to_f64(dv[:128]), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    for t, nm in ((o, "O"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert np.all(np.isfinite(oracle.bf16_to_f64(t))), nm + " has unwritten/non-finite elements"


@pytest.mark.parametrize("name", [
    "8k", "varlen",
    pytest.param("64k", marks=pytest.mark.skipif(
        os.environ.get("ULY_ORACLE_FULL") != "1",
        reason="the full fp64 oracle at 64K takes about 10 minutes on 16 host threads; set ULY_ORACLE_FULL=1")),
])
def test_workload_head_shard_full_oracle(name):
    """Rank 0's head shard at the workload's full size against the oracle on
    every query row and every key: O, LSE, dQ, dK, dV. The oracle takes about
    11 s at 8K and about a minute for the packed-document batch on 16 host
    threads."""
    w = workloads.WORKLOADS[name]
    print("workload %s N=%d hq=%d hkv=%d (full oracle)" % (name, w.N, w.hq, w.hkv), flush=True)
    qkv = workloads.gen_head_shard(w, 0)
    dy = workloads.gen_dy_head_shard(w, 0)
    cu = workloads.cu_seqlens(w) if w.varlen else None
    _check_full(qkv, dy, w.hq, w.hkv, w.scale, True, cu, name)


@pytest.mark.parametrize("N,hq,hkv,d", [
    (16384, 8, 4, 128),   # G = 2: two heads per workgroup
    (65536, 3, 1, 128),   # G = 3: one head per workgroup
    (32768, 8, 2, 64),    # d = 64
])
def test_unsplit_grids_sampled(N, hq, hkv, d):
    """Problems large enough that no kernel splits its ranges (at least 512
    blocks per grid), for the head-group sizes and head dim the workloads
    above do not reach unsplit; oracle on sampled query rows and the last
    512 keys."""
    print("unsplit N=%d hq=%d hkv=%d d=%d" % (N, hq, hkv, d), flush=True)
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=N + hq * 7 + d, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=N + hq * 11 + d)
    scale = 1.0 / np.sqrt(d)
    r = Run(qkv, hq, hkv, scale)
    o, lse = r.fwd()
    dq, dk, dv = r.bwd(dy)
    q, k, v = _split(qkv, hq, hkv)
    rows = _sample_rows(N, N // 4, 48, seed=N % 97 + hq)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, True, None, rows=rows)
    assert_close("O[rows]", oracle.bf16_to_f64(o[rows]), o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close("LSE[rows]", lse[:, rows].astype(np.float64), lse_ref, LSE_MAX_ABS, 1.0)
    klo = N - TAIL_KEYS
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dy, scale, True, None, rows=rows, key_lo=klo)
    assert_close("dQ[rows]", oracle.bf16_to_f64(dq[rows]), dq_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close("dK[tail]", oracle.bf16_to_f64(dk[klo:]), dk_ref, GRAD_MAX_ABS, GRAD_REL)
    assert_close("dV[tail]", oracle.bf16_to_f64(dv[klo:]), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    for t, nm in ((o, "O"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert np.all(np.isfinite(oracle.bf16_to_f64(t))), nm + " has unwritten/non-finite elements"


@pytest.mark.parametrize("N,max_len", [(2_100_000, 1200), (400_000, 1200), (1_000_000, 200)])
def test_long_packed_batch_sampled(N, max_len):
    """Long batches of short documents: at 2.1 M tokens more blocks than the
    work sort of the workgroup-order pass takes (the kernels keep block
    order), grids of over 16000 workgroups and the largest row offsets the
    tests reach; at 400 K tokens (about 3100 blocks per order) and 1 M tokens
    in documents of at most 200 tokens (about 7800 blocks, 9990 documents)
    sorted orders of several thousand blocks. Oracle on sampled rows and on
    the first and last 128 keys."""
    hq, hkv, d = 2, 1, 64
    rng = np.random.default_rng(0x10C + N)
    lens = []
    while sum(lens) < N:
        lens.append(int(rng.integers(1, max_len + 1)))
    lens[-1] -= sum(lens) - N
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print("long packed batch N=%d docs=%d" % (N, len(lens)), flush=True)
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=0x10D, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=0x10E)
    scale = 1.0 / np.sqrt(d)
    r = Run(qkv, hq, hkv, scale, True, cu)
    o, lse = r.fwd()
    dq, dk, dv = r.bwd(dy)
    q, k, v = _split(qkv, hq, hkv)
    rows = np.unique(np.concatenate([_sample_rows(N, N // 4, 64, seed=3), cu[-4:-1], cu[-4:-1] - 1]))
    rows = rows[(rows >= 0) & (rows < N)]
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, True, cu, rows=rows)
    assert_close("O[rows]", oracle.bf16_to_f64(o[rows]), o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close("LSE[rows]", lse[:, rows].astype(np.float64), lse_ref, LSE_MAX_ABS, 1.0)
    dq_ref, _, _ = oracle.attn_bwd(q, k, v, dy, scale, True, cu, rows=rows, want_dkv=False)
    assert_close("dQ[rows]", oracle.bf16_to_f64(dq[rows]), dq_ref, GRAD_MAX_ABS, GRAD_REL)
    for lo, hi in ((0, 128), (N - 128, N)):
        _, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dy, scale, True, cu, rows=rows[:1], key_lo=lo, key_hi=hi,
                                            want_dq=False)
        assert_close("dK[%d:%d]" % (lo, hi), oracle.bf16_to_f64(dk[lo:hi]), dk_ref, GRAD_MAX_ABS, GRAD_REL)
        assert_close("dV[%d:%d]" % (lo, hi), oracle.bf16_to_f64(dv[lo:hi]), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    for t, nm in ((o, "O"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):  # bf16 exponent all ones: NaN or Inf
        assert not np.any((t & 0x7F80) == 0x7F80), nm + " has unwritten/non-finite elements"


def test_separate_and_strided_layouts_give_identical_bits():
    """The kernels see only pointers and token strides: separate contiguous
    q, k, v and dq, dk, dv tensors, and an output that is a view inside a
    wider buffer, give the same bits as the fused q|k|v layout."""
    N, hq, hkv, d = 777, 4, 2, 128
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=606, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=607)
    scale = 1.0 / np.sqrt(d)
    fused = Run(qkv, hq, hkv, scale)
    o1, l1 = fused.fwd()
    g1 = fused.bwd(dy)
    qs, ks, vs = (dev(np.ascontiguousarray(x)) for x in _split(qkv, hq, hkv))
    wide = sentinel((N, hq + 2, d))
    o2 = wide[:, 1:1 + hq]                      # token stride (hq + 2) * d, offset d
    lse2 = torch.empty((hq, N), dtype=torch.float32, device="cuda")
    uly.attn_fwd(qs, ks, vs, o2, lse2, scale, True)
    dq2, dk2, dv2 = sentinel((N, hq, d)), sentinel((N, hkv, d)), sentinel((N, hkv, d))
    ws = torch.empty(uly.attn_bwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
    uly.attn_bwd(qs, ks, vs, o2, lse2, dev(dy), dq2, dk2, dv2, scale, True, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(o2), o1) and np.array_equal(lse2.cpu().numpy(), l1)
    assert np.all(host(wide[:, 0]) == 0xFFFF) and np.all(host(wide[:, 1 + hq]) == 0xFFFF)  # untouched
    for a, b in zip((host(dq2), host(dk2), host(dv2)), g1):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["64k", "256k"])
@pytest.mark.parametrize("zero", ["q", "k"])
def test_uniform_scores_closed_form_full_size(name, zero):
    """Q = 0 or K = 0 at the full 64K and 256K head shards, in the launch
    shape the benchmark times: every visible score is zero, so attention and
    all its gradients have closed forms in prefix and suffix sums
    (tests/uniform_scores.py). Every row of O, LSE and dV is compared, every
    row of dQ (Q = 0) or dK (K = 0), and the other of the two must be
    exactly zero. dV and dK cover every key block's whole walk through the
    dK/dV kernel (4096 tiles for the first block at 64K, 16384 at 256K)."""
    w = workloads.WORKLOADS[name]
    print("uniform scores %s N=%d hq=%d hkv=%d, %s = 0" % (name, w.N, w.hq, w.hkv, zero), flush=True)
    qkv = workloads.gen_head_shard(w, 0)
    if zero == "q":
        qkv[:, :w.hq] = 0
    else:
        qkv[:, w.hq:w.hq + w.hkv] = 0
    dy = workloads.gen_dy_head_shard(w, 0)
    r = Run(qkv, w.hq, w.hkv, w.scale, True)
    o, lse = r.fwd()
    dq, dk, dv = r.bwd(dy)
    q, k, v = (oracle.bf16_to_f64(x) for x in _split(qkv, w.hq, w.hkv))
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = uniform_scores.uniform_causal(
        q, k, v, oracle.bf16_to_f64(dy), w.scale, want_dq=zero == "q", want_dk=zero == "k")
    tag = "%s %s=0 " % (name, zero.upper())
    assert_close(tag + "O", oracle.bf16_to_f64(o), o_ref, FWD_MAX_ABS, FWD_REL)
    assert_close(tag + "LSE", lse.astype(np.float64), lse_ref, LSE_MAX_ABS, 1.0)
    assert_close(tag + "dV", oracle.bf16_to_f64(dv), dv_ref, GRAD_MAX_ABS, GRAD_REL)
    if zero == "q":
        assert_close(tag + "dQ", oracle.bf16_to_f64(dq), dq_ref, GRAD_MAX_ABS, GRAD_REL)
        assert np.all(oracle.bf16_to_f64(dk) == 0.0), "dK must be exactly 0 when Q = 0"
    else:
        assert_close(tag + "dK", oracle.bf16_to_f64(dk), dk_ref, GRAD_MAX_ABS, GRAD_REL)
        assert np.all(oracle.bf16_to_f64(dq) == 0.0), "dQ must be exactly 0 when K = 0"


def test_determinism_and_causality():
    N, hq, hkv, d = 1200, 4, 2, 128
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=77, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=78)
    r1 = Run(qkv, hq, hkv, 1 / np.sqrt(d))
    o1, l1 = r1.fwd()
    g1 = r1.bwd(dy)
    r2 = Run(qkv, hq, hkv, 1 / np.sqrt(d))
    o2, l2 = r2.fwd()
    g2 = r2.bwd(dy)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
    # perturb every token after i: rows <= i of O and LSE must not change (bits)
    i = 517
    qkv2 = qkv.copy()
    qkv2[i + 1:] = workloads.normal_bf16(qkv2[i + 1:].shape, seed=79, sigma=0.5)
    o3, l3 = Run(qkv2, hq, hkv, 1 / np.sqrt(d)).fwd()
    assert np.array_equal(o3[:i + 1], o1[:i + 1]) and np.array_equal(l3[:, :i + 1], l1[:, :i + 1])


def test_head_shards_concatenate_to_full_heads_bitexact():
    """Ulysses composition on the GPU: per-rank head-shard runs, side by side,
    equal the full-head run bit for bit (heads are independent)."""
    w = workloads.WORKLOADS["tiny"]
    X = workloads.gen_x(w, range(w.Ht))
    dY = workloads.gen_dy(w, range(w.Hq))
    full = Run(X, w.Hq, w.Hkv, w.scale)
    of, lf = full.fwd()
    dqf, dkf, dvf = full.bwd(dY)
    for r in range(w.P):
        sh = Run(workloads.gen_head_shard(w, r), w.hq, w.hkv, w.scale)
        o, l = sh.fwd()
        dq, dk, dv = sh.bwd(workloads.gen_dy_head_shard(w, r))
        hs, ks = slice(r * w.hq, (r + 1) * w.hq), slice(r * w.hkv, (r + 1) * w.hkv)
        assert np.array_equal(o, of[:, hs]) and np.array_equal(l, lf[hs])
        assert np.array_equal(dq, dqf[:, hs]) and np.array_equal(dk, dkf[:, ks]) and np.array_equal(dv, dvf[:, ks])


def test_varlen_single_document_equals_dense_and_per_doc_runs():
    N, hq, hkv, d = 900, 4, 2, 128
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=91, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=92)
    dense = Run(qkv, hq, hkv, 1 / np.sqrt(d))
    od, ld = dense.fwd()
    gd = dense.bwd(dy)
    one = Run(qkv, hq, hkv, 1 / np.sqrt(d), cu=np.array([0, N], dtype=np.int32))
    o1, l1 = one.fwd()
    g1 = one.bwd(dy)
    assert np.array_equal(od, o1) and np.array_equal(ld, l1)
    for a, b in zip(gd, g1):
        assert np.array_equal(a, b)
    cu = np.array([0, 130, 131, 500, 900], dtype=np.int32)
    packed = Run(qkv, hq, hkv, 1 / np.sqrt(d), cu=cu)
    op, lp = packed.fwd()
    gp = packed.bwd(dy)
    for a, b in zip(cu[:-1], cu[1:]):
        doc = Run(np.ascontiguousarray(qkv[a:b]), hq, hkv, 1 / np.sqrt(d))
        o_doc, l_doc = doc.fwd()
        g_doc = doc.bwd(np.ascontiguousarray(dy[a:b]))
        assert_close("doc O", oracle.bf16_to_f64(op[a:b]), oracle.bf16_to_f64(o_doc), 1e-2, 1e-2)
        assert np.max(np.abs(lp[:, a:b] - l_doc)) < 1e-4
        for x, y in zip(gp, g_doc):
            assert_close("doc grad", oracle.bf16_to_f64(x[a:b]), oracle.bf16_to_f64(y), 3e-2, 3e-2)


def test_attention_argument_errors():
    q = torch.zeros((64, 4, 128), dtype=torch.int16, device="cuda")
    kv = torch.zeros((64, 3, 128), dtype=torch.int16, device="cuda")
    o = sentinel((64, 4, 128))
    lse = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.attn_fwd(q, kv, kv, o, lse, 0.1)                  # 4 % 3 != 0
    assert e.value.name == "ULY_E_GQA"
    q96 = torch.zeros((64, 4, 96), dtype=torch.int16, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.attn_fwd(q96, q96[:, :2], q96[:, :2], q96.clone(), lse, 0.1)
    assert e.value.name == "ULY_E_HEADDIM"
    with pytest.raises(uly.UlyssesError) as e:
        uly.attn_fwd(q, q[:, :2], q[:, :2], q, lse, 0.1)      # o aliases q
    assert e.value.name == "ULY_E_ALIAS"
    # caught by the binding before the library is called: what the C
    # interface cannot see (sizes of the buffers behind the pointers, dtypes)
    k2 = torch.zeros((64, 2, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError):
        uly.attn_fwd(q, k2[:32], k2, o, lse, 0.1)              # k shorter than N
    with pytest.raises(ValueError):
        uly.attn_fwd(q, k2, k2, o, lse[:, :32], 0.1)           # lse too small
    with pytest.raises(ValueError):
        uly.attn_fwd(q, k2, k2, o, lse.double(), 0.1)          # lse not float32
    with pytest.raises(ValueError):
        uly.attn_fwd(q.float(), k2, k2, o, lse, 0.1)           # 4-byte elements
    with pytest.raises(ValueError):
        uly.attn_fwd(q, k2, k2, o, lse, 0.1, cu_seqlens=torch.tensor([0, 64], device="cuda"))  # int64
    with pytest.raises(ValueError):
        uly.attn_bwd_dq(q, k2, k2, o, lse, q, o, 0.1)          # no workspace
    torch.cuda.synchronize()
    assert np.all(host(o) == 0xFFFF)


def test_workspace_contents_do_not_matter():
    """Both workspaces are scratch: filling them with 0xFF bytes (NaN as
    float) before the calls changes no output bit. Ragged N leaves padded
    rows in every per-row workspace array, which must never be read as data."""
    for N, hq, hkv, d, cu in ((300, 4, 2, 128, None), (1000, 8, 2, 128, [0, 1, 333, 1000]),
                              (77, 2, 1, 64, None)):
        print("workspace N=%d hq=%d hkv=%d d=%d docs=%s" % (N, hq, hkv, d, cu), flush=True)
        qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=N + 5, sigma=0.5)
        dy = workloads.normal_bf16((N, hq, d), seed=N + 6)
        r = Run(qkv, hq, hkv, 1 / np.sqrt(d), cu=None if cu is None else np.array(cu, dtype=np.int32))
        outs = []
        for fill in (0x00, 0xFF):
            wsf = torch.full((uly.attn_fwd_workspace_bytes(N, hq, hkv, d),), fill, dtype=torch.uint8, device="cuda")
            wsb = torch.full((uly.attn_bwd_workspace_bytes(N, hq, hkv, d),), fill, dtype=torch.uint8, device="cuda")
            o = sentinel((N, hq, d))
            lse = torch.full((hq, N), float("nan"), dtype=torch.float32, device="cuda")
            uly.attn_fwd(r.q, r.k, r.v, o, lse, r.scale, True, r.cu_dev, r.max_seqlen, wsf)
            dqkv = sentinel((N, hq + 2 * hkv, d))
            dyd = dev(dy)
            uly.attn_bwd(r.q, r.k, r.v, o, lse, dyd, dqkv[:, :hq], dqkv[:, hq:hq + hkv], dqkv[:, hq + hkv:],
                         r.scale, True, wsb, r.cu_dev, r.max_seqlen)
            torch.cuda.synchronize()
            outs.append((host(o), lse.cpu().numpy(), host(dqkv)))
        assert np.array_equal(outs[0][0], outs[1][0])
        assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
        assert np.array_equal(outs[0][2], outs[1][2])
        assert np.all(np.isfinite(oracle.bf16_to_f64(outs[1][2])))


def test_split_backward_equals_attn_bwd():
    """attn_bwd_dq then attn_bwd_dkdv gives attn_bwd's bits."""
    N, hq, hkv, d = 700, 8, 2, 128
    qkv = workloads.normal_bf16((N, hq + 2 * hkv, d), seed=101, sigma=0.5)
    dy = workloads.normal_bf16((N, hq, d), seed=102)
    for cu in (None, np.array([0, 100, 101, 700], dtype=np.int32)):
        r = Run(qkv, hq, hkv, 1 / np.sqrt(d), cu=cu)
        r.fwd()
        ref = r.bwd(dy)
        dq = sentinel((N, hq, d))
        dkv = sentinel((N, 2 * hkv, d))
        ws = torch.empty(uly.attn_bwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
        uly.attn_bwd_dq(r.q, r.k, r.v, r.o, r.lse, r.dy, dq, r.scale, True, ws, r.cu_dev)
        uly.attn_bwd_dkdv(r.q, r.k, r.v, r.lse, r.dy, dkv[:, :hkv], dkv[:, hkv:], r.scale, True, ws, r.cu_dev)
        torch.cuda.synchronize()
        assert np.array_equal(host(dq), ref[0])
        assert np.array_equal(host(dkv)[:, :hkv], ref[1]) and np.array_equal(host(dkv)[:, hkv:], ref[2])


def _align256(n):
    return (n + 255) // 256 * 256


def _expected_order(cu, N, causal, bs, key_blocks):
    """Blocks of bs rows sorted by decreasing work, ties in id order; the work
    of a block is the number of 64-token tiles its rows' visible range spans
    (keys seen by its queries, or queries that see its keys). Visibility:
    same document, and j <= i under the causal mask."""
    t = np.arange(N, dtype=np.int64)
    doc = np.searchsorted(cu, t, side="right") - 1
    start, end = cu[doc].astype(np.int64), cu[doc + 1].astype(np.int64)
    if key_blocks:  # queries that see key j: [j or doc start, doc end)
        lo, hi = (t if causal else start), end
    else:           # keys query i sees: [doc start, i + 1 or doc end)
        lo, hi = start, (t + 1 if causal else end)
    nb = (N + bs - 1) // bs
    first = np.arange(nb) * bs
    last = np.minimum(first + bs, N) - 1
    work = (hi[last] + 63) // 64 - lo[first] // 64
    return np.array(sorted(range(nb), key=lambda i: (-int(work[i]), i)), dtype=np.int32)


@pytest.mark.parametrize("case", ["varlen-64k", "ties-ragged", "ties-ragged-full", "d64-g2"])
def test_packed_block_orders_sort_blocks_by_work(case):
    """Over packed documents the forward, dq and dK/dV kernels take their
    blocks in the order a sorting pass leaves in the workspace (its regions
    as the header lays them out): all blocks, by decreasing tile work, equal
    work in id order. Index work, so compared exactly."""
    causal = case != "ties-ragged-full"
    if case == "varlen-64k":
        cu = workloads.cu_seqlens(workloads.WORKLOADS["varlen"])
        N, hq, hkv, d = int(cu[-1]), 8, 2, 128
    elif case == "d64-g2":
        N, hq, hkv, d = 3001, 4, 2, 64
        cu = workloads.random_cu_seqlens(N, seed=77, lo=1, hi=900)
    else:  # many short documents: most blocks tie
        N, hq, hkv, d = 1000, 8, 2, 128
        cu = workloads.random_cu_seqlens(N, seed=76, lo=1, hi=70)
    hpw = 4 if (hq // hkv) % 4 == 0 else 2 if (hq // hkv) % 2 == 0 else 1
    q_bs, k_bs = 256 // hpw, 128
    np64 = (N + 63) // 64 * 64
    nq, nk = (N + q_bs - 1) // q_bs, (N + k_bs - 1) // k_bs
    print("block orders: %s N=%d hq=%d hkv=%d d=%d docs=%d" % (case, N, hq, hkv, d, len(cu) - 1), flush=True)

    g = torch.Generator(device="cuda").manual_seed(5)
    qkv = (torch.randn((N, hq + 2 * hkv, d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    q, k, v = qkv[:, :hq], qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]
    dy = torch.randn((N, hq, d), generator=g, device="cuda").to(torch.bfloat16)
    cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda")
    scale = 1 / np.sqrt(d)

    fws = torch.zeros(uly.attn_fwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, N), dtype=torch.float32, device="cuda")
    uly.attn_fwd(q, k, v, o, lse, scale, causal, cu_dev, int(np.max(np.diff(cu))), ws=fws)
    bws = torch.zeros(uly.attn_bwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
    dq = torch.empty((N, hq, d), dtype=torch.bfloat16, device="cuda")
    uly.attn_bwd_dq(q, k, v, o, lse, dy, dq, scale, causal, bws, cu_dev)
    torch.cuda.synchronize()

    # Forward: the order is the workspace's last region.
    fo = fws[fws.numel() - _align256(np64 // 64 * 4):].cpu().numpy().view(np.int32)[:nq]
    # Backward: -D, LSE*log2(e), K^T, Q^T, dO^T, then the key-block and
    # query-block orders.
    korder_at = (2 * _align256(hq * np64 * 4) + _align256(hkv * d * np64 * 2)
                 + 2 * _align256(hq * d * np64 * 2))
    qorder_at = korder_at + _align256(np64 // 64 * 4)
    b = bws.cpu().numpy()
    ko = b[korder_at:korder_at + nk * 4].view(np.int32)
    qo = b[qorder_at:qorder_at + nq * 4].view(np.int32)

    want_q = _expected_order(cu, N, causal, q_bs, key_blocks=False)
    want_k = _expected_order(cu, N, causal, k_bs, key_blocks=True)
    assert np.array_equal(fo, want_q)
    assert np.array_equal(qo, want_q)
    assert np.array_equal(ko, want_k)
