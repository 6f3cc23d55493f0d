"""The C-ABI library loads, exports every symbol include/ulysses.h declares,
and rejects bad arguments on the host before touching a device (no GPU
needed: every call here fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

uly = pytest.importorskip("long_context_attention_ulysses_amd")
L = uly.raw()

# fake, 256-byte aligned "device" addresses 32 MiB apart (never dereferenced)
A = 1 << 25
B = 2 << 25
C = 3 << 25
D_ = 4 << 25
E = 5 << 25       # lse
F = 6 << 25       # dout / cu
W = 8 << 25       # workspace


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})


def test_header_symbols_exported():
    names = declared_functions()
    assert set(names) == set(uly.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code, name in uly.STATUS.items():
        assert uly.status_string(code) and uly.status_string(code) != "unknown status", name
    assert uly.status_string(0) == "ok"
    assert uly.status_string(-999) == "unknown status"


def test_shard_len_and_cu_seqlens():
    assert uly.ulysses_shard_len(65536, 4) == 16384
    with pytest.raises(uly.UlyssesError) as e:
        uly.ulysses_shard_len(65537, 4)
    assert e.value.name == "ULY_E_DIV_P"
    with pytest.raises(uly.UlyssesError):
        uly.ulysses_shard_len(0, 4)
    uly.ulysses_check_cu_seqlens([0, 5, 6, 10], 10)
    for bad in ([1, 5, 10], [0, 5, 5, 10], [0, 5, 9], [0, 7, 3, 10]):
        with pytest.raises(uly.UlyssesError) as e:
            uly.ulysses_check_cu_seqlens(bad, 10)
        assert e.value.name == "ULY_E_SEQLENS"


def _seg(*s):
    return (ctypes.c_int32 * len(s))(*s)


@pytest.mark.parametrize("args,code", [
    ((0, B, 16, 4, 3, _seg(32, 8, 8), 128), "ULY_E_NULL"),
    ((A, B, 0, 4, 3, _seg(32, 8, 8), 128), "ULY_E_SHAPE"),
    ((A, B, 16, 4, 3, _seg(32, 6, 8), 128), "ULY_E_DIV_P"),
    ((A, B, 16, 4, 3, _seg(32, 8, 8), 100), "ULY_E_ALIGN"),
    ((A + 2, B, 16, 4, 3, _seg(32, 8, 8), 128), "ULY_E_ALIGN"),
    ((A, A + 64, 16, 4, 3, _seg(32, 8, 8), 128), "ULY_E_ALIAS"),
    ((A, B, 16, 4, 9, _seg(*([4] * 9)), 128), "ULY_E_SHAPE"),
])
def test_swap_validation(args, code):
    for fn in (L.ulysses_seq_to_head, L.ulysses_head_to_seq):
        assert fn(*args, None) == uly.CODE[code]


def _fwd(**kw):
    a = dict(q=A, k=B, v=C, o=D_, lse=E, N=1024, hq=8, hkv=2, d=128, qs=1536, ks=1536, vs=1536,
             os=1024, scale=0.088, causal=1, ws=W, wsb=1 << 25)
    a.update(kw)
    return L.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["N"], a["hq"], a["hkv"], a["d"], a["qs"],
                      a["ks"], a["vs"], a["os"], a["scale"], a["causal"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), "ULY_E_NULL"),
    (dict(lse=0), "ULY_E_NULL"),
    (dict(N=0), "ULY_E_SHAPE"),
    (dict(hkv=3), "ULY_E_GQA"),
    (dict(d=96, qs=96 * 12, ks=96 * 12, vs=96 * 12, os=96 * 8), "ULY_E_HEADDIM"),
    (dict(qs=1000), "ULY_E_STRIDE"),
    (dict(os=1000), "ULY_E_STRIDE"),
    (dict(qs=1540), "ULY_E_ALIGN"),
    (dict(k=B + 8), "ULY_E_ALIGN"),
    (dict(scale=0.0), "ULY_E_SHAPE"),
    (dict(scale=float("nan")), "ULY_E_SHAPE"),
    (dict(o=A), "ULY_E_ALIAS"),
    (dict(ws=0), "ULY_E_WORKSPACE"),
    (dict(wsb=100), "ULY_E_WORKSPACE"),
    (dict(ws=W + 64), "ULY_E_WORKSPACE"),
    (dict(ws=D_), "ULY_E_ALIAS"),
])
def test_attn_fwd_validation(kw, code):
    assert _fwd(**kw) == uly.CODE[code]


def test_attn_fwd_noalloc_validation():
    """The allocation-free forward checks its arguments like attn_fwd and
    rejects, before any device call, problems whose workspace exceeds its
    static scratch buffer (80 MiB)."""
    far = 1 << 36           # fake addresses far enough apart for 2^18 tokens

    def fwd(N=1024, hq=8, hkv=2, o=4 * far, q=far, qs=1536):
        return L.attn_fwd_noalloc(q, 2 * far, 3 * far, o, 5 * far, N, hq, hkv, 128, qs, qs, qs, hq * 128, 0.088,
                                  1, None)

    assert fwd(q=0) == uly.CODE["ULY_E_NULL"]
    assert fwd(hkv=3) == uly.CODE["ULY_E_GQA"]
    assert fwd(qs=1000) == uly.CODE["ULY_E_STRIDE"]
    assert fwd(o=far) == uly.CODE["ULY_E_ALIAS"]
    limit = uly.NOALLOC_SCRATCH_BYTES
    assert limit == 80 << 20
    # one KV head of 2^18 tokens fits (64 MiB of V^T); two heads at 2^18 or
    # more tokens do not
    assert L.attn_fwd_workspace_bytes(1 << 18, 4, 1, 128) <= limit
    assert L.attn_fwd_workspace_bytes(1 << 18, 8, 2, 128) > limit
    assert fwd(N=1 << 18, hq=8, hkv=2, qs=12 * 128) == uly.CODE["ULY_E_SCRATCH"]
    assert L.attn_fwd_workspace_bytes(327552, 4, 1, 128) <= limit < L.attn_fwd_workspace_bytes(327616, 4, 1, 128)
    assert L.attn_fwd_workspace_bytes(163776, 8, 2, 128) <= limit < L.attn_fwd_workspace_bytes(163840, 8, 2, 128)
    assert fwd(N=327616, hq=4, hkv=1, qs=6 * 128) == uly.CODE["ULY_E_SCRATCH"]
    assert "scratch" in uly.status_string(uly.CODE["ULY_E_SCRATCH"])


def test_attn_varlen_and_bwd_validation():
    r = L.attn_fwd_varlen(A, B, C, D_, E, 1024, 8, 2, 128, 1536, 1536, 1536, 1024, 0.1, 1, None, 3, 512,
                          W, 1 << 25, None)
    assert r == uly.CODE["ULY_E_NULL"]
    r = L.attn_fwd_varlen(A, B, C, D_, E, 1024, 8, 2, 128, 1536, 1536, 1536, 1024, 0.1, 1, F, 0, 512,
                          W, 1 << 25, None)
    assert r == uly.CODE["ULY_E_SHAPE"]
    N, hq, hkv, d = 1024, 8, 2, 128
    need = L.attn_bwd_workspace_bytes(N, hq, hkv, d, 1)
    assert need >= N * hq * 4 * 2 + N * d * (hkv + 2 * hq) * 2 and need % 256 == 0
    # transposed V, plus float32 partial softmax states (O, max, sum) of the
    # 4-way key split that 1024 tokens (32 query blocks x 2 head groups) get,
    # plus the 16 int32 entries of the packed-document query-block order
    # (rounded up to 256 bytes)
    assert L.attn_fwd_workspace_bytes(N, hq, hkv, d) == hkv * d * N * 2 + 4 * N * hq * (d + 2) * 4 + 256

    def bwd(ws=W, ws_bytes=need, dq=9 << 25, dk=10 << 25, dv=11 << 25):
        return L.attn_bwd(A, B, C, D_, E, F, dq, dk, dv, N, hq, hkv, d, 1536, 1536, 1536, 1024, 1024,
                          1536, 1536, 1536, 0.1, 1, ws, ws_bytes, None)

    assert bwd(ws=0) == uly.CODE["ULY_E_WORKSPACE"]
    assert bwd(ws_bytes=need - 1) == uly.CODE["ULY_E_WORKSPACE"]
    assert bwd(ws=W + 16) == uly.CODE["ULY_E_WORKSPACE"]
    assert bwd(dq=A) == uly.CODE["ULY_E_ALIAS"]
    assert bwd(dk=W + (1 << 20)) == uly.CODE["ULY_E_ALIAS"]
    assert bwd(dv=0) == uly.CODE["ULY_E_NULL"]


def test_workspaces_grow_linearly_with_n():
    """O(N) memory: no N x N buffer anywhere; the only device memory the
    attention calls use beyond their inputs and outputs is the workspace."""
    for hq, hkv, d in ((8, 2, 128), (4, 1, 64)):
        for N in (4096, 65536, 262144):
            f1, f2 = L.attn_fwd_workspace_bytes(N, hq, hkv, d), L.attn_fwd_workspace_bytes(2 * N, hq, hkv, d)
            b1, b2 = L.attn_bwd_workspace_bytes(N, hq, hkv, d, 1), L.attn_bwd_workspace_bytes(2 * N, hq, hkv, d, 1)
            # below 512 (query block, head group) pairs the forward and the dq
            # pass split their key ranges over up to 4 workgroups (float32
            # partials); below 512 (128-key block, KV head) pairs the dK/dV pass splits its
            # query ranges, and below 512 (query block, head group) pairs the dq
            # pass splits its key ranges, over up to 4 workgroups each, keeping
            # float32 partials
            dkdv_split = N // 128 * hkv < 512
            dq_split = N // 64 * (hq // 4) < 512  # 4 heads per dq workgroup here
            split_max = (4 * N * hkv * 2 * d * 4 if dkdv_split else 0) + (4 * N * hq * d * 4 if dq_split else 0)
            assert f1 <= hkv * d * N * 2 + (4 * N * hq * (d + 2) * 4 if dq_split else 0) + N // 64 * 4 + 512
            if not dq_split:
                assert f2 == 2 * f1
            assert b1 <= N * (2 * hq * 4 + (hkv + 2 * hq) * d * 2) + 2 * (N // 64 * 4) + split_max + 2048
            if not dkdv_split and not dq_split:
                assert abs(b2 - 2 * b1) <= 2048


def test_binding_rejects_host_tensors():
    """The binding refuses tensors that are not on a GPU before calling the
    library: a host pointer handed to a kernel would fault the device."""
    import torch
    import long_context_attention_ulysses_amd as uly
    x = torch.zeros((8, 4, 16), dtype=torch.int16)
    out = torch.zeros((2, 8, 2, 16), dtype=torch.int16)
    with pytest.raises(ValueError, match="must be on a GPU"):
        uly.ulysses_seq_to_head(x, out, 2, [4])
    q = torch.zeros((64, 4, 64), dtype=torch.int16)
    k = torch.zeros((64, 2, 64), dtype=torch.int16)
    lse = torch.zeros((4, 64), dtype=torch.float32)
    ws = torch.zeros((1 << 20,), dtype=torch.uint8)
    with pytest.raises(ValueError, match="must be on a GPU"):
        uly.attn_fwd(q, k, k, q.clone(), lse, 0.125, ws=ws)
    with pytest.raises(TypeError):
        uly.ring_grad_sum([q.numpy()], q)


def test_workspace_is_allocated_on_the_launch_stream(monkeypatch):
    """When the binding allocates a workspace itself (ws=None), it takes the
    memory on the stream the kernels are launched on, so torch's caching
    allocator cannot hand that block to other work before the kernels are
    done. Checked with stand-ins for torch's stream objects (no GPU)."""
    import contextlib

    import long_context_attention_ulysses_amd._lib as lib

    active, made = [], []

    class FakeStream:
        def __init__(self, handle, device=None):
            self.cuda_stream = handle

    @contextlib.contextmanager
    def enter(s):
        active.append(s.cuda_stream)
        yield
        active.pop()

    class Like:
        device = "cuda:0"

    monkeypatch.setattr(lib.torch.cuda, "current_stream", lambda device=None: FakeStream(5))
    monkeypatch.setattr(lib.torch.cuda, "ExternalStream", FakeStream)
    monkeypatch.setattr(lib.torch.cuda, "stream", enter)
    monkeypatch.setattr(lib.torch, "empty", lambda *a, **k: made.append(active[-1] if active else "current"))
    lib._workspace(100, Like(), 9)      # a side stream: allocate under it
    lib._workspace(100, Like(), 5)      # torch's current stream: no switch
    assert made == [9, "current"]
    assert lib._stream(FakeStream(11), "cuda:0") == 11 and lib._stream(12, "cuda:0") == 12
    assert lib._stream(None, "cuda:0") == 5
