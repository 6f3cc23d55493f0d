"""attn_fwd_noalloc (the forward in the library's static per-GPU scratch
buffer, for callers that cannot allocate) against attn_fwd with a caller
workspace: identical bits on two calls in a row, the second smaller (it
leaves the first call's contents behind in the buffer), and an over-limit
problem rejected before any launch."""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu import dev, host, sentinel

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")


def _both(qkv_bits, hq, hkv, scale, causal=True):
    N, _, d = qkv_bits.shape
    x = dev(qkv_bits)
    q, k, v = x[:, :hq], x[:, hq:hq + hkv], x[:, hq + hkv:]
    o1, o2 = sentinel((N, hq, d)), sentinel((N, hq, d))
    l1 = torch.full((hq, N), float("nan"), dtype=torch.float32, device="cuda")
    l2 = torch.full((hq, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(uly.attn_fwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
    uly.attn_fwd(q, k, v, o1, l1, scale, causal, ws=ws)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    uly.attn_fwd_noalloc(q, k, v, o2, l2, scale, causal)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before, "the call allocated"
    assert np.array_equal(host(o2), host(o1)), "O differs from attn_fwd"
    assert np.array_equal(l2.cpu().numpy(), l1.cpu().numpy()), "LSE differs from attn_fwd"
    assert np.all(np.isfinite(l2.cpu().numpy()))


def test_noalloc_matches_attn_fwd_on_two_calls_second_smaller():
    for name in ("64k", "8k"):             # 8k: the split path with float32 partials in the scratch buffer
        w = workloads.WORKLOADS[name]
        print("noalloc %s N=%d hq=%d hkv=%d" % (name, w.N, w.hq, w.hkv), flush=True)
        _both(workloads.gen_head_shard(w, 0), w.hq, w.hkv, w.scale)
    print("noalloc ragged N=777 G=3 d=64, non-causal", flush=True)
    _both(workloads.normal_bf16((777, 3 + 2, 64), seed=5, sigma=1.0), 3, 1, 0.125, causal=False)


def test_noalloc_rejects_problems_beyond_its_scratch():
    N, hq, hkv, d = 327744, 4, 1, 128
    assert uly.attn_fwd_workspace_bytes(N, hq, hkv, d) > uly.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((N, hq + 2 * hkv, d), dtype=torch.int16, device="cuda")
    o = sentinel((N, hq, d))
    lse = torch.zeros((hq, N), dtype=torch.float32, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.attn_fwd_noalloc(x[:, :hq], x[:, hq:hq + 1], x[:, hq + 1:], o, lse, 0.088, True)
    assert e.value.name == "ULY_E_SCRATCH"
    torch.cuda.synchronize()
    assert np.all(host(o[:64]) == 0xFFFF), "a rejected call must not launch"
