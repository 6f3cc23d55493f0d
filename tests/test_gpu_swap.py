"""GPU parity of the layout swap kernels against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import dev, host, sentinel

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")


def _pack(x_bits, P, segs):
    n, H, d = x_bits.shape
    x = dev(x_bits)
    out = sentinel((P, n, H // P, d))
    uly.ulysses_seq_to_head(x, out, P, segs)
    torch.cuda.synchronize()
    return host(out)


def _unpack(r_bits, P, segs):
    P_, n, h, d = r_bits.shape
    r = dev(r_bits)
    out = sentinel((n, h * P, d))
    uly.ulysses_head_to_seq(r, out, P, segs)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("n,P,segs,d", [
    (1, 2, [4, 2, 2], 64),
    (37, 2, [4, 2, 2], 64),
    (129, 4, [32, 8, 8], 128),
    (5, 3, [3, 6], 8),
    (11, 8, [8], 24),
    (50, 1, [4, 2, 2], 16),
    # long token rows (6144 and 4096 16-byte vectors, 96 and 64 KiB)
    (37, 4, [256, 64, 64], 128),
    (9, 8, [128, 64, 64], 128),
    # many chunks: P = 16 and 32, segment blocks of 16/4/4 and 8/2/2 heads
    # (48 and 96 runs per token row)
    (3, 16, [256, 64, 64], 128),
    (2, 32, [256, 64, 64], 128),
])
def test_swap_small_shapes_bit_exact(n, P, segs, d):
    x = workloads.normal_bf16((n, sum(segs), d), seed=n * 131 + P)
    print("swap n=%d P=%d segs=%s d=%d" % (n, P, segs, d), flush=True)
    got = _pack(x, P, segs)
    assert np.array_equal(got, oracle.seq_to_head(x, P, segs))
    back = _unpack(got, P, segs)
    assert np.array_equal(back, x)
    r = workloads.normal_bf16((P, n, sum(segs) // P, d), seed=n * 17 + 3)
    assert np.array_equal(_unpack(r, P, segs), oracle.head_to_seq(r, P, segs))


@pytest.mark.parametrize("name", ["tiny", "8k", "64k", "256k"])
def test_swap_workloads_bit_exact(name):
    """a1 / a10 (fused q|k|v) and a5 / a6 (query heads) at the workloads' shard shapes."""
    w = workloads.WORKLOADS[name]
    print("swap workload %s n=%d P=%d" % (name, w.n, w.P), flush=True)
    x = workloads.gen_seq_shard(w, 0)
    send = _pack(x, w.P, w.segments)
    assert np.array_equal(send, oracle.seq_to_head(x, w.P, w.segments))
    assert np.array_equal(_unpack(send, w.P, w.segments), x)
    dy = workloads.gen_dy_seq_shard(w, 0)
    o_send = _pack(dy, w.P, [w.Hq])
    assert np.array_equal(o_send, oracle.seq_to_head(dy, w.P, [w.Hq]))
    assert np.array_equal(_unpack(o_send, w.P, [w.Hq]), dy)


def test_swap_composition_gives_head_shard():
    """Pack on every simulated rank + exchange = rank r's head shard."""
    w = workloads.WORKLOADS["tiny"]
    sends = [_pack(workloads.gen_seq_shard(w, s), w.P, w.segments) for s in range(w.P)]
    for r in range(w.P):
        recv = np.stack([sends[s][r] for s in range(w.P)]).reshape(w.N, w.ht, w.d)
        assert np.array_equal(recv, workloads.gen_head_shard(w, r))


def test_swap_errors_leave_output_untouched():
    x = dev(workloads.normal_bf16((8, 6, 16), seed=5))
    out = sentinel((4, 8, 1, 16))
    with pytest.raises(uly.UlyssesError) as e:
        uly.ulysses_seq_to_head(x, out, 4, [2, 4])          # 2 % 4 != 0
    assert e.value.name == "ULY_E_DIV_P"
    with pytest.raises(uly.UlyssesError) as e:
        uly.ulysses_seq_to_head(x, x, 2, [2, 4])            # in place
    assert e.value.name == "ULY_E_ALIAS"
    out2 = sentinel((2, 8, 3, 16))
    with pytest.raises(ValueError):
        uly.ulysses_seq_to_head(x.transpose(0, 1).contiguous().transpose(0, 1), out2, 2, [2, 4])  # not contiguous
    with pytest.raises(ValueError):
        uly.ulysses_seq_to_head(x, out2[:1], 2, [2, 4])      # output too small
    with pytest.raises(ValueError):
        uly.ulysses_seq_to_head(x, out2, 2, [2, 2])          # segments do not add up to H
    torch.cuda.synchronize()
    assert np.all(host(out2) == 0xFFFF)
    torch.cuda.synchronize()
    assert np.all(host(out) == 0xFFFF)
