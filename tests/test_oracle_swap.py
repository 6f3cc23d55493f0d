"""Pins for the oracle's layout swap (CPU only).

The swap is pinned to (a) the two-GPU diagram of the "Ulysses sequence
parallelism" page written out as a fixture, (b) numpy's reshape/transpose,
(c) the round trip and bijectivity, (d) P = 1 being a copy.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tags(shape):
    n = int(np.prod(shape))
    assert n <= 65536, "tags must be unique uint16"
    return np.arange(n, dtype=np.uint16).reshape(shape)


def test_diagram_two_gpus():
    g = json.load(open(os.path.join(GOLDEN, "ulysses_diagram_2gpu.json")))
    N, H, P = g["N"], g["H"], g["P"]
    n = N // P
    # element (t, h) carries the tag t*H + h; d = 1
    X = np.array([[[t * H + h] for h in range(H)] for t in range(N)], dtype=np.uint16)
    seq = [X[s * n:(s + 1) * n] for s in range(P)]
    for s in range(P):
        want = [t * H + h for t, h in g["seq_sharded"][str(s)]]
        assert seq[s].reshape(-1).tolist() == want
    sends = [oracle.seq_to_head(seq[s], P, [H]) for s in range(P)]
    recvs = oracle.exchange(sends)
    for r in range(P):
        shard = recvs[r].reshape(N, H // P, 1)       # [P, n, h, d] -> [N, h, d]: source ranks in token order
        want = [t * H + h for t, h in g["head_sharded"][str(r)]]
        assert shard.reshape(-1).tolist() == want
    # the second all-to-all returns the first layout
    back_sends = recvs
    back_recvs = oracle.exchange(back_sends)
    for s in range(P):
        assert np.array_equal(oracle.head_to_seq(back_recvs[s], P, [H]), seq[s])


def _numpy_pack(x, P, segs):
    """Independent formulation: per segment, split heads into P blocks with a
    reshape and move the block axis to the front."""
    n, H, d = x.shape
    parts, off = [], 0
    for S in segs:
        blk = x[:, off:off + S, :].reshape(n, P, S // P, d).transpose(1, 0, 2, 3)
        parts.append(blk)
        off += S
    return np.concatenate(parts, axis=2)


@pytest.mark.parametrize("n,P,segs,d", [
    (3, 2, [4, 2, 2], 8),
    (5, 4, [8, 4, 4], 4),
    (7, 2, [6], 16),
    (2, 3, [3, 3, 6], 8),
    (4, 1, [4, 2, 2], 8),
])
def test_pack_matches_numpy_reshape(n, P, segs, d):
    x = _tags((n, sum(segs), d))
    got = oracle.seq_to_head(x, P, segs)
    assert got.shape == (P, n, sum(segs) // P, d)
    assert np.array_equal(got, _numpy_pack(x, P, segs))


@pytest.mark.parametrize("n,P,segs,d", [(3, 2, [4, 2, 2], 8), (6, 4, [8, 4, 4], 8), (9, 2, [4], 2)])
def test_round_trip_and_bijective(n, P, segs, d):
    x = _tags((n, sum(segs), d))
    send = oracle.seq_to_head(x, P, segs)
    assert np.array_equal(np.sort(send.reshape(-1)), np.sort(x.reshape(-1)))   # every element exactly once
    assert np.array_equal(oracle.head_to_seq(send, P, segs), x)
    # the other direction too: unpack then pack is the identity on [P, n, h, d]
    y = _tags((P, n, sum(segs) // P, d))
    assert np.array_equal(oracle.seq_to_head(oracle.head_to_seq(y, P, segs), P, segs), y)


def test_p1_is_identity():
    x = _tags((5, 8, 8))
    assert np.array_equal(oracle.seq_to_head(x, 1, [4, 2, 2])[0], x)


def test_fused_qkv_chunk_order():
    """Chunk p holds [q heads of group p | k heads of group p | v heads of group p]."""
    w = workloads.WORKLOADS["tiny"]
    x = _tags((w.n // 4, w.Ht, 8))
    send = oracle.seq_to_head(x, w.P, w.segments)
    for p in range(w.P):
        heads = workloads.rank_heads(w, p)
        assert np.array_equal(send[p], x[:, heads, :])


def test_ulysses_composition_gives_head_shard():
    """Pack on every rank + exchange = the rank's heads over the full sequence."""
    w = workloads.WORKLOADS["tiny"]
    X = workloads.gen_x(w, range(w.Ht))
    sends = [oracle.seq_to_head(X[s * w.n:(s + 1) * w.n], w.P, w.segments) for s in range(w.P)]
    recvs = oracle.exchange(sends)
    for r in range(w.P):
        assert np.array_equal(recvs[r].reshape(w.N, w.ht, w.d), X[:, workloads.rank_heads(w, r), :])
        assert np.array_equal(recvs[r].reshape(w.N, w.ht, w.d), workloads.gen_head_shard(w, r))
