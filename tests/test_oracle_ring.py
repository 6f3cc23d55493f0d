"""Pins of the ring-attention merge (oracle.lse_merge) against things other
than itself: the full attention over the whole sequence computed directly,
and identities of the softmax."""
import numpy as np
import pytest

import oracle


def _blocks(P=4, n=24, hq=4, hkv=2, d=16, seed=3):
    rng = np.random.default_rng(seed)
    N = P * n
    q = rng.standard_normal((N, hq, d))
    k = rng.standard_normal((N, hkv, d))
    v = rng.standard_normal((N, hkv, d))
    return P, n, q, k, v


def _ring_rank(P, n, q, k, v, r, scale, order=None):
    """Rank r's ring steps: its queries against block b (causal on its own
    block, full on earlier ones; later blocks see nothing)."""
    qs = q[r * n:(r + 1) * n]
    parts = []
    for b in (order if order is not None else range(r + 1)):
        kb, vb = k[b * n:(b + 1) * n], v[b * n:(b + 1) * n]
        parts.append(oracle.attn_fwd(qs, kb, vb, scale, causal=(b == r)))
    return parts


@pytest.mark.parametrize("r", [0, 1, 3])
def test_merged_ring_steps_equal_full_causal_attention(r):
    P, n, q, k, v = _blocks()
    scale = 0.3
    o_full, lse_full = oracle.attn_fwd(q, k, v, scale, causal=True)
    parts = _ring_rank(P, n, q, k, v, r, scale)
    o, lse = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_full[r * n:(r + 1) * n], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_full[:, r * n:(r + 1) * n], rtol=0, atol=1e-12)


def test_merge_identities():
    P, n, q, k, v = _blocks(seed=5)
    parts = _ring_rank(P, n, q, k, v, 2, 0.25)
    o1, l1 = oracle.lse_merge([parts[0][0]], [parts[0][1]])
    assert np.array_equal(o1, parts[0][0]) and np.allclose(l1, parts[0][1], atol=1e-15)
    # a part merged with itself: same o, lse + ln 2
    o2, l2 = oracle.lse_merge([parts[1][0]] * 2, [parts[1][1]] * 2)
    np.testing.assert_allclose(o2, parts[1][0], atol=1e-14)
    np.testing.assert_allclose(l2, parts[1][1] + np.log(2.0), atol=1e-14)
    # a part with no keys adds nothing; order does not matter
    empty = (np.full_like(parts[0][0], 7.0), np.full_like(parts[0][1], -np.inf))
    oa, la = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    ob, lb = oracle.lse_merge([empty[0]] + [p[0] for p in parts[::-1]], [empty[1]] + [p[1] for p in parts[::-1]])
    np.testing.assert_allclose(oa, ob, atol=1e-14)
    np.testing.assert_allclose(la, lb, atol=1e-14)
    # rows without keys anywhere
    oz, lz = oracle.lse_merge([empty[0], empty[0]], [empty[1], empty[1]])
    assert np.all(oz == 0) and np.all(np.isneginf(lz))


def test_planted_mistakes_fail_the_full_attention_pin():
    P, n, q, k, v = _blocks(seed=9)
    scale = 0.3
    r = 3
    o_full, _ = oracle.attn_fwd(q, k, v, scale, causal=True)
    ref = o_full[r * n:(r + 1) * n]
    parts = _ring_rank(P, n, q, k, v, r, scale)
    # dropping one block, or treating the own block as unmasked, or mixing up
    # which lse belongs to which o, each moves the result well away
    bad = [
        ([p[0] for p in parts[1:]], [p[1] for p in parts[1:]]),
        ([p[0] for p in parts[:-1]] + [oracle.attn_fwd(q[r * n:], k[r * n:], v[r * n:], scale, causal=False)[0]],
         [p[1] for p in parts[:-1]] + [oracle.attn_fwd(q[r * n:], k[r * n:], v[r * n:], scale, causal=False)[1]]),
        ([p[0] for p in parts], [p[1] for p in parts[::-1]]),
    ]
    for o_parts, l_parts in bad:
        o, _ = oracle.lse_merge(o_parts, l_parts)
        assert np.max(np.abs(o - ref)) > 1e-3
