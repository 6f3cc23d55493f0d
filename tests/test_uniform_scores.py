"""CPU pins of the full-size closed forms in tests/uniform_scores.py (used by
the GPU tests at 64K and 256K): against the oracle on problems spanning
several chunks with a ragged last one, and the chunked bilinear sums against
their O(N^2) definition."""
import numpy as np
import pytest

import oracle
from tests import uniform_scores


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def test_pair_sums_match_definition():
    N, d, e = 97, 5, 3
    x, y, z = _rand((N, d), 1), _rand((N, d), 2), _rand((N, e), 3)
    dots = x @ y.T                                        # [a, b] = x_a . y_b
    suf = np.stack([(dots[a, a:, None] * z[a:]).sum(axis=0) for a in range(N)])
    pre = np.stack([(dots[a, :a + 1, None] * z[:a + 1]).sum(axis=0) for a in range(N)])
    for chunk in (1, 7, 32, 97, 200):
        np.testing.assert_allclose(uniform_scores.suffix_pair_sum(x, y, z, chunk), suf, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(uniform_scores.prefix_pair_sum(x, y, z, chunk), pre, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("zero", ["q", "k"])
def test_uniform_closed_forms_match_oracle(zero):
    N, hq, hkv, d, scale = 600, 4, 2, 16, 0.25
    q, k, v = _rand((N, hq, d), 11), _rand((N, hkv, d), 12), _rand((N, hkv, d), 13)
    dout = _rand((N, hq, d), 14)
    if zero == "q":
        q[:] = 0.0
    else:
        k[:] = 0.0
    o, lse, dq, dk, dv = uniform_scores.uniform_causal(q, k, v, dout, scale)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, scale, True)
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, dout, scale, True)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-10, atol=1e-12)
    # the vanishing gradient is exactly zero on both sides
    assert np.all((dk if zero == "q" else dq) == 0.0)
    assert np.all((dk_ref if zero == "q" else dq_ref) == 0.0)


def test_uniform_closed_forms_reject_a_planted_sign_error():
    """A closed form with the D_i term of dK added instead of subtracted is
    caught by the oracle comparison above."""
    N, hq, hkv, d, scale = 300, 2, 1, 8, 0.5
    q, v, dout = _rand((N, hq, d), 21), _rand((N, hkv, d), 22), _rand((N, hq, d), 23)
    k = np.zeros((N, hkv, d))
    _, _, _, dk, _ = uniform_scores.uniform_causal(q, k, v, dout, scale)
    _, dk_ref, _ = oracle.attn_bwd(q, k, v, dout, scale, True)
    w = 1.0 / np.arange(1, N + 1)
    D = np.einsum("nhd,nhd->nh", dout, (np.cumsum(v, axis=0) * w[:, None, None]).repeat(hq, axis=1))
    tail = np.cumsum(((w[:, None] * D)[..., None] * q)[::-1], axis=0)[::-1].sum(axis=1, keepdims=True)
    planted = dk + 2.0 * scale * tail                    # turns "- tail" into "+ tail"
    assert np.allclose(dk, dk_ref, rtol=1e-9, atol=1e-11)
    assert not np.allclose(planted, dk_ref, rtol=1e-3, atol=1e-3)
