"""Pins of the shifted-label loss oracle and its aggregation over SP ranks
against things other than itself: torch's cross-entropy and autograd in
float64, closed forms, and the single-device loss of the whole sequence."""
import numpy as np
import pytest
import torch

import oracle


def _case(n=40, V=64, seed=0, ignore_every=5):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((n, V)) * 2.0
    labels = rng.integers(0, V, size=n)
    labels[::ignore_every] = oracle.IGNORE
    return logits, labels


def test_rank_loss_matches_torch_cross_entropy():
    logits, labels = _case()
    row_loss, row_lse, loss, good = oracle.shifted_ce(logits, labels)
    t = torch.tensor(logits, dtype=torch.float64)
    y = torch.tensor(labels)
    ref = torch.nn.functional.cross_entropy(t, y, ignore_index=-100, reduction="mean").item()
    ref_rows = torch.nn.functional.cross_entropy(t, y, ignore_index=-100, reduction="none").numpy()
    assert abs(loss - ref) < 1e-12
    np.testing.assert_allclose(row_loss, ref_rows, atol=1e-12)
    np.testing.assert_allclose(row_lse, torch.logsumexp(t, dim=1).numpy(), atol=1e-12)
    assert good == int(np.sum(labels != -100))


def test_closed_forms():
    V = 48
    row_loss, _, loss, good = oracle.shifted_ce(np.zeros((3, V)), np.array([0, 5, 47]))
    np.testing.assert_allclose(row_loss, np.log(V), atol=1e-14)     # uniform logits
    big = np.zeros((2, V))
    big[0, 7] = 60.0
    big[1, 3] = 60.0
    row_loss, _, _, _ = oracle.shifted_ce(big, np.array([7, 4]))
    assert row_loss[0] < 1e-20 and abs(row_loss[1] - 60.0) < 1e-12  # right vs wrong confident guess
    rl, _, l0, g0 = oracle.shifted_ce(np.ones((4, V)), np.full(4, -100))
    assert l0 == 0.0 and g0 == 0 and np.all(rl == 0)
    assert oracle.sp_loss_aggregate([0.0, 0.0], [0, 0]) == 0.0          # max(G, 1)


def test_shift_labels():
    lab = np.array([5, 9, 2, 7, 1])
    assert oracle.shift_labels(lab).tolist() == [9, 2, 7, 1, -100]


@pytest.mark.parametrize("P", [1, 2, 4])
def test_sp_aggregate_equals_single_device_loss(P):
    """The pages' quality check: the SP loss equals the one-GPU loss of the
    whole sequence (mean over every good token), however the good tokens
    fall over the ranks."""
    N, V = 48, 32
    rng = np.random.default_rng(P)
    logits = rng.standard_normal((N, V))
    tokens = rng.integers(0, V, size=N)
    labels = oracle.shift_labels(tokens)
    labels[: N // 3] = oracle.IGNORE                   # a prompt without loss: rank 0 may have none
    whole = oracle.shifted_ce(logits, labels)[2]
    n = N // P
    losses, goods = [], []
    for r in range(P):
        _, _, l, g = oracle.shifted_ce(logits[r * n:(r + 1) * n], labels[r * n:(r + 1) * n])
        losses.append(l)
        goods.append(g)
    assert abs(oracle.sp_loss_aggregate(losses, goods) - whole) < 1e-12


def test_gradient_matches_torch_autograd_of_the_aggregate():
    P, n, V = 3, 10, 24
    rng = np.random.default_rng(11)
    shards = [rng.standard_normal((n, V)) for _ in range(P)]
    labels = [rng.integers(0, V, size=n) for _ in range(P)]
    labels[0][:] = -100                                # a rank with no good tokens
    labels[1][::3] = -100
    G = sum(int(np.sum(l != -100)) for l in labels)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in shards]
    total = 0.0
    goods = []
    for t, l in zip(ts, labels):
        y = torch.tensor(l)
        g = int((y != -100).sum())
        goods.append(g)
        if g:
            total = total + torch.nn.functional.cross_entropy(t, y, ignore_index=-100, reduction="mean") * g
    (total / max(sum(goods), 1)).backward()
    for t, x, l in zip(ts, shards, labels):
        ref = np.zeros_like(x) if t.grad is None else t.grad.numpy()    # a rank without good tokens
        np.testing.assert_allclose(oracle.shifted_ce_grad(x, l, G), ref, atol=1e-14)


def test_gradient_finite_differences():
    logits, labels = _case(n=6, V=10, seed=4, ignore_every=4)
    G = int(np.sum(labels != -100))
    g = oracle.shifted_ce_grad(logits, labels, G)
    h = 1e-6
    for (r, c) in [(1, 3), (2, 0), (5, 9), (0, 2)]:
        xp, xm = logits.copy(), logits.copy()
        xp[r, c] += h
        xm[r, c] -= h
        fp = oracle.shifted_ce(xp, labels)
        fm = oracle.shifted_ce(xm, labels)
        num = (oracle.sp_loss_aggregate([fp[2]], [fp[3]]) - oracle.sp_loss_aggregate([fm[2]], [fm[3]])) / (2 * h)
        assert abs(num - g[r, c]) < 1e-7
