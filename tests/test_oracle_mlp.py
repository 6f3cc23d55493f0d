"""Pins of the TiledMLP oracle (the SwiGLU MLP, untiled) against torch's
float64 autograd, finite differences, closed forms and the token-tiling
invariance the method relies on."""
import numpy as np
import torch

import oracle


def _case(n=12, H=16, I=24, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, H))
    w_gu = rng.standard_normal((2 * I, H)) / np.sqrt(H)
    w_down = rng.standard_normal((H, I)) / np.sqrt(I)
    dy = rng.standard_normal((n, H))
    return x, w_gu, w_down, dy


def test_matches_torch_autograd():
    x, w_gu, w_down, dy = _case()
    I = w_down.shape[1]
    tx, tg, td = (torch.tensor(a, requires_grad=True) for a in (x, w_gu, w_down))
    y = (torch.nn.functional.silu(tx @ tg[:I].T) * (tx @ tg[I:].T)) @ td.T
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(oracle.swiglu_mlp(x, w_gu, w_down), y.detach().numpy(), atol=1e-12)
    dx, dwg, dwd = oracle.swiglu_mlp_bwd(x, w_gu, w_down, dy)
    np.testing.assert_allclose(dx, tx.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dwg, tg.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dwd, td.grad.numpy(), atol=1e-12)


def test_finite_differences():
    x, w_gu, w_down, dy = _case(n=4, H=8, I=8, seed=3)
    dx, dwg, dwd = oracle.swiglu_mlp_bwd(x, w_gu, w_down, dy)
    h = 1e-6
    f = lambda a, b, c: float(np.sum(oracle.swiglu_mlp(a, b, c) * dy))
    for arr, grad, idx in ((x, dx, (1, 3)), (w_gu, dwg, (2, 5)), (w_gu, dwg, (11, 0)), (w_down, dwd, (4, 6))):
        p, m = arr.copy(), arr.copy()
        p[idx] += h
        m[idx] -= h
        args_p = [p if a is arr else a for a in (x, w_gu, w_down)]
        args_m = [m if a is arr else a for a in (x, w_gu, w_down)]
        assert abs((f(*args_p) - f(*args_m)) / (2 * h) - grad[idx]) < 1e-7


def test_closed_forms():
    """A gate that is zero for every token while W_gate is not: x lives in
    the first half of the hidden dims and the gate rows in the second half,
    so gate = x W_gate^T = 0. Then silu(0) = 0 and d silu/dg = 1/2 give
      y = 0,  dx = (1/2) ((dy W_down) * up) W_gate,
      dW_gate = ((1/2) (dy W_down) * up)^T x,  dW_up = 0,  dW_down = 0,
    with up = x W_up^T; dx and dW_gate are not zero."""
    n, H, I = 5, 8, 6
    x, w_gu, w_down, dy = _case(n=n, H=H, I=I, seed=5)
    x[:, H // 2:] = 0.0
    w_gu[:I, :H // 2] = 0.0
    assert np.all(x @ w_gu[:I].T == 0.0) and np.any(w_gu[:I] != 0.0)
    assert np.all(oracle.swiglu_mlp(x, w_gu, w_down) == 0.0)
    dx, dwg, dwd = oracle.swiglu_mlp_bwd(x, w_gu, w_down, dy)
    up = x @ w_gu[I:].T
    dgate = 0.5 * (dy @ w_down) * up
    np.testing.assert_allclose(dx, dgate @ w_gu[:I], atol=1e-12)
    np.testing.assert_allclose(dwg[:I], dgate.T @ x, atol=1e-12)
    assert np.all(dwg[I:] == 0.0) and np.all(dwd == 0.0)
    assert np.max(np.abs(dx)) > 1e-3 and np.max(np.abs(dwg[:I])) > 1e-3


def test_token_tiles_are_independent():
    """What TiledMLP relies on: rows of y depend only on their own token, and
    the weight gradients are sums over tokens, so any tiling of the tokens
    gives the same y, dx and (summed) dW."""
    x, w_gu, w_down, dy = _case(n=10, seed=7)
    y = oracle.swiglu_mlp(x, w_gu, w_down)
    dx, dwg, dwd = oracle.swiglu_mlp_bwd(x, w_gu, w_down, dy)
    parts = [slice(0, 3), slice(3, 7), slice(7, 10)]
    np.testing.assert_allclose(np.concatenate([oracle.swiglu_mlp(x[p], w_gu, w_down) for p in parts]), y,
                               atol=1e-13)
    grads = [oracle.swiglu_mlp_bwd(x[p], w_gu, w_down, dy[p]) for p in parts]
    np.testing.assert_allclose(np.concatenate([g[0] for g in grads]), dx, atol=1e-13)
    np.testing.assert_allclose(sum(g[1] for g in grads), dwg, atol=1e-12)
    np.testing.assert_allclose(sum(g[2] for g in grads), dwd, atol=1e-12)
