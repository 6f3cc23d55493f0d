"""GPU parity of TiledMLP (SwiGLU MLP over token tiles) against the fp64
oracle, tiling invariance, gradient accumulation and argument checks."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import FWD_MAX_ABS, FWD_REL, GRAD_MAX_ABS, GRAD_REL, assert_close, dev, host, sentinel

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")


def _weights(H, I, seed):
    w_gu = workloads.normal_bf16((2 * I, H), seed=seed, sigma=1.0 / np.sqrt(H))
    w_down = workloads.normal_bf16((H, I), seed=seed + 1, sigma=1.0 / np.sqrt(I))
    return w_gu, w_down


class Mlp:
    def __init__(self, n, H, I, seed):
        self.n, self.H, self.I = n, H, I
        self.x_b = workloads.normal_bf16((n, H), seed=seed + 2)
        self.dy_b = workloads.normal_bf16((n, H), seed=seed + 3)
        self.wg_b, self.wd_b = _weights(H, I, seed)
        self.x, self.dy, self.wg, self.wd = dev(self.x_b), dev(self.dy_b), dev(self.wg_b), dev(self.wd_b)

    def run(self, tile, accumulate=False, dwg=None, dwd=None):
        y = sentinel((self.n, self.H))
        uly.tiled_mlp_fwd(self.x, self.wg, self.wd, y, tile)
        dx = sentinel((self.n, self.H))
        if dwg is None:
            dwg = torch.full((2 * self.I, self.H), float("nan"), device="cuda")
            dwd = torch.full((self.H, self.I), float("nan"), device="cuda")
        uly.tiled_mlp_bwd(self.x, self.wg, self.wd, self.dy, dx, dwg, dwd, tile, accumulate)
        torch.cuda.synchronize()
        return host(y), host(dx), dwg, dwd


@pytest.mark.parametrize("n,H,I,tile", [(100, 64, 96, 32), (37, 128, 256, 37), (5, 16, 24, 2)])
def test_mlp_matches_oracle(n, H, I, tile):
    print("mlp n=%d H=%d I=%d tile=%d" % (n, H, I, tile), flush=True)
    m = Mlp(n, H, I, seed=n + H)
    y, dx, dwg, dwd = m.run(tile)
    y_ref = oracle.swiglu_mlp(m.x_b, m.wg_b, m.wd_b)
    dx_ref, dwg_ref, dwd_ref = oracle.swiglu_mlp_bwd(m.x_b, m.wg_b, m.wd_b, m.dy_b)
    assert_close("y", oracle.bf16_to_f64(y), y_ref, FWD_MAX_ABS, FWD_REL)
    assert_close("dx", oracle.bf16_to_f64(dx), dx_ref, GRAD_MAX_ABS, GRAD_REL)
    # weight gradients are sums over all n tokens, so their max-abs bar is
    # the gradient bar relative to the largest entry
    assert_close("dW_gu", dwg.cpu().numpy().astype(np.float64), dwg_ref, GRAD_MAX_ABS * np.abs(dwg_ref).max(),
                 GRAD_REL)
    assert_close("dW_down", dwd.cpu().numpy().astype(np.float64), dwd_ref, GRAD_MAX_ABS * np.abs(dwd_ref).max(),
                 GRAD_REL)


def test_tile_size_does_not_change_the_result():
    m = Mlp(96, 64, 128, seed=5)
    a = m.run(96)
    b = m.run(7)
    f = oracle.bf16_to_f64
    assert_close("y tiles", f(b[0]), f(a[0]), 1e-2, 1e-2)
    assert_close("dx tiles", f(b[1]), f(a[1]), 1e-2, 1e-2)
    assert_close("dW_gu tiles", b[2].cpu().numpy().astype(np.float64), a[2].cpu().numpy().astype(np.float64), 1e-2,
                 1e-3)


def test_accumulate_adds_weight_gradients():
    m = Mlp(40, 32, 64, seed=9)
    _, _, dwg, dwd = m.run(16)
    g1, d1 = dwg.clone(), dwd.clone()
    m.run(16, accumulate=True, dwg=dwg, dwd=dwd)
    np.testing.assert_allclose(dwg.cpu().numpy(), 2 * g1.cpu().numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dwd.cpu().numpy(), 2 * d1.cpu().numpy(), rtol=1e-5, atol=1e-6)


def test_full_size_sampled_rows():
    """Qwen3-4B MLP shape (H = 2560, I = 9728) on 2048 tokens in tiles of
    512. Token rows are independent, so sampled rows of y and dx are checked
    against the oracle one by one. The weight gradients of intermediate unit
    j (rows j and I + j of dW_gu, column j of dW_down) depend only on x, dy
    and that unit's own weights, so the oracle run over all 2048 tokens with
    only the sampled units' weights gives their exact values."""
    n, H, I = 2048, 2560, 9728
    m = Mlp(n, H, I, seed=21)
    y, dx, dwg, dwd = m.run(512)
    rows = np.array([0, 1, 511, 512, 1000, 2047])
    y_ref = oracle.swiglu_mlp(m.x_b[rows], m.wg_b, m.wd_b)
    dx_ref, _, _ = oracle.swiglu_mlp_bwd(m.x_b[rows], m.wg_b, m.wd_b, m.dy_b[rows])
    assert_close("y rows", oracle.bf16_to_f64(y[rows]), y_ref, FWD_MAX_ABS, FWD_REL)
    assert_close("dx rows", oracle.bf16_to_f64(dx[rows]), dx_ref, GRAD_MAX_ABS, GRAD_REL)
    units = np.array([0, 1, 2047, 4864, 9000, I - 1])
    gu_rows = np.concatenate([units, I + units])
    _, dwg_ref, dwd_ref = oracle.swiglu_mlp_bwd(m.x_b, m.wg_b[gu_rows], m.wd_b[:, units], m.dy_b)
    dwg_s = dwg.cpu().numpy().astype(np.float64)[gu_rows]
    dwd_s = dwd.cpu().numpy().astype(np.float64)[:, units]
    assert_close("dW_gu units", dwg_s, dwg_ref, GRAD_MAX_ABS * np.abs(dwg_ref).max(), GRAD_REL)
    assert_close("dW_down units", dwd_s, dwd_ref, GRAD_MAX_ABS * np.abs(dwd_ref).max(), GRAD_REL)


def test_mlp_argument_errors():
    n, H, I = 8, 16, 24
    x = torch.zeros((n, H), dtype=torch.int16, device="cuda")
    wg = torch.zeros((2 * I, H), dtype=torch.int16, device="cuda")
    wd = torch.zeros((H, I), dtype=torch.int16, device="cuda")
    y = sentinel((n, H))
    small = torch.empty((1024,), dtype=torch.uint8, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.tiled_mlp_fwd(x, wg, wd, y, 4, ws=small)
    assert e.value.name == "ULY_E_WORKSPACE"
    with pytest.raises(uly.UlyssesError) as e:
        uly.tiled_mlp_fwd(x, wg, wd, x, 4)                      # y is x
    assert e.value.name == "ULY_E_ALIAS"
    x12 = torch.zeros((n, 12), dtype=torch.int16, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.tiled_mlp_fwd(x12, torch.zeros((2 * I, 12), dtype=torch.int16, device="cuda"),
                          torch.zeros((12, I), dtype=torch.int16, device="cuda"), sentinel((n, 12)), 4)
    assert e.value.name == "ULY_E_ALIGN"
    torch.cuda.synchronize()
    assert np.all(host(y) == 0xFFFF)
