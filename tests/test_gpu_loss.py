"""GPU parity of the shifted-label loss, its aggregation over SP ranks and
its gradient, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._gpu import GRAD_MAX_ABS, GRAD_REL, assert_close, dev, host, sentinel

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")


def _labels(n, V, seed, ignore_every=4):
    rng = np.random.default_rng(seed)
    lab = rng.integers(0, V, size=n).astype(np.int32)
    lab[::ignore_every] = -100
    return lab


class Rank:
    def __init__(self, logits_bits, labels):
        self.n, self.V = logits_bits.shape
        self.bits = logits_bits
        self.labels_np = labels
        self.logits = dev(logits_bits)
        self.labels = torch.from_numpy(labels.astype(np.int32)).cuda()
        self.row_loss = torch.full((self.n,), float("nan"), device="cuda")
        self.row_lse = torch.full((self.n,), float("nan"), device="cuda")
        self.loss = torch.full((1,), float("nan"), device="cuda")
        self.good = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def fwd(self):
        uly.shifted_ce_fwd(self.logits, self.labels, self.row_loss, self.row_lse, self.loss, self.good)


@pytest.mark.parametrize("n,V,sigma", [(37, 1000, 2.0), (3, 151936, 2.0), (64, 8, 4.0)])
def test_rank_loss_matches_oracle(n, V, sigma):
    print("loss n=%d V=%d" % (n, V), flush=True)
    bits = workloads.normal_bf16((n, V), seed=n + V, sigma=sigma)
    lab = _labels(n, V, seed=n)
    lab[1] = V + 3                          # outside [0, V): no loss, like -100
    r = Rank(bits, lab)
    r.fwd()
    torch.cuda.synchronize()
    row_loss, row_lse, loss, good = oracle.shifted_ce(bits, lab)
    assert int(r.good.item()) == good
    assert np.max(np.abs(r.row_lse.cpu().numpy() - row_lse)) <= 1e-4
    assert np.max(np.abs(r.row_loss.cpu().numpy() - row_loss)) <= 1e-4
    assert abs(r.loss.item() - loss) <= 1e-4


def test_rank_without_good_tokens():
    bits = workloads.normal_bf16((5, 64), seed=3)
    r = Rank(bits, np.full(5, -100, dtype=np.int32))
    r.fwd()
    total = torch.full((1,), float("nan"), device="cuda")
    scale = torch.full((1,), float("nan"), device="cuda")
    uly.sp_loss_aggregate([r.loss], [r.good], total, scale)
    g = sentinel((5, 64))
    uly.shifted_ce_bwd(r.logits, r.labels, r.row_lse, scale, g)
    torch.cuda.synchronize()
    assert r.good.item() == 0 and r.loss.item() == 0.0 and total.item() == 0.0 and scale.item() == 1.0
    assert np.all(host(g) == 0)


@pytest.mark.parametrize("P,n,V", [(4, 24, 512), (2, 50, 2048)])
def test_sp_step_loss_and_gradient(P, n, V):
    """P ranks of one sequence: per-rank losses from shifted labels, their
    weighted aggregate (== the loss of the whole sequence on one device) and
    the gradient of that aggregate with respect to every rank's logits."""
    print("sp loss P=%d n=%d V=%d" % (P, n, V), flush=True)
    N = P * n
    bits = workloads.normal_bf16((N, V), seed=N * 3 + V, sigma=2.0)
    tokens = np.random.default_rng(N).integers(0, V, size=N)
    labels = oracle.shift_labels(tokens).astype(np.int32)
    labels[: n + n // 2] = -100                # prompt: rank 0 has no good tokens
    ranks = [Rank(np.ascontiguousarray(bits[r * n:(r + 1) * n]), labels[r * n:(r + 1) * n]) for r in range(P)]
    for rk in ranks:
        rk.fwd()
    total = torch.full((1,), float("nan"), device="cuda")
    scale = torch.full((1,), float("nan"), device="cuda")
    uly.sp_loss_aggregate([rk.loss for rk in ranks], [rk.good for rk in ranks], total, scale)
    grads = []
    for rk in ranks:
        g = sentinel((n, V))
        uly.shifted_ce_bwd(rk.logits, rk.labels, rk.row_lse, scale, g)
        grads.append(g)
    torch.cuda.synchronize()
    whole = oracle.shifted_ce(bits, labels)
    assert abs(total.item() - whole[2]) <= 1e-4
    G = whole[3]
    assert abs(scale.item() * max(G, 1) - 1.0) <= 1e-6     # a float32 reciprocal
    for r, (rk, g) in enumerate(zip(ranks, grads)):
        ref = oracle.shifted_ce_grad(rk.bits, rk.labels_np, G)
        got = oracle.bf16_to_f64(host(g))
        if np.any(ref != 0):
            assert_close("dlogits rank %d" % r, got, ref, GRAD_MAX_ABS, GRAD_REL)
        else:
            assert np.all(got == 0)
    # in place: the gradient overwrites the logits with the same bits
    rk = ranks[-1]
    out_of_place = host(grads[-1])
    uly.shifted_ce_bwd(rk.logits, rk.labels, rk.row_lse, scale, rk.logits)
    torch.cuda.synchronize()
    assert np.array_equal(host(rk.logits), out_of_place)


def test_loss_argument_errors():
    n, V = 16, 64
    x = torch.zeros((n, V), dtype=torch.int16, device="cuda")
    lab = torch.zeros((n,), dtype=torch.int32, device="cuda")
    f = torch.zeros((n,), dtype=torch.float32, device="cuda")
    f2 = torch.zeros((n,), dtype=torch.float32, device="cuda")
    s = torch.zeros((1,), dtype=torch.float32, device="cuda")
    gi = torch.zeros((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.shifted_ce_fwd(torch.zeros((n, 60), dtype=torch.int16, device="cuda"), lab, f, f2, s, gi)
    assert e.value.name == "ULY_E_ALIGN"
    with pytest.raises(uly.UlyssesError) as e:
        uly.shifted_ce_fwd(x, lab, f, f, s, gi)                      # row_loss is row_lse
    assert e.value.name == "ULY_E_ALIAS"
    with pytest.raises(uly.UlyssesError) as e:
        uly.sp_loss_aggregate([s] * 17, [gi] * 17, s.clone(), s.clone())
    assert e.value.name == "ULY_E_SHAPE"
    big = torch.zeros((n + 1, V), dtype=torch.int16, device="cuda")
    with pytest.raises(uly.UlyssesError) as e:
        uly.shifted_ce_bwd(big[:n], lab, f, s, big[1:])              # partial overlap
    assert e.value.name == "ULY_E_ALIAS"
    with pytest.raises(ValueError):
        uly.shifted_ce_bwd(x, lab, f, s, big[2:])                    # dlogits one row short
    with pytest.raises(ValueError):
        uly.shifted_ce_fwd(x, lab.float(), f, f2, s, gi)             # labels must be int32
