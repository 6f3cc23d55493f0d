"""Pins for the oracle's attention forward and backward (CPU only).

Pinned to: PyTorch's CPU scaled_dot_product_attention and autograd in
float64 (a library routine the definition reduces to), central finite
differences, closed forms (Q = 0, K = 0, constant V, constant K, first row) and
invariants (causality, documents, head-shard concatenation, GQA as repeated
KV heads).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _mask(N, causal, cu):
    m = np.ones((N, N), dtype=bool)
    if causal:
        m &= np.tril(np.ones((N, N), dtype=bool))
    if cu is not None:
        doc = np.searchsorted(cu, np.arange(N), side="right") - 1
        m &= doc[:, None] == doc[None, :]
    return m


def _torch_ref(q, k, v, scale, causal, cu, dout=None):
    """Library reference: torch SDPA in float64 with KV heads repeated per group."""
    N, hq, d = q.shape
    G = hq // k.shape[1]
    tq = torch.tensor(q.transpose(1, 0, 2)[None], requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2)[None], requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2)[None], requires_grad=True)
    mask = torch.tensor(_mask(N, causal, cu))
    out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1),
                                         attn_mask=mask, scale=scale)
    scores = (tq @ tk.repeat_interleave(G, dim=1).transpose(-1, -2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)[0]
    res = {"o": out[0].detach().numpy().transpose(1, 0, 2), "lse": lse.detach().numpy()}
    if dout is not None:
        (out * torch.tensor(dout.transpose(1, 0, 2)[None])).sum().backward()
        res["dq"] = tq.grad[0].numpy().transpose(1, 0, 2)
        res["dk"] = tk.grad[0].numpy().transpose(1, 0, 2)
        res["dv"] = tv.grad[0].numpy().transpose(1, 0, 2)
    return res


CASES = [
    # N, hq, hkv, d, causal, cu
    (37, 4, 2, 16, True, None),
    (37, 4, 2, 16, False, None),
    (64, 2, 2, 8, True, None),
    (50, 4, 1, 8, True, [0, 7, 8, 30, 50]),
    (50, 3, 3, 8, False, [0, 20, 21, 50]),
]


@pytest.mark.parametrize("N,hq,hkv,d,causal,cu", CASES)
def test_fwd_bwd_vs_torch_sdpa(N, hq, hkv, d, causal, cu):
    q, k, v = _rand((N, hq, d), 1), _rand((N, hkv, d), 2), _rand((N, hkv, d), 3)
    dout = _rand((N, hq, d), 4)
    scale = 1.0 / np.sqrt(d)
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    ref = _torch_ref(q, k, v, scale, causal, cu_a, dout)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, cu_a)
    np.testing.assert_allclose(o, ref["o"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-12, atol=1e-12)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, scale, causal, cu_a)
    np.testing.assert_allclose(dq, ref["dq"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, ref["dk"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, ref["dv"], rtol=1e-10, atol=1e-11)


def test_bwd_central_differences():
    N, hq, hkv, d = 16, 2, 1, 8
    q, k, v = _rand((N, hq, d), 11), _rand((N, hkv, d), 12), _rand((N, hkv, d), 13)
    dout = _rand((N, hq, d), 14)
    scale = 0.37

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, scale, True)
        return float(np.sum(o * dout))

    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, scale, True)
    eps = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a_p, a_m = arr.copy(), arr.copy()
            a_p[idx] += eps
            a_m[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = a_p, a_m
            fd[idx] = (loss(**{x + "_": args_p[x] for x in "qkv"}) -
                       loss(**{x + "_": args_m[x] for x in "qkv"})) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("cu", [None, [0, 5, 6, 40, 64]])
def test_q_zero_closed_forms(cu):
    """Q = 0: every allowed key has the same score, so o_i is the mean of the
    allowed values, LSE_i = ln |A(i)|, dK = 0 and dV_j = sum_{i sees j} dO_i / |A(i)|."""
    N, hq, hkv, d = 64, 4, 2, 8
    G = hq // hkv
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    q = np.zeros((N, hq, d))
    k, v = _rand((N, hkv, d), 21), _rand((N, hkv, d), 22)
    dout = _rand((N, hq, d), 23)
    o, lse = oracle.attn_fwd(q, k, v, 0.125, True, cu_a)
    starts = np.zeros(N, dtype=np.int64) if cu is None else np.array(cu)[np.searchsorted(cu, np.arange(N), "right") - 1]
    cnt = np.arange(N) - starts + 1
    csum = np.cumsum(v, axis=0)
    for i in range(N):
        tot = csum[i] - (csum[starts[i] - 1] if starts[i] > 0 else 0)
        mean = tot / cnt[i]
        for h in range(hq):
            np.testing.assert_allclose(o[i, h], mean[h // G], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(cnt), (hq, N)), rtol=1e-13, atol=1e-13)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, 0.125, True, cu_a)
    assert np.max(np.abs(dk)) == 0.0
    w = dout / cnt[:, None, None]                       # dO_i / |A(i)|
    for j in range(N):
        end = N if cu is None else np.array(cu)[np.searchsorted(cu, j, "right")]
        for g in range(hkv):
            ref = w[j:end, g * G:(g + 1) * G, :].sum(axis=(0, 1))
            np.testing.assert_allclose(dv[j, g], ref, rtol=1e-11, atol=1e-12)


def _doc_bounds(N, cu):
    """Start and end (exclusive) of the document holding each token."""
    if cu is None:
        return np.zeros(N, dtype=np.int64), np.full(N, N, dtype=np.int64)
    cu = np.asarray(cu)
    b = np.searchsorted(cu, np.arange(N), "right") - 1
    return cu[b].astype(np.int64), cu[b + 1].astype(np.int64)


@pytest.mark.parametrize("cu", [None, [0, 5, 6, 40, 64]])
def test_q_zero_dq_closed_form(cu):
    """Q = 0 makes every allowed score 0, so p_ij = 1/|A(i)| and
    dQ_i = scale/|A(i)| * (sum_j (dO_i . v_j) k_j - D_i sum_j k_j), with
    D_i = dO_i . mean_j v_j. The sums over j are prefix sums inside the
    document: sum_j v_j k_j^T (a d x d matrix) and sum_j k_j."""
    N, hq, hkv, d = 64, 4, 2, 8
    G, scale = hq // hkv, 0.2
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    q = np.zeros((N, hq, d))
    k, v = _rand((N, hkv, d), 24), _rand((N, hkv, d), 25)
    dout = _rand((N, hq, d), 26)
    dq, _, _ = oracle.attn_bwd(q, k, v, dout, scale, True, cu_a)
    start, _ = _doc_bounds(N, cu)
    vk = np.cumsum(np.einsum("ngd,nge->ngde", v, k), axis=0)     # prefix sum of v_j k_j^T
    ks, vs = np.cumsum(k, axis=0), np.cumsum(v, axis=0)
    pre = lambda c, i: c[i] - (c[start[i] - 1] if start[i] > 0 else 0)  # noqa: E731
    for i in range(N):
        cnt = i - start[i] + 1
        m_vk, s_k, s_v = pre(vk, i), pre(ks, i), pre(vs, i)
        for h in range(hq):
            g = h // G
            dsum = dout[i, h] @ m_vk[g]                         # sum_j (dO_i . v_j) k_j
            D = dout[i, h] @ (s_v[g] / cnt)
            ref = scale / cnt * (dsum - D * s_k[g])
            np.testing.assert_allclose(dq[i, h], ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("cu", [None, [0, 9, 10, 33, 64]])
def test_k_zero_closed_forms(cu):
    """K = 0 also makes p_ij = 1/|A(i)|: dQ = 0, dV as for Q = 0, and
    dK_j = scale * sum_{h in g} sum_{i sees j} (dO_i . v_j - D_i) q_i / |A(i)|,
    i.e. suffix sums (inside the document) of q_i dO_i^T / |A(i)| applied to
    v_j, minus suffix sums of D_i q_i / |A(i)|."""
    N, hq, hkv, d = 64, 4, 2, 8
    G, scale = hq // hkv, 0.3
    cu_a = None if cu is None else np.array(cu, dtype=np.int32)
    q, v = _rand((N, hq, d), 27), _rand((N, hkv, d), 28)
    k = np.zeros((N, hkv, d))
    dout = _rand((N, hq, d), 29)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, scale, True, cu_a)
    assert np.max(np.abs(dq)) == 0.0
    start, end = _doc_bounds(N, cu)
    cnt = np.arange(N) - start + 1
    vs = np.cumsum(v, axis=0)
    mean_v = np.stack([(vs[i] - (vs[start[i] - 1] if start[i] > 0 else 0)) / cnt[i] for i in range(N)])
    D = np.einsum("nhd,nhd->nh", dout, mean_v[:, np.arange(hq) // G])       # dO_i . o_i
    w = 1.0 / cnt[:, None, None]
    qdo = np.cumsum((np.einsum("nhd,nhe->nhde", q, dout) * w[..., None])[::-1], axis=0)[::-1]
    dqs = np.cumsum((D[..., None] * q * w)[::-1], axis=0)[::-1]
    dos = np.cumsum((dout * w)[::-1], axis=0)[::-1]
    suf = lambda c, j: c[j] - (c[end[j]] if end[j] < N else 0)  # noqa: E731
    for j in range(N):
        s_qdo, s_dq, s_do = suf(qdo, j), suf(dqs, j), suf(dos, j)
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            ref_k = scale * ((s_qdo[hs] @ v[j, g]).sum(axis=0) - s_dq[hs].sum(axis=0))
            np.testing.assert_allclose(dk[j, g], ref_k, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(dv[j, g], s_do[hs].sum(axis=0), rtol=1e-10, atol=1e-12)


def test_constant_v_and_constant_k():
    N, hq, hkv, d = 40, 2, 1, 8
    q, k = _rand((N, hq, d), 31), _rand((N, hkv, d), 32)
    vrow = _rand((1, 1, d), 33)
    v = np.broadcast_to(vrow, (N, hkv, d)).copy()
    dout = _rand((N, hq, d), 34)
    o, _ = oracle.attn_fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, (N, hq, d)), rtol=1e-13, atol=1e-14)   # rows of p sum to 1
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, 0.3, True)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    kc = np.broadcast_to(_rand((1, 1, d), 35), (N, hkv, d)).copy()
    v2 = _rand((N, hkv, d), 36)
    dq2, _, _ = oracle.attn_bwd(q, kc, v2, dout, 0.3, True)
    assert np.max(np.abs(dq2)) < 1e-12


def test_first_row_of_each_document_is_its_value():
    N, hq, hkv, d = 48, 2, 1, 8
    cu = np.array([0, 10, 11, 30, 48], dtype=np.int32)
    q, k, v = _rand((N, hq, d), 41), _rand((N, hkv, d), 42), _rand((N, hkv, d), 43)
    o, _ = oracle.attn_fwd(q, k, v, 0.5, True, cu)
    for s in cu[:-1]:
        for h in range(hq):
            np.testing.assert_array_equal(o[s, h], v[s, 0])


def test_causality_perturb_future():
    N, hq, hkv, d = 40, 2, 1, 8
    q, k, v = _rand((N, hq, d), 51), _rand((N, hkv, d), 52), _rand((N, hkv, d), 53)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.4, True)
    i = 17
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[i + 1:] += 1.0
    k2[i + 1:] -= 2.0
    v2[i + 1:] *= 3.0
    o2, l2 = oracle.attn_fwd(q2, k2, v2, 0.4, True)
    assert np.array_equal(o1[:i + 1], o2[:i + 1]) and np.array_equal(l1[:, :i + 1], l2[:, :i + 1])


def test_varlen_equals_per_document_dense():
    N, hq, hkv, d = 60, 4, 2, 8
    cu = np.array([0, 13, 14, 41, 60], dtype=np.int32)
    q, k, v = _rand((N, hq, d), 61), _rand((N, hkv, d), 62), _rand((N, hkv, d), 63)
    dout = _rand((N, hq, d), 64)
    o, lse = oracle.attn_fwd(q, k, v, 0.35, True, cu)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, 0.35, True, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        od, ld = oracle.attn_fwd(q[a:b], k[a:b], v[a:b], 0.35, True)
        np.testing.assert_allclose(o[a:b], od, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], ld, rtol=1e-13, atol=1e-14)
        qd, kd, vd = oracle.attn_bwd(q[a:b], k[a:b], v[a:b], dout[a:b], 0.35, True)
        np.testing.assert_allclose(dq[a:b], qd, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dk[a:b], kd, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv[a:b], vd, rtol=1e-12, atol=1e-13)


def test_head_shards_concatenate_to_full_heads():
    """Ulysses composition: the P rank results, side by side, are the full-head run."""
    w = workloads.WORKLOADS["tiny"]
    X = oracle.bf16_to_f64(workloads.gen_x(w, range(w.Ht)))
    dY = oracle.bf16_to_f64(workloads.gen_dy(w, range(w.Hq)))
    Q, K, V = X[:, :w.Hq], X[:, w.Hq:w.Hq + w.Hkv], X[:, w.Hq + w.Hkv:]
    o_full, lse_full = oracle.attn_fwd(Q, K, V, w.scale, True)
    rows = np.array([0, 1, 127, 128, 129, 255])
    dq_full, dk_full, dv_full = oracle.attn_bwd(Q, K, V, dY, w.scale, True, rows=rows, key_lo=192)
    for r in range(w.P):
        sh = oracle.bf16_to_f64(workloads.gen_head_shard(w, r))
        q, k, v = sh[:, :w.hq], sh[:, w.hq:w.hq + w.hkv], sh[:, w.hq + w.hkv:]
        o, lse = oracle.attn_fwd(q, k, v, w.scale, True)
        hs = slice(r * w.hq, (r + 1) * w.hq)
        ks = slice(r * w.hkv, (r + 1) * w.hkv)
        assert np.array_equal(o, o_full[:, hs]) and np.array_equal(lse, lse_full[hs])
        dq, dk, dv = oracle.attn_bwd(q, k, v, dY[:, hs], w.scale, True, rows=rows, key_lo=192)
        assert np.array_equal(dq, dq_full[:, hs])
        assert np.array_equal(dk, dk_full[:, ks]) and np.array_equal(dv, dv_full[:, ks])


def test_gqa_equals_repeated_kv_heads():
    N, hq, hkv, d = 30, 4, 2, 8
    G = hq // hkv
    q, k, v = _rand((N, hq, d), 71), _rand((N, hkv, d), 72), _rand((N, hkv, d), 73)
    dout = _rand((N, hq, d), 74)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, True)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o2, lse2 = oracle.attn_fwd(q, kr, vr, 0.3, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, 0.3, True)
    dq2, dk2, dv2 = oracle.attn_bwd(q, kr, vr, dout, 0.3, True)
    np.testing.assert_array_equal(dq, dq2)
    np.testing.assert_allclose(dk, dk2.reshape(N, hkv, G, d).sum(axis=2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(N, hkv, G, d).sum(axis=2), rtol=1e-13, atol=1e-14)


def test_sampled_rows_and_key_ranges_match_full():
    N, hq, hkv, d = 45, 2, 1, 8
    q, k, v = _rand((N, hq, d), 81), _rand((N, hkv, d), 82), _rand((N, hkv, d), 83)
    dout = _rand((N, hq, d), 84)
    for cu in (None, np.array([0, 9, 30, 45], dtype=np.int32)):
        o, lse = oracle.attn_fwd(q, k, v, 0.3, True, cu)
        dq, dk, dv = oracle.attn_bwd(q, k, v, dout, 0.3, True, cu)
        rows = np.array([44, 0, 13, 30])
        o_s, lse_s = oracle.attn_fwd(q, k, v, 0.3, True, cu, rows=rows)
        np.testing.assert_array_equal(o_s, o[rows])
        np.testing.assert_array_equal(lse_s, lse[:, rows])
        dq_s, dk_s, dv_s = oracle.attn_bwd(q, k, v, dout, 0.3, True, cu, rows=rows, key_lo=20, key_hi=33)
        np.testing.assert_allclose(dq_s, dq[rows], rtol=0, atol=0)
        np.testing.assert_allclose(dk_s, dk[20:33], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dv_s, dv[20:33], rtol=1e-14, atol=1e-15)


def test_plants_are_caught():
    """A wrong scale, a dropped diagonal or a transposed GQA map must fail the torch pin."""
    N, hq, hkv, d = 20, 4, 2, 8
    q, k, v = _rand((N, hq, d), 91), _rand((N, hkv, d), 92), _rand((N, hkv, d), 93)
    ref = _torch_ref(q, k, v, 0.3, True, None)
    o_scale, _ = oracle.attn_fwd(q, k, v, 0.31, True)
    assert np.max(np.abs(o_scale - ref["o"])) > 1e-4
    # interleaved GQA (h % hkv) instead of contiguous groups differs
    ref_inter = _torch_ref(q[:, [0, 2, 1, 3]], k, v, 0.3, True, None)["o"][:, [0, 2, 1, 3]]
    o, _ = oracle.attn_fwd(q, k, v, 0.3, True)
    assert np.max(np.abs(o - ref_inter)) > 1e-4
    # strictly-lower mask differs from the diagonal-inclusive one at every row > 0
    o_strict = _torch_ref(q, k, v, 0.3, False, None)
    assert np.max(np.abs(o - o_strict["o"])) > 1e-4
