"""Closed forms of causal attention and its gradients when every visible
score is zero (Q = 0 or K = 0), written to run at full sequence length.

With s_ij = 0 for all j <= i, the softmax is uniform over the i + 1 visible
keys: p_ij = w_i = 1/(i+1). The definitions of the forward and backward pass
("Ulysses Sequence Parallelism for Million-Token Context Training", "The
Challenge of Long Sequence Training": tiled attention must give the exact
result) then reduce to prefix and suffix sums (fp64, numpy):

  O_i   = w_i sum_{j<=i} v_j                 LSE_i = ln(i+1)
  D_i   = dO_i . O_i
  dV_j  = sum_{h in g} sum_{i>=j} w_i dO_i
  dQ_i  = scale w_i ( sum_{j<=i} (dO_i . v_j) k_j  -  D_i sum_{j<=i} k_j )
  dK_j  = scale sum_{h in g} ( sum_{i>=j} w_i (dO_i . v_j) q_i  -  sum_{i>=j} w_i D_i q_i )

(with Q = 0 the dK sum vanishes, with K = 0 the dQ sum does). The bilinear
sums sum_{b>=a} (x_a . y_b) z_b are evaluated in token chunks from the end:
a d x d running matrix carries everything past the chunk and a masked
chunk x chunk product the rest, so no N x N or N x d x d array is formed.
These are test helpers; they share nothing with the oracle or the HIP path.
"""
from __future__ import annotations

import numpy as np


def suffix_pair_sum(x: np.ndarray, y: np.ndarray, z: np.ndarray, chunk: int = 256) -> np.ndarray:
    """out[a] = sum_{b >= a} (x[a] . y[b]) z[b] for x, y [N, d], z [N, e]."""
    N, d = x.shape
    out = np.empty((N, z.shape[1]), dtype=np.float64)
    M = np.zeros((d, z.shape[1]), dtype=np.float64)      # sum over b past the chunk of y_b z_b^T
    for hi in range(N, 0, -chunk):
        lo = max(0, hi - chunk)
        xc, yc, zc = x[lo:hi], y[lo:hi], z[lo:hi]
        inner = np.triu(xc @ yc.T)                       # [a, b], kept where b >= a
        out[lo:hi] = xc @ M + inner @ zc
        M += yc.T @ zc
    return out


def prefix_pair_sum(x: np.ndarray, y: np.ndarray, z: np.ndarray, chunk: int = 256) -> np.ndarray:
    """out[a] = sum_{b <= a} (x[a] . y[b]) z[b] (the suffix sum on reversed tokens)."""
    return suffix_pair_sum(x[::-1], y[::-1], z[::-1], chunk)[::-1]


def uniform_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float,
                   want_dq: bool = True, want_dk: bool = True):
    """Closed forms for causal attention over one document when every
    visible score is zero. q [N, hq, d], k, v [N, hkv, d], dout [N, hq, d]
    (float64; q or k all zeros). Returns o [N, hq, d], lse [hq, N],
    dq [N, hq, d] (or None), dk, dv [N, hkv, d] (dk None when not wanted)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    w = 1.0 / np.arange(1, N + 1, dtype=np.float64)
    o = np.empty((N, hq, d))
    dq = np.zeros((N, hq, d)) if want_dq else None
    dk = np.zeros((N, hkv, d)) if want_dk else None
    dv = np.zeros((N, hkv, d))
    for g in range(hkv):
        mean_v = np.cumsum(v[:, g], axis=0) * w[:, None]
        ksum = np.cumsum(k[:, g], axis=0)
        for h in range(g * G, (g + 1) * G):
            o[:, h] = mean_v
            D = np.einsum("nd,nd->n", dout[:, h], mean_v)
            wdo = dout[:, h] * w[:, None]
            dv[:, g] += np.cumsum(wdo[::-1], axis=0)[::-1]
            if want_dq:
                dq[:, h] = scale * w[:, None] * (prefix_pair_sum(dout[:, h], v[:, g], k[:, g])
                                                 - D[:, None] * ksum)
            if want_dk:
                tail = np.cumsum((w * D)[::-1, None] * q[::-1, h], axis=0)[::-1]
                dk[:, g] += scale * (suffix_pair_sum(v[:, g], wdo, q[:, h]) - tail)
    lse = np.broadcast_to(np.log(np.arange(1, N + 1, dtype=np.float64)), (hq, N))
    return o, lse, dq, dk, dv
