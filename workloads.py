"""Seeded synthetic workloads for the Ulysses head-shard path.

This module only describes shapes and draws random numbers. It holds none of
the method's arithmetic (no permutation, no attention), so that both the
oracle and the HIP path can consume identical bits from it without sharing
any code with each other.

Workload shapes follow the Qwen3-4B attention geometry used by the
"Ulysses Sequence Parallelism for Million-Token Context Training" page
(Performance Benchmarks): 32 query heads, 8 KV heads, head_dim 128, split
over P sequence-parallel ranks.

Random streams are blocked per (kind, head, token block) so that any head
range or token range can be drawn without generating the whole tensor:
stream = numpy PCG64 seeded with [seed, kind, head, block], drawing
``block * d`` float32 standard normals in token-major order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

KIND_X = 1      # fused QKV activations [N, Hq + 2*Hkv, d]
KIND_DY = 2     # upstream gradient of the attention output [N, Hq, d]
KIND_DOCS = 3   # packed document lengths
TOKEN_BLOCK = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int              # total tokens of the sequence (all simulated ranks)
    P: int              # simulated sequence-parallel degree
    Hq: int             # query heads of the model
    Hkv: int            # key/value heads of the model
    d: int              # head dim
    x_sigma: float      # X ~ N(0,1) * x_sigma, rounded to bf16
    seed: int
    causal: bool = True
    varlen: bool = False
    doc_lo: int = 512
    doc_hi: int = 8192

    @property
    def n(self) -> int:           # tokens per simulated rank
        return self.N // self.P

    @property
    def Ht(self) -> int:          # fused q|k|v heads
        return self.Hq + 2 * self.Hkv

    @property
    def hq(self) -> int:
        return self.Hq // self.P

    @property
    def hkv(self) -> int:
        return self.Hkv // self.P

    @property
    def ht(self) -> int:
        return self.ht_of(self.P)

    def ht_of(self, P: int) -> int:
        return (self.Hq + 2 * self.Hkv) // P

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def segments(self) -> List[int]:
        return [self.Hq, self.Hkv, self.Hkv]


# The five workloads: a tiny two-rank check, Qwen3-4B-shaped SP=4 shards at
# 8K and 64K tokens, a packed variable-length batch, and an SP=8 shard at 256K.
WORKLOADS = {
    "tiny": Workload("tiny", N=256, P=2, Hq=4, Hkv=2, d=64, x_sigma=1.0, seed=0x5EED + 0),
    "8k": Workload("8k", N=8192, P=4, Hq=32, Hkv=8, d=128, x_sigma=0.5, seed=0x5EED + 1),
    "64k": Workload("64k", N=65536, P=4, Hq=32, Hkv=8, d=128, x_sigma=0.5, seed=0x5EED + 2),
    "varlen": Workload("varlen", N=65536, P=4, Hq=32, Hkv=8, d=128, x_sigma=0.5,
                       seed=0x5EED + 3, varlen=True),
    "256k": Workload("256k", N=262144, P=8, Hq=32, Hkv=8, d=128, x_sigma=0.5, seed=0x5EED + 4),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_normals(seed: int, kind: int, head: int, block: int, count: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, kind, head, block])))
    return rng.standard_normal(count, dtype=np.float32)


def head_stream(seed: int, kind: int, head: int, t0: int, t1: int, d: int, sigma: float) -> np.ndarray:
    """bf16 bits [t1 - t0, d] of head ``head`` for tokens [t0, t1)."""
    out = np.empty((t1 - t0, d), dtype=np.uint16)
    b0, b1 = t0 // TOKEN_BLOCK, (t1 - 1) // TOKEN_BLOCK
    for b in range(b0, b1 + 1):
        vals = _block_normals(seed, kind, head, b, TOKEN_BLOCK * d).reshape(TOKEN_BLOCK, d)
        if sigma != 1.0:
            vals = vals * np.float32(sigma)
        lo = max(t0, b * TOKEN_BLOCK)
        hi = min(t1, (b + 1) * TOKEN_BLOCK)
        out[lo - t0:hi - t0] = f32_to_bf16_bits(vals[lo - b * TOKEN_BLOCK:hi - b * TOKEN_BLOCK])
    return out


def gen_x(w: Workload, heads: Sequence[int], t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """Fused activations X[t0:t1, heads, :] as bf16 bits [t1-t0, len(heads), d]."""
    t1 = w.N if t1 is None else t1
    out = np.empty((t1 - t0, len(heads), w.d), dtype=np.uint16)
    for i, h in enumerate(heads):
        out[:, i, :] = head_stream(w.seed, KIND_X, h, t0, t1, w.d, w.x_sigma)
    return out


def gen_dy(w: Workload, heads: Sequence[int], t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """Upstream gradient dY[t0:t1, heads, :] (query heads) ~ N(0,1), bf16 bits."""
    t1 = w.N if t1 is None else t1
    out = np.empty((t1 - t0, len(heads), w.d), dtype=np.uint16)
    for i, h in enumerate(heads):
        out[:, i, :] = head_stream(w.seed, KIND_DY, h, t0, t1, w.d, 1.0)
    return out


def gen_seq_shard(w: Workload, s: int) -> np.ndarray:
    """Rank s's sequence shard of the fused activations: [n, Ht, d] bf16 bits."""
    return gen_x(w, range(w.Ht), s * w.n, (s + 1) * w.n)


def gen_dy_seq_shard(w: Workload, s: int) -> np.ndarray:
    return gen_dy(w, range(w.Hq), s * w.n, (s + 1) * w.n)


def rank_heads(w: Workload, r: int) -> List[int]:
    """Fused-head indices (into X's head axis) that rank r owns after the
    sequence-to-head exchange, in local order [q..., k..., v...].

    Contiguous head blocks per rank, as the intro diagram of the
    "Ulysses sequence parallelism" page draws them (GPU 0 gets the first half
    of the heads, GPU 1 the second)."""
    hq, hkv = w.hq, w.hkv
    q = [r * hq + c for c in range(hq)]
    k = [w.Hq + r * hkv + c for c in range(hkv)]
    v = [w.Hq + w.Hkv + r * hkv + c for c in range(hkv)]
    return q + k + v


def gen_head_shard(w: Workload, r: int) -> np.ndarray:
    """Rank r's head shard over the full sequence: [N, ht, d] bf16 bits."""
    return gen_x(w, rank_heads(w, r))


def gen_dy_head_shard(w: Workload, r: int) -> np.ndarray:
    return gen_dy(w, [r * w.hq + c for c in range(w.hq)])


def doc_lengths(w: Workload) -> List[int]:
    """Packed-document lengths: integers uniform in [doc_lo, doc_hi] drawn until
    the total reaches N, the last one truncated so the total is exactly N."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, KIND_DOCS])))
    lens: List[int] = []
    total = 0
    while total < w.N:
        L = int(rng.integers(w.doc_lo, w.doc_hi, endpoint=True))
        L = min(L, w.N - total)
        lens.append(L)
        total += L
    return lens


def cu_seqlens(w: Workload) -> np.ndarray:
    if not w.varlen:
        return np.array([0, w.N], dtype=np.int32)
    lens = doc_lengths(w)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def random_cu_seqlens(N: int, seed: int, lo: int, hi: int) -> np.ndarray:
    """Small helper for tests: document lengths uniform in [lo, hi], last truncated."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, KIND_DOCS, N])))
    lens = []
    total = 0
    while total < N:
        L = min(int(rng.integers(lo, hi, endpoint=True)), N - total)
        lens.append(L)
        total += L
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def normal_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, sigma^2) tensor rounded to bf16 bits (for tests)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    vals = rng.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(vals).reshape(shape)


# Vocabulary of the Qwen3-4B-shaped workloads (the model the pages benchmark).
VOCAB = 151936


def gen_normal_device(shape, seed: int, sigma: float = 1.0):
    """N(0, sigma^2) values rounded to bf16, as bit patterns (int16), drawn
    directly on the GPU with torch's seeded generator (large inputs do not
    round-trip through the host)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device="cuda", dtype=torch.bfloat16)
    x.mul_(sigma)
    return x.view(torch.int16)


def gen_logits_device(n: int, V: int, seed: int, sigma: float = 2.0):
    """Synthetic logits [n, V] (see gen_normal_device)."""
    return gen_normal_device((n, V), seed, sigma)


# MLP shape of the Qwen3-4B-shaped workloads: hidden size and SwiGLU
# intermediate size.
MLP_HIDDEN, MLP_INTER = 2560, 9728


def gen_shift_labels(n: int, V: int, seed: int, ignore_frac: float = 0.1) -> np.ndarray:
    """Pre-shifted labels of one rank's n tokens: uniform token ids in
    [0, V), with a leading prompt-like run of -100 (no loss) covering
    ignore_frac of the tokens."""
    rng = np.random.default_rng(seed)
    lab = rng.integers(0, V, size=n).astype(np.int32)
    lab[: int(n * ignore_frac)] = -100
    return lab
