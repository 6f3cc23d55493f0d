"""Streams and HIP graphs: the swap and attention calls launch kernels only,
on the stream they are given (no allocation, copy, memset or
synchronisation inside the library), so one Ulysses layer runs the same on a
side stream and can be captured in a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import workloads
from tests._gpu import dev, host

pytestmark = pytest.mark.gpu

uly = pytest.importorskip("long_context_attention_ulysses_amd")

P, n, Hq, Hkv, d = 2, 500, 8, 4, 128
hq, hkv = Hq // P, Hkv // P
N, Ht, ht = P * n, Hq + 2 * Hkv, hq + 2 * hkv
SEGS = [Hq, Hkv, Hkv]
SCALE = 1.0 / np.sqrt(d)


class Layer:
    """Rank 0's share of one layer on preallocated buffers: pack q|k|v, take
    this rank's chunk as its head shard (the other rank's tokens stand in
    for what the exchange would bring), attention forward and backward,
    unpack O and dq|dk|dv."""

    def __init__(self, seed=71):
        self.x = dev(workloads.normal_bf16((n, Ht, d), seed=seed, sigma=0.5))
        self.shard = dev(workloads.normal_bf16((N, ht, d), seed=seed + 1, sigma=0.5))
        self.dy = dev(workloads.normal_bf16((N, hq, d), seed=seed + 2))
        self.send = torch.empty((P, n, ht, d), dtype=torch.int16, device="cuda")
        self.o = torch.empty((N, hq, d), dtype=torch.int16, device="cuda")
        self.lse = torch.empty((hq, N), dtype=torch.float32, device="cuda")
        self.dqkv = torch.empty((N, ht, d), dtype=torch.int16, device="cuda")
        self.o_seq = torch.empty((n, Hq, d), dtype=torch.int16, device="cuda")
        self.g_seq = torch.empty((n, Ht, d), dtype=torch.int16, device="cuda")
        self.wsf = torch.empty(uly.attn_fwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")
        self.wsb = torch.empty(uly.attn_bwd_workspace_bytes(N, hq, hkv, d), dtype=torch.uint8, device="cuda")

    def outputs(self):
        return (self.send, self.o, self.lse, self.dqkv, self.o_seq, self.g_seq)

    def clear(self):
        for t in self.outputs():
            t.fill_(-1)

    def run(self, stream=None):
        s = self.shard
        q, k, v = s[:, :hq], s[:, hq:hq + hkv], s[:, hq + hkv:]
        uly.ulysses_seq_to_head(self.x, self.send, P, SEGS, stream=stream)
        uly.attn_fwd(q, k, v, self.o, self.lse, SCALE, True, ws=self.wsf, stream=stream)
        g = self.dqkv
        uly.attn_bwd(q, k, v, self.o, self.lse, self.dy, g[:, :hq], g[:, hq:hq + hkv], g[:, hq + hkv:], SCALE, True,
                     ws=self.wsb, stream=stream)
        uly.ulysses_head_to_seq(self.o.view(P, n, hq, d), self.o_seq, P, [Hq], stream=stream)
        uly.ulysses_head_to_seq(self.dqkv.view(P, n, ht, d), self.g_seq, P, SEGS, stream=stream)

    def bits(self):
        return [t.cpu().numpy().copy() if t.dtype == torch.float32 else host(t) for t in self.outputs()]


def test_side_stream_gives_default_stream_bits():
    layer = Layer()
    layer.clear()
    layer.run()
    torch.cuda.synchronize()
    ref = layer.bits()
    layer.clear()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()                 # default priority
    side.wait_stream(torch.cuda.current_stream())  # the fills ran on the default stream
    layer.run(stream=side.cuda_stream)
    side.synchronize()
    for a, b in zip(layer.bits(), ref):
        assert np.array_equal(a, b)


def test_side_stream_with_binding_allocated_workspaces():
    """ws=None on a side stream: the binding allocates the workspaces on that
    stream, so memory the default stream allocates and overwrites right
    after each call cannot be the workspace the side stream's kernels are
    still using."""
    layer = Layer(seed=75)
    layer.clear()
    layer.run()
    torch.cuda.synchronize()
    ref = layer.bits()
    layer.clear()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()                 # default priority
    side.wait_stream(torch.cuda.current_stream())
    s = layer.shard
    q, k, v = s[:, :hq], s[:, hq:hq + hkv], s[:, hq + hkv:]
    g = layer.dqkv
    junk = []
    uly.ulysses_seq_to_head(layer.x, layer.send, P, SEGS, stream=side.cuda_stream)
    uly.attn_fwd(q, k, v, layer.o, layer.lse, SCALE, True, stream=side.cuda_stream)
    junk.append(torch.full((layer.wsf.numel(),), 0x7F, dtype=torch.uint8, device="cuda"))
    uly.attn_bwd(q, k, v, layer.o, layer.lse, layer.dy, g[:, :hq], g[:, hq:hq + hkv], g[:, hq + hkv:], SCALE,
                 True, stream=side.cuda_stream)
    junk.append(torch.full((layer.wsb.numel(),), 0x7F, dtype=torch.uint8, device="cuda"))
    uly.ulysses_head_to_seq(layer.o.view(P, n, hq, d), layer.o_seq, P, [Hq], stream=side.cuda_stream)
    uly.ulysses_head_to_seq(layer.dqkv.view(P, n, ht, d), layer.g_seq, P, SEGS, stream=side.cuda_stream)
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(layer.bits(), ref):
        assert np.array_equal(a, b)


def test_layer_captured_in_a_hip_graph_replays_exactly():
    layer = Layer()
    layer.clear()
    layer.run()
    torch.cuda.synchronize()
    ref = layer.bits()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):              # the calls launch on torch's capture stream
        layer.run()
    torch.cuda.synchronize()
    for replay in range(3):
        layer.clear()                          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(layer.bits(), ref)):
            assert np.array_equal(a, b), "replay %d, output %d" % (replay, i)


def test_two_layers_on_two_streams_at_once():
    """The library keeps no mutable state between calls: two different
    layers launched on two side streams at the same time each give the bits
    they give alone."""
    a, b = Layer(seed=81), Layer(seed=91)
    refs = []
    for layer in (a, b):
        layer.clear()
        layer.run()
        torch.cuda.synchronize()
        refs.append(layer.bits())
        layer.clear()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for _ in range(2):                                   # interleave the launches of both
        a.run(stream=s1.cuda_stream)
        b.run(stream=s2.cuda_stream)
    torch.cuda.synchronize()
    for layer, ref in ((a, refs[0]), (b, refs[1])):
        for x, y in zip(layer.bits(), ref):
            assert np.array_equal(x, y)
