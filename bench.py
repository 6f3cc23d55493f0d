#!/usr/bin/env python3
"""Benchmark of one Ulysses rank's hot path on one MI355X.

One step is one pass over every step of the path for one simulated rank, on
seeded synthetic inputs already resident in HBM:
  seq->head pack of fused QKV -> attention forward -> head->seq unpack of O
  -> seq->head pack of dO -> attention backward (D + dQ, then dK/dV)
  -> head->seq unpack of the fused dQKV.
The all-to-all between the packs and the attention (a re-indexing of buffers
across ranks) is not a kernel of this rank and is not timed: the attention
reads the rank's head shard generated directly.

Prints ONE JSON line on stdout. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd+bwd TFLOP/s (% bf16 MFMA peak) at 64K head-shard; swap GB/s"
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4        # the engine clock the published bf16 peak assumes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def unmasked_pairs(w, cu):
    """U: (query, key) pairs the mask allows, per query head."""
    if cu is None:
        return w.N * (w.N + 1) // 2
    lens = [int(b - a) for a, b in zip(cu[:-1], cu[1:])]
    return sum(L * (L + 1) // 2 for L in lens)


def cpu_baseline(w, tokens: int):
    """The oracle, as it stands, on a bounded sample of the same workload:
    causal fwd + bwd (all dQ rows, all dK/dV keys) over the first `tokens`
    tokens of rank 0's head shard, all its heads. Counted like the GPU:
    14 * d flop per unmasked (query, key) pair per query head."""
    import numpy as np

    import oracle
    import workloads
    qkv = workloads.gen_x(w, workloads.rank_heads(w, 0), 0, tokens)
    dy = workloads.gen_dy(w, [c for c in range(w.hq)], 0, tokens)
    q, k, v = qkv[:, :w.hq], qkv[:, w.hq:w.hq + w.hkv], qkv[:, w.hq + w.hkv:]
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, w.scale, True)
    oracle.attn_bwd(q, k, v, dy, w.scale, True)
    dt = time.perf_counter() - t0
    U = tokens * (tokens + 1) // 2
    flops = 14.0 * w.d * U * w.hq
    del np
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": "fp64 oracle causal attention fwd+bwd over the first %d of %d tokens of the head shard "
                  "(%d q / %d kv heads, d=%d); %.1f s" % (tokens, w.N, w.hq, w.hkv, w.d, dt),
        "seconds": dt,
        "host_cpus": os.cpu_count(),
    }


KERNEL_OF = {"a3_attn_fwd": "attn_fwd_kernel", "a7a9_attn_bwd_dq": "attn_bwd_dq_kernel",
             "a8_attn_bwd_dkdv": "attn_bwd_dkdv_kernel"}


def swap_cold_warm(torch, fns, reps=15, batch=20):
    """Each swap timed alone, outside the step, cold and warm, beside a
    device-to-device copy of the same bytes as the achievable-copy reference.
    Bytes counted: one read + one write.

    An event recorded right before a kernel holds that kernel back by about
    6 us (the marker's own completion), and after a synchronization the first
    event fires before the host has submitted the launch. So neither timing
    puts an event directly in front of the kernel it measures:
      warm: `batch` launches back to back between two events, per launch;
      cold: [MALL-evicting 512 MiB scratch write, then the swap] minus [the
            same scratch write alone], both between two events, medians of
            `reps` alternating pairs.
    fns: {name: (launch, src, dst)} with src/dst the swap's tensors."""
    import numpy as np
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def between(*calls):
        torch.cuda.synchronize()
        e0.record()
        for c in calls:
            c()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    evict = lambda: scratch.fill_(1)  # noqa: E731

    def rate(ms, nbytes):
        return {"ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    def timed_cold(fn, nbytes):
        with_fn, alone = [], []
        for _ in range(reps):
            with_fn.append(between(evict, fn))
            alone.append(between(evict))
        return rate(float(np.median(with_fn)) - float(np.median(alone)), nbytes)

    def timed_warm(fn, nbytes):
        fn()
        ts = [between(*([fn] * batch)) / batch for _ in range(max(3, reps // 5))]
        return rate(float(np.median(ts)), nbytes)

    out = {}
    for name, (launch, src, dst) in fns.items():
        nbytes = 2 * src.numel() * src.element_size()
        flat_src, flat_dst = src.reshape(-1), dst.view(-1)
        copy = lambda: flat_dst.copy_(flat_src)  # noqa: E731
        out[name] = {"bytes": nbytes, "cold": timed_cold(launch, nbytes), "warm": timed_warm(launch, nbytes),
                     "d2d_copy_cold": timed_cold(copy, nbytes), "d2d_copy_warm": timed_warm(copy, nbytes)}
    del scratch
    return out


def ring_step(uly, torch, w, reps=3):
    """Ring attention at the same sequence and P: rank P-1 (the one with the
    most work) attends its n tokens x all Hq heads to all P key/value blocks
    (its own block causal, the P-1 earlier ones unmasked), merges the P
    results, then runs the P backward steps with the merged o and lse and sums
    the P dQ shares. Every block reuses the rank's own q|k|v data (timing does
    not depend on the values). Medians over `reps`."""
    import numpy as np

    import workloads
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    x_seq = dev(workloads.gen_seq_shard(w, 0))
    dy_seq = dev(workloads.gen_dy_seq_shard(w, 0))
    P, n, Hq, Hkv, d = w.P, w.n, w.Hq, w.Hkv, w.d
    q, k, v = x_seq[:, :Hq], x_seq[:, Hq:Hq + Hkv], x_seq[:, Hq + Hkv:]
    o_parts = [torch.empty((n, Hq, d), dtype=torch.int16, device="cuda") for _ in range(P)]
    l_parts = [torch.empty((Hq, n), dtype=torch.float32, device="cuda") for _ in range(P)]
    o = torch.empty((n, Hq, d), dtype=torch.int16, device="cuda")
    lse = torch.empty((Hq, n), dtype=torch.float32, device="cuda")
    g_parts = [torch.empty((n, Hq + 2 * Hkv, d), dtype=torch.int16, device="cuda") for _ in range(P)]
    dq = torch.empty((n, Hq, d), dtype=torch.int16, device="cuda")
    wsf = torch.empty(uly.attn_fwd_workspace_bytes(n, Hq, Hkv, d), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(uly.attn_bwd_workspace_bytes(n, Hq, Hkv, d), dtype=torch.uint8, device="cuda")
    causal = [b == P - 1 for b in range(P)]

    def fwd():
        for b in range(P):
            uly.attn_fwd(q, k, v, o_parts[b], l_parts[b], w.scale, causal[b], None, None, wsf)

    def merge():
        uly.attn_lse_merge(o_parts, l_parts, o, lse)

    def bwd():
        for b in range(P):
            g = g_parts[b]
            uly.attn_bwd(q, k, v, o, lse, dy_seq, g[:, :Hq], g[:, Hq:Hq + Hkv], g[:, Hq + Hkv:], w.scale, causal[b],
                         wsb)

    def gsum():
        uly.ring_grad_sum([g[:, :Hq] for g in g_parts], dq)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    t_fwd, t_merge, t_bwd, t_sum = timed(fwd), timed(merge), timed(bwd), timed(gsum)
    pairs = (P - 1) * n * n + n * (n + 1) // 2  # per query head
    merge_bytes = P * (n * Hq * d * 2 + Hq * n * 4) + n * Hq * d * 2 + Hq * n * 4
    sum_bytes = (P + 1) * n * Hq * d * 2
    return {
        "rank": P - 1, "blocks": P, "tokens_per_block": n, "heads": [Hq, Hkv], "d": d,
        "fwd_ms": round(t_fwd, 3), "fwd_tflops": round(4.0 * d * pairs * Hq / (t_fwd * 1e-3) / 1e12, 2),
        "bwd_ms": round(t_bwd, 3), "bwd_tflops": round(10.0 * d * pairs * Hq / (t_bwd * 1e-3) / 1e12, 2),
        "merge_ms": round(t_merge, 4), "merge_gbps": round(merge_bytes / (t_merge * 1e-3) / 1e9, 1),
        "merge_frac_hbm": round(merge_bytes / (t_merge * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "grad_sum_ms": round(t_sum, 4), "grad_sum_gbps": round(sum_bytes / (t_sum * 1e-3) / 1e9, 1),
        "grad_sum_frac_hbm": round(sum_bytes / (t_sum * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
    }


def loss_step(uly, torch, w, reps=3):
    """The shifted-label loss of one rank's n tokens at the Qwen3-4B vocabulary:
    the rank's cross-entropy (reads the logits once), the aggregation over the
    P ranks' scalars, and the gradient (reads the logits once, writes the
    gradient once). Medians over `reps`."""
    import numpy as np

    import workloads
    n, V, P = w.n, workloads.VOCAB, w.P
    logits = workloads.gen_logits_device(n, V, seed=w.seed + 77).view(n, V)
    labels = torch.from_numpy(workloads.gen_shift_labels(n, V, seed=w.seed + 78)).cuda()
    grad = torch.empty_like(logits)
    row_loss = torch.empty((n,), dtype=torch.float32, device="cuda")
    row_lse = torch.empty((n,), dtype=torch.float32, device="cuda")
    loss = torch.empty((P,), dtype=torch.float32, device="cuda")
    good = torch.empty((P,), dtype=torch.int32, device="cuda")
    total = torch.empty((1,), dtype=torch.float32, device="cuda")
    scale = torch.empty((1,), dtype=torch.float32, device="cuda")

    def fwd():
        uly.shifted_ce_fwd(logits, labels, row_loss, row_lse, loss[0:1], good[0:1])

    def agg():  # the other ranks' scalars stand in as copies of this one's
        loss[1:].fill_(0.0)
        uly.sp_loss_aggregate([loss[r:r + 1] for r in range(P)], [good[r:r + 1] for r in range(P)], total, scale)

    def bwd():
        uly.shifted_ce_bwd(logits, labels, row_lse, scale, grad)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    good[1:].fill_(0)
    t_fwd = timed(fwd)
    agg()
    t_bwd = timed(bwd)
    nbytes = n * V * 2
    out = {
        "tokens": n, "vocab": V,
        "fwd_ms": round(t_fwd, 4), "fwd_gbps": round(nbytes / (t_fwd * 1e-3) / 1e9, 1),
        "fwd_frac_hbm": round(nbytes / (t_fwd * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "bwd_ms": round(t_bwd, 4), "bwd_gbps": round(2 * nbytes / (t_bwd * 1e-3) / 1e9, 1),
        "bwd_frac_hbm": round(2 * nbytes / (t_bwd * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "rank_loss": round(float(loss[0].item()), 5),
    }
    del logits, grad
    return out


def mlp_step(uly, torch, w, tile=4096, reps=3):
    """TiledMLP over one rank's n tokens at the Qwen3-4B MLP shape (H = 2560,
    I = 9728), tiles of `tile` tokens: forward, and backward with the
    recompute. Counted work: 6nHI flop forward, 12nHI backward (the
    recompute of the gate/up GEMM, 4nHI more, is executed but not counted).
    Medians over `reps`."""
    import numpy as np

    import workloads
    n, H, I = w.n, workloads.MLP_HIDDEN, workloads.MLP_INTER
    x = workloads.gen_normal_device((n, H), seed=w.seed + 80)
    dy = workloads.gen_normal_device((n, H), seed=w.seed + 81)
    w_gu = workloads.gen_normal_device((2 * I, H), seed=w.seed + 82, sigma=1.0 / np.sqrt(H))
    w_down = workloads.gen_normal_device((H, I), seed=w.seed + 83, sigma=1.0 / np.sqrt(I))
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dw_gu = torch.empty((2 * I, H), dtype=torch.float32, device="cuda")
    dw_down = torch.empty((H, I), dtype=torch.float32, device="cuda")
    ws = torch.empty(uly.tiled_mlp_workspace_bytes(tile, H, I), dtype=torch.uint8, device="cuda")

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    t_fwd = timed(lambda: uly.tiled_mlp_fwd(x, w_gu, w_down, y, tile, ws))
    t_bwd = timed(lambda: uly.tiled_mlp_bwd(x, w_gu, w_down, dy, dx, dw_gu, dw_down, tile, False, ws))
    nhi = float(n) * H * I
    out = {
        "tokens": n, "hidden": H, "intermediate": I, "tile": tile,
        "fwd_ms": round(t_fwd, 3), "fwd_tflops": round(6 * nhi / (t_fwd * 1e-3) / 1e12, 2),
        "bwd_ms": round(t_bwd, 3), "bwd_tflops": round(12 * nhi / (t_bwd * 1e-3) / 1e12, 2),
        "bwd_exec_tflops": round(16 * nhi / (t_bwd * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(6 * nhi / (t_fwd * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "intermediate_bytes_tiled": int(ws.numel()),
        "intermediate_bytes_untiled": int(n * 6 * I * 2),
    }
    del x, dy, y, dx, dw_gu, dw_down, ws
    return out


def measure_workload(uly, torch, w, steps, warmup, swaps_alone):
    """One workload's step (a1, a3, a5, a6, a7+a9, a8, a10 on inputs already
    resident in HBM): `warmup` untimed steps, then `steps` timed between two
    synchronizations; per-kernel times from HIP events recorded on the
    launch stream (torch's current stream, which the library launches on)."""
    import numpy as np

    import workloads
    cu = workloads.cu_seqlens(w) if w.varlen else None
    log("workload %s: N=%d P=%d hq=%d hkv=%d d=%d" % (w.name, w.N, w.P, w.hq, w.hkv, w.d))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    t_gen = time.perf_counter()
    x_seq = dev(workloads.gen_seq_shard(w, 0))            # [n, Ht, d]  this rank's tokens
    recv = dev(workloads.gen_head_shard(w, 0))            # [N, ht, d]  its head shard
    dy_seq = dev(workloads.gen_dy_seq_shard(w, 0))        # [n, Hq, d]
    dy_head = dev(workloads.gen_dy_head_shard(w, 0))      # [N, hq, d]
    log("inputs generated in %.1f s" % (time.perf_counter() - t_gen))
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")

    n, P, hq, hkv, ht, d = w.n, w.P, w.hq, w.hkv, w.ht, w.d
    send = torch.empty((P, n, ht, d), dtype=torch.int16, device="cuda")
    q, k, v = recv[:, :hq], recv[:, hq:hq + hkv], recv[:, hq + hkv:]
    o = torch.empty((w.N, hq, d), dtype=torch.int16, device="cuda")
    lse = torch.empty((hq, w.N), dtype=torch.float32, device="cuda")
    o_seq = torch.empty((n, w.Hq, d), dtype=torch.int16, device="cuda")
    dsend = torch.empty((P, n, hq, d), dtype=torch.int16, device="cuda")
    dqkv = torch.empty((w.N, ht, d), dtype=torch.int16, device="cuda")
    dq, dk, dv = dqkv[:, :hq], dqkv[:, hq:hq + hkv], dqkv[:, hq + hkv:]
    dqkv_seq = torch.empty((n, w.Ht, d), dtype=torch.int16, device="cuda")
    ws = torch.empty(uly.attn_bwd_workspace_bytes(w.N, hq, hkv, d, 1 if cu is None else len(cu) - 1),
                     dtype=torch.uint8, device="cuda")
    ws_fwd = torch.empty(uly.attn_fwd_workspace_bytes(w.N, hq, hkv, d), dtype=torch.uint8, device="cuda")
    o_chunks = o.view(P, n, hq, d)          # O's P destination chunks (token blocks)
    g_chunks = dqkv.view(P, n, ht, d)

    names = ["a1_pack_qkv", "a3_attn_fwd", "a5_unpack_o", "a6_pack_do", "a7a9_attn_bwd_dq",
             "a8_attn_bwd_dkdv", "a10_unpack_dqkv"]
    launches = [
        lambda: uly.ulysses_seq_to_head(x_seq, send, P, w.segments),
        lambda: uly.attn_fwd(q, k, v, o, lse, w.scale, True, cu_dev, None, ws_fwd),
        lambda: uly.ulysses_head_to_seq(o_chunks, o_seq, P, [w.Hq]),
        lambda: uly.ulysses_seq_to_head(dy_seq, dsend, P, [w.Hq]),
        lambda: uly.attn_bwd_dq(q, k, v, o, lse, dy_head, dq, w.scale, True, ws, cu_dev),
        lambda: uly.attn_bwd_dkdv(q, k, v, lse, dy_head, dk, dv, w.scale, True, ws, cu_dev),
        lambda: uly.ulysses_head_to_seq(g_chunks, dqkv_seq, P, w.segments),
    ]
    swap_bytes = {
        "a1_pack_qkv": 2 * n * w.Ht * d * 2,
        "a5_unpack_o": 2 * n * w.Hq * d * 2,
        "a6_pack_do": 2 * n * w.Hq * d * 2,
        "a10_unpack_dqkv": 2 * n * w.Ht * d * 2,
    }
    U = unmasked_pairs(w, cu)
    flops = {
        "a3_attn_fwd": 4.0 * d * U * hq,
        "a7a9_attn_bwd_dq": 2.0 * d * U * hq,      # dQ; its recompute of S and dP is not counted
        "a8_attn_bwd_dkdv": 8.0 * d * U * hq,      # S recompute, dP, dV, dK
    }
    total_flops = 14.0 * d * U * hq

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    # The dK/dV kernel carries 8 of the 14 counted d-units per pair, so it
    # is the dominant kernel of every workload; the timed steps bracket only
    # it with events.
    DOM = names.index("a8_attn_bwd_dkdv")
    dom_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]

    def step(ev=None, dom_ev=None):
        if ev is not None:
            ev[0].record()
        for i, f in enumerate(launches):
            if dom_ev is not None and i == DOM:
                dom_ev[0].record()
            f()
            if ev is not None:
                ev[i + 1].record()
            if dom_ev is not None and i == DOM:
                dom_ev[1].record()

    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        log("warmup step %d done" % (i + 1))
    # An event recorded between two kernels holds the second one back by
    # about 6 us, so the timed steps record events only around the dominant
    # kernel; the per-kernel breakdown comes from a second pass of the same
    # number of steps with an event after every launch.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(dom_ev=dom_events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    log("timed %d steps: %.3f ms/step" % (steps, ms_per_step))
    t2 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_per_step_events = (time.perf_counter() - t2) * 1e3 / steps
    log("breakdown pass: %.3f ms/step with an event after every launch" % ms_per_step_events)

    kern_all = {nm: [events[s_][i].elapsed_time(events[s_][i + 1]) for s_ in range(steps)]
                for i, nm in enumerate(names)}
    kern_ms = {nm: float(np.mean(v_)) for nm, v_ in kern_all.items()}
    kern_med = {nm: float(np.median(v_)) for nm, v_ in kern_all.items()}
    attn_ms = kern_ms["a3_attn_fwd"] + kern_ms["a7a9_attn_bwd_dq"] + kern_ms["a8_attn_bwd_dkdv"]
    swap_gbps = {nm: swap_bytes[nm] / (kern_ms[nm] * 1e-3) / 1e9 for nm in swap_bytes}
    dom = names[DOM]
    dom_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dom_events]))
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    roofline = {
        "kernel": dom,
        "launch_ms": round(dom_ms, 4),   # HIP events around each of its launches in the timed steps
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": None,
    }
    out = {
        "value": round(value, 3),
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_with_events": round(ms_per_step_events, 4),
        "config": {
            "workload": "Qwen3-4B-shaped SP=%d head shard, %s: N=%d tokens, %d q / %d kv heads, d=%d, causal%s"
                        % (P, w.name, w.N, hq, hkv, d, ", packed docs" if cu is not None else ""),
            "N": w.N, "P": P, "hq": hq, "hkv": hkv, "d": d, "seq_shard": [n, w.Ht, d],
            "n_docs": None if cu is None else len(cu) - 1,
        },
        "roofline": roofline,
        "attn_tflops": round(total_flops / (attn_ms * 1e-3) / 1e12, 2),
        "attn_frac_peak": round(total_flops / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "value_frac_peak": round(value / BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": round(w.N / (attn_ms * 1e-3), 1),
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in kern_ms.items()},
        "kernel_ms_median": {k_: round(v_, 4) for k_, v_ in kern_med.items()},
        "kernel_tflops": {k_: round(flops[k_] / (kern_ms[k_] * 1e-3) / 1e12, 2) for k_ in flops},
        "fwd_tflops": round(4.0 * d * U * hq / (kern_ms["a3_attn_fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10.0 * d * U * hq / ((kern_ms["a7a9_attn_bwd_dq"] + kern_ms["a8_attn_bwd_dkdv"]) * 1e-3)
                            / 1e12, 2),
        # from the breakdown pass: each includes the ~6 us by which the event
        # recorded in front of it holds it back
        "swap_gbps_breakdown": {k_: round(v_, 1) for k_, v_ in swap_gbps.items()},
        "counted_flop_per_step": total_flops,
        "peak_device_bytes": torch.cuda.max_memory_allocated(),
        "unmasked_pairs_per_head": U,
    }
    if swaps_alone:
        out["swaps_alone"] = swap_cold_warm(torch, {
            "a1_pack_qkv": (launches[0], x_seq, send),
            "a5_unpack_o": (launches[2], o_chunks, o_seq),
            "a6_pack_do": (launches[3], dy_seq, dsend),
            "a10_unpack_dqkv": (launches[6], g_chunks, dqkv_seq),
        })
        # The swaps' rates: each alone and cold (timed without an event in
        # front of it; they agree with the kernel trace's durations).
        out["swap_gbps"] = {k_: v_["cold"]["gbps"] for k_, v_ in out["swaps_alone"].items()}
        out["swap_frac_hbm"] = {k_: v_["cold"]["frac_hbm"] for k_, v_ in out["swaps_alone"].items()}
    del x_seq, recv, dy_seq, dy_head, send, o, lse, o_seq, dsend, dqkv, dqkv_seq, ws, ws_fwd
    torch.cuda.empty_cache()
    return out


def csrc_digest():
    """sha256 over the HIP sources (names and bytes), to tell whether stored
    counter readings still describe the kernels being run."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "long_context_attention_ulysses_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_profile(workload: str, step_name: str):
    """What the committed rocprofv3 counter summary (profiles/traffic_<workload>.txt)
    says about a kernel's last dispatch in the profiled steps: HBM bytes
    (FETCH_SIZE + WRITE_SIZE, scaled by the readings of a copy of known size)
    and the engine clock (GRBM_GUI_ACTIVE cycles over the 8 XCDs / the
    dispatch's duration). None when there is no summary for this workload or
    the HIP sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        doc = json.load(fh)
    if doc.get("source_sha256") != csrc_digest():
        return None
    prefix = KERNEL_OF[step_name]
    # the kernel's last dispatch: the last profiled step (after a warm-up step)
    hits = [d for d in doc["dispatches"] if d["kernel"].startswith(prefix)]
    if not hits:
        return None
    out = {"hbm_bytes": hits[-1]["hbm_bytes"]}
    if hits[-1].get("clock_ghz"):
        out["clock_ghz"] = hits[-1]["clock_ghz"]
        out["clock_source"] = ("GRBM_GUI_ACTIVE / 8 XCDs / kernel duration of the same dispatch "
                               "(profiles/traffic_%s.txt)" % workload)
    return out


def add_measured_profile(workload: str, roofline: dict):
    """traffic (HBM bytes per launch) and the clock of the roofline kernel from
    the committed counter summary of this workload, with the fraction of the
    peak at that clock; traffic None when there is no summary of the current
    sources."""
    prof = measured_profile(workload, roofline["kernel"])
    roofline["traffic"] = prof and prof["hbm_bytes"]
    if prof and prof.get("clock_ghz"):
        # clock measured by the committed counter pass of the same sources
        ghz = prof["clock_ghz"]
        roofline["clock_ghz"] = ghz
        roofline["peak_at_clock"] = round(BF16_PEAK_TFLOPS * ghz / PEAK_CLOCK_GHZ, 1)
        roofline["frac_clock_adjusted"] = round(roofline["achieved"] / roofline["peak_at_clock"], 4)
        roofline["clock_source"] = prof["clock_source"]


def short_kernel_name(full: str) -> str:
    """'void uly::(anonymous namespace)::f<128, 4>(args)' -> 'f<128, 4>'."""
    name = full.replace("(anonymous namespace)::", "")
    name = name.split("(")[0].replace("void ", "", 1)
    return name.split("::")[-1].strip()


def write_traffic_summary(workload: str, pmc_dir: str):
    """Turn the rocprofv3 counter runs of `bench.py --steps 2 --warmup 1`
    into profiles/traffic_<workload>.txt (the dispatches of the bench steps:
    warm-up, timed steps and breakdown pass):
      - FETCH_SIZE in <pmc_dir>/fetch_counter_collection.csv and WRITE_SIZE in
        <pmc_dir>/write_counter_collection.csv: HBM bytes per dispatch. Both
        counters are scaled by what they read for the step's first launch,
        the seq->head pack, which reads and writes exactly the sequence
        shard's bytes once.
      - optionally GRBM_GUI_ACTIVE with the kernel trace of the same run
        (<pmc_dir>/grbm_counter_collection.csv, grbm_kernel_trace.csv): the
        engine clock of each dispatch, as its busy cycles summed over the 8
        XCDs / 8 / its duration."""
    import csv

    import workloads
    w = workloads.WORKLOADS[workload]

    def read(name, counter):
        rows = []
        with open(os.path.join(pmc_dir, "%s_counter_collection.csv" % name)) as fh:
            for r in csv.DictReader(fh):
                assert r["Counter_Name"] == counter, r["Counter_Name"]
                rows.append((int(r["Dispatch_Id"]), short_kernel_name(r["Kernel_Name"]),
                             float(r["Counter_Value"])))
        return sorted(rows)

    fetch, write = read("fetch", "FETCH_SIZE"), read("write", "WRITE_SIZE")
    assert [(d, k) for d, k, _ in fetch] == [(d, k) for d, k, _ in write], "runs launched different kernels"
    clocks = {}
    grbm_path = os.path.join(pmc_dir, "grbm_counter_collection.csv")
    if os.path.exists(grbm_path):
        grbm = read("grbm", "GRBM_GUI_ACTIVE")
        assert [(d, k) for d, k, _ in grbm] == [(d, k) for d, k, _ in fetch], "runs launched different kernels"
        dur = {}
        with open(os.path.join(pmc_dir, "grbm_kernel_trace.csv")) as fh:
            for r in csv.DictReader(fh):
                dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for d, _, cyc in grbm:
            if dur.get(d, 0) > 0:
                clocks[d] = (cyc / 8.0 / dur[d], dur[d])   # cycles per ns = GHz
    # The bench steps start at the first seq->head pack (runtime copies, e.g.
    # of a cu_seqlens table, can come before it).
    lib_kernels = ("swap_kernel", "to_trans_kernel", "attn_", "fwd_merge_kernel", "dq_part_sum_kernel",
                   "dkdv_part_sum_kernel", "block_order_kernel")
    first = next(i for i, (_, k, _) in enumerate(fetch) if k.startswith("swap_kernel"))
    fetch, write = fetch[first:], write[first:]
    shard_bytes = w.n * w.Ht * w.d * 2
    fetch_scale = shard_bytes / (fetch[0][2] * 1024)
    write_scale = shard_bytes / (write[0][2] * 1024)
    run = ("-- python3 $REPO/bench.py --workload %s --steps 2 --warmup 1 --cpu-tokens 0 --no-ring --no-loss "
           "--no-mlp --no-workloads" % workload)
    doc = {
        "workload": "%s head shard, one warm-up and two timed bench steps (--steps 2 --warmup 1)" % workload,
        "commands": [
            "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $PMC -o fetch " + run,
            "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $PMC -o write " + run,
            "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc GRBM_GUI_ACTIVE --kernel-trace --output-format csv "
            "-d $PMC -o grbm " + run,
            "python3 $REPO/bench.py --workload %s --traffic-summary $PMC" % workload,
        ],
        "calibration": {
            "kernel": "%s (a1 pack of the %d x %d x %d bf16 sequence shard: reads and writes exactly %d bytes)"
                      % (fetch[0][1], w.n, w.Ht, w.d, shard_bytes),
            "fetch_scale": fetch_scale,
            "write_scale": write_scale,
        },
        "host": os.uname().nodename,
        "source_sha256": csrc_digest(),
        "dispatches": [],
    }
    # Only the bench steps' dispatches: the first kernel that is not the
    # library's (torch's fill before the swaps timed alone) ends them.
    for (d, k, fv), (_, _, wv) in zip(fetch, write):
        if not k.startswith(lib_kernels):
            doc["dispatches_left_out"] = len(fetch) - len(doc["dispatches"])
            break
        e = {"dispatch": d, "kernel": k, "fetch_kb": fv, "write_kb": wv,
             "hbm_bytes": int(round((fv * fetch_scale + wv * write_scale) * 1024))}
        if d in clocks:
            # the counter's window is only meaningful against dispatches of a
            # millisecond or more (short ones read above the 2.4 GHz maximum)
            if clocks[d][1] >= 1_000_000:
                e["clock_ghz"] = round(clocks[d][0], 4)
            e["duration_ns"] = clocks[d][1]
        doc["dispatches"].append(e)
    out = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    log("wrote %s" % out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="64k", choices=["tiny", "8k", "64k", "varlen", "256k"])
    ap.add_argument("--cpu-tokens", type=int, default=9216,
                    help="tokens of the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-ring", action="store_true", help="skip the ring-attention measurement")
    ap.add_argument("--no-loss", action="store_true", help="skip the shifted-label loss measurement")
    ap.add_argument("--no-mlp", action="store_true", help="skip the TiledMLP measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the short runs of the 8k, varlen and 256k workloads after the 64k one")
    ap.add_argument("--traffic-summary", metavar="PMC_DIR",
                    help="write profiles/traffic_<workload>.txt from two rocprofv3 counter runs and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        write_traffic_summary(args.workload, args.traffic_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the Ulysses path; runs on more than one GPU "
              "are not supported: the exchange between GPUs is not implemented (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_ulysses_amd as uly
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.WORKLOADS[args.workload]
    cu = workloads.cu_seqlens(w) if w.varlen else None
    r = measure_workload(uly, torch, w, args.steps, args.warmup, swaps_alone=True)
    result = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": r.pop("config"),
    }
    add_measured_profile(args.workload, r["roofline"])
    result["roofline"] = r.pop("roofline")
    for key in ("value", "ms_per_step"):
        r.pop(key)
    result.update(r)
    if not args.no_workloads and args.workload == "64k":
        result["workloads"] = {}
        for name in ("8k", "varlen", "256k"):
            steps = 3 if name == "256k" else 10
            log("workload %s (%d steps) ..." % (name, steps))
            wr = measure_workload(uly, torch, workloads.WORKLOADS[name], steps, 2, swaps_alone=False)
            add_measured_profile(name, wr["roofline"])
            result["workloads"][name] = {
                "config": wr["config"]["workload"], "steps": steps, "ms_per_step": wr["ms_per_step"],
                "value_tflops": wr["value"], "attn_tflops": wr["attn_tflops"], "attn_frac_peak": wr["attn_frac_peak"],
                "kernel_ms": wr["kernel_ms"], "kernel_tflops": wr["kernel_tflops"],
                "swap_gbps_breakdown": wr["swap_gbps_breakdown"], "roofline": wr["roofline"],
            }
    if not args.no_ring and cu is None:
        log("ring attention step (rank %d of %d) ..." % (w.P - 1, w.P))
        result["ring"] = ring_step(uly, torch, w)
    if not args.no_loss:
        log("shifted-label loss (%d tokens x %d vocab) ..." % (w.n, 151936))
        result["loss"] = loss_step(uly, torch, w)
    if not args.no_mlp:
        log("TiledMLP (%d tokens) ..." % w.n)
        result["mlp"] = mlp_step(uly, torch, w)
    if args.cpu_tokens > 0:
        log("cpu baseline: oracle on %d tokens ..." % args.cpu_tokens)
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_tokens, w.N))
        log("cpu baseline done in %.1f s" % result["cpu_baseline"]["seconds"])
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
