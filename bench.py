#!/usr/bin/env python3
"""Benchmark of librha's hot path on one MI355X.

A step is one pass of the whole path over the Wan 2.1 1.3B 480p workload
(B=1, H=12, d=128, 21 latent frames x 1560 tokens, 3-frame window, bf16):
rha_state_scan followed by rha_hybrid_fwd.  Inputs are seeded synthetic
Gaussians resident in HBM before timing starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Extra modes used for profiling (not part of the contract):
    --only fwd|scan|stream|stream_sparse|sparse|bidir|anchor|bwd|bwd_bidir|bwd_anchor|bwd_sparse
                          run just that call --steps times (for rocprofv3)
    --copy-calib             run a plain device copy of a known size (counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn query tokens/s + % MFMA bf16 peak, Wan-1.3B shape (H12 d128 32760 tok)"
# MI355X dense bf16 matrix-core peak: 256 CUs x 2.4 GHz x 4096 flop per clock per CU
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # 2516.58
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_wan13b_traffic.md")
# the dominant kernel at this shape (head_dim 128, bf16)
FWD_SOURCE = os.path.join(ROOT, "linear_attention_video_chunked_amd", "csrc", "rha_fwd_bf16_qb2.hip")


def fwd_flops(C, N, w, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_fwd call: 4d per (query, window key)
    pair (QK^T and PV) plus 2d^2 + 2d per query whose state is non-empty."""
    f = 0
    for c in range(N):
        nwin = min(c + 1, w) * C if w > 0 else 0
        f += C * (4 * d * nwin + ((2 * d * d + 2 * d) if (w == 0 or c >= w) else 0))
    return f * BH


def fwd_bytes(C, N, w, d, BH, elem=2):
    """Algorithmic HBM bytes of one rha_hybrid_fwd call: q, k, v read once, the
    state slots of chunks with history read once, out written once."""
    L = N * C
    n_state = sum(1 for c in range(N) if (w == 0 or c >= w))
    return BH * (4 * L * d * elem + n_state * (d * d + d) * 4)


def scan_bytes(C, N, w, d, BH, elem=2):
    """Algorithmic HBM bytes of rha_state_scan: k, v of the folded chunks read
    once, every state slot written once."""
    return BH * (2 * max(0, N - w) * C * d * elem + N * (d * d + d) * 4)


def sparse_fwd_flops(C, N, w, d, mask, qtile=256, ktile=64):
    """Algorithmic FLOPs of one rha_hybrid_fwd_sparse call: as fwd_flops, but
    only the (query, key) pairs of kept blocks count.  mask: numpy [B,H,N,nqt,nkt]."""
    B, H = mask.shape[:2]
    f = 0
    for c in range(N):
        wk = min(c + 1, w) * C if w > 0 else 0  # keys in this chunk's window
        keys = [max(0, min(ktile, wk - ktile * j)) for j in range(mask.shape[4])]
        for i in range(mask.shape[3]):
            rows = min(C, qtile * (i + 1)) - qtile * i
            kept = (mask[:, :, c, i, :].astype(int) * keys).sum()  # over b, h
            f += rows * 4 * d * kept
            if w == 0 or c >= w:
                f += rows * (2 * d * d + 2 * d) * B * H
    return f


def bidir_fwd_flops(C, N, w, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_fwd_bidir call: 4d per (query, key) in
    the symmetric window, plus 2d^2 + 2d per query with any chunk outside it."""
    f = 0
    for c in range(N):
        if w > 0:
            lo, hi = max(0, c - w + 1), min(N - 1, c + w - 1)
            nwin, outside = (hi - lo + 1) * C, lo > 0 or hi < N - 1
        else:
            nwin, outside = 0, True
        f += C * (4 * d * nwin + ((2 * d * d + 2 * d) if outside else 0))
    return f * BH


def anchor_fwd_flops(C, N, w, a, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_fwd call with a anchor chunks: 4d per
    (query, key) over the window and the anchors, 2d^2 + 2d per query whose
    history (chunks a .. c-w) is non-empty."""
    f = 0
    for c in range(N):
        lo = max(0, c - w + 1) if w > 0 else c + 1
        keys = set(range(lo, c + 1)) | set(range(0, min(a, c + 1)))
        f += C * (4 * d * len(keys) * C + ((2 * d * d + 2 * d) if c - w >= a else 0))
    return f * BH


def bwd_flops(C, N, w, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_bwd call: 10d per (query, window key)
    pair (scores recomputed once, dP, dV, dQ, dK: the usual five products), 4d^2
    per query with a state (dS and the query gradient of the linear term) and
    4d^2 per token folded into some state (its value and key gradients)."""
    f = 0
    for c in range(N):
        nwin = min(c + 1, w) * C if w > 0 else 0
        f += C * 10 * d * nwin
        if w == 0 or c >= w:
            f += C * 4 * d * d
        if c <= N - 1 - w:
            f += C * 4 * d * d
    return f * BH


def bidir_bwd_flops(C, N, w, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_bwd_bidir call: 10d per (query, key)
    pair of the symmetric window, 4d^2 per query with any chunk outside its
    window (dS and the query gradient of the linear term) and 4d^2 per token
    in some other chunk's state (its value and key gradients)."""
    f = 0
    first = max(w, 1)
    for c in range(N):
        if w > 0:
            lo, hi = max(0, c - w + 1), min(N - 1, c + w - 1)
            nwin, outside = (hi - lo + 1) * C, lo > 0 or hi < N - 1
        else:
            nwin, outside = 0, True
        f += C * 10 * d * nwin
        if outside:
            f += C * 4 * d * d
        if c <= N - 1 - w or c >= first:  # key chunk c is in some chunk's past or future state
            f += C * 4 * d * d
    return f * BH


def anchor_bwd_flops(C, N, w, a, d, BH):
    """Algorithmic FLOPs of one rha_hybrid_bwd call with a anchor chunks: 10d
    per (query, key) pair over the window and the anchors not in the query's
    future, 4d^2 per query with a history (chunks a .. c-w) and 4d^2 per token
    of a non-anchor chunk in some history."""
    f = 0
    for c in range(N):
        lo = max(0, c - w + 1) if w > 0 else c + 1
        keys = set(range(lo, c + 1)) | set(range(0, min(a, c + 1)))
        f += C * 10 * d * len(keys) * C
        if c - w >= a:
            f += C * 4 * d * d
        if a <= c <= N - 1 - w:
            f += C * 4 * d * d
    return f * BH


def sparse_bwd_flops(C, N, w, d, mask, qtile=256, ktile=64):
    """Algorithmic FLOPs of one rha_hybrid_bwd_sparse call: as bwd_flops, but
    the 10d per (query, key) pair counts only the pairs of kept blocks.
    mask: numpy [B,H,N,nqt,nkt]."""
    B, H = mask.shape[:2]
    f = 0
    for c in range(N):
        wk = min(c + 1, w) * C if w > 0 else 0  # keys in this chunk's window
        keys = [max(0, min(ktile, wk - ktile * j)) for j in range(mask.shape[4])]
        for i in range(mask.shape[3]):
            rows = min(C, qtile * (i + 1)) - qtile * i
            f += rows * 10 * d * int((mask[:, :, c, i, :].astype(int) * keys).sum())
        if w == 0 or c >= w:
            f += C * 4 * d * d * B * H
        if c <= N - 1 - w:
            f += C * 4 * d * d * B * H
    return f


def stream_step_flops(C, w, d, BH):
    """Algorithmic FLOPs of one rha_stream_step with a full window: the new
    chunk's queries against w cached chunks (4d per pair) and the state (2d^2
    + 2d per query), plus the fold of the evicted chunk (2d^2 + 2d per key)."""
    return BH * C * (4 * d * w * C + 2 * d * d + 2 * d) + BH * C * (2 * d * d + 2 * d)


def stream_sparse_step_flops(C, w, d, mask, qtile=256, ktile=64):
    """Algorithmic FLOPs of one rha_stream_step_sparse with a full window: as
    stream_step_flops, but the window's 4d per (query, key) pair counts only
    the pairs of kept blocks.  mask: numpy [B, H, nqt, nkt] of the step."""
    B, H = mask.shape[:2]
    keys = [max(0, min(ktile, w * C - ktile * j)) for j in range(mask.shape[3])]
    f = 0
    for i in range(mask.shape[2]):
        rows = min(C, qtile * (i + 1)) - qtile * i
        f += rows * 4 * d * int((mask[:, :, i, :].astype(int) * keys).sum())
    return f + B * H * C * (2 * d * d + 2 * d) * 2


def stream_step_bytes(C, w, d, BH, elem=2):
    """Algorithmic HBM bytes of one rha_stream_step with a full window, the
    method's own traffic: new q, k, v read and out written; the new k, v
    written into their cache slot; the w - 1 cached chunks' k, v read; S, z
    read; the evicted chunk's k, v read and S, z written back by the fold."""
    chunk = C * d * elem
    state = (d * d + d) * 4
    return BH * (3 * chunk + chunk + 2 * chunk + 2 * (w - 1) * chunk + state + 2 * chunk + state)


def stream_step_impl_extra_bytes(C, w, d, BH, elem=2):
    """Traffic of the implementation beyond the method's: the attention reads
    the new chunk's k, v back from its cache slot (the whole window comes from
    one buffer), and S, z are read once more by the fold's merge."""
    return BH * (2 * C * d * elem + (d * d + d) * 4)


def read_traffic():
    """HBM traffic per fwd launch from the committed rocprofv3 counter summary,
    valid only while the kernel source is the one that was measured."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^\s*[-*]?\s*`?([a-z_0-9]+)`?\s*:\s*`?([0-9a-fA-F.eE+-]+)`?\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    sha = hashlib.sha256(open(FWD_SOURCE, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_model() -> str:
    """The host's CPU model (lscpu's "Model name", else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=12.0, per_config=True):
    """The fp64 oracle on the host: whole heads of the headline workload, run
    until the time budget is spent (at least one head); then one head of each
    other full-size configuration (one step of the streaming one), so the
    oracle's rate is stated per configuration too."""
    import oracle
    from synth import CONFIGS, gen_head
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def head(w, h, L=None, t0=0):
        return [gen_head(w, t, 0, h, L=L, t0=t0).double().numpy() for t in ("q", "k", "v")]

    heads, elapsed = 0, 0.0
    while True:
        q, k, v = head(wl, heads)
        ts = time.perf_counter()
        oracle.hybrid(q, k, v, wl.C, wl.w)
        elapsed += time.perf_counter() - ts  # input generation stays off the clock
        heads += 1
        if elapsed > budget_s or heads >= wl.H:
            break
    # query tokens/s in the metric's unit: one query token = one row across all H heads
    value = wl.B * wl.L * heads / wl.H / elapsed
    res = {"value": value, "unit": "query tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"fp64 chunked oracle on {heads} of {wl.H} heads (b=0) of the full "
                     f"{wl.N}x{wl.C}-token sequence, {elapsed:.1f} s"}
    if per_config:
        pc = {wl.name: {"heads": heads, "oracle_s": elapsed, "query_tokens_per_s": value}}
        for name in ("wan14b", "long"):
            ow = CONFIGS[name]
            q, k, v = head(ow, 0)
            ts = time.perf_counter()
            oracle.hybrid(q, k, v, ow.C, ow.w)
            t = time.perf_counter() - ts
            pc[name] = {"heads": 1, "oracle_s": t, "query_tokens_per_s": ow.B * ow.L / ow.H / t}
        # streaming: the step after the prefill, one head, as the oracle states
        # it (its window's rows over the concatenated sequence up to that step)
        sw = CONFIGS["stream"]
        T = sw.prefill + 1
        q, k, v = head(sw, 0, L=T * sw.C)
        rows = list(range((T - 1) * sw.C, T * sw.C))
        ts = time.perf_counter()
        oracle.hybrid_rows(q, k, v, sw.C, sw.w, rows)
        t = time.perf_counter() - ts
        pc["stream"] = {"heads": 1, "steps": 1, "oracle_s": t, "chunks_per_s": 1.0 / (t * sw.H)}
        res["per_config"] = pc
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~0.2 s of work before the timed region, so the GPU clocks have settled
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["fwd", "scan", "stream", "stream_sparse", "sparse", "bidir", "anchor", "bwd", "bwd_bidir",
                                       "bwd_anchor", "bwd_sparse"],
                    default=None)
    # the GPU's clocks ramp up over the first ~0.1-0.2 s of load after an idle
    # gap: before the W warm-up steps, steps run untimed for this many seconds,
    # so the timed steps see settled clocks whatever W is
    ap.add_argument("--settle", type=float, default=0.25)
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library computes "
              f"on one GPU; heads (and chunk ranges, with a halo and a scan of state sums) "
              f"would be the units to shard across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import linear_attention_video_chunked_amd as rha
    from synth import CONFIGS, gen_block_mask, gen_qkv

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    if args.copy_calib:
        n = 256 << 20  # 256 MiB
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))
        return

    def timed(fn, n):
        """(mean, median, min) seconds per call on the launch stream: the mean
        from two events around all n calls, median and min from an event pair
        around each call.  One untimed call first: the binding's first call
        allocates its outputs and workspace through torch's caching
        allocator, later calls reuse those blocks."""
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            ev[2 * i].record(stream)
            fn()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]) / 1e3
        return e0.elapsed_time(e1) / 1e3 / n, float(np.median(per)), float(per.min())

    def run_only(fn, n):
        for _ in range(n):
            fn()
        torch.cuda.synchronize()

    wl = CONFIGS["wan13b"]
    BH = wl.B * wl.H

    # ---- streaming workload (9-frame window, 21-chunk prefill, 60 steps): it
    # allocates its own tensors and needs nothing from the other sections
    def stream_run(pruned=False):
        sw = CONFIGS["stream"]
        sq, sk, sv = (t.to(dev) for t in gen_qkv(sw))
        sout = torch.empty_like(sq)  # step outputs land in place, with the inputs' strides
        st = rha.StreamState(sw.B, sw.H, sw.d, sw.C, sw.w, device=dev)
        # pruned steps: half of each step's blocks kept (seeded, one mask per chunk)
        smask_cpu = (gen_block_mask((sw.N,) + rha.stream_mask_shape(sw.B, sw.H, sw.C, sw.w), 0.5, seed=43)
                     if pruned else None)
        smask = smask_cpu.to(dev) if pruned else None

        def push(t):
            sl = slice(t * sw.C, (t + 1) * sw.C)
            if pruned:
                rha.stream_step_sparse(st, sq[:, :, sl], sk[:, :, sl], sv[:, :, sl], smask[t], out=sout[:, :, sl],
                                       stream=stream)
            else:
                rha.stream_step(st, sq[:, :, sl], sk[:, :, sl], sv[:, :, sl], out=sout[:, :, sl], stream=stream)

        for t in range(sw.prefill):
            push(t)
        # untimed steps with a full window first (the inputs of the timed
        # steps, later cursor positions), so the timed steps do not start from
        # an idle GPU: measured, the first steps after an idle gap run slower
        for t in range(sw.prefill, sw.prefill + sw.steps):
            push(t)
        torch.cuda.synchronize()
        # the mean from two events around the timed steps; median and min from
        # an event after each of the same steps run again (later cursor
        # positions, the same inputs: the window is full in every pass)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(sw.prefill, sw.prefill + sw.steps):
            push(t)
        e1.record(stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(sw.steps + 1)]
        ev[0].record(stream)
        for i, t in enumerate(range(sw.prefill, sw.prefill + sw.steps)):
            push(t)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(sw.steps)]) / 1e3
        mean = e0.elapsed_time(e1) / 1e3 / sw.steps
        del sq, sk, sv, sout, st
        torch.cuda.empty_cache()
        if pruned:  # the timed steps' mean algorithmic FLOPs
            flops = np.mean([stream_sparse_step_flops(sw.C, sw.w, sw.d, smask_cpu[t].numpy())
                             for t in range(sw.prefill, sw.prefill + sw.steps)])
            return sw, float(mean), float(np.median(per)), float(per.min()), float(flops)
        return sw, float(mean), float(np.median(per)), float(per.min())

    if args.only == "stream":
        stream_run()
        torch.cuda.synchronize()
        return
    if args.only == "stream_sparse":
        stream_run(pruned=True)
        torch.cuda.synchronize()
        return

    q, k, v = (t.to(dev) for t in gen_qkv(wl))
    S = torch.empty((wl.B, wl.H, wl.N, wl.d, wl.d), dtype=torch.float32, device=dev)
    z = torch.empty((wl.B, wl.H, wl.N, wl.d), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)

    def step():
        rha.state_scan(k, v, wl.C, wl.w, S=S, z=z, stream=stream)
        rha.hybrid_fwd(q, k, v, S, z, wl.C, wl.w, out=out, stream=stream)

    def fwd_call():
        rha.hybrid_fwd(q, k, v, S, z, wl.C, wl.w, out=out, stream=stream)

    def scan_call():
        rha.state_scan(k, v, wl.C, wl.w, S=S, z=z, stream=stream)

    if args.only == "fwd":
        scan_call()
        run_only(fwd_call, args.steps)
        return
    if args.only == "scan":
        run_only(scan_call, args.steps)
        return

    # ---- pruned window: half of the (query block, key block) pairs kept (seeded)
    mask_cpu = gen_block_mask(rha.sparse_mask_shape(wl.B, wl.H, wl.C, wl.N, wl.w), 0.5, seed=31)
    mask = mask_cpu.to(dev)

    def sparse_call():
        rha.hybrid_fwd_sparse(q, k, v, S, z, wl.C, wl.w, mask, out=out, stream=stream)

    if args.only == "sparse":
        scan_call()
        run_only(sparse_call, args.steps)
        return

    # ---- bidirectional hybrid at the same shape (window of 3 chunks each way)
    bstates = [None]

    def bidir_scan():
        bstates[0] = rha.state_scan_bidir(k, v, wl.C, wl.w, stream=stream)

    def bidir_call():
        rha.hybrid_fwd_bidir(q, k, v, bstates[0], wl.C, wl.w, out=out, stream=stream)

    if args.only == "bidir":
        bidir_scan()
        run_only(bidir_call, args.steps)
        return

    # ---- the first frame as an anchor (sink) chunk, same shape
    SA = torch.empty_like(S)
    zA = torch.empty_like(z)

    def anchor_call():
        rha.hybrid_fwd(q, k, v, SA, zA, wl.C, wl.w, out=out, stream=stream, anchors=1)

    def anchor_setup():
        rha.state_scan(k, v, wl.C, wl.w, S=SA, z=zA, stream=stream, anchors=1)

    if args.only == "anchor":
        anchor_setup()
        run_only(anchor_call, args.steps)
        return

    # ---- backward pass at the same shape (seeded dout)
    gen = torch.Generator(device="cpu").manual_seed(77)
    dout = torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(dev)
    lse_f = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)
    out_f = torch.empty_like(q)

    def bwd_setup():
        scan_call()
        rha.hybrid_fwd(q, k, v, S, z, wl.C, wl.w, out=out_f, lse=lse_f, stream=stream)

    def bwd_call():
        rha.hybrid_bwd(q, k, v, S, z, out_f, lse_f, dout, wl.C, wl.w, stream=stream)

    if args.only == "bwd":
        bwd_setup()
        run_only(bwd_call, args.steps)
        return

    # ---- backward pass of the bidirectional hybrid at the same shape
    out_b = torch.empty_like(q)
    lse_b = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)

    def bwd_bidir_setup():
        bidir_scan()
        rha.hybrid_fwd_bidir(q, k, v, bstates[0], wl.C, wl.w, out=out_b, lse=lse_b, stream=stream)

    def bwd_bidir_call():
        rha.hybrid_bwd_bidir(q, k, v, bstates[0], out_b, lse_b, dout, wl.C, wl.w, stream=stream)

    if args.only == "bwd_bidir":
        bwd_bidir_setup()
        run_only(bwd_bidir_call, args.steps)
        return

    # ---- backward pass with the first frame as an anchor chunk, same shape
    out_a = torch.empty_like(q)
    lse_a = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)

    def bwd_anchor_setup():
        anchor_setup()
        rha.hybrid_fwd(q, k, v, SA, zA, wl.C, wl.w, out=out_a, lse=lse_a, stream=stream, anchors=1)

    def bwd_anchor_call():
        rha.hybrid_bwd(q, k, v, SA, zA, out_a, lse_a, dout, wl.C, wl.w, stream=stream, anchors=1)

    if args.only == "bwd_anchor":
        bwd_anchor_setup()
        run_only(bwd_anchor_call, args.steps)
        return

    # ---- backward pass of the pruned window (the half-kept mask above)
    out_s = torch.empty_like(q)
    lse_s = torch.empty((wl.B, wl.H, wl.L), dtype=torch.float32, device=dev)

    def bwd_sparse_setup():
        scan_call()
        rha.hybrid_fwd_sparse(q, k, v, S, z, wl.C, wl.w, mask, out=out_s, lse=lse_s, stream=stream)

    def bwd_sparse_call():
        rha.hybrid_bwd_sparse(q, k, v, S, z, mask, out_s, lse_s, dout, wl.C, wl.w, stream=stream)

    if args.only == "bwd_sparse":
        bwd_sparse_setup()
        run_only(bwd_sparse_call, args.steps)
        return

    # ---- the contract: W warmup steps, then exactly K timed steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle0 < args.settle:
        for _ in range(8):
            step()
        n_settle += 8
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = e0.elapsed_time(e1) / 1e3 / args.steps

    # ---- per-kernel timings over timed regions (same stream)
    n_k = max(args.steps, 10)
    t_fwd, t_fwd_med, t_fwd_min = timed(fwd_call, n_k)
    t_scan, t_scan_med, t_scan_min = timed(scan_call, n_k)
    scan_call()
    t_sparse = timed(sparse_call, n_k)[0]
    bidir_scan()
    t_bidir = timed(bidir_call, n_k)[0]
    t_bidir_scan = timed(bidir_scan, n_k)[0]
    bF = bidir_fwd_flops(wl.C, wl.N, wl.w, wl.d, BH)
    anchor_setup()
    t_anchor = timed(anchor_call, n_k)[0]
    bwd_setup()
    t_bwd, t_bwd_med, t_bwd_min = timed(bwd_call, max(args.steps // 5, 5))
    gF = bwd_flops(wl.C, wl.N, wl.w, wl.d, BH)
    bwd_bidir_setup()
    t_bbwd, t_bbwd_med, t_bbwd_min = timed(bwd_bidir_call, max(args.steps // 5, 5))
    gbF = bidir_bwd_flops(wl.C, wl.N, wl.w, wl.d, BH)
    bwd_anchor_setup()
    t_abwd, t_abwd_med, _ = timed(bwd_anchor_call, max(args.steps // 5, 5))
    gaF = anchor_bwd_flops(wl.C, wl.N, wl.w, 1, wl.d, BH)
    bwd_sparse_setup()
    t_sbwd, t_sbwd_med, _ = timed(bwd_sparse_call, max(args.steps // 5, 5))
    gsF = sparse_bwd_flops(wl.C, wl.N, wl.w, wl.d, mask_cpu.numpy())
    aF = anchor_fwd_flops(wl.C, wl.N, wl.w, 1, wl.d, BH)
    spF = sparse_fwd_flops(wl.C, wl.N, wl.w, wl.d, mask_cpu.numpy())
    scan_call()  # S, z of the headline problem again (the backward set-up wrote them too)

    sw, t_stream, t_stream_med, t_stream_min = stream_run()
    _, t_sstream, t_sstream_med, _, ssF = stream_run(pruned=True)

    # ---- the two larger shapes (scan + fwd, each timed on its own); inputs
    # drawn on the GPU from a seeded generator with the same distribution (the
    # parity tests check these shapes against the oracle on sampled rows)
    def other_shape(name, n_calls=5, ow=None):
        ow = CONFIGS[name] if ow is None else ow
        g = torch.Generator(device=dev).manual_seed(1000 + ow.wid)
        shape = (ow.B, ow.H, ow.L, ow.d)
        oq, ok, ov = (torch.randn(shape, generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
        oS, oz = rha.state_scan(ok, ov, ow.C, ow.w, stream=stream)
        oo = torch.empty_like(oq)
        rha.hybrid_fwd(oq, ok, ov, oS, oz, ow.C, ow.w, out=oo, stream=stream)
        t_f = timed(lambda: rha.hybrid_fwd(oq, ok, ov, oS, oz, ow.C, ow.w, out=oo, stream=stream), n_calls)[0]
        t_s = timed(lambda: rha.state_scan(ok, ov, ow.C, ow.w, S=oS, z=oz, stream=stream), n_calls)[0]
        obh = ow.B * ow.H
        oF = fwd_flops(ow.C, ow.N, ow.w, ow.d, obh)
        dense_causal = obh * sum(ow.C * 4 * ow.d * (c + 1) * ow.C for c in range(ow.N))
        dense_full = obh * ow.L * 4 * ow.d * ow.L
        res = {f"{name}_fwd_us": t_f * 1e6, f"{name}_query_tokens_per_s": ow.B * ow.L / t_f,
               f"{name}_TFLOPs": oF / t_f / 1e12, f"{name}_mfma_frac": oF / t_f / 1e12 / PEAK_BF16_TFLOPS,
               f"{name}_scan_us": t_s * 1e6,
               f"{name}_flop_reduction_vs_dense_block_causal": dense_causal / oF,
               f"{name}_flop_reduction_vs_dense_full": dense_full / oF}
        if name == "long":
            # the two limits on the first 21 chunks: w = all (block-causal
            # softmax attention, MFMA-bound) and w = 0 (linear attention only:
            # q, the state slots and out stream through, HBM-bound)
            n21 = 21
            sl = [t[:, :, : n21 * ow.C].contiguous() for t in (oq, ok, ov)]
            so = torch.empty_like(sl[0])
            for wlim, tag in ((n21, "wall"), (0, "w0")):
                sS, sz = rha.state_scan(sl[1], sl[2], ow.C, wlim, stream=stream)
                fn = lambda: rha.hybrid_fwd(sl[0], sl[1], sl[2], sS, sz, ow.C, wlim, out=so, stream=stream)
                fn()
                t_l = timed(fn, n_calls)[0]
                lF = fwd_flops(ow.C, n21, wlim, ow.d, obh)
                res[f"{name}_slice21_{tag}_fwd_us"] = t_l * 1e6
                res[f"{name}_slice21_{tag}_TFLOPs"] = lF / t_l / 1e12
                if wlim > 0:
                    res[f"{name}_slice21_{tag}_mfma_frac"] = lF / t_l / 1e12 / PEAK_BF16_TFLOPS
                else:
                    # q read, out written (bf16), one state slot per chunk read
                    lB = obh * (2 * n21 * ow.C * ow.d * 2 + n21 * (ow.d * ow.d + ow.d) * 4)
                    res[f"{name}_slice21_{tag}_GBps"] = lB / t_l / 1e9
                    res[f"{name}_slice21_{tag}_hbm_frac"] = lB / t_l / 1e9 / PEAK_HBM_GBS
                del sS, sz
            del sl, so
        del oq, ok, ov, oS, oz, oo
        torch.cuda.empty_cache()
        return res

    more = {}
    for name in ("wan14b", "long"):
        more.update(other_shape(name))
    # head_dim 64 at the Wan-1.3B model width (24 heads x 64 = 1536 features):
    # the d = 64 kernel, measured only (its parity is tested at mid sizes)
    more.update(other_shape("wan13b_d64", ow=CONFIGS["wan13b"].replace(name="wan13b_d64", wid=90, H=24, d=64)))
    F = fwd_flops(wl.C, wl.N, wl.w, wl.d, BH)
    achieved = F / t_fwd / 1e12
    traffic = read_traffic()
    tokens = wl.B * wl.L
    sF = stream_step_flops(sw.C, sw.w, sw.d, sw.B * sw.H)
    sB = stream_step_bytes(sw.C, sw.w, sw.d, sw.B * sw.H)
    sX = stream_step_impl_extra_bytes(sw.C, sw.w, sw.d, sw.B * sw.H)
    scB = scan_bytes(wl.C, wl.N, wl.w, wl.d, BH)
    result = {
        "metric": METRIC,
        "value": tokens / t_step,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": settle_s, "steps": n_settle},
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "wan2.1-1.3b-480p: B1 H12 d128, 21 chunks x 1560 tokens (L=32760), "
                               "window 3 chunks, bf16 q/v~N(0,1), k~0.5*N(0,1); step = state_scan + hybrid_fwd",
                   "global_batch": wl.B, "seq_len": wl.L, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "fwd_bf16_qb2_kernel (rha_hybrid_fwd)", "flops_per_launch": F,
                     "algorithmic_bytes_per_launch": fwd_bytes(wl.C, wl.N, wl.w, wl.d, BH),
                     "avg_launch_us": t_fwd * 1e6, "median_launch_us": t_fwd_med * 1e6,
                     "min_launch_us": t_fwd_min * 1e6},
        "detail": {
            "fwd_query_tokens_per_s": tokens / t_fwd,
            "fwd_us": t_fwd * 1e6,
            "fwd_median_us": t_fwd_med * 1e6,
            "fwd_min_us": t_fwd_min * 1e6,
            "fwd_mfma_frac_at_min": F / t_fwd_min / 1e12 / PEAK_BF16_TFLOPS,
            "scan_us": t_scan * 1e6,
            "scan_median_us": t_scan_med * 1e6,
            "scan_min_us": t_scan_min * 1e6,
            "scan_GBps": scB / t_scan / 1e9,
            "scan_hbm_frac": scB / t_scan / 1e9 / PEAK_HBM_GBS,
            "stream_step_us": t_stream * 1e6,
            "stream_step_median_us": t_stream_med * 1e6,
            "stream_step_min_us": t_stream_min * 1e6,
            "stream_chunks_per_s": 1.0 / t_stream,
            "stream_step_TFLOPs": sF / t_stream / 1e12,
            "stream_sparse_half_step_us": t_sstream * 1e6,
            "stream_sparse_half_step_median_us": t_sstream_med * 1e6,
            "stream_sparse_half_step_TFLOPs": ssF / t_sstream / 1e12,
            "stream_sparse_half_step_mfma_frac": ssF / t_sstream / 1e12 / PEAK_BF16_TFLOPS,
            "stream_step_mfma_frac": sF / t_stream / 1e12 / PEAK_BF16_TFLOPS,
            "stream_step_bytes": sB,
            "stream_step_GBps": sB / t_stream / 1e9,
            "stream_step_hbm_frac": sB / t_stream / 1e9 / PEAK_HBM_GBS,
            "stream_step_impl_extra_bytes": sX,
            "sparse_half_fwd_us": t_sparse * 1e6,
            "sparse_half_kept_frac": float(mask_cpu.float().mean()),
            "sparse_half_TFLOPs": spF / t_sparse / 1e12,
            "sparse_half_mfma_frac": spF / t_sparse / 1e12 / PEAK_BF16_TFLOPS,
            "bidir_fwd_us": t_bidir * 1e6,
            "bidir_TFLOPs": bF / t_bidir / 1e12,
            "bidir_mfma_frac": bF / t_bidir / 1e12 / PEAK_BF16_TFLOPS,
            "bidir_scan_us": t_bidir_scan * 1e6,
            "anchor1_fwd_us": t_anchor * 1e6,
            "anchor1_TFLOPs": aF / t_anchor / 1e12,
            "anchor1_mfma_frac": aF / t_anchor / 1e12 / PEAK_BF16_TFLOPS,
            "bwd_us": t_bwd * 1e6,
            "bwd_median_us": t_bwd_med * 1e6,
            "bwd_min_us": t_bwd_min * 1e6,
            "bwd_TFLOPs": gF / t_bwd / 1e12,
            "bwd_mfma_frac": gF / t_bwd / 1e12 / PEAK_BF16_TFLOPS,
            "bidir_bwd_us": t_bbwd * 1e6,
            "bidir_bwd_median_us": t_bbwd_med * 1e6,
            "bidir_bwd_TFLOPs": gbF / t_bbwd / 1e12,
            "bidir_bwd_mfma_frac": gbF / t_bbwd / 1e12 / PEAK_BF16_TFLOPS,
            "anchor1_bwd_us": t_abwd * 1e6,
            "anchor1_bwd_median_us": t_abwd_med * 1e6,
            "anchor1_bwd_TFLOPs": gaF / t_abwd / 1e12,
            "anchor1_bwd_mfma_frac": gaF / t_abwd / 1e12 / PEAK_BF16_TFLOPS,
            "sparse_half_bwd_us": t_sbwd * 1e6,
            "sparse_half_bwd_median_us": t_sbwd_med * 1e6,
            "sparse_half_bwd_TFLOPs": gsF / t_sbwd / 1e12,
            "sparse_half_bwd_mfma_frac": gsF / t_sbwd / 1e12 / PEAK_BF16_TFLOPS,
            **more,
            "timed_wall_s": wall,
        },
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
