#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-secondary] [--no-cpu]
  python bench.py --calibration


Prints ONE JSON line.  The headline workload is the fp8-KV decode step at
256 sequences (n_head 32, n_head_kv 8, head_dim 128, page 16, contexts
log-uniform in [2048, 32768]); one step is the append/quantise of each
sequence's newest K/V row followed by the decode attention call.  `value` is
the step's algorithmic HBM bytes divided by its wall time (inputs resident in
HBM).  `roofline` times the split-K attention kernel alone with HIP events
(recorded by the library on the call's stream) and prices its algorithmic
bytes against 8 TB/s.  `secondary` times the other workloads the same way:
single-sequence decode (latency), 64-sequence bf16 decode at head_dim 256,
the 8-row verify round, the 4096-row prefill chunk (bf16 MFMA TFLOP/s), and
the extended calls on the same shapes: a 4096-key sliding window, rounds of
widths 1/2/4/8, the fp8-cache chunk with QK^T on the fp8 unit, 8-row tree
rounds and the mixed decode + chunk step.  `cpu_baseline` is the CPU oracle
timed over the whole headline workload on this host (repeated to about 10 s,
median pass).

Every timed line first repeats its call untimed: at least W calls and at
least WARM_S seconds of them.  The GPU's clocks rise over the first tens of
milliseconds of load after an idle spell (measured per launch: the prefill
chunk takes 2.6 ms at a cold start and settles at 1.83 ms after about 40 ms
of launches; after 2 s idle it starts again at 2.2 ms), so a line timed
within that ramp would report the ramp, not the kernel.

`roofline.traffic` is the measured HBM bytes per launch of the timed kernel,
read from profiles/hbm_traffic.json when that file was taken on the current
kernel sources (else null).  It comes from rocprofv3 FETCH_SIZE and
WRITE_SIZE passes over this script, each scaled by what the same counter
reads for `--calibration`, which runs two kernels of known traffic: a fill
that writes 1 GiB and a sum that reads 1 GiB.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk, dense
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak
METRIC = "paged-attn decode µs/step & HBM GB/s (% peak) at 256 seqs; prefill MFMA TFLOP/s"
WARM_S = 0.25  # least untimed run time of a call before it is timed (seconds)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (torch's events only see
    torch's own streams)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        assert self.hip.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def decode_bytes(lengths, w, with_out=True):
    """Algorithmic bytes of one decode/verify call: K and V of every cached
    token of every kv head (1 byte per element for fp8, 2 for bf16), the fp8
    scales and block-table entries of every page read, Q, the lengths, and
    (with_out) the output."""
    b = 1 if w.kv_fp8 else 2
    tot = 0
    for c in lengths:
        pages = -(-c // 16)
        tot += c * w.n_head_kv * w.head_dim * 2 * b + pages * 4
        if w.kv_fp8:
            tot += pages * w.n_head_kv * 2 * 4
    q = w.n_seq * w.rows * w.n_head * w.head_dim * 2
    tot += q + 4 * w.n_seq + (q if with_out else 0)
    return tot


def append_bytes(n_tok, w):
    """Append of n_tok rows: bf16 K and V read, stored K and V written, the
    slot list, and (fp8) the page scales read."""
    e = n_tok * w.n_head_kv * w.head_dim
    return e * 2 * 2 + e * 2 * (1 if w.kv_fp8 else 2) + 4 * n_tok + \
        (n_tok * w.n_head_kv * 2 * 4 if w.kv_fp8 else 0)


def prefill_flops(n_rows, ctx, w):
    """4 * n_head * head_dim per (row, key) pair the causal mask admits."""
    cached = ctx - n_rows
    pairs = n_rows * cached + n_rows * (n_rows + 1) // 2
    return 4 * w.n_head * w.head_dim * pairs


# The source file each profiled kernel is built from.
KERNEL_SOURCE = {"split_kernel": "decode.hip", "combine_kernel": "decode.hip",
                 "prefill_kernel": "prefill.hip", "prefill_pipe_kernel": "prefill_pipe.hip"}


def kernel_source_hash(kernel_key):
    """First 16 hex digits of the sha256 of the kernel's source file."""
    src = KERNEL_SOURCE[max((k for k in KERNEL_SOURCE if kernel_key.startswith(k)), key=len)]
    with open(os.path.join(ROOT, "paged_kv_cache_20_amd", "csrc", src), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return e.get("bytes_per_launch")


class Bench:
    def __init__(self, torch, pa, synth):
        self.torch, self.pa, self.synth = torch, pa, synth
        self.ev = HipEvents()

    def warm(self, fn, n):
        """Untimed calls of fn: at least n, and at least WARM_S seconds of
        them (the device drained every 8 calls, so the time is the GPU's)."""
        t0 = time.perf_counter()
        i = 0
        while i < n or time.perf_counter() - t0 < WARM_S:
            fn()
            i += 1
            if i % 8 == 0:
                self.torch.cuda.synchronize()
        self.torch.cuda.synchronize()

    def setup_split(self, name, spare_pages=0):
        torch, pa, synth = self.torch, self.pa, self.synth
        w = synth.WORKLOADS[name]
        if spare_pages:
            need = sum(-(-c // 16) for c in synth.draw_lengths(
                w, torch.Generator(device="cpu").manual_seed(w.seed)).tolist())
            w = synth.scaled(w, pool_pages=need + w.n_seq + spare_pages)
        inp = synth.draw(w, "cuda")
        k, v, ks, vs = synth.poison_pools(inp.n_pages, w, "cuda")
        kv = pa.KV_FP8_E4M3 if w.kv_fp8 else pa.KV_BF16
        pa.attn_kv_append(inp.k_src, inp.v_src, inp.slots, inp.slots.numel(), k, v, ks, vs,
                          inp.n_pages, w.n_head_kv, w.head_dim, 16, kv)
        op = {"decode": 0, "verify": 1}[w.kind]
        wsb = pa.attn_paged_workspace_bytes(op, w.n_seq, w.max_pages, w.n_head, w.head_dim)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(inp.q)
        # the step's own new rows: the last `rows` tokens of every sequence
        lens = inp.lengths.to(torch.int64)
        ends = torch.cumsum(lens, 0)
        idx = torch.cat([torch.arange(int(e) - w.rows, int(e), device="cuda") for e in ends])
        st = dict(w=w, inp=inp, k=k, v=v, ks=ks, vs=vs, kv=kv, ws=ws, wsb=wsb, out=out,
                  k_new=inp.k_src[idx].contiguous(), v_new=inp.v_src[idx].contiguous(),
                  slots_new=inp.slots[idx].contiguous(),
                  lengths_host=inp.lengths.cpu().tolist())
        torch.cuda.synchronize()
        return st

    def split_step(self, st, timer=None, marks=None):
        """One step: the append (A0) of every sequence's new rows, then the
        attention call.  `timer`: HIP events around the split kernel;
        `marks`: three torch events recorded before the append, between the
        two calls and after the attention call (the library launches on
        torch's current stream)."""
        pa = self.pa
        w, inp = st["w"], st["inp"]
        if marks is not None:
            marks[0].record()
        pa.attn_kv_append(st["k_new"], st["v_new"], st["slots_new"], st["slots_new"].numel(),
                          st["k"], st["v"], st["ks"], st["vs"], inp.n_pages, w.n_head_kv,
                          w.head_dim, 16, st["kv"])
        if marks is not None:
            marks[1].record()
        if timer is not None:
            pa.attn_set_kernel_timer(timer[0], timer[1])
        fn = pa.attn_paged_decode if w.kind == "decode" else pa.attn_paged_verify
        fn(inp.q, st["k"], st["v"], st["ks"], st["vs"], inp.n_pages, inp.table, w.max_pages,
           inp.lengths, w.n_seq, w.n_head, w.n_head_kv, w.head_dim, 16, st["kv"], st["out"],
           st["ws"], st["wsb"])
        if marks is not None:
            marks[2].record()

    def time_split(self, st, steps, warmup):
        torch = self.torch
        self.warm(lambda: self.split_step(st), warmup)
        evs = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.split_step(st, evs[i], marks[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        kern = [self.ev.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            self.ev.destroy(a)
            self.ev.destroy(b)
        app = sorted(m[0].elapsed_time(m[1]) for m in marks)
        call = sorted(m[1].elapsed_time(m[2]) for m in marks)
        st["append_us_median"] = round(app[len(app) // 2] * 1e3, 2)
        st["call_us_median"] = round(call[len(call) // 2] * 1e3, 2)
        return wall, sum(kern) / len(kern), sorted(kern)[len(kern) // 2]

    def setup_prefill(self, name, w=None):
        torch, pa, synth = self.torch, self.pa, self.synth
        w = synth.WORKLOADS[name] if w is None else w
        inp = synth.draw(w, "cuda")
        k, v, ks, vs = synth.poison_pools(inp.n_pages, w, "cuda")
        kv = pa.KV_FP8_E4M3 if w.kv_fp8 else pa.KV_BF16
        pa.attn_kv_append(inp.k_src, inp.v_src, inp.slots, inp.slots.numel(), k, v, ks, vs,
                          inp.n_pages, w.n_head_kv, w.head_dim, 16, kv)
        out = torch.empty((w.rows, w.n_head, w.head_dim), dtype=torch.bfloat16, device="cuda")
        C = int(inp.lengths[0])
        st = dict(w=w, inp=inp, k=k, v=v, ks=ks, vs=vs, kv=kv, out=out, C=C,
                  q=inp.q.view(w.rows, w.n_head, w.head_dim),
                  k_new=inp.k_src[C - w.rows:].contiguous(),
                  v_new=inp.v_src[C - w.rows:].contiguous(),
                  slots_new=inp.slots[C - w.rows:].contiguous())
        torch.cuda.synchronize()
        return st

    def prefill_step(self, st, timer=None):
        pa = self.pa
        w, inp = st["w"], st["inp"]
        pa.attn_kv_append(st["k_new"], st["v_new"], st["slots_new"], w.rows, st["k"], st["v"],
                          st["ks"], st["vs"], inp.n_pages, w.n_head_kv, w.head_dim, 16, st["kv"])
        if timer is not None:
            pa.attn_set_kernel_timer(timer[0], timer[1])
        pa.attn_paged_prefill(st["q"], w.rows, st["k"], st["v"], st["ks"], st["vs"],
                              inp.n_pages, inp.table, w.max_pages, st["C"], w.n_head,
                              w.n_head_kv, w.head_dim, 16, st["kv"], st["out"])

    def time_mixed(self, steps=20, warmup=5):
        """The mixed step as one attn_paged_mixed call, against its decode
        half (attn_paged_decode) and its chunk half (attn_paged_prefill)
        called alone."""
        torch, pa, synth = self.torch, self.pa, self.synth
        w, inp, q, cu, lens = synth.mixed_step()
        k, v, ks, vs = synth.poison_pools(inp.n_pages, w, "cuda")
        kv = pa.KV_FP8_E4M3
        pa.attn_kv_append(inp.k_src, inp.v_src, inp.slots, inp.slots.numel(), k, v, ks, vs,
                          inp.n_pages, w.n_head_kv, w.head_dim, 16, kv)
        mp = inp.table.shape[1]
        wsb = pa.attn_paged_workspace_bytes(3, 256, mp, w.n_head, w.head_dim)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)
        n_tok = int(q.shape[0])

        def mixed():
            pa.attn_paged_mixed(q, n_tok, cu, 257, 256, 2048, k, v, ks, vs, inp.n_pages,
                                inp.table, mp, inp.lengths, w.n_head, w.n_head_kv, w.head_dim,
                                16, kv, out, ws, wsb)

        def dec_half():
            pa.attn_paged_decode(q[:256].view(256, 1, w.n_head, w.head_dim), k, v, ks, vs,
                                 inp.n_pages, inp.table, mp, inp.lengths, 256, w.n_head,
                                 w.n_head_kv, w.head_dim, 16, kv, out[:256], ws, wsb)

        def chunk_half():
            pa.attn_paged_prefill(q[256:], 2048, k, v, ks, vs, inp.n_pages, inp.table[256], mp,
                                  8192, w.n_head, w.n_head_kv, w.head_dim, 16, kv, out[256:])

        res = {}
        for tag, fn in (("mixed_call", mixed), ("decode_half", dec_half),
                        ("chunk_half", chunk_half)):
            self.warm(fn, warmup)
            # The library launches on torch's current stream, so torch's
            # events bracket each whole call (all of its kernels).
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            for i in range(steps):
                evs[i][0].record()
                fn()
                evs[i][1].record()
            torch.cuda.synchronize()
            kern = sorted(a.elapsed_time(b) for a, b in evs)
            res[tag] = kern[len(kern) // 2] * 1e3
        dw = synth.scaled(synth.WORKLOADS["decode_256seq_fp8"], n_seq=256)
        by = decode_bytes(lens[:256], dw, with_out=False)
        fl = prefill_flops(2048, 8192, w)
        return {"us_median": round(res["mixed_call"], 2),
                "decode_half_alone_us": round(res["decode_half"], 2),
                "chunk_half_alone_us": round(res["chunk_half"], 2),
                "decode_bytes": by, "chunk_flops": fl,
                "note": "medians of whole-call spans (every kernel of the call) by events on "
                        "the call's stream"}

    def time_window(self, window=4096, steps=20, warmup=5):
        """The 256-sequence fp8 decode step with a sliding window: split
        kernel time (library kernel timer) and the bytes of the keys in
        each row's window."""
        torch, pa = self.torch, self.pa
        st = self.setup_split("decode_256seq_fp8")
        w, inp = st["w"], st["inp"]

        def call():
            pa.attn_paged_decode_window(inp.q, 1, st["k"], st["v"], st["ks"], st["vs"],
                                        inp.n_pages, inp.table, w.max_pages, inp.lengths,
                                        w.n_seq, window, None, w.n_head, w.n_head_kv,
                                        w.head_dim, 16, st["kv"], st["out"], st["ws"], st["wsb"])
        self.warm(call, warmup)
        evs = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
        for i in range(steps):
            pa.attn_set_kernel_timer(evs[i][0], evs[i][1])
            call()
        torch.cuda.synchronize()
        kern = sorted(self.ev.elapsed_ms(a, b) for a, b in evs)
        for a, b in evs:
            self.ev.destroy(a)
            self.ev.destroy(b)
        us = kern[len(kern) // 2] * 1e3
        # keys in the window of each row; pages (scales, table) from the first
        # page holding one of them
        b = 1
        tot = 0
        for c in st["lengths_host"]:
            lo = max(0, c - window)
            pages = -(-c // 16) - lo // 16
            tot += (c - lo) * w.n_head_kv * w.head_dim * 2 * b + pages * 4 + \
                pages * w.n_head_kv * 2 * 4
        tot += w.n_seq * w.n_head * w.head_dim * 2 + 4 * w.n_seq
        return {"window": window, "kernel_median_us": round(us, 2), "bytes": tot,
                "kernel_gbs": round(tot / (us * 1e-6) / 1e9, 1),
                "hbm_frac": round(tot / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    def time_widths(self, widths=(1, 2, 4, 8), steps=20, warmup=5):
        """Rounds of several widths over the 32-sequence verify cache (d 256,
        bf16, 4,104 tokens each): split-kernel time per width (HIP events
        from the library's kernel timer) and the bytes it streams."""
        torch, pa = self.torch, self.pa
        st = self.setup_split("verify_32seq_8rows")
        w, inp = st["w"], st["inp"]
        res = {}
        for width in widths:
            q = inp.q[:, :width].contiguous()
            out = torch.empty_like(q)

            def call():
                pa.attn_paged_verify_width(q, st["k"], st["v"], st["ks"], st["vs"], inp.n_pages,
                                           inp.table, w.max_pages, inp.lengths, w.n_seq, width,
                                           w.n_head, w.n_head_kv, w.head_dim, 16, st["kv"], out,
                                           st["ws"], st["wsb"])
            self.warm(call, warmup)
            evs = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
            for i in range(steps):
                pa.attn_set_kernel_timer(evs[i][0], evs[i][1])
                call()
            torch.cuda.synchronize()
            kern = sorted(self.ev.elapsed_ms(a, b) for a, b in evs)
            for a, b in evs:
                self.ev.destroy(a)
                self.ev.destroy(b)
            by = decode_bytes(st["lengths_host"], self.synth.scaled(w, rows=width),
                              with_out=False)
            us = kern[len(kern) // 2] * 1e3
            res["w%d" % width] = {"kernel_median_us": round(us, 2), "bytes": by,
                                  "hbm_frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        return res

    def time_tree(self, width=8, steps=20, warmup=5):
        """A tree-shaped round of 8 rows per sequence (each row's parent drawn
        at random among the earlier rows, seed 1008) over the 32-sequence
        verify cache: the whole call (branch staging, split kernel, combine)
        and its split kernel alone, medians of HIP events."""
        import numpy as np
        torch, pa = self.torch, self.pa
        st = self.setup_split("verify_32seq_8rows", spare_pages=2 * 32 * width)
        w, inp = st["w"], st["inp"]
        S = w.n_seq
        masks = self.synth.tree_masks(S, width, 1008)
        used = set(inp.table.cpu().numpy().ravel().tolist())
        free = [p for p in range(inp.n_pages) if p not in used][:2 * S * width]
        scratch = torch.tensor(free, dtype=torch.int32, device="cuda")
        mask_d = torch.from_numpy(masks).cuda()
        wsb = pa.attn_paged_workspace_bytes(4, S, w.max_pages, w.n_head, w.head_dim)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        q = inp.q[:, :width].contiguous()
        out = torch.empty_like(q)

        def call():
            pa.attn_paged_verify_tree(q, st["k"], st["v"], st["ks"], st["vs"], inp.n_pages,
                                      inp.table, w.max_pages, inp.lengths, S, width, mask_d,
                                      scratch, w.n_head, w.n_head_kv, w.head_dim, 16, st["kv"],
                                      out, ws, wsb)
        self.warm(call, warmup)
        kev = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i in range(steps):
            pa.attn_set_kernel_timer(kev[i][0], kev[i][1])
            cev[i][0].record()
            call()
            cev[i][1].record()
        torch.cuda.synchronize()
        kern = sorted(self.ev.elapsed_ms(a, b) for a, b in kev)
        whole = sorted(a.elapsed_time(b) for a, b in cev)
        for a, b in kev:
            self.ev.destroy(a)
            self.ev.destroy(b)
        depth = int(sum(bin(int(m)).count("1") for m in masks.ravel()))
        return {"call_median_us": round(whole[len(whole) // 2] * 1e3, 2),
                "split_kernel_median_us": round(kern[len(kern) // 2] * 1e3, 2),
                "rows": S * width, "mean_branch_depth": round(depth / (S * width), 3)}

    def time_prefill_fp8(self, steps=10, warmup=3, rounds=3):
        """The 4,096-row chunk over 28,672 cached rows with an fp8 cache:
        the plain prefill (bf16 MFMA on the decoded codes) against
        ATTN_PREFILL_FP8_QK (QK^T on the fp8 matrix unit) and QK | PV (PV on
        it too), kernel medians by the library's kernel timer, best of
        interleaved rounds."""
        torch, pa = self.torch, self.pa
        w = self.synth.scaled(self.synth.WORKLOADS["prefill_4096_over_28672"], kv_fp8=True,
                              name="prefill_4096_over_28672_fp8kv")
        st = self.setup_prefill(None, w)
        inp = st["inp"]
        fl = prefill_flops(w.rows, st["C"], w)
        best = {}
        for _ in range(rounds):
            for bits in (0, pa.ATTN_PREFILL_FP8_QK,
                         pa.ATTN_PREFILL_FP8_QK | pa.ATTN_PREFILL_FP8_PV):
                def call(timer=None):
                    if timer is not None:
                        pa.attn_set_kernel_timer(timer[0], timer[1])
                    pa.attn_paged_prefill_fp8(st["q"], w.rows, st["k"], st["v"], st["ks"],
                                              st["vs"], inp.n_pages, inp.table, w.max_pages,
                                              st["C"], w.n_head, w.n_head_kv, w.head_dim, 16,
                                              st["kv"], bits, st["out"])
                self.warm(call, warmup)
                evs = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
                for i in range(steps):
                    call(evs[i])
                torch.cuda.synchronize()
                kern = sorted(self.ev.elapsed_ms(a, b) for a, b in evs)
                for a, b in evs:
                    self.ev.destroy(a)
                    self.ev.destroy(b)
                med = kern[len(kern) // 2]
                best[bits] = min(best.get(bits, med), med)
        res = {}
        qkpv = pa.ATTN_PREFILL_FP8_QK | pa.ATTN_PREFILL_FP8_PV
        for bits, tag in ((0, "bits0_bf16_qk"), (pa.ATTN_PREFILL_FP8_QK, "qk_fp8"),
                          (qkpv, "qk_pv_fp8")):
            ms = best[bits]
            res[tag] = {"kernel_median_ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                        "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
        # With both bits every product runs on the fp8 matrix unit.
        res["qk_pv_fp8"]["frac_of_fp8_peak"] = round(
            fl / (best[qkpv] * 1e-3) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4)
        res["flops_per_launch"] = fl
        res["speedup"] = round(best[0] / best[pa.ATTN_PREFILL_FP8_QK], 3)
        res["speedup_qk_pv"] = round(best[0] / best[qkpv], 3)
        del st
        torch.cuda.empty_cache()
        return res

    def time_prefill(self, st, steps, warmup):
        torch = self.torch
        self.warm(lambda: self.prefill_step(st), warmup)
        evs = [(self.ev.create(), self.ev.create()) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.prefill_step(st, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        kern = [self.ev.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            self.ev.destroy(a)
            self.ev.destroy(b)
        return wall, sum(kern) / len(kern), sorted(kern)[len(kern) // 2]


def cpu_baseline(st, torch, synth, min_seconds=10.0, max_runs=15):
    """The CPU oracle timed on the whole headline workload (every sequence),
    run repeatedly until about `min_seconds` of CPU work have passed, priced
    with the same byte accounting as the GPU value (median run)."""
    import numpy as np
    import oracle

    w, inp = st["w"], st["inp"]
    lens = st["lengths_host"]
    n = len(lens)
    need = [-(-c // 16) for c in lens]
    table = inp.table.cpu().numpy()
    old = np.concatenate([table[s, :k] for s, k in enumerate(need)])
    new_table = np.full((n, w.max_pages), -1, np.int32)
    pos = 0
    for s, k in enumerate(need):
        new_table[s, :k] = np.arange(pos, pos + k)
        pos += k
    idx = torch.from_numpy(old.astype(np.int64)).cuda()
    kp = synth.bits(st["k"].index_select(0, idx))
    vp = synth.bits(st["v"].index_select(0, idx))
    ks = st["ks"].index_select(0, idx).cpu().numpy() if w.kv_fp8 else None
    vs = st["vs"].index_select(0, idx).cpu().numpy() if w.kv_fp8 else None
    del idx
    q = synth.bits(inp.q)
    threads = oracle.default_threads()
    oracle.build()
    runs = []
    while len(runs) < max_runs and (len(runs) < 3 or sum(runs) < min_seconds):
        t0 = time.perf_counter()
        oracle.paged_attention(q, kp, vp, new_table, np.asarray(lens, np.int32),
                               n_head=w.n_head, n_head_kv=w.n_head_kv, head_dim=w.head_dim,
                               page_size=16,
                               kv_dtype=oracle.KV_FP8 if w.kv_fp8 else oracle.KV_BF16,
                               k_scale=ks, v_scale=vs, threads=threads)
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[len(runs) // 2]
    gbs = decode_bytes(lens, w) / dt / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "decode attention of all %d sequences (%d cached tokens), fp64 oracle, "
                      "median of %d runs (%.2f s each, %.1f s in all)"
                      % (n, sum(lens), len(runs), dt, sum(runs))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_256seq_fp8")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibration", action="store_true",
                    help="run a 1 GiB fill and a 1 GiB sum (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibration:
        import torch
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        s = None
        for _ in range(3):
            x.fill_(1.0)   # writes 1 GiB
            s = x.sum()    # reads 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "fill 1 GiB, sum 1 GiB", "sum": float(s)}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_20_amd as pa
    from paged_kv_cache_20_amd import synth

    torch.cuda.set_device(0)
    b = Bench(torch, pa, synth)
    name = args.workload
    w = synth.WORKLOADS[name]
    log("[bench] headline", name)
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "fp8-e4m3 KV, bf16 MFMA, fp32 accumulation" if w.kv_fp8 else "bf16",
              "data": "synthetic"}
    if w.kind == "prefill":
        st = b.setup_prefill(name)
        wall, kavg, kmed = b.time_prefill(st, args.steps, args.warmup)
        fl = prefill_flops(w.rows, st["C"], w)
        result.update(value=round(fl / wall / 1e12, 2), unit="TFLOP/s",
                      ms_per_step=round(wall * 1e3, 4))
        achieved = fl / (kavg * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2),
                              "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                              "traffic": traffic_from_profiles(
                                  "prefill_pipe_kernel" if not w.kv_fp8 else "prefill_kernel")}
    else:
        st = b.setup_split(name)
        wall, kavg, kmed = b.time_split(st, args.steps, args.warmup)
        lens = st["lengths_host"]
        step_bytes = decode_bytes(lens, w) + append_bytes(w.n_seq * w.rows, w)
        split_bytes = decode_bytes(lens, w, with_out=False)
        result.update(value=round(step_bytes / wall / 1e9, 2), unit="GB/s",
                      ms_per_step=round(wall * 1e3, 4))
        achieved = split_bytes / (kavg * 1e-3) / 1e9
        result["us_per_step"] = round(wall * 1e6, 2)
        result["hbm_frac"] = round(step_bytes / wall / 1e9 / HBM_PEAK_GBS, 4)
        result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBS, 4),
                              "traffic": traffic_from_profiles("split_kernel_" + name),
                              "kernel": "split_kernel", "kernel_avg_us": round(kavg * 1e3, 2),
                              "kernel_median_us": round(kmed * 1e3, 2),
                              "algorithmic_bytes_per_launch": split_bytes}
        # The step's parts by events on the stream: the append (A0) of the
        # step's new rows, and the attention call (split + combine kernels).
        result["append_us_median"] = st["append_us_median"]
        result["attention_call_us_median"] = st["call_us_median"]
        result["append_bytes"] = append_bytes(w.n_seq * w.rows, w)
    result["config"] = {"workload": name, "n_seq": w.n_seq, "rows": w.rows, "n_head": w.n_head,
                        "n_head_kv": w.n_head_kv, "head_dim": w.head_dim, "page_size": 16,
                        "kv_dtype": "fp8-e4m3" if w.kv_fp8 else "bf16",
                        "ctx": "%s[%d,%d]" % (w.lengths, w.ctx_lo, w.ctx_hi),
                        "sum_ctx": int(sum(st["inp"].lengths.cpu().tolist())),
                        "seed": w.seed}
    log("[bench] headline done", json.dumps(result))

    if not args.no_cpu and w.kind != "prefill":
        log("[bench] cpu baseline")
        result["cpu_baseline"] = cpu_baseline(st, torch, synth)
        log("[bench] cpu baseline done", result["cpu_baseline"])
    del st
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        for other in ("decode_1seq_ctx512", "decode_64seq_hd256", "verify_32seq_8rows",
                      "prefill_4096_over_28672"):
            if other == name:
                continue
            ow = synth.WORKLOADS[other]
            log("[bench] secondary", other)
            try:
                if ow.kind == "prefill":
                    s2 = b.setup_prefill(other)
                    wall, kavg, kmed = b.time_prefill(s2, 10, 3)
                    fl = prefill_flops(ow.rows, s2["C"], ow)
                    sec[other] = {"ms_per_step": round(wall * 1e3, 4),
                                  "kernel_avg_ms": round(kavg, 4),
                                  "tflops": round(fl / (kavg * 1e-3) / 1e12, 2),
                                  "mfma_frac": round(fl / (kavg * 1e-3) / 1e12 /
                                                     BF16_MFMA_PEAK_TFLOPS, 4),
                                  "flops_per_launch": fl}
                else:
                    s2 = b.setup_split(other)
                    wall, kavg, kmed = b.time_split(s2, 30, 5)
                    lens = s2["lengths_host"]
                    by = decode_bytes(lens, ow, with_out=False)
                    sec[other] = {"us_per_step": round(wall * 1e6, 2),
                                  "kernel_avg_us": round(kavg * 1e3, 2),
                                  "kernel_gbs": round(by / (kavg * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(by / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "bytes_per_launch": by}
                    if ow.kind == "verify":
                        fl = 4 * ow.n_head * ow.head_dim * sum(
                            8 * c - 28 for c in lens)  # pairs of 8 causal rows
                        sec[other]["tflops"] = round(fl / (kavg * 1e-3) / 1e12, 2)
                del s2
            except Exception as e:  # report, keep the headline
                sec[other] = {"error": str(e)[:200]}
            torch.cuda.empty_cache()
            log("[bench] secondary done", other, sec[other])
        log("[bench] secondary windowed decode")
        try:
            sec["decode_256seq_fp8_window4096"] = b.time_window()
        except Exception as e:  # report, keep the headline
            sec["decode_256seq_fp8_window4096"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
        log("[bench] secondary done", sec["decode_256seq_fp8_window4096"])
        log("[bench] secondary verify widths")
        try:
            sec["verify_32seq_widths_1_2_4_8"] = b.time_widths()
        except Exception as e:  # report, keep the headline
            sec["verify_32seq_widths_1_2_4_8"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
        log("[bench] secondary done", sec["verify_32seq_widths_1_2_4_8"])
        log("[bench] secondary fp8 prefill")
        try:
            sec["prefill_4096_over_28672_fp8kv_qk"] = b.time_prefill_fp8()
        except Exception as e:  # report, keep the headline
            sec["prefill_4096_over_28672_fp8kv_qk"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
        log("[bench] secondary done", sec["prefill_4096_over_28672_fp8kv_qk"])
        log("[bench] secondary tree round")
        try:
            sec["verify_32seq_tree8"] = b.time_tree()
        except Exception as e:  # report, keep the headline
            sec["verify_32seq_tree8"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
        log("[bench] secondary done", sec["verify_32seq_tree8"])
        log("[bench] secondary mixed_256dec_fp8_plus_2048chunk")
        try:
            sec["mixed_256dec_fp8_plus_2048chunk"] = b.time_mixed()
        except Exception as e:  # report, keep the headline
            sec["mixed_256dec_fp8_plus_2048chunk"] = {"error": str(e)[:200]}
        torch.cuda.empty_cache()
        log("[bench] secondary done", sec["mixed_256dec_fp8_plus_2048chunk"])
        result["secondary"] = sec
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
