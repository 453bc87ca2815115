#!/usr/bin/env python3
"""Decode-step attention benchmark for Windowed-MTP on one MI355X.

One step is the attention of one speculative decode step at 1,048,576 tokens
of context (the per-decode-step cost model): gamma = 3 draft steps of one MTP
draft layer (append one entry, draft attention, LSE combine) followed by the
verify attention of 10 full-attention target layers (append gamma+1 entries,
verify over all keys with 4 causal queries, LSE combine).  16 query heads,
2 KV heads, head_dim 256, bf16 KV, fp32 accumulation, paged pools of 16-token
blocks with a random-permutation block table.

The draft runs in both modes: native (full context from the paged pool) and
Windowed-MTP (4 sinks + 4,096-token window from the compact ring).  `value` is
the Windowed-MTP step time in microseconds; the native step and the ratio are
reported beside it.  Inputs are synthetic and resident in HBM before timing.

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from long_context_decode_gqa_amd import wmtp as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "draft+verify attention µs/decode-step and HBM GB/s (% of peak) at 1M context"

# HBM bytes per verify launch at the 1M-token workload, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the factors a plain
# 256 MiB device copy gives in the same run (FETCH x2.0, WRITE x1.0).  Valid only
# for the kernel code they were taken with (sha256 of the sources without
# comments and whitespace, below); otherwise null.
VERIFY_TRAFFIC = {"sources_sha256": "054721d1e60e93c91416d13fd54f3e69225322b1b9e9135995521abbe247011c",
                  "fetch_kib": 1049653.28, "write_kib": 8232.00, "fetch_factor": 2.0, "write_factor": 1.0}
VERIFY_SOURCES = ("long_context_decode_gqa_amd/csrc/wmtp_verify.hip", "long_context_decode_gqa_amd/csrc/wmtp_row_tile.hpp",
                  "long_context_decode_gqa_amd/csrc/wmtp_teams.hpp", "long_context_decode_gqa_amd/csrc/wmtp_device.hpp")


def verify_sources_sha256() -> str:
    """sha256 of the verify kernel's sources with comments and whitespace removed."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in VERIFY_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def verify_kernel_name(t_q, group):
    """The kernel a verify launch of t_q queries at G = group, head_dim 256, runs on."""
    row_tiles = (t_q * group + 31) // 32
    if row_tiles == 1:
        return f"mfma_attn_kernel<256, {group}, false, false>"
    return f"mfma_attn_teams_kernel<256, {group}, {row_tiles}>"


def verify_traffic_bytes():
    t = VERIFY_TRAFFIC
    if t["fetch_kib"] is None or t["sources_sha256"] != verify_sources_sha256():
        return None
    return int(round((t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]) * 1024))


# Untimed launches (~0.3 ms each over 2 GiB) before a probe's timed ones: the device's
# rate settles only after ~20 ms of sustained load.
SETTLE_LAUNCHES = 60


def stream_ceiling_gbps(dev, nbytes=2 << 30):
    """Best rate of the library's streaming-read probe over a 2 GiB buffer."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    best = 0.0
    for wgs in (256, 512, 1024, 2048):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
        for _ in range(SETTLE_LAUNCHES):
            W.stream_read(src, sink, wgs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            W.stream_read(src, sink, wgs)
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) / 10 * 1e-3) / 1e9)
    del src
    torch.cuda.empty_cache()
    return best


def paged_ceiling_gbps(step, run_kib=16):
    """Best rate of the paged streaming-read probe over one verify layer's pool, read in the
    block table's order, one head's blocks after another: per (block, head) the 8 KiB of K and
    the 8 KiB of V after it, i.e. the verify's own access pattern without its arithmetic.
    run_kib=32 (K|V pools): per block the 32 KiB of both heads instead."""
    wl, n = step.wl, step.n0 + step.wl.gamma + 1
    pool = step.layers[1][0]
    nb = synth.blocks_for(n, 16)
    Hk = wl.num_kv_heads
    run_bytes = 16 * wl.head_dim * 2                       # one (block, head) half: K or V
    bt = step.bt[0, :nb].to(torch.int64)
    runs = torch.cat([bt * Hk + h for h in range(Hk)])
    if step.kv_runs and run_kib == 32:
        # both heads of a block, 32 KiB in the K|V pool: halves of 16 KiB read back to back
        flat = pool.view(-1)
        run_bytes = Hk * run_bytes
        k, v = flat, flat[run_bytes // 2:]
        runs = 2 * bt
    elif step.kv_runs:
        flat = pool.view(-1)
        k, v = flat, flat[run_bytes // 2:]                 # V of a run starts 8 KiB after its K
        runs = 2 * runs
    else:
        k, v = pool
    runs = runs.to(torch.int32).contiguous()
    nbytes = 2 * runs.numel() * run_bytes
    best = 0.0
    for wgs in (256, 512):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device=k.device)
        for _ in range(SETTLE_LAUNCHES):
            W.stream_read_paged(k, v, runs, run_bytes, sink, wgs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            W.stream_read_paged(k, v, runs, run_bytes, sink, wgs)
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) / 10 * 1e-3) / 1e9)
    return best


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Device state of one decode step: draft layer (pool + ring) and target layers."""

    def __init__(self, wl, n0, target_layers, chunk_full, chunk_win, split, dev, kv_runs=True):
        self.wl, self.n0, self.dev = wl, n0, dev
        Hq, Hk, D, g = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma
        self.sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
        self.chunk_full, self.chunk_win, self.split = chunk_full, chunk_win, split
        blocks = synth.blocks_for(n0 + g + 1, 16)
        bt, total = synth.block_table(wl.seed, [blocks], permuted=True)
        self.bt = torch.from_numpy(bt).to(dev)
        self.total_blocks = total
        # (pool, desc): index 0 is the draft layer's native pool.  kv_runs: each pool holds K and V
        # of a (block, head) side by side, [blocks][H_kv][2][16][D] (one 16 KiB run per block and
        # head); else separate K and V pools [blocks][H_kv][16][D] (pool = (k, v)).
        self.kv_runs = kv_runs
        self.layers = []
        for layer in range(target_layers + 1):
            if kv_runs:
                pool = synth.normal((total, Hk, 2, 16, D), wl.seed, ("pool_kv", layer), wl.kv_scale, "bf16", dev)
                self.layers.append((pool, W.make_paged_interleaved(pool, self.bt)))
            else:
                k = synth.normal((total, Hk, 16, D), wl.seed, ("pool_k", layer), wl.kv_scale, "bf16", dev)
                v = synth.normal((total, Hk, 16, D), wl.seed, ("pool_v", layer), wl.kv_scale, "bf16", dev)
                self.layers.append(((k, v), W.make_paged(k, v, self.bt)))
            log(f"  pool {layer} ready")
        S, Wn = wl.sink, wl.window
        self.R = R = g - 1                    # headroom for rolling back rejected drafts
        self.rk = torch.zeros((1, Hk, S + Wn + R, D), dtype=torch.bfloat16, device=dev)
        self.rv = torch.zeros_like(self.rk)
        self.tags = torch.full((1, S + Wn + R), -1, dtype=torch.int32, device=dev)
        self.ring = W.make_ring(self.rk, self.rv, self.tags, S, Wn, R)
        # ring holds the sinks and the last W context tokens of the draft layer's sequence
        sink_k = synth.normal((1, S, Hk, D), wl.seed, "ring_sink_k", wl.kv_scale, "bf16", dev)
        sink_v = synth.normal((1, S, Hk, D), wl.seed, "ring_sink_v", wl.kv_scale, "bf16", dev)
        tail_k = synth.normal((1, Wn, Hk, D), wl.seed, "ring_tail_k", wl.kv_scale, "bf16", dev)
        tail_v = synth.normal((1, Wn, Hk, D), wl.seed, "ring_tail_v", wl.kv_scale, "bf16", dev)
        s_eff = min(S, n0)                        # contexts shorter than S + W fill what they have
        t_eff = min(n0 - s_eff, Wn)
        if s_eff:
            W.ring_append(self.sh, self.ring, sink_k[:, :s_eff].contiguous(), sink_v[:, :s_eff].contiguous(), [0])
        if t_eff:
            W.ring_append(self.sh, self.ring, tail_k[:, Wn - t_eff:].contiguous(), tail_v[:, Wn - t_eff:].contiguous(),
                          [n0 - t_eff])
        self.tail_k, self.tail_v = tail_k, tail_v
        # per-step inputs
        self.q_draft = synth.normal((g, 1, Hq, D), wl.seed, "q_draft", 1.0, "bf16", dev)
        self.k_draft = synth.normal((g, 1, 1, Hk, D), wl.seed, "k_new", wl.kv_scale, "bf16", dev)
        self.v_draft = synth.normal((g, 1, 1, Hk, D), wl.seed, "v_new", wl.kv_scale, "bf16", dev)
        self.q_ver = [synth.normal((1, g + 1, Hq, D), wl.seed, ("q_verify", l), 1.0, "bf16", dev)
                      for l in range(target_layers)]
        self.k_ver = synth.normal((1, g + 1, Hk, D), wl.seed, "k_new_layer", wl.kv_scale, "bf16", dev)
        self.v_ver = synth.normal((1, g + 1, Hk, D), wl.seed, "v_new_layer", wl.kv_scale, "bf16", dev)
        # workspaces and outputs
        lens_d = [n0 + g]
        self.ws_full = W.workspace(W.draft_workspace_bytes(W.FULL, self.sh, lens_d, chunk_full), dev)
        self.ws_win = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, self.sh, lens_d, chunk_win, S, Wn, R), dev)
        self.ws_ver = W.workspace(W.verify_workspace_bytes(self.sh, g + 1, [n0 + g + 1], split), dev)
        self.out_d = torch.empty((1, Hq, D), dtype=torch.float32, device=dev)
        self.lse_d = torch.empty((1, Hq), dtype=torch.float32, device=dev)
        self.out_v = torch.empty((1, (g + 1) * Hq, D), dtype=torch.float32, device=dev)
        self.lse_v = torch.empty((1, (g + 1) * Hq), dtype=torch.float32, device=dev)
        self._calls = {}

    def draft(self, mode, flag, ev=None, fused=True):
        """gamma draft steps.  fused: each step's append runs inside its attention launch
        (wmtp_draft_attn_append); else an append call precedes wmtp_draft_attn.  ev brackets
        the first step's attention launch (with the fused append, that launch includes it)."""
        g, n0 = self.wl.gamma, self.n0
        for j in range(g):
            pos, n = n0 + j, n0 + j + 1
            kw = dict(paged=self.layers[0][1], chunk_tokens=self.chunk_full) if mode == W.FULL else \
                dict(ring=self.ring, chunk_tokens=self.chunk_win)
            ws = self.ws_full if mode == W.FULL else self.ws_win
            if not fused:
                if mode == W.FULL:
                    W.paged_append(self.sh, self.layers[0][1], self.k_draft[j], self.v_draft[j], [pos])
                else:
                    W.ring_append(self.sh, self.ring, self.k_draft[j], self.v_draft[j], [pos])
            if ev is not None:
                ev[0].record()
            if fused:
                parts = W.draft_attn_append(mode | flag, self.sh, self.q_draft[j], self.k_draft[j], self.v_draft[j],
                                            [n], ws, **kw)
            else:
                parts = W.draft_attn(mode | flag, self.sh, self.q_draft[j], [n], ws, **kw)
            if ev is not None:
                ev[1].record()
                ev = None
            W.combine(parts, self.out_d, self.lse_d)

    def verify(self, ev_list=None, fused=True):
        """The target layers' verify; fused: each layer's append runs inside its verify launch."""
        g, n0 = self.wl.gamma, self.n0
        for l in range(len(self.layers) - 1):
            desc = self.layers[l + 1][1]
            if not fused:
                W.paged_append(self.sh, desc, self.k_ver, self.v_ver, [n0])
            if ev_list is not None:
                ev_list[l][0].record()
            if fused:
                parts = W.verify_attn_append(self.sh, self.q_ver[l], g + 1, desc, self.k_ver, self.v_ver,
                                             [n0 + g + 1], self.ws_ver, self.split)
            else:
                parts = W.verify_attn(self.sh, self.q_ver[l], g + 1, desc, [n0 + g + 1], self.ws_ver, self.split)
            if ev_list is not None:
                ev_list[l][1].record()
            W.combine(parts, self.out_v, self.lse_v)


    def calls(self, mode, flag, fused=True):
        """The launches of one decode step as prepared C-ABI calls, in launch order: a list of
        (kind, index, call) with kind in draft / draft_combine / verify / verify_combine (and append
        for the unfused step).  The calls run once here, which fills each attention call's partials
        before the combine that reads them is prepared."""
        key = (mode, flag, fused)
        if key in self._calls:
            return self._calls[key]
        g, n0 = self.wl.gamma, self.n0
        out = []
        for j in range(g):
            pos, n = n0 + j, n0 + j + 1
            full = mode == W.FULL
            kw = dict(paged=self.layers[0][1], chunk_tokens=self.chunk_full) if full else \
                dict(ring=self.ring, chunk_tokens=self.chunk_win)
            ws = self.ws_full if full else self.ws_win
            if fused:
                a = W.prepare_draft_attn_append(mode | flag, self.sh, self.q_draft[j], self.k_draft[j],
                                                self.v_draft[j], [n], ws, **kw)
            else:
                app = (W.prepare_paged_append(self.sh, self.layers[0][1], self.k_draft[j], self.v_draft[j], [pos])
                       if full else W.prepare_ring_append(self.sh, self.ring, self.k_draft[j], self.v_draft[j], [pos]))
                app()
                out.append(("append", j, app))
                a = W.prepare_draft_attn(mode | flag, self.sh, self.q_draft[j], [n], ws, **kw)
            a()
            c = W.prepare_combine(a.parts, self.out_d, self.lse_d)
            c()
            out += [("draft", j, a), ("draft_combine", j, c)]
        for l in range(len(self.layers) - 1):
            desc = self.layers[l + 1][1]
            if fused:
                a = W.prepare_verify_attn_append(self.sh, self.q_ver[l], g + 1, desc, self.k_ver, self.v_ver,
                                                 [n0 + g + 1], self.ws_ver, self.split)
            else:
                app = W.prepare_paged_append(self.sh, desc, self.k_ver, self.v_ver, [n0])
                app()
                out.append(("append", 100 + l, app))
                a = W.prepare_verify_attn(self.sh, self.q_ver[l], g + 1, desc, [n0 + g + 1], self.ws_ver, self.split)
            a()
            c = W.prepare_combine(a.parts, self.out_v, self.lse_v)
            c()
            out += [("verify", l, a), ("verify_combine", l, c)]
        self._calls[key] = out
        return out


def kv_bytes(tokens, wl):
    return tokens * wl.num_kv_heads * wl.head_dim * 2 * 2


def verify_launch_bytes(n, wl, t_q):
    """Algorithmic bytes of one verify launch: visible K/V, queries, block-table entries, and the
    t_q new tokens' K/V written into the cache (the append runs inside the launch)."""
    return kv_bytes(n, wl) + t_q * wl.num_q_heads * wl.head_dim * 2 + synth.blocks_for(n, 16) * 4 + kv_bytes(t_q, wl)


def draft_launch_bytes(entries, wl, paged):
    """Algorithmic bytes of one draft launch: visible K/V, the query, block-table entries (or ring
    tags), and the step's new token's K/V written into the cache (the append runs inside the launch)."""
    b = kv_bytes(entries, wl) + wl.num_q_heads * wl.head_dim * 2 + kv_bytes(1, wl)
    return b + (synth.blocks_for(entries, 16) * 4 if paged else entries * 4)


def time_steps(step, mode, flag, steps, warmup, fused=True, per_launch=True):
    """Warmup, then `steps` decode steps of prepared C-ABI calls with the garbage collector off.

    Two timed passes over the same launches: the first records events only at step boundaries
    (the step times: an event recorded between two launches costs device time, 2-5 us each at
    this size); the second records an event after every launch as well, and the interval ending
    at a launch's event is that launch's time on the device's timeline, any idle gap before it
    included.  Returns {"step": [ms per step], kind: [[ms per launch of that kind] per step]}
    (launch kinds from the second pass, or none with per_launch=False)."""
    calls = step.calls(mode, flag, fused)
    torch.cuda.synchronize()
    for _ in range(warmup):
        for _, _, c in calls:
            c()
    res = {}
    for every in ((False, True) if per_launch else (False,)):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        gc_was = gc.isenabled()
        gc.disable()
        try:
            for s in range(steps):
                ev = evs[s]
                ev[0].record()
                for i, (_, _, c) in enumerate(calls):
                    c()
                    if every:
                        ev[i + 1].record()
                if not every:
                    ev[-1].record()
            torch.cuda.synchronize()
        finally:
            if gc_was:
                gc.enable()
        if not every:
            res["step"] = [ev[0].elapsed_time(ev[-1]) for ev in evs]
            continue
        res["step_with_launch_events"] = [ev[0].elapsed_time(ev[-1]) for ev in evs]
        for i, (kind, _, _) in enumerate(calls):
            res.setdefault(kind, [[] for _ in range(steps)])
            for s in range(steps):
                res[kind][s].append(evs[s][i].elapsed_time(evs[s][i + 1]))
    return res


def flat(per_step):
    return [x for row in per_step for x in row]


def med(ms):
    return float(np.median(np.asarray(ms, dtype=np.float64)))


def pct(ms, full=False):
    """median / p10 / p90 (and with full=True mean, max and the count above 1.1 x median) of a list of
    milliseconds, in microseconds."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    m = float(np.median(a))
    out = {"median": round(m, 1), "p10": round(float(np.percentile(a, 10)), 1),
           "p90": round(float(np.percentile(a, 90)), 1), "n": int(a.size)}
    if full:
        out.update(mean=round(float(a.mean()), 1), max=round(float(a.max()), 1),
                   above_1_1x_median=int((a > 1.1 * m).sum()))
    return out


def _hold(cycles=100000):
    """Keep the GPU busy for a bounded spin (tens of µs) while the host queues the timed launches,
    so the events measure device time rather than Python launch overhead."""
    torch.cuda._sleep(cycles)


def _timed(fn, reps, before=_hold):
    """Per-repetition milliseconds of fn() between events on the current stream (`before` runs untimed)."""
    out = []
    for _ in range(reps):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def graph_step(step, mode, flag, reps):
    """One whole decode step captured in a HIP graph and replayed.

    Eager work (clearing the outputs, snapshotting them) runs between replays,
    and every replay's outputs are compared with an eager step's, bit for bit
    (the kernels are deterministic).  Replays are queued back to back after an
    untimed one, as the eager steps are, so that no replay starts from an idle
    GPU.  Returns (per-replay ms, all replays matched).
    """
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step.draft(mode, flag)
        step.verify()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    ref_d, ref_v = step.out_d.clone(), step.out_v.clone()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step.draft(mode, flag)
        step.verify()
    torch.cuda.synchronize()
    for _ in range(5):          # settle under sustained load, as the eager warmup does
        gr.replay()
    _hold()
    evs, outs = [], []
    for _ in range(reps):
        step.out_d.zero_()
        step.out_v.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gr.replay()
        b.record()
        evs.append((a, b))
        outs.append((step.out_d.clone(), step.out_v.clone()))
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ok = all(torch.equal(d, ref_d) and torch.equal(v, ref_v) for d, v in outs)
    del gr
    torch.cuda.synchronize()
    return times, ok


def window_step_fn(step, flag, n):
    """One windowed draft step at length n (append at n - 1 and attend in one launch, combine)."""
    g0 = 0

    def run():
        parts = W.draft_attn_append(W.SINK_WINDOW | flag, step.sh, step.q_draft[g0], step.k_draft[g0],
                                    step.v_draft[g0], [n], step.ws_win, ring=step.ring, chunk_tokens=step.chunk_win)
        W.combine(parts, step.out_d, step.lse_d)
    return run


def window_measurements(step, flag, reps, dev, contexts):
    """Windowed draft step: warm and cold (1 GiB written between repetitions), and across contexts."""
    wl, n0 = step.wl, step.n0
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    run = window_step_fn(step, flag, n0 + 1)
    run()
    torch.cuda.synchronize()
    res = {"warm": pct(_timed(run, reps)), "cold_after_1GiB_write": pct(_timed(run, reps, lambda: flush.fill_(1)))}
    res["launches"] = ("draft attention with the ring append inside + combine; host launches queued behind a "
                       "spin or the flush")
    by_ctx = {}
    for n in contexts:
        # the ring of a sequence at length n: sinks at 0..S-1, the last W context tokens before n
        W.ring_append(step.sh, step.ring, step.tail_k, step.tail_v, [n - wl.window])
        r = window_step_fn(step, flag, n + 1)
        r()
        torch.cuda.synchronize()
        by_ctx[str(n)] = pct(_timed(r, reps, lambda: flush.fill_(1)))["median"]
    W.ring_append(step.sh, step.ring, step.tail_k, step.tail_v, [n0 - wl.window])   # back to n0
    torch.cuda.synchronize()
    del flush
    res["cold_median_by_context"] = by_ctx
    # rollback after a partial acceptance: forget the drafts past n0 + 1
    res["ring_rollback_us"] = pct(_timed(lambda: W.ring_rollback(step.ring, [n0 + 1]), reps))["median"]
    # The step is two short launches, so latency sets its cost.  Queued back to back (the device's
    # throughput for them) beside a one-block torch kernel as the floor of any launch; the figures
    # above, one step between two events, add the events' own cost (compare the empty launch).
    a = W.prepare_draft_attn_append(W.SINK_WINDOW | flag, step.sh, step.q_draft[0], step.k_draft[0],
                                    step.v_draft[0], [n0 + 1], step.ws_win, ring=step.ring, chunk_tokens=step.chunk_win)
    a()
    c = W.prepare_combine(a.parts, step.out_d, step.lse_d)
    x = torch.zeros(64, device=dev)

    def back_to_back(fn, count=20):
        fn()
        torch.cuda.synchronize()
        _hold(2000000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(count):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / count * 1e3, 2)
    res["back_to_back_us"] = {"step": back_to_back(lambda: (a(), c())), "attention": back_to_back(a),
                              "combine": back_to_back(c), "empty_launch": back_to_back(lambda: x.add_(1))}
    res["empty_launch_between_events_us"] = pct(_timed(lambda: x.add_(1), reps))["median"]
    return res


def native_split_measurements(step, flag, reps, dev):
    """Native draft launch at 1M with literal 256-key splits and with the library default."""
    n = step.n0 + 1
    out = {}
    for chunk, name in ((256, "split_256"), (0, "split_default")):
        ws = W.workspace(W.draft_workspace_bytes(W.FULL, step.sh, [n], chunk), dev)
        run = lambda: W.draft_attn(W.FULL | flag, step.sh, step.q_draft[0], [n], ws, paged=step.layers[0][1],
                                   chunk_tokens=chunk)
        run()
        out[name] = pct(_timed(run, reps))["median"]
        del ws
    return out


def other_head_reading(flag, reps, dev):
    """The 1M paged draft workload under the other reading of its head shapes: 4 query heads on
    1 KV head, d=64, bf16 (256 B per token).  Native and windowed draft step (append inside the
    attention launch, then the combine) in the launch configuration of the main step."""
    wl = synth.workload("paged_1m_bf16", num_q_heads=4, num_kv_heads=1, head_dim=64)
    Hq, Hk, D, S, Wn, R = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window, wl.gamma - 1
    n0 = wl.contexts[0]
    n = n0 + 1
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    bt, total = synth.block_table(wl.seed, [synth.blocks_for(n, 16)], permuted=True)
    pool = synth.normal((total, Hk, 2, 16, D), wl.seed, "pool_kv", wl.kv_scale, "bf16", dev)   # K|V runs
    btd = torch.from_numpy(bt).to(dev)
    desc = W.make_paged_interleaved(pool, btd)
    q = synth.normal((1, Hq, D), wl.seed, "q_draft", 1.0, "bf16", dev)
    kn = synth.normal((1, 1, Hk, D), wl.seed, "k_new", wl.kv_scale, "bf16", dev)
    vn = synth.normal((1, 1, Hk, D), wl.seed, "v_new", wl.kv_scale, "bf16", dev)
    out = torch.empty((1, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, Hq), dtype=torch.float32, device=dev)
    ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, [n], 0), dev)

    def native():
        W.combine(W.draft_attn_append(W.FULL | flag, sh, q, kn, vn, [n], ws, paged=desc), out, lse)
    native()
    t_nat = pct(_timed(native, reps))["median"]
    rk = torch.zeros((1, Hk, S + Wn + R, D), dtype=torch.bfloat16, device=dev)
    rv = torch.zeros_like(rk)
    tags = torch.full((1, S + Wn + R), -1, dtype=torch.int32, device=dev)
    ring = W.make_ring(rk, rv, tags, S, Wn, R)
    W.ring_append(sh, ring, synth.normal((1, S, Hk, D), wl.seed, "ring_sink_k", wl.kv_scale, "bf16", dev),
                  synth.normal((1, S, Hk, D), wl.seed, "ring_sink_v", wl.kv_scale, "bf16", dev), [0])
    W.ring_append(sh, ring, synth.normal((1, Wn, Hk, D), wl.seed, "ring_tail_k", wl.kv_scale, "bf16", dev),
                  synth.normal((1, Wn, Hk, D), wl.seed, "ring_tail_v", wl.kv_scale, "bf16", dev), [n0 - Wn])
    wsw = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, [n], 0, S, Wn, R), dev)

    def window():
        W.combine(W.draft_attn_append(W.SINK_WINDOW | flag, sh, q, kn, vn, [n], wsw, ring=ring), out, lse)
    window()
    t_win = pct(_timed(window, reps))["median"]
    res = {"shape": "4 q heads / 1 KV head, d=64, bf16", "context": n0,
           "native_draft_step_us": t_nat,
           "native_gbps": round(draft_launch_bytes(n, wl, True) / (t_nat * 1e-6) / 1e9, 1),
           "window_draft_step_us": t_win}
    del pool, ws, wsw, rk, rv, tags
    torch.cuda.empty_cache()
    return res


def mixed_batch(flag, reps, dev):
    """Four sequences of mixed length in one call: native draft, then the window draft at three W."""
    wl = synth.workload("mixed_4seq_bf16")
    Hq, Hk, D, S = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    lens = [n + 1 for n in wl.contexts]                 # after this step's append
    B = len(lens)
    bt, total = synth.block_table(wl.seed, [synth.blocks_for(n, 16) for n in lens], permuted=True)
    pool = synth.normal((total, Hk, 2, 16, D), wl.seed, "pool_kv", wl.kv_scale, "bf16", dev)   # K|V runs
    btd = torch.from_numpy(bt).to(dev)
    desc = W.make_paged_interleaved(pool, btd)
    q = synth.normal((B, Hq, D), wl.seed, "q_draft", 1.0, "bf16", dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, lens, 0), dev)

    def native():
        W.combine(W.draft_attn(W.FULL | flag, sh, q, lens, ws, paged=desc), out, lse)
    native()
    t = pct(_timed(native, reps))["median"]
    res = {"contexts": list(wl.contexts), "native_draft_step_us": t,
           "native_gbps": round(sum(lens) * Hk * D * 4 / (t * 1e-6) / 1e9, 1), "window_draft_step_us": {}}
    del ws
    for Wn in wl.windows:
        R = wl.gamma - 1
        rk = torch.zeros((B, Hk, S + Wn + R, D), dtype=torch.bfloat16, device=dev)
        rv = torch.zeros_like(rk)
        tags = torch.full((B, S + Wn + R), -1, dtype=torch.int32, device=dev)
        ring = W.make_ring(rk, rv, tags, S, Wn, R)
        sk = synth.normal((B, S, Hk, D), wl.seed, ("ring_sink_k", Wn), wl.kv_scale, "bf16", dev)
        sv = synth.normal((B, S, Hk, D), wl.seed, ("ring_sink_v", Wn), wl.kv_scale, "bf16", dev)
        tk = synth.normal((B, Wn, Hk, D), wl.seed, ("ring_tail_k", Wn), wl.kv_scale, "bf16", dev)
        tv = synth.normal((B, Wn, Hk, D), wl.seed, ("ring_tail_v", Wn), wl.kv_scale, "bf16", dev)
        W.ring_append(sh, ring, sk, sv, [0] * B)
        W.ring_append(sh, ring, tk, tv, [n - Wn for n in lens])
        wsw = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, lens, 0, S, Wn, R), dev)

        def window():
            W.combine(W.draft_attn(W.SINK_WINDOW | flag, sh, q, lens, wsw, ring=ring), out, lse)
        window()
        res["window_draft_step_us"][str(Wn)] = pct(_timed(window, reps))["median"]
        if Wn == max(wl.windows):
            # adaptive windows: every sequence its own W_b (and S_b) in one call on this ring layout
            mix_w = [wl.windows[b % len(wl.windows)] for b in range(B)]
            mix_s = [S if b % 2 == 0 else 0 for b in range(B)]
            pol = W.with_policy(ring, mix_s, mix_w)

            def mixed():
                W.combine(W.draft_attn(W.SINK_WINDOW | flag, sh, q, lens, wsw, ring=pol), out, lse)
            mixed()
            res["per_sequence_policy"] = {"sinks": mix_s, "windows": mix_w,
                                          "window_draft_step_us": pct(_timed(mixed, reps))["median"]}
        del rk, rv, tags, wsw
    del pool
    torch.cuda.empty_cache()
    return res


def draft_131k_measurements(flag, reps, dev):
    """The single-draft-layer workload at 131,072 tokens: gamma = 3 draft steps (each the append inside
    the attention launch, then the combine) in native mode over a contiguous K|V pool and in
    sink_window mode (S = 4, W = 4,096) over a ring of S + W slots.  Timed cold (1 GiB written
    between repetitions, as a real step's verify evicts the draft's KV) and warm."""
    wl = synth.workload("draft_131k_bf16")
    Hq, Hk, D, S, Wn, g = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window, wl.gamma
    n0 = wl.contexts[0]
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    nb = synth.blocks_for(n0 + g, 16)
    bt, total = synth.block_table(wl.seed, [nb], permuted=False)
    pool = synth.normal((total, Hk, 2, 16, D), wl.seed, "c2kv", wl.kv_scale, "bf16", dev)
    desc = W.make_paged_interleaved(pool, torch.from_numpy(bt).to(dev))
    rk = torch.zeros((1, Hk, S + Wn, D), dtype=torch.bfloat16, device=dev)
    rv = torch.zeros_like(rk)
    tags = torch.full((1, S + Wn), -1, dtype=torch.int32, device=dev)
    ring = W.make_ring(rk, rv, tags, S, Wn)
    W.ring_append(sh, ring, synth.normal((1, S, Hk, D), wl.seed, "c2_sink_k", wl.kv_scale, "bf16", dev),
                  synth.normal((1, S, Hk, D), wl.seed, "c2_sink_v", wl.kv_scale, "bf16", dev), [0])
    W.ring_append(sh, ring, synth.normal((1, Wn, Hk, D), wl.seed, "c2_tail_k", wl.kv_scale, "bf16", dev),
                  synth.normal((1, Wn, Hk, D), wl.seed, "c2_tail_v", wl.kv_scale, "bf16", dev), [n0 - Wn])
    q = synth.normal((g, 1, Hq, D), wl.seed, "c2q", 1.0, "bf16", dev)
    kn = synth.normal((g, 1, 1, Hk, D), wl.seed, "c2kn", wl.kv_scale, "bf16", dev)
    vn = synth.normal((g, 1, 1, Hk, D), wl.seed, "c2vn", wl.kv_scale, "bf16", dev)
    out = torch.empty((1, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, Hq), dtype=torch.float32, device=dev)
    lens = [n0 + g]
    ws_full = W.workspace(W.draft_workspace_bytes(W.FULL, sh, lens, 0), dev)
    ws_win = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, lens, 0, S, Wn, 0), dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    res = {"context": n0, "gamma": g, "sink": S, "window": Wn, "pool": "contiguous K|V runs (identity table)"}
    for mode, name in ((W.FULL, "native"), (W.SINK_WINDOW, "windowed")):
        calls = []
        for j in range(g):
            kw = dict(paged=desc) if mode == W.FULL else dict(ring=ring)
            a = W.prepare_draft_attn_append(mode | flag, sh, q[j], kn[j], vn[j], [n0 + j + 1],
                                            ws_full if mode == W.FULL else ws_win, **kw)
            a()
            c = W.prepare_combine(a.parts, out, lse)
            c()
            calls += [a, c]

        def run():
            for c in calls:
                c()
        run()
        torch.cuda.synchronize()
        cold = pct(_timed(run, reps, lambda: (flush.fill_(1), _hold(400000))))
        warm = pct(_timed(run, reps, lambda: _hold(400000)))
        nbytes = sum(draft_launch_bytes(min(n0 + j + 1, S + Wn) if mode == W.SINK_WINDOW else n0 + j + 1, wl,
                                        mode == W.FULL) for j in range(g))
        gbps = nbytes / (cold["median"] * 1e-6) / 1e9
        res[name] = {"cold_us": cold, "warm_us_median": warm["median"], "algorithmic_bytes": nbytes,
                     "gbps": round(gbps, 1), "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}
    res["ratio_native_over_windowed"] = round(res["native"]["cold_us"]["median"] /
                                              res["windowed"]["cold_us"]["median"], 3)
    res["launches"] = (f"{g} x (draft attention with the append inside + combine); host launches queued behind "
                       f"a spin (and the flush when cold)")
    del pool, flush, rk, rv, tags, ws_full, ws_win
    torch.cuda.empty_cache()
    return res


def native_draft_pv_measurements(step, reps):
    """The 1M native draft step (append inside the attention launch, then the combine) with fp32 softmax
    weights in the PV product (the whole-tile vector kernel) beside bf16 weight pairs (the matrix-core
    kernel), in the main step's launch configuration.  Every launch streams the 2 GiB pool, far past
    the caches, so each repetition reads it from HBM."""
    n = step.n0 + 1
    res = {}
    for flag, name in ((0, "fp32_weights_vector_kernel"), (W.DRAFT_FAST_PV, "bf16_weights_matrix_core_kernel")):
        a = W.prepare_draft_attn_append(W.FULL | flag, step.sh, step.q_draft[0], step.k_draft[0], step.v_draft[0],
                                        [n], step.ws_full, paged=step.layers[0][1], chunk_tokens=step.chunk_full)
        a()
        c = W.prepare_combine(a.parts, step.out_d, step.lse_d)

        def run():
            a()
            c()
        run()
        torch.cuda.synchronize()
        t = pct(_timed(run, reps, lambda: _hold(400000)), full=True)
        nbytes = draft_launch_bytes(n, step.wl, True)
        gbps = nbytes / (t["median"] * 1e-6) / 1e9
        res[name] = {"us": t, "gbps": round(gbps, 1), "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}
    res["algorithmic_bytes"] = draft_launch_bytes(n, step.wl, True)
    return res


def _per_rep(fn, budget_s):
    """Mean seconds per call of fn(rep), repeating until `budget_s` has passed (at least once)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(reps)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return el / reps, reps, el


def cpu_baseline(wl, n0, budget_s=12.0):
    """The float64 oracle on a bounded sample, scaled to one decode step (both draft modes).

    Sample, for one KV head: verify layers over all n0 + gamma + 1 keys (gamma + 1
    causal queries x G heads, a fresh query set each repetition), native draft
    steps over n0 + 1 keys and windowed draft steps over the sink + window
    entries, each repeated until its share of `budget_s` (3/4, 1/5, the rest)
    has passed; the mean per repetition is scaled by KV heads, target layers and
    draft steps.  Keys and values are synthetic bf16.
    """
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=cores)          # BLAS threads = the cores this process may use
    except ImportError:
        limits = None
    rng = np.random.default_rng(0)
    D, G, g = wl.head_dim, wl.group, wl.gamma
    n = n0 + g + 1
    kb = torch.from_numpy(rng.standard_normal((n, 1, D), dtype=np.float32) * 0.5).to(torch.bfloat16)
    vb = torch.from_numpy(rng.standard_normal((n, 1, D), dtype=np.float32) * 0.5).to(torch.bfloat16)
    src_k = O.LogicalKV(kb.view(torch.int16).numpy().view(np.uint16), "bf16")
    src_v = O.LogicalKV(vb.view(torch.int16).numpy().view(np.uint16), "bf16")
    qs = rng.standard_normal((4, g + 1, G, D))
    win = O.visible_positions(n0 + 1, O.SINK_WINDOW, wl.sink, wl.window)

    def verify_layer(r):
        for i in range(g + 1):
            O.attention_over(qs[r % 4, i], src_k, src_v, np.arange(n0 + i + 1), 0, wl.scale)

    t_verify, r_v, e_v = _per_rep(verify_layer, 0.75 * budget_s)
    t_native, r_n, e_n = _per_rep(
        lambda r: O.attention_over(qs[r % 4, 0], src_k, src_v, np.arange(n0 + 1), 0, wl.scale), 0.2 * budget_s)
    t_win, r_w, e_w = _per_rep(
        lambda r: O.attention_over(qs[r % 4, 0], src_k, src_v, win, 0, wl.scale), 0.05 * budget_s)
    if limits is not None:
        limits.restore_original_limits()
    Hk, L = wl.num_kv_heads, wl.target_layers
    verify_step = t_verify * Hk * L
    win_s, nat_s = verify_step + t_win * Hk * g, verify_step + t_native * Hk * g
    return {
        "value": round(win_s * 1e6, 1),
        "unit": "us/decode-step",
        "native_value": round(nat_s * 1e6, 1),
        # oracle-equivalent rate: the step's algorithmic K/V bytes over the oracle's time
        "gbps": round(step_bytes(n0, wl, True) / win_s / 1e9, 3),
        "native_gbps": round(step_bytes(n0, wl, False) / nat_s / 1e9, 3),
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 oracle on 1 KV head: {r_v} verify layer(s) ({g + 1} causal queries x {G} heads over "
                   f"{n} keys), {r_n} native draft step(s) ({n0 + 1} keys), {r_w} windowed draft step(s) "
                   f"({wl.sink}+{wl.window} entries); mean per repetition scaled x{Hk} KV heads, x{L} target "
                   f"layers, x{g} draft steps; measured {e_v + e_n + e_w:.1f} s"),
    }


def step_bytes(n0, wl, windowed):
    """Algorithmic K/V bytes of one decode step (gamma draft steps + the target layers' verify)."""
    g = wl.gamma
    draft = sum(kv_bytes(min(n0 + j, wl.sink + wl.window) if windowed else n0 + j, wl) for j in range(1, g + 1))
    return draft + wl.target_layers * kv_bytes(n0 + g + 1, wl)


def sweep(flag, steps, warmup, dev, contexts, gammas):
    """Decode steps across context length and draft depth, both draft modes, beside the
    bytes model's native/windowed ratio (which widens as the context grows)."""
    rows = []
    # Largest contexts first: they are bandwidth-bound and the most sensitive to the
    # device's state after minutes of sustained load; the small, launch-bound ones
    # come last.  Rows are reported in context order.
    for n0 in sorted(contexts, reverse=True):
        for g in gammas:
            wl = synth.workload("step_1m_bf16", contexts=(n0,), gamma=g)
            log(f"sweep n0={n0} gamma={g}")
            step = Step(wl, n0, wl.target_layers, 0, 0, 0, dev)
            rw = time_steps(step, W.SINK_WINDOW, flag, steps, warmup)
            rn = time_steps(step, W.FULL, flag, steps, warmup)
            win_ms, nat_ms = med(rw["step"]), med(rn["step"])
            ver_ms, dwin_ms, dnat_ms = med(flat(rw["verify"])), med(flat(rw["draft"])), med(flat(rn["draft"]))
            # the same steps replayed from a HIP graph: no host launch cost (small contexts are host-bound eagerly)
            gw, okw = graph_step(step, W.SINK_WINDOW, flag, 5)
            gn, okn = graph_step(step, W.FULL, flag, 5)
            bw, bn = step_bytes(n0, wl, True), step_bytes(n0, wl, False)
            rows.append({"context": n0, "gamma": g, "windowed_us": round(win_ms * 1e3, 1),
                         "native_us": round(nat_ms * 1e3, 1), "ratio": round(nat_ms / win_ms, 4),
                         "bytes_model_ratio": round(bn / bw, 4),
                         "windowed_gbps": round(bw / (win_ms * 1e-3) / 1e9, 1),
                         "native_gbps": round(bn / (nat_ms * 1e-3) / 1e9, 1),
                         "draft_window_us": round(dwin_ms * 1e3, 2), "draft_native_us": round(dnat_ms * 1e3, 2),
                         "verify_us": round(ver_ms * 1e3, 2),
                         "graph_windowed_us": pct(gw)["median"], "graph_native_us": pct(gn)["median"],
                         "graph_ratio": round(float(np.median(gn)) / float(np.median(gw)), 4),
                         "graph_replays_match_eager": bool(okw and okn)})
            del step
            torch.cuda.empty_cache()
    return sorted(rows, key=lambda r: (r["context"], r["gamma"]))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # ~35 ms of sustained load at 1M: after an idle spell the first launches run fast, then
    # slow for a few ms, and settle after ~20 ms of load; the warmup absorbs that
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--context", type=int, default=1 << 20)
    ap.add_argument("--gamma", type=int, default=3, help="draft steps per decode step (verify takes gamma + 1 queries)")
    ap.add_argument("--chunk-full", type=int, default=0, help="draft split size, native mode (0 = library default)")
    ap.add_argument("--chunk-window", type=int, default=0, help="draft split size, window mode (0 = default)")
    ap.add_argument("--split", type=int, default=0, help="verify split size (0 = library default)")
    ap.add_argument("--exact-pv", action="store_true", help="draft PV with fp32 weights instead of bf16 pairs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-details", action="store_true",
                    help="skip the extra measurements (graph replay, cold window, split and batch variants)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step at --context: steps over contexts 2K..1M and gamma 3/5/8")
    ap.add_argument("--pool-layout", choices=("kv_runs", "separate"), default="kv_runs",
                    help="paged pools: K and V of a (block, head) side by side (default), or separate K and V")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a plain 256 MiB device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    W.load()
    dev = "cuda"
    if args.calibrate:
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flag = 0 if args.exact_pv else W.DRAFT_FAST_PV
    if args.sweep:
        rows = sweep(flag, args.steps, args.warmup, dev, (2048, 8192, 32768, 131072, 524288, 1 << 20), (3, 5, 8))
        print(json.dumps({"metric": "decode-step attention us across context and gamma", "unit": "us/decode-step",
                          "data": "synthetic", "dtype": "bf16", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "rows": rows}), flush=True)
        return
    wl = synth.workload("step_1m_bf16", contexts=(args.context,), gamma=args.gamma)
    n0 = args.context
    log("streaming-read ceiling")
    ceiling = stream_ceiling_gbps(dev)
    log(f"setup: {wl.target_layers} target layers + 1 draft layer at {n0} tokens")
    step = Step(wl, n0, wl.target_layers, args.chunk_full, args.chunk_window,
                args.split, dev, kv_runs=args.pool_layout == "kv_runs")

    log("paged streaming-read ceiling")
    paged_ceiling = paged_ceiling_gbps(step)
    paged_ceiling_32k = paged_ceiling_gbps(step, 32) if args.pool_layout == "kv_runs" else None
    log("timing windowed step")
    rw = time_steps(step, W.SINK_WINDOW, flag, args.steps, args.warmup)
    log("timing native step")
    rn = time_steps(step, W.FULL, flag, args.steps, args.warmup)
    win_ms, nat_ms = med(rw["step"]), med(rn["step"])
    ver_ms = med(flat(rw["verify"]))                  # verify launches of the windowed (headline) step
    ver_ms_nat = med(flat(rn["verify"]))
    dwin_ms, dnat_ms = med(flat(rw["draft"])), med(flat(rn["draft"]))
    L = wl.target_layers
    details = {
        "step_us": {"windowed": pct(rw["step"], True), "native": pct(rn["step"], True)},
        "launch_us": {arm: {kind: pct(flat(r[kind]), True) for kind in ("draft", "draft_combine", "verify",
                                                                          "verify_combine")}
                      for arm, r in (("windowed", rw), ("native", rn))},
        "verify_us_by_layer": [round(med([r[l] for r in rw["verify"]]) * 1e3, 1) for l in range(L)],
        "self_check": {
            # the step contains its verify launches: L x their median cannot exceed the step's median
            "verify_layers_within_step": bool(L * ver_ms <= win_ms and L * ver_ms_nat <= nat_ms),
            # the launches' medians add up to the step's median within 2% (nothing else is timed)
            "launch_sum_over_step": {arm: round(sum(med(flat(r[k])) * len(r[k][0]) for k in r if k.islower()
                                                    and not k.startswith("step")) / med(r["step_with_launch_events"]),
                                                4) for arm, r in (("windowed", rw), ("native", rn))},
            # device time the per-launch events add to a step (the step times above have none)
            "launch_events_cost_us": {arm: round((med(r["step_with_launch_events"]) - med(r["step"])) * 1e3, 1)
                                      for arm, r in (("windowed", rw), ("native", rn))},
        },
        "timing": ("median over the timed steps, events at step boundaries only; per-launch times from a second "
                   "pass with an event after every launch on the launch stream; prepared C-ABI calls with the "
                   "garbage collector off"),
    }
    if not details["self_check"]["verify_layers_within_step"]:
        log("WARNING: verify launches exceed their step")
    if not args.no_details:
        reps = 20
        log("unfused steps (append calls before the attention calls)")
        uw = time_steps(step, W.SINK_WINDOW, flag, args.steps, args.warmup, fused=False, per_launch=False)
        un = time_steps(step, W.FULL, flag, args.steps, args.warmup, fused=False, per_launch=False)
        details["unfused_step_us"] = {"windowed": pct(uw["step"]), "native": pct(un["step"])}
        log("graph-captured steps")
        gw, okw = graph_step(step, W.SINK_WINDOW, flag, 20)
        gn, okn = graph_step(step, W.FULL, flag, 20)
        details["graph_step_us"] = {"windowed": pct(gw), "native": pct(gn), "replays_match_eager": bool(okw and okn),
                                    "ratio": round(med(gn) / med(gw), 4)}
        log("window draft: warm, cold, across contexts")
        details["window_draft_step_us"] = window_measurements(
            step, flag, reps, dev, (32768, 131072, 524288, n0))
        total_mem = torch.cuda.get_device_properties(0).total_memory
        details["memory_plan"] = dict(W.plan_memory(step.sh, wl.target_layers, n0 + wl.gamma + 1, wl.sink, wl.window,
                                                    step.R, total_mem),
                                      budget="the GPU's whole memory", budget_bytes=int(total_mem))
        log("native draft launch: literal 256-key splits vs default")
        details["native_draft_launch_us"] = native_split_measurements(step, flag, 10, dev)
        log("native draft step: fp32 vs bf16 PV weights")
        details["native_draft_step_1m_pv"] = native_draft_pv_measurements(step, reps)
        del step
        torch.cuda.empty_cache()
        log("131K draft layer: native vs windowed, 3 steps")
        details["draft_131k_3_steps"] = draft_131k_measurements(flag, reps, dev)
        log("mixed batch (4 sequences)")
        details["mixed_batch"] = mixed_batch(flag, reps, dev)
        log("1M draft step, 4 q heads / 1 KV head / d=64")
        details["draft_1m_4q_1kv_d64"] = other_head_reading(flag, reps, dev)

    g = wl.gamma
    bytes_win, bytes_nat = step_bytes(n0, wl, True), step_bytes(n0, wl, False)
    ver_bytes = verify_launch_bytes(n0 + g + 1, wl, g + 1)
    achieved = ver_bytes / (ver_ms * 1e-3) / 1e9
    ver_all = np.asarray(flat(rw["verify"]), dtype=np.float64)
    res = {
        "metric": METRIC,
        "value": round(win_ms * 1e3, 1),
        "unit": "us/decode-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(win_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"per-decode-step attention at {n0} tokens: {wl.target_layers} target layers x verify "
                         f"({g + 1} causal queries) + 1 draft layer x {g} steps, 16 q heads / 2 KV heads, "
                         f"d=256, bf16 KV, paged 16-token blocks (random permutation); draft in sink_window "
                         f"mode S={wl.sink} W={wl.window}"),
            "context": n0, "gamma": g, "target_layers": wl.target_layers,
            "draft_pv": "fp32 weights" if args.exact_pv else "bf16 weight pairs",
            "pool_layout": ("[blocks][H_kv][K|V][16][D]" if args.pool_layout == "kv_runs"
                            else "[blocks][H_kv][16][D] per K and V"),
            "statistic": "median of the timed steps",
        },
        "windowed_us_per_step": round(win_ms * 1e3, 1),
        "native_us_per_step": round(nat_ms * 1e3, 1),
        "ratio_native_over_windowed": round(nat_ms / win_ms, 4),
        "windowed_gbps": round(bytes_win / (win_ms * 1e-3) / 1e9, 1),
        "native_gbps": round(bytes_nat / (nat_ms * 1e-3) / 1e9, 1),
        "windowed_pct_peak": round(100 * bytes_win / (win_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "native_pct_peak": round(100 * bytes_nat / (nat_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "kernels_us": {
            "verify_per_layer": round(ver_ms * 1e3, 2),
            "verify_per_layer_native_arm": round(ver_ms_nat * 1e3, 2),
            "draft_window_per_step": round(dwin_ms * 1e3, 2),
            "draft_native_per_step": round(dnat_ms * 1e3, 2),
            "verify_combine": round(med(flat(rw["verify_combine"])) * 1e3, 2),
            "draft_combine_window": round(med(flat(rw["draft_combine"])) * 1e3, 2),
        },
        "roofline": {
            "kernel": (f"{verify_kernel_name(g + 1, wl.group)} (verify, {wl.target_layers} launches per step)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            # counters were taken on the default workload (1M keys, gamma 3, K|V-run pools)
            "traffic": (verify_traffic_bytes() if (n0, g, args.pool_layout) == (1 << 20, 3, "kv_runs") else None),
            "algorithmic_bytes": ver_bytes,
            "launch_us_median": round(ver_ms * 1e3, 2),
            "launch_us_mean": round(float(ver_all.mean()) * 1e3, 2),
            "launches": int(ver_all.size),
            "measured_read_ceiling": round(ceiling, 1),
            "frac_of_measured_ceiling": round(achieved / ceiling, 4),
            "measured_paged_read_ceiling": round(paged_ceiling, 1),
            "frac_of_paged_ceiling": round(achieved / paged_ceiling, 4),
            # the same probe over runs of both heads of a block (32 KiB), what one work item per
            # block covering both heads would read
            "measured_paged_read_ceiling_32k_runs": (round(paged_ceiling_32k, 1) if paged_ceiling_32k else None),
        },
    }
    native_draft_bytes = draft_launch_bytes(n0 + 1, wl, True)
    res["draft_native_gbps"] = round(native_draft_bytes / (dnat_ms * 1e-3) / 1e9, 1)
    res["draft_native_pct_peak"] = round(100 * native_draft_bytes / (dnat_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
    res["details"] = details
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        res["cpu_baseline"] = cpu_baseline(wl, n0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
