"""The no-allocation draft call (wmtp_draft_attn_noalloc) against the workspace calls it stands for.

Callers that cannot allocate get one draft step into final outputs with the split partials in
the library's fixed scratch.  Two calls in a row, the second with a smaller input, in both
draft modes, with and without the append inside the launch, with both PV variants: each output
must equal, bit for bit, wmtp_draft_attn (or wmtp_draft_attn_append) into a torch workspace
followed by wmtp_combine (the same kernels and plan), and match the float64 oracle within the
bf16 tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
from long_context_decode_gqa_amd import wmtp as W
from tests.gpu_cases import DEV, TOL, PagedCache, RingCache, max_err, run_combine

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fast_pv", [True, False])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_noalloc_draft_matches_workspace_calls(mode, fused, fast_pv):
    wl = synth.workload("draft_131k_bf16", window=512)
    Hq, Hk, D, S, Wn = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    for call, contexts in enumerate(((700, 5000, 63), (300,))):          # the second call is smaller
        say("noalloc", mode, fused, fast_pv, "call", call, contexts)
        case = synth.draft_case(wl, contexts, seed=40 + call)
        B = len(contexts)
        lens = [n + 1 for n in contexts]
        q = case.q[0].contiguous().to(DEV)
        kn, vn = case.k_new[0].contiguous().to(DEV), case.v_new[0].contiguous().to(DEV)
        if mode == O.FULL:
            cache = PagedCache(case.k_ctx, case.v_ctx, contexts, extra=1, seed=40 + call, interleaved=True)
            kw = dict(paged=cache.desc)
        else:
            ring = RingCache(B, Hk, D, S, Wn, torch.bfloat16, headroom=2)
            for b in range(B):
                sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), S, Wn, 2)
                W.ring_append(sh, sub, case.k_ctx[b:b + 1, :contexts[b]].contiguous().to(DEV),
                              case.v_ctx[b:b + 1, :contexts[b]].contiguous().to(DEV), [0])
            kw = dict(ring=ring.desc)
        if not fused:                      # the step's own entry, appended by its own call first
            if mode == O.FULL:
                W.paged_append(sh, cache.desc, kn, vn, contexts)
            else:
                W.ring_append(sh, ring.desc, kn, vn, contexts)
        # the existing entry points with a workspace
        ws = W.workspace(W.draft_workspace_bytes(mode, sh, lens, 0, S, Wn, 2), DEV)
        if fused:
            parts = W.draft_attn_append(mode | flag, sh, q, kn, vn, lens, ws, **kw)
        else:
            parts = W.draft_attn(mode | flag, sh, q, lens, ws, **kw)
        want_o, want_l = run_combine(parts, Hq, D, B)
        # the no-allocation call (the fused append rewrites the same token at the same position)
        got_o = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        got_l = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        W.draft_attn_noalloc(mode | flag, sh, q, lens, got_o, got_l, k_new=kn if fused else None,
                             v_new=vn if fused else None, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got_o, want_o) and torch.equal(got_l, want_l), (call, "differs from the workspace calls")
        kb, vb = synth.bf16_bits(case.k_ctx), synth.bf16_bits(case.v_ctx)
        nkb, nvb = synth.bf16_bits(case.k_new[0]), synth.bf16_bits(case.v_new[0])
        qf = O.to_f64(synth.bf16_bits(case.q[0]), "bf16")
        for b in range(B):
            sk = O.ConcatKV(O.LogicalKV(kb[b], "bf16", contexts[b]), O.LogicalKV(nkb[b], "bf16"))
            sv = O.ConcatKV(O.LogicalKV(vb[b], "bf16", contexts[b]), O.LogicalKV(nvb[b], "bf16"))
            o_ref, l_ref = O.draft_attention(qf[b], sk, sv, lens[b], mode, S, Wn, wl.scale)
            eo, el = max_err(got_o[b], o_ref), max_err(got_l[b], l_ref)
            assert eo <= TOL["bf16"] and el <= TOL["bf16"], (call, b, eo, el)


@pytest.mark.parametrize("fast_pv", [True, False])
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_noalloc_draft_steps_in_a_graph(mode, fast_pv):
    """Callers under graph capture: three no-allocation draft steps (the append inside) captured
    in a HIP graph.  Every replay, with eager work and synchronisations between replays, gives the
    eager calls' outputs bit for bit; the eager calls match the oracle."""
    wl = synth.workload("draft_131k_bf16", window=512)
    Hq, Hk, D, S, Wn, g = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window, wl.gamma
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    n0 = 3000
    say("noalloc graph", mode, fast_pv)
    case = synth.draft_case(wl, (n0,), seed=47)
    if mode == O.FULL:
        cache = PagedCache(case.k_ctx, case.v_ctx, (n0,), extra=g, seed=47, interleaved=True)
        kw = dict(paged=cache.desc)
    else:
        ring = RingCache(1, Hk, D, S, Wn, torch.bfloat16, headroom=g - 1)
        W.ring_append(sh, ring.desc, case.k_ctx[:, :n0].contiguous().to(DEV), case.v_ctx[:, :n0].contiguous().to(DEV),
                      [0])
        kw = dict(ring=ring.desc)
    q = case.q.contiguous().to(DEV)
    kn, vn = case.k_new.contiguous().to(DEV), case.v_new.contiguous().to(DEV)
    out = torch.zeros((g, 1, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.zeros((g, 1, Hq), dtype=torch.float32, device=DEV)

    def steps():
        for j in range(g):
            W.draft_attn_noalloc(mode | flag, sh, q[j], [n0 + j + 1], out[j], lse[j], k_new=kn[j], v_new=vn[j], **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps()                      # eager (the appends rewrite the same tokens at the same positions)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    qf = O.to_f64(synth.bf16_bits(case.q[:, 0]), "bf16")
    kb, vb = synth.bf16_bits(case.k_ctx[0]), synth.bf16_bits(case.v_ctx[0])
    for j in range(g):
        nkb = synth.bf16_bits(case.k_new[:j + 1, 0, 0])
        nvb = synth.bf16_bits(case.v_new[:j + 1, 0, 0])
        sk = O.ConcatKV(O.LogicalKV(kb, "bf16", n0), O.LogicalKV(nkb, "bf16"))
        sv = O.ConcatKV(O.LogicalKV(vb, "bf16", n0), O.LogicalKV(nvb, "bf16"))
        o_ref, l_ref = O.draft_attention(qf[j], sk, sv, n0 + j + 1, mode, S, Wn, wl.scale)
        eo, el = max_err(ref_o[j, 0], o_ref), max_err(ref_l[j, 0], l_ref)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (j, eo, el)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), rep
    del graph
