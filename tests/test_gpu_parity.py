"""GPU parity: the HIP library (through the C ABI) against the float64 oracle.

Index resolution, ring and paged appends are compared bit for bit; attention
outputs within max-abs 1e-5 (fp32 workloads) or 2e-3 (bf16 KV, fp32
accumulation).  Inputs come from `synth` with the workloads' shapes at context
lengths the oracle finishes in seconds, spanning several tiles and splits with
ragged tails; the 1M-token cases compare sampled KV heads.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
from long_context_decode_gqa_amd import wmtp as W
from tests.gpu_cases import (DEV, TOL, PagedCache, RingCache, host_array, max_err, needles, plant_logical,
                              plant_paged, run_combine, top_block_positions)

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ============================================================== index resolution
def test_resolve_paged_bit_exact_past_2_pow_31():
    rng = np.random.default_rng(1)
    nb_pool = 1 << 22                                   # block ids up to 4M: offsets beyond 2^31 elements
    bt = rng.integers(0, nb_pool, size=(2, 4096)).astype(np.int32)
    bt_dev = torch.from_numpy(bt).to(DEV)
    desc = W.Paged(0, 0, bt_dev.data_ptr(), 16, bt.shape[1], nb_pool)
    pos = rng.integers(0, 4096 * 16, size=5000).astype(np.int32)
    pos_dev = torch.from_numpy(pos).to(DEV)
    for b in range(2):
        for h in range(2):
            got = W.debug_resolve_paged(desc, 2, 256, b, h, pos_dev).cpu().numpy()
            want = np.array([O.paged_element_offset(bt[b], int(t), h, 2, 16, 256) for t in pos], dtype=np.int64)
            assert np.array_equal(got, want)
    assert want.max() > 2 ** 31
    # K|V runs of 32 rows (K and V of a block and head side by side)
    desc32 = W.Paged(0, 0, bt_dev.data_ptr(), 16, bt.shape[1], nb_pool, 32)
    for b in range(2):
        for h in range(2):
            got = W.debug_resolve_paged(desc32, 2, 256, b, h, pos_dev).cpu().numpy()
            want = np.array([O.paged_element_offset(bt[b], int(t), h, 2, 16, 256, 32) for t in pos], dtype=np.int64)
            assert np.array_equal(got, want)


@pytest.mark.parametrize("S,Wn", [(4, 4096), (0, 7), (1, 1), (4, 256), (16, 1000)])
def test_resolve_ring_and_window_sets_bit_exact(S, Wn):
    rng = np.random.default_rng(S * 31 + Wn)
    pos = np.concatenate([np.arange(0, 300), rng.integers(0, 1 << 24, size=3000)]).astype(np.int32)
    got = W.debug_resolve_ring(S, Wn, torch.from_numpy(pos).to(DEV)).cpu().numpy()
    want = np.array([O.ring_slot(int(p), S, Wn) for p in pos])
    assert np.array_equal(got, want)
    for n in [0, 1, S, S + 1, S + Wn - 1, S + Wn, S + Wn + 1, 3 * Wn + 5, 1048579]:
        g = W.debug_window_positions(S, Wn, n, DEV).cpu().numpy()
        assert np.array_equal(g, O.window_slot_positions(n, S, Wn)), n


# ============================================================== appends
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ring_append_sequence_bit_exact(dtype):
    S, Wn, Hk, D, B = 4, 40, 2, 64, 2
    sh = W.make_shape(4, Hk, D, TDT[dtype])
    ring = RingCache(B, Hk, D, S, Wn, TDT[dtype])
    total = 300
    k_all = synth.normal((B, total, Hk, D), 7, "rk", 1.0, dtype)
    v_all = synth.normal((B, total, Hk, D), 7, "rv", 1.0, dtype)
    tags = [np.full(S + Wn, -1, dtype=np.int64) for _ in range(B)]
    at = 0
    for t_new in [3, 1, 70, 1, 1, 45, 100, 1, 2, 50]:          # bulk appends longer than W, single steps
        if at + t_new > total:
            break
        W.ring_append(sh, ring.desc, k_all[:, at:at + t_new].contiguous().to(DEV),
                      v_all[:, at:at + t_new].contiguous().to(DEV), [at] * B)
        for b in range(B):
            O.ring_append(tags[b], at, t_new, S, Wn)
        at += t_new
        torch.cuda.synchronize()
        got_tags = ring.tags.cpu().numpy()
        kr, vr = ring.k.cpu(), ring.v.cpu()
        for b in range(B):
            assert np.array_equal(got_tags[b], tags[b])
            for s_, p in enumerate(tags[b]):
                if p >= 0:
                    assert torch.equal(kr[b, :, s_], k_all[b, p]) and torch.equal(vr[b, :, s_], v_all[b, p])


@pytest.mark.parametrize("interleaved", [False, True])
def test_paged_append_bit_exact(interleaved):
    Hk, D, B = 2, 256, 3
    sh = W.make_shape(16, Hk, D, torch.bfloat16)
    n0 = [5, 16, 33]
    T = 20
    k_ctx = synth.normal((B, 40, Hk, D), 8, "pk", 0.5, "bf16")
    cache = PagedCache(k_ctx, k_ctx, n0, extra=T, seed=8, interleaved=interleaved)
    k_new = synth.normal((B, T, Hk, D), 8, "pkn", 0.5, "bf16")
    v_new = synth.normal((B, T, Hk, D), 8, "pvn", 0.5, "bf16")
    # flat memory of k and v, and the element offset of v's rows relative to k's
    if interleaved:
        flat = lambda: (cache.pool.cpu().reshape(-1),) * 2
        v_shift = 16 * D
    else:
        flat = lambda: (cache.k.cpu().reshape(-1), cache.v.cpu().reshape(-1))
        v_shift = 0
    before_k, before_v = (x.clone() for x in flat())
    W.paged_append(sh, cache.desc, k_new.to(DEV), v_new.to(DEV), n0)
    torch.cuda.synchronize()
    kf, vf = flat()
    touched_k = np.zeros(kf.numel(), dtype=bool)
    touched_v = np.zeros(vf.numel(), dtype=bool)
    for b in range(B):
        for i in range(T):
            for h in range(Hk):
                off = cache.element_offset(b, n0[b] + i, h)
                assert torch.equal(kf[off:off + D], k_new[b, i, h])
                assert torch.equal(vf[off + v_shift:off + v_shift + D], v_new[b, i, h])
                touched_k[off:off + D] = True
                touched_v[off + v_shift:off + v_shift + D] = True
    if interleaved:                      # one pool: every row not appended is unchanged
        untouched = torch.from_numpy(~(touched_k | touched_v))
        assert torch.equal(kf[untouched], before_k[untouched])
    else:
        for f, before, touched in ((kf, before_k, touched_k), (vf, before_v, touched_v)):
            untouched = torch.from_numpy(~touched)
            assert torch.equal(f[untouched], before[untouched])


# ============================================================== headroom and rollback
@pytest.mark.parametrize("S,Wn,R", [(4, 4096, 2), (0, 7, 3), (1, 1, 5), (16, 1000, 7)])
def test_resolve_ring_with_headroom_bit_exact(S, Wn, R):
    rng = np.random.default_rng(S * 7 + Wn + R)
    pos = np.concatenate([np.arange(0, 300), rng.integers(0, 1 << 24, size=3000)]).astype(np.int32)
    got = W.debug_resolve_ring(S, Wn, torch.from_numpy(pos).to(DEV), headroom=R).cpu().numpy()
    assert np.array_equal(got, np.array([O.ring_slot(int(p), S, Wn, R) for p in pos]))
    for n in [0, 1, S, S + Wn, S + Wn + R, S + Wn + R + 1, 3 * Wn + 5, 1048579]:
        g = W.debug_window_positions(S, Wn, n, DEV, headroom=R).cpu().numpy()
        assert np.array_equal(g, O.window_slot_positions(n, S, Wn, R)), n


def test_ring_append_with_headroom_bit_exact():
    S, Wn, R, Hk, D, B = 4, 40, 3, 2, 64, 2
    sh = W.make_shape(4, Hk, D, torch.bfloat16)
    ring = RingCache(B, Hk, D, S, Wn, torch.bfloat16, headroom=R)
    total = 300
    k_all = synth.normal((B, total, Hk, D), 9, "rk", 1.0, "bf16")
    v_all = synth.normal((B, total, Hk, D), 9, "rv", 1.0, "bf16")
    tags = [np.full(S + Wn + R, -1, dtype=np.int64) for _ in range(B)]
    at = 0
    for t_new in [3, 1, 70, 1, 1, 45, 100, 1, 2, 50]:
        if at + t_new > total:
            break
        W.ring_append(sh, ring.desc, k_all[:, at:at + t_new].contiguous().to(DEV),
                      v_all[:, at:at + t_new].contiguous().to(DEV), [at] * B)
        for b in range(B):
            O.ring_append(tags[b], at, t_new, S, Wn, R)
        at += t_new
        torch.cuda.synchronize()
        got = ring.tags.cpu().numpy()
        kr, vr = ring.k.cpu(), ring.v.cpu()
        for b in range(B):
            assert np.array_equal(got[b], tags[b])
            for s_, p in enumerate(tags[b]):
                if p >= 0:
                    assert torch.equal(kr[b, :, s_], k_all[b, p]) and torch.equal(vr[b, :, s_], v_all[b, p])


@pytest.mark.parametrize("fast_pv", [False, True])
def test_speculative_rollback_draft_parity(fast_pv):
    """Draft cycles with partial acceptance on a ring with R = gamma - 1 headroom slots.

    Prefill: one bulk append of n0 tokens.  Cycle c drafts gamma tokens (fresh K/V
    per cycle) at positions n..n+gamma-1, each followed by a window draft query;
    verification accepts the first a of them, wmtp_ring_rollback forgets the rest,
    and the next cycle starts at n + a.  Every query is compared with the oracle
    over the accepted sequence plus the current cycle's drafts; the ring's tags
    with the oracle's ring model after every call, bit for bit.
    """
    S, Wn, gamma, Hq, Hk, D, B = 4, 64, 3, 8, 2, 128, 2
    R = gamma - 1
    scale = D ** -0.5
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, scale)
    n0 = [150, 97]
    accepts = [[1, 3, 2, 1, 3, 1], [3, 1, 1, 2, 3, 2]]
    ring = RingCache(B, Hk, D, S, Wn, torch.bfloat16, headroom=R)
    cap = max(n0) + gamma * len(accepts[0]) + 1
    k_pre = synth.normal((B, cap, Hk, D), 21, "pre_k", 0.5, "bf16")
    v_pre = synth.normal((B, cap, Hk, D), 21, "pre_v", 0.5, "bf16")
    truth_k = [synth.bf16_bits(k_pre[b]).copy() for b in range(B)]   # [cap][Hk][D] accepted content
    truth_v = [synth.bf16_bits(v_pre[b]).copy() for b in range(B)]
    tags = [np.full(S + Wn + R, -1, dtype=np.int64) for _ in range(B)]
    for b in range(B):                                     # bulk init from the prefill
        sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), S, Wn, R)
        W.ring_append(sh, sub, k_pre[b:b + 1, :n0[b]].contiguous().to(DEV),
                      v_pre[b:b + 1, :n0[b]].contiguous().to(DEV), [0])
        O.ring_append(tags[b], 0, n0[b], S, Wn, R)
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    n = list(n0)
    worst = 0.0
    for c in range(len(accepts[0])):
        kd = synth.normal((gamma, B, 1, Hk, D), 22, ("draft_k", c), 0.5, "bf16")
        vd = synth.normal((gamma, B, 1, Hk, D), 22, ("draft_v", c), 0.5, "bf16")
        q = synth.normal((gamma, B, Hq, D), 22, ("draft_q", c), 1.0, "bf16")
        cur_k = [truth_k[b].copy() for b in range(B)]      # accepted prefix + this cycle's drafts
        cur_v = [truth_v[b].copy() for b in range(B)]
        for j in range(gamma):
            pos = [n[b] + j for b in range(B)]
            lens = [p + 1 for p in pos]
            W.ring_append(sh, ring.desc, kd[j].contiguous().to(DEV), vd[j].contiguous().to(DEV), pos)
            for b in range(B):
                O.ring_append(tags[b], pos[b], 1, S, Wn, R)
                cur_k[b][pos[b]] = synth.bf16_bits(kd[j, b, 0])
                cur_v[b][pos[b]] = synth.bf16_bits(vd[j, b, 0])
            ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW | flag, sh, lens, 0, S, Wn, R), DEV)
            parts = W.draft_attn(W.SINK_WINDOW | flag, sh, q[j].contiguous().to(DEV), lens, ws, ring=ring.desc)
            out, lse = run_combine(parts, Hq, D, B)
            torch.cuda.synchronize()
            assert np.array_equal(ring.tags.cpu().numpy(), np.stack(tags))
            qf = O.to_f64(synth.bf16_bits(q[j]), "bf16")
            for b in range(B):
                o_ref, l_ref = O.draft_attention(qf[b], O.LogicalKV(cur_k[b], "bf16", lens[b]),
                                                 O.LogicalKV(cur_v[b], "bf16", lens[b]), lens[b], O.SINK_WINDOW,
                                                 S, Wn, scale)
                worst = max(worst, max_err(out[b], o_ref), max_err(lse[b], l_ref))
        for b in range(B):                                 # verification: accept the first a drafts
            a = accepts[b][c]
            truth_k[b][n[b]:n[b] + a] = cur_k[b][n[b]:n[b] + a]
            truth_v[b][n[b]:n[b] + a] = cur_v[b][n[b]:n[b] + a]
            n[b] += a
            O.ring_rollback(tags[b], n[b])
        W.ring_rollback(ring.desc, n)
        torch.cuda.synchronize()
        assert np.array_equal(ring.tags.cpu().numpy(), np.stack(tags))
    say("speculative rollback worst", worst)
    assert worst <= TOL["bf16"], worst


@pytest.mark.parametrize("fast_pv", [False, True])
def test_per_sequence_sinks_and_windows_parity(fast_pv):
    """Adaptive windows / dynamic sinks: one batched window-mode call where every sequence has
    its own S_b <= S and W_b <= W + R, changing from step to step, on one ring layout."""
    S, Wn, R, Hq, Hk, D, B = 8, 96, 2, 16, 2, 256, 4
    scale = D ** -0.5
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, scale)
    n0 = [40, 200, 1000, 7]
    steps = 4
    policies = [([8, 0, 4, 2], [98, 1, 50, 96]), ([1, 8, 8, 0], [10, 98, 97, 5]),
                ([0, 3, 8, 8], [96, 64, 2, 98]), ([8, 8, 0, 5], [1, 33, 98, 40])]
    ring = RingCache(B, Hk, D, S, Wn, torch.bfloat16, headroom=R)
    cap = max(n0) + steps
    kc = synth.normal((B, cap, Hk, D), 31, "pol_k", 0.5, "bf16")
    vc = synth.normal((B, cap, Hk, D), 31, "pol_v", 0.5, "bf16")
    for b in range(B):
        sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), S, Wn, R)
        W.ring_append(sh, sub, kc[b:b + 1, :n0[b]].contiguous().to(DEV), vc[b:b + 1, :n0[b]].contiguous().to(DEV), [0])
    kb = [synth.bf16_bits(kc[b]) for b in range(B)]
    vb = [synth.bf16_bits(vc[b]) for b in range(B)]
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    worst = 0.0
    for j in range(steps):
        pos = [n + j for n in n0]
        lens = [p + 1 for p in pos]
        W.ring_append(sh, ring.desc, torch.stack([kc[b, pos[b]] for b in range(B)])[:, None].contiguous().to(DEV),
                      torch.stack([vc[b, pos[b]] for b in range(B)])[:, None].contiguous().to(DEV), pos)
        sinks, wins = policies[j]
        pol = W.with_policy(ring.desc, sinks, wins)
        q = synth.normal((B, Hq, D), 31, ("pol_q", j), 1.0, "bf16")
        ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW | flag, sh, lens, 64, S, Wn, R), DEV)
        parts = W.draft_attn(W.SINK_WINDOW | flag, sh, q.to(DEV), lens, ws, ring=pol, chunk_tokens=64)
        out, lse = run_combine(parts, Hq, D, B)
        torch.cuda.synchronize()
        qf = O.to_f64(synth.bf16_bits(q), "bf16")
        for b in range(B):
            o_ref, l_ref = O.draft_attention(qf[b], O.LogicalKV(kb[b], "bf16", lens[b]),
                                             O.LogicalKV(vb[b], "bf16", lens[b]), lens[b], O.SINK_WINDOW,
                                             sinks[b], wins[b], scale)
            worst = max(worst, max_err(out[b], o_ref), max_err(lse[b], l_ref))
    say("per-sequence policy worst", worst)
    assert worst <= TOL["bf16"], worst


@pytest.mark.parametrize("poison", [False, True])
@pytest.mark.parametrize("fast_pv", [False, True])
def test_window_holes_are_masked(fast_pv, poison):
    """A visible entry whose slot tag does not hold its position is left out.

    The ring is rolled back below the query's length, so the newest visible
    positions are holes (tag -1); the result must equal attention over the rest
    of the window set.  Sequence 0 has wrapped (n > S + W); sequence 1 is
    shorter than S + W, so sinks and window overlap.  Both kernels that serve
    window mode are covered (bf16 PV weights at d = 256: the matrix-core one).
    poison: the holes' K and V are then overwritten with NaN (a slot that does not
    hold its position may hold any bits; 0 x NaN would be NaN).
    """
    S, Wn, R, Hq, Hk, D, B = 4, 64, 2, 16, 2, 256, 2
    G = Hq // Hk
    scale = D ** -0.5
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, scale)
    n0, kept = [200, 61], [198, 60]
    ring = RingCache(B, Hk, D, S, Wn, torch.bfloat16, headroom=R)
    kc = synth.normal((B, max(n0), Hk, D), 41, "hole_k", 0.5, "bf16")
    vc = synth.normal((B, max(n0), Hk, D), 41, "hole_v", 0.5, "bf16")
    for b in range(B):
        sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), S, Wn, R)
        W.ring_append(sh, sub, kc[b:b + 1, :n0[b]].contiguous().to(DEV), vc[b:b + 1, :n0[b]].contiguous().to(DEV), [0])
    W.ring_rollback(ring.desc, kept)
    if poison:
        holes = (ring.tags < 0).unsqueeze(1).unsqueeze(-1).expand_as(ring.k)
        assert bool(holes.any())
        ring.k.masked_fill_(holes, float("nan"))
        ring.v.masked_fill_(holes, float("nan"))
    q = synth.normal((B, Hq, D), 41, "hole_q", 1.0, "bf16")
    qf = O.to_f64(synth.bf16_bits(q), "bf16")
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    worst = 0.0
    for chunk in (64, 0):
        say("window holes", fast_pv, chunk)
        ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW | flag, sh, n0, chunk, S, Wn, R), DEV)
        parts = W.draft_attn(W.SINK_WINDOW | flag, sh, q.to(DEV), n0, ws, ring=ring.desc, chunk_tokens=chunk)
        out, lse = run_combine(parts, Hq, D, B)
        torch.cuda.synchronize()
        for b in range(B):
            pos = O.visible_positions(n0[b], O.SINK_WINDOW, S, Wn)
            pos = pos[pos < kept[b]]
            kk = O.LogicalKV(synth.bf16_bits(kc[b]), "bf16", n0[b])
            vv = O.LogicalKV(synth.bf16_bits(vc[b]), "bf16", n0[b])
            for h in range(Hk):
                o_ref, l_ref = O.attention_over(qf[b, h * G:(h + 1) * G], kk, vv, pos, h, scale)
                worst = max(worst, max_err(out[b, h * G:(h + 1) * G], o_ref), max_err(lse[b, h * G:(h + 1) * G], l_ref))
    say("window holes worst", worst)
    assert worst <= TOL["bf16"], worst


# ============================================================== draft attention
def draft_steps(wl, contexts, mode, chunk=0, fast_pv=False, steps=None, out_dtype=torch.float32, fused=False,
                headroom=0, record=None, interleaved=False, fill=0.0):
    """Run gamma draft steps on the GPU and the oracle; return the worst max-abs errors (o, lse).

    fused: append and attend in one call (wmtp_draft_attn_append) instead of an
    append call followed by wmtp_draft_attn.  record: a list that receives each
    step's (out, lse) and, last, the cache tensors the steps leave."""
    case = synth.draft_case(wl, contexts)
    B, Hq, Hk, D = len(case.n0), wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    dt = wl.dtype
    sh = W.make_shape(Hq, Hk, D, TDT[dt], wl.scale)
    steps = wl.gamma if steps is None else steps
    ctx_k = host_array(case.k_ctx, dt)
    ctx_v = host_array(case.v_ctx, dt)
    new_k = host_array(case.k_new, dt)      # [gamma][B][1][Hk][D]
    new_v = host_array(case.v_new, dt)
    if mode == O.FULL:
        cache = PagedCache(case.k_ctx, case.v_ctx, case.n0, extra=steps, seed=wl.seed, permuted=wl.permuted,
                           interleaved=interleaved, fill=fill)
    else:
        ring = RingCache(B, Hk, D, wl.sink, wl.window, TDT[dt], headroom, fill=fill)
        for b in range(B):                   # bulk-fill each sequence's ring with its context
            if case.n0[b] == 0:
                continue
            sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), wl.sink, wl.window,
                         headroom)
            W.ring_append(sh, sub, case.k_ctx[b:b + 1, :case.n0[b]].contiguous().to(DEV),
                          case.v_ctx[b:b + 1, :case.n0[b]].contiguous().to(DEV), [0])
    flag = W.DRAFT_FAST_PV if fast_pv else 0
    worst_o = worst_l = 0.0
    for j in range(steps):
        kn = case.k_new[j].contiguous().to(DEV)
        vn = case.v_new[j].contiguous().to(DEV)
        pos = [n + j for n in case.n0]
        lens = [n + j + 1 for n in case.n0]
        qj = case.q[j].contiguous().to(DEV)
        if mode == O.FULL:
            nbytes = W.draft_workspace_bytes(mode | flag, sh, lens, chunk)
            ws = W.workspace(nbytes, DEV)
            if fused:
                parts = W.draft_attn_append(mode | flag, sh, qj, kn, vn, lens, ws, paged=cache.desc,
                                            chunk_tokens=chunk)
            else:
                W.paged_append(sh, cache.desc, kn, vn, pos)
                parts = W.draft_attn(mode | flag, sh, qj, lens, ws, paged=cache.desc, chunk_tokens=chunk)
        else:
            nbytes = W.draft_workspace_bytes(mode | flag, sh, lens, chunk, wl.sink, wl.window, headroom)
            ws = W.workspace(nbytes, DEV)
            if fused:
                parts = W.draft_attn_append(mode | flag, sh, qj, kn, vn, lens, ws, ring=ring.desc,
                                            chunk_tokens=chunk)
            else:
                W.ring_append(sh, ring.desc, kn, vn, pos)
                parts = W.draft_attn(mode | flag, sh, qj, lens, ws, ring=ring.desc, chunk_tokens=chunk)
        out, lse = run_combine(parts, Hq, D, B, out_dtype)
        if record is not None:
            record.append((out, lse))
        torch.cuda.synchronize()
        qf = O.to_f64(host_array(case.q[j], dt), dt)
        for b in range(B):
            src_k = O.ConcatKV(O.LogicalKV(ctx_k[b], dt, case.n0[b]), O.LogicalKV(new_k[:j + 1, b, 0], dt))
            src_v = O.ConcatKV(O.LogicalKV(ctx_v[b], dt, case.n0[b]), O.LogicalKV(new_v[:j + 1, b, 0], dt))
            o_ref, l_ref = O.draft_attention(qf[b], src_k, src_v, lens[b], mode, wl.sink, wl.window, wl.scale)
            worst_o = max(worst_o, max_err(out[b], o_ref))
            worst_l = max(worst_l, max_err(lse[b], l_ref))
    if record is not None:
        record.append((cache.k, cache.v) if mode == O.FULL else (ring.k, ring.v, ring.tags))
    return worst_o, worst_l


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_tiny_fp32_4k_three_steps(mode):
    wl = synth.workload("tiny_fp32_4k")
    say("draft tiny fp32 4k", mode)
    eo, el = draft_steps(wl, None, mode)
    assert eo <= TOL["f32"] and el <= TOL["f32"], (eo, el)
    eo, el = draft_steps(wl, None, mode, chunk=32)                 # splits of half a 64-key tile
    assert eo <= TOL["f32"] and el <= TOL["f32"], (eo, el)


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
@pytest.mark.parametrize("fast_pv", [False, True])
@pytest.mark.parametrize("n0,chunk", [(1, 64), (63, 64), (64, 0), (700, 128), (5000, 256), (9001, 1024),
                                      (90, 32), (1500, 96)])
def test_draft_bf16_16q_2kv_d256(mode, fast_pv, n0, chunk):
    wl = synth.workload("draft_131k_bf16", window=1024)
    say("draft bf16", mode, fast_pv, n0, chunk)
    eo, el = draft_steps(wl, (n0,), mode, chunk=chunk, fast_pv=fast_pv)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_mixed_batch_paged_permuted(mode):
    wl = synth.workload("mixed_4seq_bf16", window=1024)
    say("draft mixed batch", mode)
    eo, el = draft_steps(wl, (300, 2000, 0, 7777), mode, chunk=256, fast_pv=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


def test_partials_keep_their_workspace_alive():
    """The partials a call returns point into its workspace and keep it alive: a workspace made
    inline in the call stays valid until the combine, and is freed with the partials."""
    import gc
    import weakref
    wl = synth.workload("draft_131k_bf16", window=256)
    case = synth.draft_case(wl, (700,))
    sh = W.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, torch.bfloat16, wl.scale)
    cache = PagedCache(case.k_ctx, case.v_ctx, case.n0, extra=1, seed=wl.seed)
    q = case.q[0].contiguous().to(DEV)
    lens = [case.n0[0]]
    parts = W.draft_attn(W.FULL, sh, q, lens, W.workspace(W.draft_workspace_bytes(W.FULL, sh, lens, 64), DEV),
                         paged=cache.desc, chunk_tokens=64)
    ref = weakref.ref(parts._workspace)
    gc.collect()
    torch.empty(1 << 22, dtype=torch.uint8, device=DEV).fill_(255)      # would reuse a freed workspace
    out, lse = run_combine(parts, wl.num_q_heads, wl.head_dim, 1)
    torch.cuda.synchronize()
    qf = O.to_f64(host_array(case.q[0], wl.dtype), wl.dtype)
    k, v = host_array(case.k_ctx, wl.dtype), host_array(case.v_ctx, wl.dtype)
    o_ref, l_ref = O.draft_attention(qf[0], O.LogicalKV(k[0], wl.dtype, lens[0]), O.LogicalKV(v[0], wl.dtype, lens[0]),
                                     lens[0], O.FULL, wl.sink, wl.window, wl.scale)
    assert max_err(out[0], o_ref) <= TOL["bf16"] and max_err(lse[0], l_ref) <= TOL["bf16"]
    del parts
    gc.collect()
    assert ref() is None


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
@pytest.mark.parametrize("hq,hk,d", [(2, 2, 256), (4, 2, 256), (8, 2, 256), (4, 1, 256),
                                     (4, 2, 128), (8, 1, 128), (2, 2, 128), (4, 1, 64), (8, 8, 64), (16, 2, 64)])
def test_draft_matrix_core_groupings(mode, hq, hk, d):
    """bf16 PV weights run the draft step on the matrix-core kernel in both modes (paged pool or
    ring): every query-head grouping G = 1, 2, 4, 8 at head_dim 256, 128 and 64 (four, two or one
    wave per work item), with fused appends, several splits and a wrapped ring."""
    wl = synth.workload("draft_131k_bf16", num_q_heads=hq, num_kv_heads=hk, head_dim=d, window=300)
    say("draft matrix-core groupings", mode, hq, hk, d)
    eo, el = draft_steps(wl, (1500, 77), mode, chunk=128, fast_pv=True, fused=True, headroom=2)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_draft_fp32_weight_groupings(g, d):
    """fp32 PV weights in full mode run the whole-tile vector kernel: every grouping G = 1, 2, 4, 8
    at head_dim 64, 128 and 256 (16- or 32-key tiles; the lanes of a key hold whole scores of
    G / parts rows after the part sums), with fused appends, ragged lengths, an empty sequence
    and splits of 96 keys (a partial last tile)."""
    wl = synth.workload("draft_131k_bf16", num_q_heads=2 * g, num_kv_heads=2, head_dim=d, window=300)
    say("draft fp32-weight groupings", g, d)
    eo, el = draft_steps(wl, (1500, 0, 77), O.FULL, chunk=96, fast_pv=False, fused=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("hq,hk,d", [(8, 8, 64), (4, 2, 128), (4, 1, 64), (16, 4, 256)])
def test_draft_other_head_shapes(hq, hk, d):
    wl = synth.workload("draft_131k_bf16", num_q_heads=hq, num_kv_heads=hk, head_dim=d, window=300)
    say("draft shapes", hq, hk, d)
    for mode in (O.FULL, O.SINK_WINDOW):
        eo, el = draft_steps(wl, (1500,), mode, chunk=192, steps=1)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (mode, eo, el)


def test_draft_bf16_output_rounding():
    wl = synth.workload("draft_131k_bf16", window=512)
    say("draft bf16 out")
    eo, _ = draft_steps(wl, (3000,), O.FULL, chunk=256, steps=1, out_dtype=torch.bfloat16)
    assert eo <= TOL["bf16"] + 2 ** -8, eo


def test_window_covering_context_equals_full_on_gpu():
    wl = synth.workload("draft_131k_bf16", window=4096)
    say("window covering")
    for mode in (O.FULL, O.SINK_WINDOW):
        eo, el = draft_steps(wl, (2000,), mode, chunk=256, steps=1)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"]


# ============================================================== unused cache rows may hold any bits
# Keys past a sequence's end share their block with its last keys, and ring slots that no
# append has written (or whose tag is stale) sit beside visible ones.  They get weight 0, but
# 0 x NaN is NaN: every kernel must keep their values out of the PV product.  Pools and rings
# filled with NaN before the context is placed must give the oracle's result.
NAN = float("nan")


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
@pytest.mark.parametrize("fast_pv", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_draft_unused_rows_hold_nan(mode, fast_pv, d):
    wl = synth.workload("draft_131k_bf16", num_q_heads=8, num_kv_heads=2, head_dim=d, window=300)
    say("draft NaN-filled cache", mode, fast_pv, d)
    eo, el = draft_steps(wl, (1500, 77, 5), mode, chunk=96, fast_pv=fast_pv, fused=True, headroom=3, fill=NAN)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_fp32_unused_rows_hold_nan(mode):
    wl = synth.workload("tiny_fp32_4k")
    say("draft fp32 NaN-filled cache", mode)
    eo, el = draft_steps(wl, (300, 7), mode, chunk=64, fused=True, headroom=2, fill=NAN)
    assert eo <= TOL["f32"] and el <= TOL["f32"], (eo, el)


@pytest.mark.parametrize("t_q,hq,hk,d", [(4, 16, 2, 256), (6, 16, 2, 256), (9, 16, 2, 256), (4, 8, 2, 128),
                                         (12, 8, 2, 128), (4, 4, 1, 64), (24, 4, 1, 64)])
def test_verify_unused_rows_hold_nan(t_q, hq, hk, d):
    wl = synth.workload("step_1m_bf16", num_q_heads=hq, num_kv_heads=hk, head_dim=d)
    say("verify NaN-filled pool", t_q, hq, hk, d)
    for contexts, split in (((1500, 3), 96), ((29,), 32), ((700,), 0)):
        eo, el = verify_run(wl, contexts, t_q, split, fused=True, fill=NAN)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (contexts, split, eo, el)


# ============================================================== verify attention
def verify_run(wl, contexts, t_q, split=0, layer=0, fused=False, record=None, interleaved=False, fill=0.0):
    """Verify on the GPU (append + verify, or the fused call) against the oracle: worst (o, lse) errors.
    record: a list that receives (out, lse, k pool, v pool)."""
    case = synth.verify_case(wl, contexts, t_q, layer=layer)
    B, Hq, Hk, D = len(case.n0), wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    dt = wl.dtype
    sh = W.make_shape(Hq, Hk, D, TDT[dt], wl.scale)
    cache = PagedCache(case.k_ctx, case.v_ctx, case.n0, extra=t_q, seed=wl.seed + 100 + layer,
                       interleaved=interleaved, fill=fill)
    kn, vn = case.k_new.contiguous().to(DEV), case.v_new.contiguous().to(DEV)
    lens = [n + t_q for n in case.n0]
    ws = W.workspace(W.verify_workspace_bytes(sh, t_q, lens, split), DEV)
    if fused:
        parts = W.verify_attn_append(sh, case.q.to(DEV), t_q, cache.desc, kn, vn, lens, ws, split)
    else:
        W.paged_append(sh, cache.desc, kn, vn, list(case.n0))
        parts = W.verify_attn(sh, case.q.to(DEV), t_q, cache.desc, lens, ws, split)
    out, lse = run_combine(parts, t_q * Hq, D, B)
    if record is not None:
        record.append((out, lse, cache.k, cache.v))
    torch.cuda.synchronize()
    qf = O.to_f64(host_array(case.q, dt), dt)
    ck, cv = host_array(case.k_ctx, dt), host_array(case.v_ctx, dt)
    nk, nv = host_array(case.k_new, dt), host_array(case.v_new, dt)
    eo = el = 0.0
    for b in range(B):
        sk = O.ConcatKV(O.LogicalKV(ck[b], dt, case.n0[b]), O.LogicalKV(nk[b], dt))
        sv = O.ConcatKV(O.LogicalKV(cv[b], dt, case.n0[b]), O.LogicalKV(nv[b], dt))
        o_ref, l_ref = O.verify_attention(qf[b], sk, sv, lens[b], wl.scale)
        eo = max(eo, max_err(out[b], o_ref.reshape(t_q * Hq, D)))
        el = max(el, max_err(lse[b], l_ref.reshape(t_q * Hq)))
    return eo, el


@pytest.mark.parametrize("n0,split", [(0, 32), (1, 0), (28, 32), (500, 64), (4000, 512), (9000, 2048)])
def test_verify_bf16_gamma3(n0, split):
    wl = synth.workload("step_1m_bf16")
    say("verify", n0, split)
    eo, el = verify_run(wl, (n0,), 4, split)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("t_q,hq,hk", [(1, 16, 2), (2, 16, 2), (3, 16, 2), (4, 8, 1), (8, 8, 2), (32, 2, 2),
                                       (5, 16, 2), (6, 16, 2), (8, 16, 2), (9, 16, 2), (12, 16, 2), (48, 4, 2),
                                       (33, 1, 1), (17, 4, 2), (12, 8, 2), (24, 8, 2), (70, 1, 1)])
def test_verify_row_packings(t_q, hq, hk):
    wl = synth.workload("step_1m_bf16", num_q_heads=hq, num_kv_heads=hk)
    say("verify rows", t_q, hq, hk)
    eo, el = verify_run(wl, (1234,), t_q, 128)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("t_q,hq,hk,contexts,split,fused,interleaved", [
    (4, 16, 2, (1234,), 64, False, False),          # G = 8: one full row tile
    (1, 8, 2, (0, 777), 0, True, False),            # G = 4, a sequence with no context
    (3, 4, 4, (300, 5000), 32, False, True),        # G = 1, K|V runs
    (8, 8, 2, (2044, 17), 256, True, True),         # G = 4, 32 rows, tokens across a split boundary
    (2, 16, 2, (200000,), 0, False, False),         # a long context, default splits
    (6, 16, 2, (29, 300), 32, True, False),         # G = 8, 48 rows: two row tiles (two wave teams)
    (9, 16, 2, (2044, 17), 256, True, True),        # 72 rows: three row tiles, straddling a split
    (12, 8, 1, (5000,), 0, False, False),           # 96 rows, the maximum
    (33, 1, 1, (100, 40), 32, True, False),         # G = 1, 33 rows: a second row tile of one row
    (40, 4, 2, (3000, 41), 64, False, True),        # G = 2, 80 rows, a ragged third row tile
])
def test_verify_small_head_dims(d, t_q, hq, hk, contexts, split, fused, interleaved):
    """Verify at head_dim 64 and 128: one or two waves per work item up to 32 packed
    rows; two wave teams (one loader wave per slice of D, one compute wave per row
    tile) for 33..96 rows."""
    wl = synth.workload("step_1m_bf16", num_q_heads=hq, num_kv_heads=hk, head_dim=d)
    say("verify small d", d, t_q, hq, hk, contexts, split, fused, interleaved)
    eo, el = verify_run(wl, contexts, t_q, split, fused=fused, interleaved=interleaved)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


def test_verify_mixed_batch():
    wl = synth.workload("mixed_4seq_bf16")
    say("verify mixed")
    eo, el = verify_run(wl, (100, 3000, 17, 6000), 4, 256)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


# ============================================================== fused append + attention
# One launch that appends the step's new tokens and attends must leave the
# same cache and produce the same partials, bit for bit, as the append call
# followed by the attention call; and it must match the oracle.  The cases put
# the new tokens across a split boundary, at position 0, in a sink slot, in a
# ring that has wrapped (with headroom), and on every kernel that serves them.
@pytest.mark.parametrize("contexts,t_q,split,hq,hk", [
    ((62, 99), 4, 64, 16, 2),       # 62..65 straddle the split at 64
    ((0, 1234), 4, 32, 16, 2),      # first tokens of an empty sequence
    ((29, 300), 6, 32, 16, 2),      # two row tiles (two wave teams), straddling 32
    ((2044, 17), 9, 256, 16, 2),    # three row tiles, straddling 2048
    ((1000, 4000), 4, 0, 16, 2),    # library default split
    ((33, 500), 4, 32, 8, 1),       # G = 8 on one KV head
    ((100, 40), 33, 32, 1, 1),      # 33 new tokens over two splits of 32 (G = 1, two row tiles)
    ((64, 5), 4, 32, 16, 2),        # a split made only of new tokens (64..67)
])
def test_verify_fused_append_equals_separate_calls(contexts, t_q, split, hq, hk):
    wl = synth.workload("step_1m_bf16", num_q_heads=hq, num_kv_heads=hk)
    say("verify fused append", contexts, t_q, split, hq, hk)
    fused, sep = [], []
    eo, el = verify_run(wl, contexts, t_q, split, fused=True, record=fused)
    verify_run(wl, contexts, t_q, split, fused=False, record=sep)
    for a, b in zip(fused[0], sep[0]):
        assert torch.equal(a, b)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
@pytest.mark.parametrize("fast_pv", [False, True])
@pytest.mark.parametrize("contexts,chunk,window,headroom", [
    ((63, 0, 2000), 64, 1024, 0),       # step tokens at 63..65 cross the split at 64; an empty sequence
    ((1, 5000), 128, 1024, 2),          # a sink slot; a wrapped ring with headroom
    ((700, 4096), 0, 256, 3),           # library default split
])
def test_draft_fused_append_equals_separate_calls(mode, fast_pv, contexts, chunk, window, headroom):
    wl = synth.workload("draft_131k_bf16", window=window)
    say("draft fused append", mode, fast_pv, contexts, chunk, window, headroom)
    fused, sep = [], []
    eo, el = draft_steps(wl, contexts, mode, chunk=chunk, fast_pv=fast_pv, fused=True, headroom=headroom,
                         record=fused)
    draft_steps(wl, contexts, mode, chunk=chunk, fast_pv=fast_pv, fused=False, headroom=headroom, record=sep)
    assert len(fused) == len(sep) == wl.gamma + 1
    for got, want in zip(fused, sep):
        for a, b in zip(got, want):
            assert torch.equal(a, b)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_fused_append_fp32_and_other_shapes(mode):
    cases = [(synth.workload("tiny_fp32_4k"), None, TOL["f32"]),
             (synth.workload("draft_131k_bf16", num_q_heads=4, num_kv_heads=2, head_dim=128, window=300), (1500,),
              TOL["bf16"]),
             (synth.workload("draft_131k_bf16", num_q_heads=8, num_kv_heads=8, head_dim=64, window=300), (777,),
              TOL["bf16"])]
    for wl, contexts, tol in cases:
        say("draft fused append shapes", mode, wl.num_q_heads, wl.num_kv_heads, wl.head_dim)
        fused, sep = [], []
        eo, el = draft_steps(wl, contexts, mode, chunk=192 if contexts else 0, fused=True, record=fused)
        draft_steps(wl, contexts, mode, chunk=192 if contexts else 0, fused=False, record=sep)
        for got, want in zip(fused, sep):
            for a, b in zip(got, want):
                assert torch.equal(a, b)
        assert eo <= tol and el <= tol, (eo, el)


# ============================================================== K|V runs: one pool, K and V of a (block, head) side by side
# The same tokens in a [blocks][H_kv][2][16][D] pool must give the oracle's
# result and, bit for bit, the result over separate K and V pools.
@pytest.mark.parametrize("contexts,t_q,split,fused", [((500, 7), 4, 64, False), ((62, 4000), 4, 0, True),
                                                      ((29, 300), 6, 32, True), ((2044, 17), 9, 256, False)])
def test_verify_kv_runs_pool(contexts, t_q, split, fused):
    wl = synth.workload("step_1m_bf16")
    say("verify K|V runs", contexts, t_q, split, fused)
    runs, sep = [], []
    eo, el = verify_run(wl, contexts, t_q, split, fused=fused, record=runs, interleaved=True)
    verify_run(wl, contexts, t_q, split, fused=fused, record=sep, interleaved=False)
    for a, b in zip(runs[0], sep[0]):            # out, lse, and the K and V token rows (views)
        assert torch.equal(a, b)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)


@pytest.mark.parametrize("fast_pv", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_draft_kv_runs_pool(fast_pv, fused):
    wl = synth.workload("draft_131k_bf16", window=1024)
    say("draft K|V runs", fast_pv, fused)
    runs, sep = [], []
    eo, el = draft_steps(wl, (63, 0, 2000), O.FULL, chunk=64, fast_pv=fast_pv, fused=fused, record=runs,
                         interleaved=True)
    draft_steps(wl, (63, 0, 2000), O.FULL, chunk=64, fast_pv=fast_pv, fused=fused, record=sep)
    for got, want in zip(runs, sep):
        for a, b in zip(got, want):
            assert torch.equal(a, b)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)
    wl = synth.workload("tiny_fp32_4k")
    eo, el = draft_steps(wl, None, O.FULL, fused=fused, interleaved=True)
    assert eo <= TOL["f32"] and el <= TOL["f32"], (eo, el)


# ============================================================== 1M-token cases
# The inputs carry needles (see synth): every checked row's softmax rests on 32 known positions
# spread over the context (or over the window), with fresh values there, so the outputs are of
# order one and a wrong value read fails the 2e-3 bar (tests/test_oracle_needles.py shows that on
# the CPU).  Needles sit also in the block at the pool's highest addresses: in a K|V pool of
# 65,537 blocks its K and V bytes start at 2^31.
def _paged_1m(seed, hk=2, d=256, extra=8, interleaved=False):
    """A 1,048,576-token paged layer (random block permutation): separate K and V pools, or one
    K|V pool as the benchmark lays them out.  Returns n0, the block table (host and device), the k
    and v token views, the descriptor and views(): after any needles are planted, src(part, n),
    the oracle's view of K (0) or V (1) positions < n of the pool."""
    n0 = 1 << 20
    blocks = synth.blocks_for(n0 + extra, 16)
    bt, total = synth.block_table(seed, [blocks], permuted=True)
    btd = torch.from_numpy(bt).to(DEV)
    if interleaved:
        pool = synth.normal((total, hk, 2, 16, d), seed, "pool_kv", 0.5, "bf16", DEV)
        k, v = pool[:, :, 0], pool[:, :, 1]
        desc = W.make_paged_interleaved(pool, btd)

        def views():
            bits = synth.bf16_bits(pool)
            return lambda part, n: O.PagedKV(bits, bt[0], 16, "bf16", n, part=part)
    else:
        k = synth.normal((total, hk, 16, d), seed, "pool_k", 0.5, "bf16", DEV)
        v = synth.normal((total, hk, 16, d), seed, "pool_v", 0.5, "bf16", DEV)
        desc = W.make_paged(k, v, btd)

        def views():
            kb, vb = synth.bf16_bits(k), synth.bf16_bits(v)
            return lambda part, n: O.PagedKV(kb if part == 0 else vb, bt[0], 16, "bf16", n)
    return n0, bt, k, v, btd, desc, views


def _check_rows(out, lse, q_rows, sk, sv, positions, h, scale, what):
    """Rows q_rows (float64 [8][D]) of KV head h against the oracle over `positions`; returns the errors."""
    o_ref, l_ref = O.attention_over(q_rows, sk, sv, positions, h, scale)
    eo, el = max_err(out, o_ref), max_err(lse, l_ref)
    say(what, "max|o|", float(np.abs(o_ref).max()), "errors", eo, el)
    assert np.abs(o_ref).max() > 0.1, (what, "needles did not take the softmax")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (what, eo, el)


@pytest.mark.slow
def test_draft_full_1m_paged_exact_pv():
    """Native draft step over a 1,048,576-token paged pool (random block permutation, separate K and
    V pools), fp32 PV weights and 256-token splits (the whole-tile vector kernel); every query head of
    both KV heads checked, on needle inputs that include the pool's last block."""
    say("draft 1M exact PV")
    n0, bt, k, v, btd, desc, views = _paged_1m(2)
    sh = W.make_shape(16, 2, 256, torch.bfloat16, 1 / 16)
    kn = synth.normal((1, 1, 2, 256), 2, "kn1m", 0.5, "bf16", DEV)
    vn = synth.normal((1, 1, 2, 256), 2, "vn1m", 0.5, "bf16", DEV)
    q = synth.normal((1, 16, 256), 2, "q1m", 1.0, "bf16", DEV)
    top = top_block_positions(bt[0], n0, k.shape[0] - 1)
    plant_paged(k, v, bt[0], needles(q[0], np.arange(16) // 8, 0, n0, 2, ("d1m",), 1 / 16, include=top))
    src = views()
    W.paged_append(sh, desc, kn, vn, [n0])
    n = n0 + 1
    ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, [n], 256), DEV)
    parts = W.draft_attn(W.FULL, sh, q, [n], ws, paged=desc, chunk_tokens=256)
    out, lse = run_combine(parts, 16, 256, 1)
    torch.cuda.synchronize()
    # oracle: context from the pool as planted (never the appended pool), plus the new token
    sk = O.ConcatKV(src(0, n0), O.LogicalKV(synth.bf16_bits(kn[0]), "bf16"))
    sv = O.ConcatKV(src(1, n0), O.LogicalKV(synth.bf16_bits(vn[0]), "bf16"))
    qf = O.to_f64(synth.bf16_bits(q[0]), "bf16")
    for h in range(2):
        rows = slice(h * 8, h * 8 + 8)
        _check_rows(out[0, rows], lse[0, rows], qf[rows], sk, sv, np.arange(n), h, 1 / 16, ("draft 1M", h))


@pytest.mark.slow
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_1m_other_head_reading(mode):
    """The 1M paged draft workload under the other reading of its head shapes (4 query heads on
    1 KV head, d = 64, bf16), in the launch configuration the benchmark times: bf16 PV weights,
    default splits, the step's token appended inside the launch.  Native over a K|V-run pool with
    a random block permutation, window over a ring with headroom; needles over the context (native)
    or over the sinks and the window; all heads checked against the oracle."""
    n0, Hq, Hk, D, S, Wn, R = 1 << 20, 4, 1, 64, 4, 4096, 2
    scale = D ** -0.5
    say("draft 1M 4q/1kv/64", mode)
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, scale)
    kc = synth.normal((1, n0, Hk, D), 7, "ctx_k_4q", 0.5, "bf16", DEV)
    vc = synth.normal((1, n0, Hk, D), 7, "ctx_v_4q", 0.5, "bf16", DEV)
    kn = synth.normal((1, 1, Hk, D), 7, "kn_4q", 0.5, "bf16", DEV)
    vn = synth.normal((1, 1, Hk, D), 7, "vn_4q", 0.5, "bf16", DEV)
    q = synth.normal((1, Hq, D), 7, "q_4q", 1.0, "bf16", DEV)
    n = n0 + 1
    if mode == O.FULL:
        nd = needles(q[0], [0] * Hq, 0, n0, 7, ("4q", mode), scale, include=[1, n0 - 1])
    else:
        nd = needles(q[0], [0] * Hq, n - Wn, n0, 7, ("4q", mode), scale, include=[n - Wn, n0 - 1])
        sinks = needles(q[0], [0] * Hq, 0, S, 7, ("4q_sink",), scale, per_row=1)
        plant_logical(kc, vc, 0, sinks)
    plant_logical(kc, vc, 0, nd)
    flag = W.DRAFT_FAST_PV
    if mode == O.FULL:
        bt, total = synth.block_table(7, [synth.blocks_for(n, 16)], permuted=True)
        pool = torch.zeros((total, Hk, 2, 16, D), dtype=torch.bfloat16, device=DEV)
        btd = torch.from_numpy(bt).to(DEV)
        desc = W.make_paged_interleaved(pool, btd)
        W.paged_append(sh, desc, kc, vc, [0])
        ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, [n], 0), DEV)
        parts = W.draft_attn_append(W.FULL | flag, sh, q, kn, vn, [n], ws, paged=desc)
    else:
        ring = RingCache(1, Hk, D, S, Wn, torch.bfloat16, headroom=R)
        W.ring_append(sh, ring.desc, kc, vc, [0])
        ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, [n], 0, S, Wn, R), DEV)
        parts = W.draft_attn_append(W.SINK_WINDOW | flag, sh, q, kn, vn, [n], ws, ring=ring.desc)
    out, lse = run_combine(parts, Hq, D, 1)
    torch.cuda.synchronize()
    sk = O.ConcatKV(O.LogicalKV(synth.bf16_bits(kc[0]), "bf16"), O.LogicalKV(synth.bf16_bits(kn[0]), "bf16"))
    sv = O.ConcatKV(O.LogicalKV(synth.bf16_bits(vc[0]), "bf16"), O.LogicalKV(synth.bf16_bits(vn[0]), "bf16"))
    qf = O.to_f64(synth.bf16_bits(q[0]), "bf16")
    _check_rows(out[0], lse[0], qf, sk, sv, O.visible_positions(n, mode, S, Wn), 0, scale, ("4q/1kv/64", mode))


@pytest.mark.slow
def test_verify_1m_paged_all_rows():
    """One target layer's verify at 1M context in the benchmark's launch configuration (K|V pool,
    default splits, the 4 new tokens appended inside the launch): 4 causal queries over 1,048,580
    keys, every query token and both KV heads checked, on needle inputs aimed at all 64 packed rows
    (including the block whose bytes start at 2^31)."""
    say("verify 1M")
    n0, bt, k, v, btd, desc, views = _paged_1m(3, interleaved=True)
    sh = W.make_shape(16, 2, 256, torch.bfloat16, 1 / 16)
    kn = synth.normal((1, 4, 2, 256), 3, "kn1m", 0.5, "bf16", DEV)
    vn = synth.normal((1, 4, 2, 256), 3, "vn1m", 0.5, "bf16", DEV)
    q = synth.normal((1, 4, 16, 256), 3, "q1m", 1.0, "bf16", DEV)
    top = top_block_positions(bt[0], n0, k.shape[0] - 1)
    row_heads = (np.arange(64) % 16) // 8                      # row i * 16 + hq is on KV head hq // 8
    plant_paged(k, v, bt[0], needles(q[0].reshape(64, 256), row_heads, 0, n0, 3, ("v1m",), 1 / 16, include=top))
    src = views()
    n = n0 + 4
    ws = W.workspace(W.verify_workspace_bytes(sh, 4, [n], 0), DEV)
    parts = W.verify_attn_append(sh, q, 4, desc, kn, vn, [n], ws, 0)
    out, lse = run_combine(parts, 64, 256, 1)
    torch.cuda.synchronize()
    sk = O.ConcatKV(src(0, n0), O.LogicalKV(synth.bf16_bits(kn[0]), "bf16"))
    sv = O.ConcatKV(src(1, n0), O.LogicalKV(synth.bf16_bits(vn[0]), "bf16"))
    qf = O.to_f64(synth.bf16_bits(q[0]), "bf16")          # [4][16][256]
    for i in range(4):
        for h in range(2):
            rows = slice(i * 16 + h * 8, i * 16 + h * 8 + 8)
            _check_rows(out[0, rows], lse[0, rows], qf[i, h * 8:(h + 1) * 8], sk, sv, np.arange(n0 + i + 1), h,
                        1 / 16, ("verify 1M", i, h))


# ============================================================== full sizes, benchmark launch configuration
def _gather(pool, bt_row, positions):
    """Tokens [T][H_kv][D] of a paged pool at `positions` (device gather through the block table)."""
    return pool[bt_row[positions // 16].long(), :, positions % 16, :]


def _fill_ring(sh, ring, k, v, bt_row, n0, S, Wn, R):
    """Ring of one sequence at length n0: sinks 0..S-1 and the last W + R context tokens, gathered from the pool."""
    pos_s = torch.arange(0, S, device=DEV)
    pos_t = torch.arange(n0 - (Wn + R), n0, device=DEV)
    W.ring_append(sh, ring, _gather(k, bt_row, pos_s)[None].contiguous(), _gather(v, bt_row, pos_s)[None].contiguous(), [0])
    W.ring_append(sh, ring, _gather(k, bt_row, pos_t)[None].contiguous(), _gather(v, bt_row, pos_t)[None].contiguous(),
                  [n0 - (Wn + R)])


def _window_needles(q_rows, heads, lo, hi, S, seed, stream, scale):
    """Needles of a sink + window draft: one in each sink for the first S rows of each KV head, and
    32 per row at context positions [lo, hi), which the caller picks inside every window checked."""
    heads = np.asarray(heads)
    first = np.concatenate([np.nonzero(heads == h)[0][:S] for h in np.unique(heads)])
    sinks = needles(q_rows[torch.from_numpy(first).to(q_rows.device)], heads[first], 0, S, seed,
                    stream + ("sink",), scale, per_row=1)
    win = needles(q_rows, heads, lo, hi, seed, stream, scale, include=[lo, hi - 1])
    return sinks, win


@pytest.mark.slow
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_1m_benchmark_launch_config(mode):
    """Draft step at 1,048,576 tokens (permuted K|V pool) in the benchmark's configuration: bf16 PV
    weights, default splits (the native step runs on the matrix-core kernel), ring with gamma - 1
    headroom; both KV heads checked, on needle inputs over the context and its last block (native)
    or over the sinks and the window."""
    S, Wn, R = 4, 4096, 2
    say("draft 1M bench config", mode)
    n0, bt, k, v, btd, desc, views = _paged_1m(6, interleaved=True)
    sh = W.make_shape(16, 2, 256, torch.bfloat16, 1 / 16)
    kn = synth.normal((1, 1, 2, 256), 6, "kn", 0.5, "bf16", DEV)
    vn = synth.normal((1, 1, 2, 256), 6, "vn", 0.5, "bf16", DEV)
    q = synth.normal((1, 16, 256), 6, "q", 1.0, "bf16", DEV)
    heads = np.arange(16) // 8
    n = n0 + 1
    if mode == O.FULL:
        top = top_block_positions(bt[0], n0, k.shape[0] - 1)
        plant_paged(k, v, bt[0], needles(q[0], heads, 0, n0, 6, ("b1m",), 1 / 16, include=top))
    else:
        for nd in _window_needles(q[0], heads, n - Wn, n0, S, 6, ("b1m_w",), 1 / 16):
            plant_paged(k, v, bt[0], nd)
    src = views()
    if mode == O.FULL:
        ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, [n], 0), DEV)
        parts = W.draft_attn_append(W.FULL | W.DRAFT_FAST_PV, sh, q, kn, vn, [n], ws, paged=desc)
    else:
        ring = RingCache(1, 2, 256, S, Wn, torch.bfloat16, headroom=R)
        _fill_ring(sh, ring.desc, k, v, btd[0], n0, S, Wn, R)
        ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, [n], 0, S, Wn, R), DEV)
        parts = W.draft_attn_append(W.SINK_WINDOW | W.DRAFT_FAST_PV, sh, q, kn, vn, [n], ws, ring=ring.desc)
    out, lse = run_combine(parts, 16, 256, 1)
    torch.cuda.synchronize()
    sk = O.ConcatKV(src(0, n0), O.LogicalKV(synth.bf16_bits(kn[0]), "bf16"))
    sv = O.ConcatKV(src(1, n0), O.LogicalKV(synth.bf16_bits(vn[0]), "bf16"))
    qf = O.to_f64(synth.bf16_bits(q[0]), "bf16")
    for h in range(2):
        rows = slice(h * 8, h * 8 + 8)
        _check_rows(out[0, rows], lse[0, rows], qf[rows], sk, sv, O.visible_positions(n, mode, S, Wn), h, 1 / 16,
                    ("draft 1M bench", mode, h))


@pytest.mark.slow
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_draft_131k_three_steps_full_size(mode):
    """Single draft layer at 131,072 tokens (identity block table), gamma = 3 draft steps,
    ring of S + W slots, benchmark launch configuration; both KV heads checked at every step, on
    needle inputs aimed at each step's query (over the context, or over the sinks and the window
    every step sees)."""
    wl = synth.workload("draft_131k_bf16")
    S, Wn = wl.sink, wl.window
    say("draft 131K full size", mode)
    n0 = wl.contexts[0]
    nb = synth.blocks_for(n0 + wl.gamma, 16)
    bt, total = synth.block_table(wl.seed, [nb], permuted=False)
    btd = torch.from_numpy(bt).to(DEV)
    pool = synth.normal((total, 2, 2, 16, 256), wl.seed, "c2kv", wl.kv_scale, "bf16", DEV)   # K|V runs
    k, v = pool[:, :, 0], pool[:, :, 1]
    kn = synth.normal((wl.gamma, 1, 1, 2, 256), wl.seed, "c2kn", wl.kv_scale, "bf16", DEV)
    vn = synth.normal((wl.gamma, 1, 1, 2, 256), wl.seed, "c2vn", wl.kv_scale, "bf16", DEV)
    q = synth.normal((wl.gamma, 1, 16, 256), wl.seed, "c2q", 1.0, "bf16", DEV)
    heads = np.arange(16) // 8
    for j in range(wl.gamma):
        if mode == O.FULL:
            plant_paged(k, v, bt[0], needles(q[j, 0], heads, 0, n0, wl.seed, ("c2", j), wl.scale,
                                             include=[5 + j, n0 - 1 - j]))
        else:   # visible at every step: the window at length n0 + 1 .. n0 + gamma covers [n0 + gamma - W, n0)
            for nd in _window_needles(q[j, 0], heads, n0 + wl.gamma - Wn, n0, S, wl.seed, ("c2w", j), wl.scale):
                plant_paged(k, v, bt[0], nd)
    bits = synth.bf16_bits(pool)                                    # the context as planted (before appends)
    sh = W.make_shape(16, 2, 256, torch.bfloat16, wl.scale)
    desc = W.make_paged_interleaved(pool, btd)
    if mode == O.SINK_WINDOW:
        ring = RingCache(1, 2, 256, S, Wn, torch.bfloat16)
        _fill_ring(sh, ring.desc, k, v, btd[0], n0, S, Wn, 0)
    for j in range(wl.gamma):
        n = n0 + j + 1
        if mode == O.FULL:
            ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, [n], 0), DEV)
            parts = W.draft_attn_append(W.FULL | W.DRAFT_FAST_PV, sh, q[j], kn[j], vn[j], [n], ws, paged=desc)
        else:
            ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, [n], 0, S, Wn), DEV)
            parts = W.draft_attn_append(W.SINK_WINDOW | W.DRAFT_FAST_PV, sh, q[j], kn[j], vn[j], [n], ws,
                                        ring=ring.desc)
        out, lse = run_combine(parts, 16, 256, 1)
        torch.cuda.synchronize()
        new_k = synth.bf16_bits(kn[:j + 1, 0, 0])                   # [j+1][H_kv][D]
        new_v = synth.bf16_bits(vn[:j + 1, 0, 0])
        sk = O.ConcatKV(O.PagedKV(bits, bt[0], 16, "bf16", n0, part=0), O.LogicalKV(new_k, "bf16"))
        sv = O.ConcatKV(O.PagedKV(bits, bt[0], 16, "bf16", n0, part=1), O.LogicalKV(new_v, "bf16"))
        qf = O.to_f64(synth.bf16_bits(q[j, 0]), "bf16")
        for h in range(2):
            rows = slice(h * 8, h * 8 + 8)
            _check_rows(out[0, rows], lse[0, rows], qf[rows], sk, sv, O.visible_positions(n, mode, S, Wn), h,
                        wl.scale, ("draft 131K", mode, j, h))


@pytest.mark.slow
def test_mixed_batch_full_sizes():
    """Mixed batch: 4 sequences of 32K / 131K / 512K / 1M tokens in one call, one block table
    permutation split over them (a K|V pool of 108,548 blocks, 3.6 GB: most blocks of the longer
    sequences lie past 2^31 bytes); window mode with W in {1,024, 4,096, 16,384}, then full mode
    (default splits, bf16 PV weights).  Every sequence and both KV heads checked in both modes, on
    needle inputs: per sequence, one set in the sinks and the last 1,024 positions (seen by every
    window) and one set spread over the whole context, so the full mode reads needles in blocks
    far apart."""
    wl = synth.workload("mixed_4seq_bf16")
    S, R = wl.sink, wl.gamma - 1
    say("mixed batch full sizes")
    lens0 = list(wl.contexts)
    B = len(lens0)
    bt, total = synth.block_table(wl.seed, [synth.blocks_for(n + 1, 16) for n in lens0], permuted=True)
    btd = torch.from_numpy(bt).to(DEV)
    pool = synth.normal((total, 2, 2, 16, 256), wl.seed, "c5kv", wl.kv_scale, "bf16", DEV)   # K|V runs
    k, v = pool[:, :, 0], pool[:, :, 1]
    kn = synth.normal((B, 1, 2, 256), wl.seed, "c5kn", wl.kv_scale, "bf16", DEV)
    vn = synth.normal((B, 1, 2, 256), wl.seed, "c5vn", wl.kv_scale, "bf16", DEV)
    q = synth.normal((B, 16, 256), wl.seed, "c5q", 1.0, "bf16", DEV)
    heads = np.arange(16) // 8
    w_min = min(wl.windows)
    for b in range(B):
        for nd in _window_needles(q[b], heads, lens0[b] + 1 - w_min, lens0[b], S, wl.seed, ("c5w", b), wl.scale):
            plant_paged(k, v, bt[b], nd)
        # spread over the context, clear of the window needles' range
        plant_paged(k, v, bt[b], needles(q[b], heads, S, lens0[b] - w_min, wl.seed, ("c5f", b), wl.scale,
                                         include=[S]))
    bits = synth.bf16_bits(pool)
    sh = W.make_shape(16, 2, 256, torch.bfloat16, wl.scale)
    desc = W.make_paged_interleaved(pool, btd)
    qf = O.to_f64(synth.bf16_bits(q), "bf16")
    lens = [n + 1 for n in lens0]

    def check(b, mode, Wn, out, lse):
        sk = O.ConcatKV(O.PagedKV(bits, bt[b], 16, "bf16", lens0[b], part=0),
                        O.LogicalKV(synth.bf16_bits(kn[b]), "bf16"))
        sv = O.ConcatKV(O.PagedKV(bits, bt[b], 16, "bf16", lens0[b], part=1),
                        O.LogicalKV(synth.bf16_bits(vn[b]), "bf16"))
        for h in range(2):
            rows = slice(h * 8, h * 8 + 8)
            _check_rows(out[b, rows], lse[b, rows], qf[b, rows], sk, sv, O.visible_positions(lens[b], mode, S, Wn),
                        h, wl.scale, ("mixed", mode, Wn, b, h))

    # window mode first (the pool is left as planted), one ring per W
    for Wn in wl.windows:
        ring = RingCache(B, 2, 256, S, Wn, torch.bfloat16, headroom=R)
        for b in range(B):
            sub = W.Ring(ring.k[b].data_ptr(), ring.v[b].data_ptr(), ring.tags[b].data_ptr(), S, Wn, R)
            _fill_ring(sh, sub, k, v, btd[b], lens0[b], S, Wn, R)
        W.ring_append(sh, ring.desc, kn, vn, lens0)
        ws = W.workspace(W.draft_workspace_bytes(W.SINK_WINDOW, sh, lens, 0, S, Wn, R), DEV)
        parts = W.draft_attn(W.SINK_WINDOW | W.DRAFT_FAST_PV, sh, q, lens, ws, ring=ring.desc)
        out, lse = run_combine(parts, 16, 256, B)
        torch.cuda.synchronize()
        for b in range(B):
            check(b, O.SINK_WINDOW, Wn, out, lse)
    # full mode over the paged pool
    W.paged_append(sh, desc, kn, vn, lens0)
    ws = W.workspace(W.draft_workspace_bytes(W.FULL, sh, lens, 0), DEV)
    parts = W.draft_attn(W.FULL | W.DRAFT_FAST_PV, sh, q, lens, ws, paged=desc)
    out, lse = run_combine(parts, 16, 256, B)
    torch.cuda.synchronize()
    for b in range(B):
        check(b, O.FULL, 1, out, lse)


# ============================================================== LSE combine alone
@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("counts", [(1, 5, 0, 100), (200,), (400, 3), (700,), (1500, 1)])
def test_combine_synthetic_partials(counts, D):
    """wmtp_combine on seeded partials whose split counts reach every workgroup shape the
    launch picks (4 waves x 4 splits per thread up to 128 splits, 4 x 8 up to 256, 8 x 8 up
    to 512, 16 x 8 beyond, two rounds of loads at 1,500), with a sequence of no splits and
    about 10% empty splits (lse = -inf, o = 0); lse spread over N(0, 5^2).  Checked against
    the oracle's float64 merge within the fp32 tolerance."""
    rows, B = 3, len(counts)
    say(f"combine counts={counts} D={D}")
    base = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    P = int(base[-1])
    o = synth.normal((P, rows, D), 7, ("comb_o", D, P), 1.0, "f32")
    lse = synth.normal((P, rows), 7, ("comb_lse", D, P), 5.0, "f32")
    empty = synth.normal((P, rows), 7, ("comb_empty", D, P), 1.0, "f32") > 1.2816   # ~10%
    lse[empty] = -math.inf
    o[empty] = 0.0
    parts = W.Partials()
    od, ld = o.to(DEV), lse.to(DEV)
    parts.o, parts.lse = od.data_ptr(), ld.data_ptr()
    parts.batch, parts.rows_per_seq, parts.head_dim, parts.total_splits = B, rows, D, P
    for b in range(B + 1):
        parts.split_base[b] = int(base[b])
    out, lse_out = run_combine(parts, rows, D, B)
    torch.cuda.synchronize()
    on, ln = o.double().numpy(), lse.double().numpy()
    for b in range(B):
        o_ref, l_ref = O.lse_combine(on[base[b]:base[b + 1]], ln[base[b]:base[b + 1]])
        got_o, got_l = out[b].double().cpu().numpy(), lse_out[b].double().cpu().numpy()
        if counts[b] == 0:
            assert np.all(got_o == 0.0) and np.all(np.isneginf(got_l))
            continue
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(got_l), fin), (b, got_l, l_ref)
        assert np.abs(got_o - o_ref).max() <= TOL["f32"], (b, np.abs(got_o - o_ref).max())
        assert np.abs(got_l[fin] - l_ref[fin]).max(initial=0.0) <= TOL["f32"] * max(1.0, np.abs(l_ref[fin]).max(initial=0.0))


# ============================================================== HIP graph capture
@pytest.mark.parametrize("mode", [O.FULL, O.SINK_WINDOW])
def test_decode_step_graph_replays_match_eager(mode):
    """A small decode step (3 fused draft steps + combines, 2 fused verify layers + combines)
    captured in a HIP graph: every replay, with eager work and synchronisations between replays,
    gives the eager step's outputs bit for bit (the kernels are deterministic), and the eager
    step matches the oracle."""
    wl = synth.workload("draft_131k_bf16", window=256)
    say("graph replay", mode)
    Hq, Hk, D, S, Wn, g = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window, wl.gamma
    sh = W.make_shape(Hq, Hk, D, torch.bfloat16, wl.scale)
    n0, layers = 3000, 2
    case = synth.draft_case(wl, (n0,))
    vcases = [synth.verify_case(wl, (n0 + g,), g + 1, layer=l) for l in range(layers)]
    draft_cache = PagedCache(case.k_ctx, case.v_ctx, case.n0, extra=g, seed=wl.seed, interleaved=True)
    ring = RingCache(1, Hk, D, S, Wn, torch.bfloat16, headroom=g - 1)
    W.ring_append(sh, ring.desc, case.k_ctx[:, :n0].contiguous().to(DEV), case.v_ctx[:, :n0].contiguous().to(DEV),
                  [0])
    # each target layer: the context (n0 + g tokens) already cached, then g + 1 new tokens
    vkeys = [torch.cat([case.k_ctx[:, :n0], case.k_new[:, :, 0].transpose(0, 1)], dim=1) for _ in range(layers)]
    vvals = [torch.cat([case.v_ctx[:, :n0], case.v_new[:, :, 0].transpose(0, 1)], dim=1) for _ in range(layers)]
    vcache = [PagedCache(vkeys[l], vvals[l], [n0 + g], extra=g + 1, seed=wl.seed + 7 + l, interleaved=True)
              for l in range(layers)]
    q = case.q.contiguous().to(DEV)
    kn, vn = case.k_new.contiguous().to(DEV), case.v_new.contiguous().to(DEV)
    qv = [c.q.contiguous().to(DEV) for c in vcases]
    knv = [c.k_new.contiguous().to(DEV) for c in vcases]
    vnv = [c.v_new.contiguous().to(DEV) for c in vcases]
    R = g - 1
    lens_d = [n0 + g]
    ws_d = W.workspace(W.draft_workspace_bytes(mode, sh, lens_d, 0, S, Wn, R), DEV)
    ws_v = W.workspace(W.verify_workspace_bytes(sh, g + 1, [n0 + 2 * g + 1], 0), DEV)
    out_d = torch.zeros((g, 1, Hq, D), dtype=torch.float32, device=DEV)
    out_v = torch.zeros((layers, 1, (g + 1) * Hq, D), dtype=torch.float32, device=DEV)

    def step():
        for j in range(g):
            kw = dict(paged=draft_cache.desc) if mode == O.FULL else dict(ring=ring.desc)
            parts = W.draft_attn_append(mode | W.DRAFT_FAST_PV, sh, q[j], kn[j], vn[j], [n0 + j + 1], ws_d, **kw)
            W.combine(parts, out_d[j])
        for l in range(layers):
            parts = W.verify_attn_append(sh, qv[l], g + 1, vcache[l].desc, knv[l], vnv[l], [n0 + 2 * g + 1], ws_v)
            W.combine(parts, out_v[l])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                     # eager (appends are idempotent: the same tokens at the same positions)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_d, ref_v = out_d.clone(), out_v.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out_d.zero_()
        out_v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, ref_d) and torch.equal(out_v, ref_v), rep
    del graph
    # the eager step against the oracle: the last draft step, and the last verify layer
    dt = "bf16"
    kb, vb = host_array(case.k_ctx, dt)[0], host_array(case.v_ctx, dt)[0]
    nk, nvv = host_array(case.k_new, dt)[:, 0, 0], host_array(case.v_new, dt)[:, 0, 0]
    sk = O.ConcatKV(O.LogicalKV(kb, dt, n0), O.LogicalKV(nk, dt))
    sv = O.ConcatKV(O.LogicalKV(vb, dt, n0), O.LogicalKV(nvv, dt))
    qf = O.to_f64(host_array(case.q[g - 1], dt), dt)[0]
    o_ref, _ = O.draft_attention(qf, sk, sv, n0 + g, mode, S, Wn, wl.scale)
    assert max_err(ref_d[g - 1, 0], o_ref) <= TOL["bf16"]
    vc = vcases[layers - 1]
    vk = O.ConcatKV(sk, O.LogicalKV(host_array(vc.k_new, dt)[0], dt))
    vv = O.ConcatKV(sv, O.LogicalKV(host_array(vc.v_new, dt)[0], dt))
    o_ref, _ = O.verify_attention(O.to_f64(host_array(vc.q, dt)[0], dt), vk, vv, n0 + 2 * g + 1, wl.scale)
    assert max_err(ref_v[layers - 1, 0], o_ref.reshape((g + 1) * Hq, D)) <= TOL["bf16"]


# ============================================================== the batch limit
def test_max_batch_of_64_sequences():
    """64 sequences (the ABI's limit) of mixed lengths in one call: draft in both modes and
    verify, each checked against the oracle on every sequence."""
    wl = synth.workload("draft_131k_bf16", window=128)
    rng = np.random.default_rng(64)
    contexts = tuple(int(x) for x in rng.integers(0, 400, size=64))
    say("batch of 64")
    for mode in (O.FULL, O.SINK_WINDOW):
        eo, el = draft_steps(wl, contexts, mode, chunk=64, fast_pv=True, steps=1, fused=True)
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (mode, eo, el)
    wlv = synth.workload("step_1m_bf16")
    eo, el = verify_run(wlv, contexts, 4, 64, fused=True, interleaved=True)
    assert eo <= TOL["bf16"] and el <= TOL["bf16"], (eo, el)
