"""Pins for the oracle's LSE combine and decode-step cost model (no GPU)."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parts(rng, n, D, R, cuts):
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    q = rng.standard_normal((R, D))
    bounds = [0] + list(cuts) + [n]
    os_, ls_ = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = O.softmax_attention(q, k[a:b], v[a:b], 0.3)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_), O.softmax_attention(q, k, v, 0.3)


@pytest.mark.parametrize("cuts", [[], [1], [5, 6, 40], [10, 20, 30, 40, 50]])
def test_combine_of_disjoint_parts_equals_whole(cuts):
    rng = np.random.default_rng(len(cuts))
    op, lp, (o, lse) = _parts(rng, 64, 8, 3, cuts)
    oc, lc = O.lse_combine(op, lp)
    assert np.max(np.abs(oc - o)) < 1e-12 and np.max(np.abs(lc - lse)) < 1e-12


def test_combine_is_permutation_invariant_and_ignores_empty_parts():
    rng = np.random.default_rng(9)
    op, lp, (o, lse) = _parts(rng, 50, 8, 2, [7, 30])
    perm = [2, 0, 1]
    a = O.lse_combine(op[perm], lp[perm])
    empty_o = np.full((1, 2, 8), 123.0)       # garbage values must not leak in
    empty_l = np.full((1, 2), -np.inf)
    b = O.lse_combine(np.concatenate([op, empty_o]), np.concatenate([lp, empty_l]))
    for oc, lc in (a, b):
        assert np.max(np.abs(oc - o)) < 1e-12 and np.max(np.abs(lc - lse)) < 1e-12
    one = O.lse_combine(op[:1], lp[:1])
    assert np.allclose(one[0], op[0], atol=1e-15, rtol=0) and np.allclose(one[1], lp[0], atol=1e-15, rtol=0)
    none = O.lse_combine(empty_o, empty_l)
    assert np.all(none[0] == 0) and np.all(np.isneginf(none[1]))


def _pages():
    return json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))


def test_window_drops_roughly_99_percent_at_1m():
    g = _pages()["dropped_fraction_at_1m"]
    n = 1 << 20
    frac = 1 - O.draft_entries_read(n, O.SINK_WINDOW, 4, 4096) / O.draft_entries_read(n, O.FULL)
    assert frac >= g["min"]


def test_step_bytes_ratio_sits_in_the_reported_speedup_range():
    g = _pages()["speedup_range_at_1m"]
    n0, gamma = 1 << 20, _pages()["draft_steps_per_cycle"]["value"]
    nat = O.step_kv_bytes(n0, gamma, 10, 2, 256, 2, O.FULL)
    win = O.step_kv_bytes(n0, gamma, 10, 2, 256, 2, O.SINK_WINDOW, 4, 4096)
    assert g["lo"] <= nat / win <= g["hi"]
    # hand count: 10 layers x (n0+4) tokens + 3 draft steps at n0+1..n0+3, 2048 B per token
    assert nat == 2048 * (10 * (n0 + 4) + (n0 + 1) + (n0 + 2) + (n0 + 3))
    assert win == 2048 * (10 * (n0 + 4) + 3 * 4100)


def test_one_draft_step_costs_a_tenth_of_the_target_read():
    g = _pages()["draft_to_target_tax"]
    n0 = 131072
    per_draft_step = O.step_kv_bytes(n0, 1, 0, 2, 256, 2, O.FULL)
    target = O.step_kv_bytes(n0, 0, g["layers_target"], 2, 256, 2, O.FULL)
    ratio = per_draft_step / target
    assert abs(ratio - g["layers_draft"] / g["layers_target"]) < 1e-3
    assert abs(ratio - g["measured"]) < 0.015     # the case study measured 8.8%


# ---------------------------------------------------------------- sweeps over context and gamma (row f2)
def _ratio(n0, gamma, L=10, S=4, Wn=4096):
    nat = O.step_kv_bytes(n0, gamma, L, 2, 256, 2, O.FULL)
    win = O.step_kv_bytes(n0, gamma, L, 2, 256, 2, O.SINK_WINDOW, S, Wn)
    return nat / win


def test_wedge_widens_with_context():
    """[P3 Abstract] the speedup increases with the context length: the bytes ratio never falls as n0 grows,
    and it is exactly 1 while the window still covers the whole context."""
    for gamma in (3, 5, 8):
        ctx = [2048, 4096 - gamma, 8192, 32768, 131072, 524288, 1 << 20, 1 << 22]
        r = [_ratio(n, gamma) for n in ctx]
        assert r[0] == 1.0 and r[1] == 1.0                 # n0 + gamma <= S + W: same entries read
        assert all(b >= a for a, b in zip(r, r[1:]))
        assert r[-1] > r[2]


def test_deeper_drafts_pay_more_at_long_context():
    """More draft forwards per cycle multiply the native draft's cost; the windowed draft's stays constant."""
    for n0 in (131072, 1 << 20):
        r = [_ratio(n0, g) for g in (1, 3, 5, 8)]
        assert all(b > a for a, b in zip(r, r[1:]))


def test_ratio_tends_to_one_plus_gamma_over_layers():
    """Closed form at long context: the draft steps read gamma full caches against L target layers,
    so step_nat / step_win -> (L + gamma) / L as n0 -> infinity with S + W fixed."""
    for gamma, L in ((3, 10), (5, 10), (8, 10), (3, 4)):
        lim = (L + gamma) / L
        gap1 = lim - _ratio(1 << 22, gamma, L)
        gap2 = lim - _ratio(1 << 23, gamma, L)
        assert 0 < gap2 < gap1 and gap2 < 2e-3
        assert abs(gap1 / gap2 - 2.0) < 0.01             # the gap is O(1/n0): halves as the context doubles


# ---------------------------------------------------------------- memory accounting (row f3)
def test_ring_reclaims_the_dead_draft_pool_share_of_kv():
    """[P3 Abstract] 7.7-11.1% of total KV at 1M: one draft layer among L target layers of equal
    per-layer KV is 1/(L+1) of it (1/13, 1/11, 1/9 for L = 12, 10, 8), less the ring's 8 MB."""
    g = _pages()["reclaimed_pool_fraction"]
    fr = {}
    for L in (8, 10, 12):
        m = O.memory_plan(2, 256, 2, L, 1 << 20, 4, 4096, 2, 1 << 40)
        fr[L] = m["reclaimed_fraction"]
        assert abs(fr[L] - 1 / (L + 1)) < 1e-3
    assert g["lo"] - 5e-4 <= min(fr.values()) and max(fr.values()) <= g["hi"] + 5e-4


def test_hand_counted_bytes_at_1m():
    m = O.memory_plan(2, 256, 2, 10, 1 << 20, 4, 4096, 2, 0)
    assert m["layer_bytes"] == 65536 * 16 * 2 * 256 * 2 * 2 == 2 << 30          # 2 GiB per layer
    assert m["ring_bytes"] == 4102 * (2048 + 4)
    assert m["native_seq_bytes"] == 11 * (2 << 30) + 65536 * 4
    assert m["windowed_seq_bytes"] == 10 * (2 << 30) + 4102 * 2052 + 65536 * 4


def test_one_more_1m_request_fits():
    """[P3 Abstract] the reclaimed pool made room for one additional concurrent 1M request: with a
    budget that holds N native 1M sequences (N > L), the windowed draft admits at least N + 1 (at
    N = L exactly, the ring and block table leave it just short)."""
    for L in (8, 10, 12):
        m = O.memory_plan(2, 256, 2, L, 1 << 20, 4, 4096, 2, 0)
        p = O.memory_plan(2, 256, 2, L, 1 << 20, 4, 4096, 2, L * m["native_seq_bytes"])
        assert p["windowed_sequences"] == L
        for n in range(L + 1, 3 * L):
            budget = n * m["native_seq_bytes"]
            p = O.memory_plan(2, 256, 2, L, 1 << 20, 4, 4096, 2, budget)
            assert p["native_sequences"] == n
            assert p["windowed_sequences"] >= n + 1
