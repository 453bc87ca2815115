"""Pins for the oracle's visible sets, ring buffer and paged addressing (no GPU)."""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _list_model_visible(n, S, W):
    """First S plus last W of the list [0..n-1], duplicates removed (list slicing, no arithmetic)."""
    xs = list(range(n))
    keep = xs[:S] + (xs[-W:] if W > 0 else [])
    return sorted(set(keep))


@settings(max_examples=300, deadline=None)
@given(n=st.integers(0, 400), S=st.integers(0, 16), W=st.integers(1, 128))
def test_visible_set_is_first_sinks_plus_last_window(n, S, W):
    got = O.visible_positions(n, O.SINK_WINDOW, S, W)
    assert list(got) == _list_model_visible(n, S, W)
    assert len(got) == min(n, S + W)
    assert O.draft_entries_read(n, O.SINK_WINDOW, S, W) == min(n, S + W)


@settings(max_examples=100, deadline=None)
@given(n=st.integers(1, 200), S=st.integers(0, 8), W=st.integers(1, 64))
def test_window_covering_context_is_full_attention(n, S, W):
    if S + W < n:
        W = n  # force the covering case
    assert np.array_equal(O.visible_positions(n, O.SINK_WINDOW, S, W), O.visible_positions(n, O.FULL))
    rng = np.random.default_rng(n)
    k = rng.standard_normal((n, 2, 8)).astype(np.float32)
    v = rng.standard_normal((n, 2, 8)).astype(np.float32)
    q = rng.standard_normal((4, 8))
    a = O.draft_attention(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), n, O.SINK_WINDOW, S, W, 0.35)
    b = O.draft_attention(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), n, O.FULL, 0, 0, 0.35)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])   # bitwise


def test_window_read_is_constant_in_context():
    S, W = 4, 4096
    reads = [O.draft_entries_read(n, O.SINK_WINDOW, S, W) for n in (4100, 131072, 524288, 1048576, 1048579)]
    assert reads == [S + W] * len(reads)
    full = [O.draft_entries_read(n, O.FULL) for n in (131072, 1048576)]
    assert full == [131072, 1048576]


def test_window_attention_matches_attention_over_the_kept_tokens():
    """sink_window = plain attention over the explicitly sliced sinks + tail of the sequence."""
    rng = np.random.default_rng(8)
    n, S, W, D = 300, 3, 40, 8
    k = rng.standard_normal((n, 1, D)).astype(np.float32)
    v = rng.standard_normal((n, 1, D)).astype(np.float32)
    q = rng.standard_normal((2, D))
    o, lse = O.draft_attention(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), n, O.SINK_WINDOW, S, W, 0.2)
    ks = np.concatenate([k[:S, 0], k[n - W:, 0]]).astype(np.float64)
    vs = np.concatenate([v[:S, 0], v[n - W:, 0]]).astype(np.float64)
    s = (q @ ks.T) * 0.2
    w = np.exp(s)
    assert np.max(np.abs(o - (w @ vs) / w.sum(1, keepdims=True))) < 1e-12
    assert np.max(np.abs(lse - np.log(w.sum(1)))) < 1e-12


def test_ring_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "ring_s2_w3.json")))
    S, W = g["sink"], g["window"]
    assert [O.ring_slot(p, S, W) for p in range(len(g["slot_of_position"]))] == g["slot_of_position"]
    for n, tags in g["tags_after_n"].items():
        assert list(O.ring_expected_tags(int(n), S, W)) == tags
    for n, vis in g["visible_after_n"].items():
        assert list(O.visible_positions(int(n), O.SINK_WINDOW, S, W)) == vis


@pytest.mark.parametrize("S,W,N", [(4, 16, 3), (4, 16, 10), (4, 16, 20), (4, 16, 500), (0, 7, 50), (1, 1, 9), (3, 5, 8)])
def test_ring_after_n_appends_holds_sinks_and_last_window(S, W, N):
    """Append one token at a time; the ring must hold exactly the list model's positions."""
    tags = np.full(S + W, -1, dtype=np.int64)
    kept = []
    for p in range(N):
        O.ring_append(tags, p, 1, S, W)
        kept.append(p)
        kept = kept[:S] + kept[S:][-W:]           # list model: first S, last W
        assert sorted(t for t in tags if t >= 0) == sorted(kept)
    assert len(set(int(t) for t in tags if t >= 0)) == min(N, S + W)
    # every held position is visible, and every visible position is held
    assert sorted(t for t in tags if t >= 0) == list(O.visible_positions(N, O.SINK_WINDOW, S, W))
    assert np.array_equal(tags, O.window_slot_positions(N, S, W))


@pytest.mark.parametrize("S,W,pos,T", [(4, 16, 0, 100), (4, 16, 7, 3), (2, 8, 30, 17), (4, 16, 0, 4), (0, 5, 3, 12)])
def test_bulk_append_equals_sequential_appends(S, W, pos, T):
    a = np.full(S + W, -1, dtype=np.int64)
    b = np.full(S + W, -1, dtype=np.int64)
    O.ring_append(a, 0, pos, S, W) if pos else None
    O.ring_append(b, 0, pos, S, W) if pos else None
    writes = O.ring_append(a, pos, T, S, W)
    for i in range(T):
        O.ring_append(b, pos + i, 1, S, W)
    assert np.array_equal(a, b)
    slots = [s for _, s in writes]
    assert len(slots) == len(set(slots))                # no slot written twice


@pytest.mark.parametrize("S,W,R,N", [(4, 16, 3, 25), (4, 16, 2, 500), (0, 7, 1, 50), (1, 1, 4, 30), (3, 5, 7, 9)])
def test_ring_with_headroom_holds_sinks_and_last_cycle(S, W, R, N):
    """With R headroom slots the ring keeps the first S and the last W + R positions (list model)."""
    tags = np.full(S + W + R, -1, dtype=np.int64)
    kept = []
    for p in range(N):
        O.ring_append(tags, p, 1, S, W, R)
        kept.append(p)
        kept = kept[:S] + kept[S:][-(W + R):]
        assert sorted(t for t in tags if t >= 0) == sorted(kept)
    assert np.array_equal(tags, O.ring_expected_tags(N, S, W, R))
    # what a query at length N reads: exactly its sink_window set, each in slot(p)
    vis = O.ring_visible(tags, N, S, W)
    assert sorted(int(t) for t in vis if t >= 0) == list(O.visible_positions(N, O.SINK_WINDOW, S, W))
    assert np.array_equal(vis, O.window_slot_positions(N, S, W, R))


@pytest.mark.parametrize("S,W,R,pos,T", [(4, 16, 3, 0, 100), (2, 8, 2, 30, 17), (0, 5, 4, 3, 12), (4, 16, 7, 19, 40)])
def test_bulk_append_with_headroom_equals_sequential(S, W, R, pos, T):
    a = np.full(S + W + R, -1, dtype=np.int64)
    b = np.full(S + W + R, -1, dtype=np.int64)
    if pos:
        O.ring_append(a, 0, pos, S, W, R)
        O.ring_append(b, 0, pos, S, W, R)
    writes = O.ring_append(a, pos, T, S, W, R)
    for i in range(T):
        O.ring_append(b, pos + i, 1, S, W, R)
    assert np.array_equal(a, b)
    slots = [sl for _, sl in writes]
    assert len(slots) == len(set(slots))


def _speculate(S, W, R, gamma, n0, accepts, rollback, vis=None):
    """Run draft cycles on a ring and return the first (cycle, step, missing position) a
    draft query fails to read with the right content, or None.

    Content model: every slot holds (position, version).  The prefill writes version
    "p"; cycle c drafts positions n..n+gamma-1 with version c.  After verification the
    first a drafted tokens are accepted (they keep version c), the rest are rejected;
    the next cycle starts at n + a (its first token is the target's correction).
    """
    C = S + W + R
    Sv, Wv = vis if vis is not None else (S, W)          # the queries' sinks and window (<= the layout's)
    tags = np.full(C, -1, dtype=np.int64)
    content = {}
    truth = {}                                           # position -> version of the accepted sequence
    for i, sl in O.ring_append(tags, 0, n0, S, W, R):   # bulk init from the prefill
        content[sl] = (i, "p")
    for p in range(n0):
        truth[p] = "p"
    n = n0
    for c, a in enumerate(accepts):
        for j in range(gamma):                           # draft step j: append, then query at n + j + 1
            p = n + j
            (_, sl), = O.ring_append(tags, p, 1, S, W, R)
            content[sl] = (p, c)
            m = p + 1
            want = {q: (truth[q] if q < n else c) for q in O.visible_positions(m, O.SINK_WINDOW, Sv, Wv)}
            got = {}
            for sl2, q in enumerate(O.ring_visible(tags, m, Sv, Wv)):
                if q >= 0:
                    got[int(q)] = content[sl2][1]
            for q, ver in want.items():
                if got.get(q) != ver:
                    return (c, j, q)
        for j in range(a):                               # accepted drafted tokens join the sequence
            truth[n + j] = c
        n += a
        if rollback:
            O.ring_rollback(tags, n)
            assert all(t < n for t in tags)
    return None


@settings(max_examples=200, deadline=None)
@given(S=st.integers(0, 6), W=st.integers(1, 24), gamma=st.integers(1, 6), extra=st.integers(0, 3),
       n0=st.integers(1, 80), data=st.data())
def test_rollback_with_headroom_keeps_every_needed_entry(S, W, gamma, extra, n0, data):
    """With R >= gamma - 1 headroom slots, every draft query after any acceptance pattern reads
    exactly its sink_window set with the accepted (or current-cycle) content."""
    accepts = data.draw(st.lists(st.integers(1, gamma), min_size=1, max_size=8))
    R = gamma - 1 + extra
    assert _speculate(S, W, R, gamma, n0, accepts, rollback=True) is None
    assert _speculate(S, W, R, gamma, n0, accepts, rollback=False) is None   # tags alone already hide rejects


def test_rollback_without_headroom_loses_a_window_entry():
    """The failure the headroom prevents: with R = 0 a rejected draft overwrites the slot of
    position p - W, which the next cycle's window still needs."""
    S, W, gamma = 4, 16, 3
    assert _speculate(S, W, 0, gamma, 100, [1, 3], rollback=True) == (1, 0, 86)
    assert _speculate(S, W, gamma - 1, gamma, 100, [1, 3], rollback=True) is None


def test_ring_rollback_clears_exactly_the_rejected_positions():
    S, W, R = 2, 5, 2
    tags = np.full(S + W + R, -1, dtype=np.int64)
    O.ring_append(tags, 0, 20, S, W, R)                 # holds 0, 1 and 13..19
    cleared = O.ring_rollback(tags, 17)
    assert sorted(cleared) == sorted(O.ring_slot(p, S, W, R) for p in (17, 18, 19))
    assert sorted(t for t in tags if t >= 0) == [0, 1, 13, 14, 15, 16]
    assert O.ring_rollback(tags, 17) == []              # idempotent


@settings(max_examples=200, deadline=None)
@given(S=st.integers(0, 8), Wn=st.integers(1, 40), R=st.integers(0, 6), data=st.data())
def test_per_sequence_sinks_and_windows_read_from_one_ring_layout(S, Wn, R, data):
    """Adaptive windows / dynamic sinks: a ring laid out for (S, W, R) and appended in order
    holds every position of the sink_window set of any S_b <= S and W_b <= W + R, and a query
    reads exactly that set, so S_b and W_b may change from one step to the next."""
    tags = np.full(S + Wn + R, -1, dtype=np.int64)
    N = data.draw(st.integers(1, 3 * (S + Wn + R) + 5))
    for p in range(N):
        O.ring_append(tags, p, 1, S, Wn, R)
        Sb = data.draw(st.integers(0, S))
        Wb = data.draw(st.integers(1, Wn + R))
        got = sorted(int(t) for t in O.ring_visible(tags, p + 1, Sb, Wb) if t >= 0)
        assert got == _list_model_visible(p + 1, Sb, Wb)


def test_per_sequence_windows_with_rollback():
    """Per-sequence windows W_b with W_b + gamma - 1 <= W + R keep every needed entry through
    draft cycles with partial acceptance (the ring layout stays (S, W, R))."""
    S, Wn, R, gamma = 4, 16, 2, 3
    for Sb, Wb in ((4, 16), (2, 10), (0, 16), (4, 1), (1, 16)):
        assert _speculate(S, Wn, R, gamma, 100, [1, 3, 2, 1, 1, 3], rollback=True, vis=(Sb, Wb)) is None
    # a window past the safe bound loses an entry after a partial acceptance
    assert _speculate(S, Wn, R, gamma, 100, [1, 3], rollback=True, vis=(4, Wn + R)) is not None


def _place_paged(logical, bt_row, bs, num_blocks):
    """Build a paged pool from a logical [n][H][D] array by block-level slicing."""
    n, H, D = logical.shape
    pool = np.zeros((num_blocks, H, bs, D), dtype=logical.dtype)
    for j in range(-(-n // bs)):
        seg = logical[j * bs:(j + 1) * bs]               # [<=bs][H][D]
        pool[bt_row[j], :, :seg.shape[0], :] = seg.transpose(1, 0, 2)
    return pool


@pytest.mark.parametrize("n,bs", [(1, 16), (16, 16), (17, 16), (300, 16), (100, 8)])
def test_paged_gather_equals_contiguous(n, bs):
    rng = np.random.default_rng(n)
    H, D = 2, 8
    nb = -(-n // bs) + 3
    bt = rng.permutation(nb).astype(np.int32)
    logical = rng.standard_normal((n, H, D)).astype(np.float32)
    pool = _place_paged(logical, bt, bs, nb)
    src = O.PagedKV(pool, bt, bs, "f32", n)
    pos = rng.permutation(n)
    for h in range(H):
        assert np.array_equal(src.rows(pos, h), logical[pos, h].astype(np.float64))
    q = rng.standard_normal((4, D))
    a = O.draft_attention(q, src, src, n, O.FULL, 0, 0, 0.3)
    b = O.draft_attention(q, O.LogicalKV(logical, "f32"), O.LogicalKV(logical, "f32"), n, O.FULL, 0, 0, 0.3)
    assert np.array_equal(a[0], b[0])


def _place_paged_kv_runs(k_logical, v_logical, bt_row, bs, num_blocks):
    """Build a K|V pool [block][H][2][bs][D] from logical K and V by block-level slicing."""
    n, H, D = k_logical.shape
    pool = np.zeros((num_blocks, H, 2, bs, D), dtype=k_logical.dtype)
    for j in range(-(-n // bs)):
        for part, logical in ((0, k_logical), (1, v_logical)):
            seg = logical[j * bs:(j + 1) * bs]
            pool[bt_row[j], :, part, :seg.shape[0], :] = seg.transpose(1, 0, 2)
    return pool


@pytest.mark.parametrize("n,bs", [(1, 16), (16, 16), (17, 16), (300, 16), (100, 8)])
def test_paged_kv_runs_gather_equals_contiguous(n, bs):
    rng = np.random.default_rng(100 + n)
    H, D = 2, 8
    nb = -(-n // bs) + 3
    bt = rng.permutation(nb).astype(np.int32)
    k_log = rng.standard_normal((n, H, D)).astype(np.float32)
    v_log = rng.standard_normal((n, H, D)).astype(np.float32)
    pool = _place_paged_kv_runs(k_log, v_log, bt, bs, nb)
    ks, vs = O.PagedKV(pool, bt, bs, "f32", n, part=0), O.PagedKV(pool, bt, bs, "f32", n, part=1)
    pos = rng.permutation(n)
    for h in range(H):
        assert np.array_equal(ks.rows(pos, h), k_log[pos, h].astype(np.float64))
        assert np.array_equal(vs.rows(pos, h), v_log[pos, h].astype(np.float64))
    # the same tokens in separate pools give the same attention, bit for bit
    q = rng.standard_normal((4, D))
    a = O.draft_attention(q, ks, vs, n, O.FULL, 0, 0, 0.3)
    b = O.draft_attention(q, O.PagedKV(_place_paged(k_log, bt, bs, nb), bt, bs, "f32", n),
                          O.PagedKV(_place_paged(v_log, bt, bs, nb), bt, bs, "f32", n), n, O.FULL, 0, 0, 0.3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_paged_offsets_hand_worked_and_past_2_pow_31():
    # pool [block][kv_head][16][D]: block 5, head 1, offset 3, D 256, 2 heads
    assert O.paged_element_offset([9, 5], 16 + 3, 1, 2, 16, 256) == ((5 * 2 + 1) * 16 + 3) * 256
    # a block id of 300,000 (a 4.8M-token pool) puts the element offset past 2**31
    big = 300000
    off = O.paged_element_offset([big] * 2, 15, 1, 2, 16, 256)
    assert off == big * 2 * 16 * 256 + 1 * 16 * 256 + 15 * 256
    assert off > 2 ** 31
    # K|V runs of 32 rows: block 5, head 1, offset 3 -> run (5 * 2 + 1), row 3 of its K half
    assert O.paged_element_offset([9, 5], 16 + 3, 1, 2, 16, 256, 32) == ((5 * 2 + 1) * 32 + 3) * 256
    # run_rows = block_size is the separate-pool layout
    assert O.paged_element_offset([9, 5], 16 + 3, 1, 2, 16, 256, 16) == O.paged_element_offset([9, 5], 19, 1, 2,
                                                                                                16, 256)
