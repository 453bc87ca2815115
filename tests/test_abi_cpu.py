"""C-ABI checks that need no GPU: exports, argument validation, workspace sizing.

Every call here returns before making any HIP call (the library validates all
arguments first), so nothing is launched.
"""
import ctypes
import os
import re

import pytest
import torch

from long_context_decode_gqa_amd import wmtp as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wmtp.h")

FAKE = 1 << 20          # a 16-byte aligned non-null "device" address; never dereferenced
FAKE_ODD = FAKE + 8     # not 16-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wmtp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = W.load()
    declared = header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(W.EXPORTS)
    assert W.version().startswith("wmtp")


def test_status_strings():
    lib = W.load()
    for st in (W.OK, W.EINVAL, W.EUNSUPPORTED, W.EALIGN, W.EWORKSPACE, W.ELAUNCH):
        assert lib.wmtp_status_str(st).decode() not in ("", "unknown status")
    assert lib.wmtp_status_str(-99).decode() == "unknown status"


def shape(hq=16, hk=2, d=256, dt=W.BF16, scale=0.0625):
    return W.Shape(hq, hk, d, scale, dt)


def lens(*xs):
    return ctypes.cast((ctypes.c_int32 * len(xs))(*xs), ctypes.c_void_p)


def paged(k=FAKE, v=FAKE, bt=FAKE, bs=16, mb=100, nb=100, rr=0):
    return W.Paged(k, v, bt, bs, mb, nb, rr)


def ring(k=FAKE, v=FAKE, tags=FAKE, s=4, w=64, r=0):
    return W.Ring(k, v, tags, s, w, r)


def draft(mode=W.FULL, sh=None, q=FAKE, kv="default", rg="default", seq=(1000,), chunk=0, ws=FAKE, wsb=1 << 30,
          parts=True):
    lib = W.load()
    sh = shape() if sh is None else sh
    kv = paged() if kv == "default" else kv
    rg = ring() if rg == "default" else rg
    p = W.Partials()
    return lib.wmtp_draft_attn(mode, ctypes.byref(sh) if sh is not False else None, q,
                               ctypes.byref(kv) if kv is not None else None,
                               ctypes.byref(rg) if rg is not None else None, lens(*seq), len(seq), chunk, ws, wsb,
                               ctypes.byref(p) if parts else None, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(), None),                                             # valid (not launched here)
    (dict(sh=False), W.EINVAL),
    (dict(sh=shape(hq=12, hk=8)), W.EINVAL),                    # H_q % H_kv != 0
    (dict(sh=shape(hq=48, hk=3)), W.EUNSUPPORTED),              # G = 16
    (dict(sh=shape(d=96)), W.EUNSUPPORTED),
    (dict(sh=shape(dt=7)), W.EINVAL),
    (dict(sh=shape(scale=float("nan"))), W.EINVAL),
    (dict(mode=5), W.EINVAL),
    (dict(mode=W.FULL | 0x40), W.EINVAL),
    (dict(q=None), W.EINVAL),
    (dict(q=FAKE_ODD), W.EALIGN),
    (dict(kv=None), W.EINVAL),
    (dict(kv=paged(bs=32)), W.EUNSUPPORTED),
    (dict(kv=paged(k=FAKE_ODD)), W.EALIGN),
    (dict(kv=paged(mb=10)), W.EINVAL),                          # table too short for 1000 tokens
    (dict(kv=paged(rr=8)), W.EINVAL),                           # runs closer than 16 rows overlap
    (dict(kv=paged(rr=-16)), W.EINVAL),
    (dict(seq=(-1,)), W.EINVAL),
    (dict(chunk=100), W.EINVAL),                                # not a multiple of 32
    (dict(chunk=16), W.EINVAL),
    (dict(ws=None), W.EINVAL),
    (dict(ws=FAKE + 16), W.EALIGN),
    (dict(wsb=16), W.EWORKSPACE),
    (dict(parts=False), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=None), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=ring(w=0)), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=ring(s=-1)), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=ring(r=-1)), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=ring(w=1 << 30, r=1 << 30)), W.EINVAL),
    (dict(mode=W.SINK_WINDOW, rg=ring(k=FAKE_ODD)), W.EALIGN),
])
def test_draft_argument_checks(kwargs, status):
    if status is None:
        # the valid call must pass every check; planning alone shows that without launching
        sh = shape()
        n = W.load().wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(1000), 1, 0, 0, 1, 0)
        assert n > 0
        return
    assert draft(**kwargs) == status


def test_draft_batch_limits():
    lib = W.load()
    sh = shape()
    assert lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(1), 0, 0, 0, 1, 0) == W.EINVAL
    big = (ctypes.c_int32 * 65)(*([10] * 65))
    assert lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), ctypes.cast(big, ctypes.c_void_p), 65, 0, 0,
                                          1, 0) == W.EINVAL


def _splits_of(ws_bytes, rows, d):
    """Total splits recorded in a workspace size: align256(P rows d 4) + align256(P rows 4)."""
    for p in range(1, 1 << 20):
        if ((p * rows * d * 4 + 255) // 256 + (p * rows * 4 + 255) // 256) * 256 == ws_bytes:
            return p
    raise AssertionError(ws_bytes)


def _rule(vis, hk, slots, lo):
    """The default-split rule, by exhaustive search over multiples of 64."""
    target = slots
    while target < len(vis) * hk:
        target += slots
    items = lambda s: hk * sum(-(-v // s) for v in vis)
    s = lo
    while s < 65536 and items(s) > target:
        s += 64
    return s


@pytest.mark.parametrize("lens", [[1048577], [1048580], [262144] * 4, [32769, 131073, 524289, 1048577], [1000],
                                  [5, 70000, 3, 9000, 1 << 20]])
def test_default_split_fits_one_round_of_work_items(lens):
    # 0 = library default: the smallest split (multiple of 64) whose work items
    # (sequence, KV head, split) fit one round of 256 (one per compute unit)
    sh = shape()                                                   # 2 KV heads
    s = _rule(lens, 2, 256, 64)
    assert W.draft_workspace_bytes(W.FULL, sh, lens, 0) == W.draft_workspace_bytes(W.FULL, sh, lens, s)
    if min(lens) >= 4:
        assert W.verify_workspace_bytes(sh, 4, lens, 0) == W.verify_workspace_bytes(sh, 4, lens, s)
    total = _splits_of(W.draft_workspace_bytes(W.FULL, sh, lens, 0), 16, 256)
    assert total * 2 <= 256
    if s > 64:                                                     # minimal: one tile less does not fit
        assert 2 * sum(-(-v // (s - 64)) for v in lens) > 256


def test_default_split_values():
    sh = shape()
    assert _rule([1048577], 2, 256, 64) == 8256                    # 128 splits x 2 heads = 256 items
    assert _rule([32769, 131073, 524289, 1048577], 2, 256, 64) > 13568    # plain division would give 260 items
    # short contexts: splits of 64 entries (two verify tiles), not a floor of 256
    assert _rule([2052], 2, 256, 64) == 64
    assert W.verify_workspace_bytes(sh, 4, [2052], 0) == W.verify_workspace_bytes(sh, 4, [2052], 64)
    assert W.draft_workspace_bytes(W.FULL, sh, [8193], 0) == W.draft_workspace_bytes(W.FULL, sh, [8193], 128)
    # very long contexts hit the 65536 cap
    big = shape(hq=64, hk=8)
    assert W.draft_workspace_bytes(W.FULL, big, [8 << 20], 0) == W.draft_workspace_bytes(W.FULL, big, [8 << 20], 65536)
    # the window draft scans min(n, S+W) entries and targets 512 items of at least 64 entries
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, [1048577], 0, 4, 4096) == \
        W.draft_workspace_bytes(W.SINK_WINDOW, sh, [1048577], 64, 4, 4096)
    lens = [32769, 131073, 524289, 1048577]
    s = _rule([min(n, 4 + 16384) for n in lens], 2, 512, 64)
    assert s == 320                                                # 256 would give 520 items
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, lens, 0, 4, 16384) == \
        W.draft_workspace_bytes(W.SINK_WINDOW, sh, lens, s, 4, 16384)


def test_workspace_sizes_follow_the_split_plan():
    sh = shape()
    # full mode at 1M+1 tokens, 1024-token splits: 1025 splits x 16 rows x (256 + 1) floats, 256-byte aligned
    n = W.draft_workspace_bytes(W.FULL, sh, [1048577], 1024)
    o = 1025 * 16 * 256 * 4
    assert n == o + ((1025 * 16 * 4 + 255) // 256) * 256
    # window mode scans min(n, S+W) slots
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, [1048577], 256, 4, 4096) == \
        W.draft_workspace_bytes(W.FULL, sh, [4100], 256)
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, [100], 256, 4, 4096) == \
        W.draft_workspace_bytes(W.FULL, sh, [100], 256)
    # verify: rows = t_q * H_q
    nv = W.verify_workspace_bytes(sh, 4, [1048580], 2048)
    splits = -(-1048580 // 2048)
    assert nv == splits * 64 * 256 * 4 + ((splits * 64 * 4 + 255) // 256) * 256
    # an empty sequence needs no split
    assert W.draft_workspace_bytes(W.FULL, sh, [0, 64], 64) == W.draft_workspace_bytes(W.FULL, sh, [64], 64)


@pytest.mark.parametrize("args,status", [
    (dict(sh=shape(dt=W.F32)), W.EUNSUPPORTED),
    (dict(sh=shape(d=128), t_q=13), W.EUNSUPPORTED),               # 13 x 8 rows > 96 at every head_dim
    (dict(sh=shape(d=64), t_q=13), W.EUNSUPPORTED),
    (dict(t_q=0), W.EINVAL),
    (dict(t_q=13), W.EUNSUPPORTED),                              # 13 x 8 rows > 96
    (dict(seq=(3,)), W.EINVAL),                                  # fewer keys than queries
    (dict(split=48), W.EINVAL),
])
def test_verify_argument_checks(args, status):
    lib = W.load()
    sh = args.get("sh", shape())
    seq = args.get("seq", (1000,))
    assert lib.wmtp_verify_workspace_bytes(ctypes.byref(sh), args.get("t_q", 4), lens(*seq), len(seq),
                                           args.get("split", 0)) == status
    p = W.Partials()
    kv = paged()
    assert lib.wmtp_verify_attn(ctypes.byref(sh), FAKE, args.get("t_q", 4), ctypes.byref(kv), lens(*seq), len(seq),
                                args.get("split", 0), FAKE, 1 << 30, ctypes.byref(p), None) == status


def test_verify_pointer_checks():
    lib = W.load()
    sh = shape()
    p = W.Partials()
    kv = paged()
    call = lambda q=FAKE, kvp=ctypes.byref(kv), ws=FAKE, wsb=1 << 30: lib.wmtp_verify_attn(
        ctypes.byref(sh), q, 4, kvp, lens(1000), 1, 0, ws, wsb, ctypes.byref(p), None)
    assert call(q=None) == W.EINVAL
    assert call(q=FAKE_ODD) == W.EALIGN
    assert call(kvp=None) == W.EINVAL
    assert call(wsb=64) == W.EWORKSPACE
    bad = paged(mb=2)
    assert call(kvp=ctypes.byref(bad)) == W.EINVAL
    bad = paged(rr=15)
    assert call(kvp=ctypes.byref(bad)) == W.EINVAL


def test_combine_checks():
    lib = W.load()
    p = W.Partials()
    p.o, p.lse, p.batch, p.rows_per_seq, p.head_dim, p.total_splits = FAKE, FAKE, 1, 16, 256, 3
    p.split_base[0], p.split_base[1] = 0, 3
    # argument order: parts, out, lse_out, out_dtype, stream
    assert lib.wmtp_combine(None, FAKE, None, W.F32, None) == W.EINVAL
    assert lib.wmtp_combine(ctypes.byref(p), None, None, W.F32, None) == W.EINVAL
    assert lib.wmtp_combine(ctypes.byref(p), FAKE, None, 9, None) == W.EINVAL
    assert lib.wmtp_combine(ctypes.byref(p), FAKE_ODD, None, W.F32, None) == W.EALIGN
    assert lib.wmtp_combine(ctypes.byref(p), FAKE, FAKE + 2, W.F32, None) == W.EALIGN   # lse_out not 4-byte aligned
    p.split_base[1] = 2
    assert lib.wmtp_combine(ctypes.byref(p), FAKE, None, W.F32, None) == W.EINVAL   # inconsistent total
    p.split_base[1] = 3
    p.head_dim = 80
    assert lib.wmtp_combine(ctypes.byref(p), FAKE, None, W.F32, None) == W.EUNSUPPORTED
    p.head_dim = 256
    p.batch = 0
    assert lib.wmtp_combine(ctypes.byref(p), FAKE, None, W.F32, None) == W.EINVAL


def test_append_checks():
    lib = W.load()
    sh = shape()
    r = ring()
    kv = paged(mb=4)
    pos = lens(10)
    assert lib.wmtp_ring_append(ctypes.byref(sh), None, FAKE, FAKE, pos, 1, 1, None) == W.EINVAL
    assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(r), None, FAKE, pos, 1, 1, None) == W.EINVAL
    assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(r), FAKE_ODD, FAKE, pos, 1, 1, None) == W.EALIGN
    assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, lens(-3), 1, 1, None) == W.EINVAL
    assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, pos, 1, -1, None) == W.EINVAL
    assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(r), FAKE, FAKE, pos, 0, 1, None) == W.EINVAL
    # paged: 4 blocks cover positions < 64
    assert lib.wmtp_paged_append(ctypes.byref(sh), ctypes.byref(kv), FAKE, FAKE, lens(60), 1, 5, None) == W.EINVAL
    short_runs = paged(rr=1)
    assert lib.wmtp_paged_append(ctypes.byref(sh), ctypes.byref(short_runs), FAKE, FAKE, lens(0), 1, 1,
                                 None) == W.EINVAL
    assert lib.wmtp_paged_append(ctypes.byref(sh), None, FAKE, FAKE, lens(0), 1, 1, None) == W.EINVAL


def test_fused_append_checks():
    lib = W.load()
    sh = shape()
    kv = paged()
    r = ring()
    p = W.Partials()

    def draft(mode=W.FULL, k_new=FAKE, v_new=FAKE, seq=(1000,), rg=r, wsb=1 << 30):
        return lib.wmtp_draft_attn_append(mode, ctypes.byref(sh), FAKE, ctypes.byref(kv),
                                          ctypes.byref(rg) if rg is not None else None, k_new, v_new, lens(*seq),
                                          len(seq), 0, FAKE, wsb, ctypes.byref(p), None)

    def verify(t_q=4, k_new=FAKE, v_new=FAKE, seq=(1000,)):
        return lib.wmtp_verify_attn_append(ctypes.byref(sh), FAKE, t_q, ctypes.byref(kv), k_new, v_new, lens(*seq),
                                           len(seq), 0, FAKE, 1 << 30, ctypes.byref(p), None)

    for mode in (W.FULL, W.SINK_WINDOW):
        assert draft(mode, k_new=None) == W.EINVAL
        assert draft(mode, v_new=None) == W.EINVAL
        assert draft(mode, k_new=FAKE_ODD) == W.EALIGN
        assert draft(mode, v_new=FAKE_ODD) == W.EALIGN
        assert draft(mode, seq=(5, 0)) == W.EINVAL          # the new token needs a position: n >= 1
        assert draft(mode, wsb=16) == W.EWORKSPACE
    assert draft(W.SINK_WINDOW, rg=None) == W.EINVAL
    assert verify(k_new=None) == W.EINVAL
    assert verify(v_new=FAKE_ODD) == W.EALIGN
    assert verify(seq=(3,)) == W.EINVAL                      # fewer keys than new tokens
    assert verify(t_q=13) == W.EUNSUPPORTED
    # the binding checks that k_new / v_new hold [batch][t_new][H_kv][D] of the cache dtype
    pyshape = W.make_shape(16, 2, 256, torch.bfloat16)
    q = torch.zeros((1, 16, 256), dtype=torch.bfloat16)
    ws = torch.zeros(256, dtype=torch.uint8)
    good = torch.zeros((1, 1, 2, 256), dtype=torch.bfloat16)
    for bad in (torch.zeros((1, 2, 2, 256), dtype=torch.bfloat16), torch.zeros((1, 1, 2, 256)),
                torch.zeros((1, 1, 2, 512), dtype=torch.bfloat16)[..., ::2]):
        with pytest.raises(ValueError):
            W.draft_attn_append(W.FULL, pyshape, q, bad, good, [10], ws, paged=kv)
        with pytest.raises(ValueError):
            W.verify_attn_append(pyshape, q, 3, kv, bad, bad, [10], ws)


def test_per_sequence_policy_checks():
    """Per-sequence sinks <= S and windows in [1, W + R] (window mode only)."""
    lib = W.load()
    sh = shape()
    base = ring(s=4, w=64, r=2)
    for sinks, wins, want in (([4], [66], W.OK), ([5], [64], W.EINVAL), ([-1], [64], W.EINVAL),
                              ([0], [0], W.EINVAL), ([0], [67], W.EINVAL), (None, [66], W.OK), ([2], None, W.OK)):
        r = W.with_policy(base, sinks, wins)
        p = W.Partials()
        st = lib.wmtp_draft_attn(W.SINK_WINDOW, ctypes.byref(sh), FAKE, None, ctypes.byref(r), lens(1000), 1, 0,
                                 FAKE, 1 << 30, ctypes.byref(p), None)
        if want == W.OK:
            assert st != W.EINVAL      # passes validation (no GPU here: the launch itself reports ELAUNCH)
        else:
            assert st == want, (sinks, wins, st)


def test_rollback_checks():
    lib = W.load()
    r = ring(r=2)
    assert lib.wmtp_ring_rollback(None, lens(10), 1, None) == W.EINVAL
    assert lib.wmtp_ring_rollback(ctypes.byref(r), None, 1, None) == W.EINVAL
    assert lib.wmtp_ring_rollback(ctypes.byref(r), lens(-1), 1, None) == W.EINVAL
    assert lib.wmtp_ring_rollback(ctypes.byref(r), lens(10), 0, None) == W.EINVAL
    assert lib.wmtp_ring_rollback(ctypes.byref(r), lens(10), 65, None) == W.EINVAL
    bad = ring(r=-1)
    assert lib.wmtp_ring_rollback(ctypes.byref(bad), lens(10), 1, None) == W.EINVAL


def test_window_workspace_covers_headroom_slots():
    # the window draft scans min(n, S+W+R) slots: R extra entries in the plan
    sh = shape()
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, [1 << 20], 64, 4, 4096, 2) == \
        W.draft_workspace_bytes(W.FULL, sh, [4102], 64)
    assert W.draft_workspace_bytes(W.SINK_WINDOW, sh, [100], 64, 4, 4096, 2) == \
        W.draft_workspace_bytes(W.FULL, sh, [100], 64)
    with pytest.raises(W.WmtpError):
        W.draft_workspace_bytes(W.SINK_WINDOW, sh, [100], 64, 4, 4096, -1)


def test_stream_read_checks():
    lib = W.load()
    assert lib.wmtp_stream_read(None, 1024, FAKE, 4, None) == W.EINVAL
    assert lib.wmtp_stream_read(FAKE, 8, FAKE, 4, None) == W.EINVAL
    assert lib.wmtp_stream_read(FAKE, 1024, FAKE, 0, None) == W.EINVAL
    assert lib.wmtp_stream_read(FAKE_ODD, 1024, FAKE, 4, None) == W.EALIGN
    assert lib.wmtp_stream_read(FAKE, 1000, FAKE, 4, None) == W.EALIGN


def test_stream_read_paged_checks():
    lib = W.load()
    f = lib.wmtp_stream_read_paged
    assert f(FAKE, FAKE, 1 << 20, FAKE, 4, 8192, FAKE, 4, None) not in (W.EINVAL, W.EALIGN)   # valid: passes the checks
    assert f(None, FAKE, 1 << 20, FAKE, 4, 8192, FAKE, 4, None) == W.EINVAL
    assert f(FAKE, FAKE, 1 << 20, None, 4, 8192, FAKE, 4, None) == W.EINVAL
    assert f(FAKE, FAKE, 1 << 20, FAKE, 0, 8192, FAKE, 4, None) == W.EINVAL
    assert f(FAKE, FAKE, 1 << 20, FAKE, 4, 6000, FAKE, 4, None) == W.EINVAL          # not a power of two
    assert f(FAKE, FAKE, 1 << 20, FAKE, 4, 2048, FAKE, 4, None) == W.EINVAL          # below 4 KiB
    assert f(FAKE, FAKE, 4096, FAKE, 4, 8192, FAKE, 4, None) == W.EINVAL              # pool smaller than a run
    assert f(FAKE_ODD, FAKE, 1 << 20, FAKE, 4, 8192, FAKE, 4, None) == W.EALIGN


def test_debug_hook_checks():
    lib = W.load()
    kv = paged()
    assert lib.wmtp_debug_resolve_paged(ctypes.byref(kv), 2, 256, 0, 2, FAKE, 1, FAKE, None) == W.EINVAL   # h >= H_kv
    assert lib.wmtp_debug_resolve_paged(None, 2, 256, 0, 0, FAKE, 1, FAKE, None) == W.EINVAL
    short_runs = paged(rr=4)
    assert lib.wmtp_debug_resolve_paged(ctypes.byref(short_runs), 2, 256, 0, 0, FAKE, 1, FAKE, None) == W.EINVAL
    assert lib.wmtp_debug_resolve_ring(4, 0, 0, FAKE, 1, FAKE, None) == W.EINVAL
    assert lib.wmtp_debug_window_positions(-1, 4, 0, 10, FAKE, None) == W.EINVAL
    assert lib.wmtp_debug_window_positions(4, 4, 0, 10, None, None) == W.EINVAL
    assert lib.wmtp_debug_window_positions(4, 4, -1, 10, FAKE, None) == W.EINVAL
    assert lib.wmtp_debug_resolve_ring(4, 4, -1, FAKE, 1, FAKE, None) == W.EINVAL


def test_memory_plan_matches_the_oracle():
    """Host-only planner (row f3) against the oracle's independent count, exact integers."""
    import oracle as O
    for hq, hk, d, dt, eb in ((16, 2, 256, W.BF16, 2), (4, 1, 64, W.F32, 4), (8, 8, 128, W.BF16, 2)):
        sh = shape(hq=hq, hk=hk, d=d, dt=dt)
        for L in (0, 1, 10):
            for ctx in (0, 1, 15, 16, 17, 131072, 1 << 20, 3_000_001):
                for S, Wn, R in ((4, 4096, 2), (0, 1, 0), (16, 16384, 7)):
                    if ctx == 0:
                        continue
                    budget = 288 * 10 ** 9
                    got = W.plan_memory(sh, L, ctx, S, Wn, R, budget)
                    want = O.memory_plan(hk, d, eb, L, ctx, S, Wn, R, budget)
                    for key, val in want.items():
                        if key == "reclaimed_fraction":
                            assert abs(got[key] - val) < 1e-12, (key, got[key], val)
                        else:
                            assert got[key] == val, (key, got[key], val)


def test_memory_plan_checks():
    lib = W.load()
    sh = shape()
    out = W.MemoryPlan()
    assert lib.wmtp_plan_memory(ctypes.byref(sh), -1, 10, 4, 64, 0, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, -1, 4, 64, 0, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, 10, 4, 0, 0, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, 10, 4, 64, -1, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, 10, 4, 64, 0, -5, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, 10, 4, 64, 0, 0, None) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 1 << 30, 1 << 60, 4, 64, 0, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(None, 10, 10, 4, 64, 0, 0, ctypes.byref(out)) == W.EINVAL
    # a sequence with no KV has no reclaimed share: both sides reject it
    for L in (0, 10):
        assert lib.wmtp_plan_memory(ctypes.byref(sh), L, 0, 4, 64, 0, 0, ctypes.byref(out)) == W.EINVAL
    assert lib.wmtp_plan_memory(ctypes.byref(sh), 10, 1, 4, 64, 0, 0, ctypes.byref(out)) == W.OK


def test_memory_plan_oracle_rejects_an_empty_sequence():
    import oracle as O
    for L in (0, 10):
        with pytest.raises(ValueError):
            O.memory_plan(2, 256, 2, L, 0, 4, 4096, 2, 1 << 40)
    one = O.memory_plan(2, 256, 2, 0, 1, 4, 4096, 2, 1 << 40)
    assert one["native_seq_bytes"] == 16 * 2 * 256 * 2 * 2 + 4      # one block of K and V, one table entry


def test_lengths_past_the_maximum_are_rejected():
    """Lengths near INT32_MAX would overflow the kernels' 32-bit position arithmetic and the
    planner's block count: every entry point that takes lengths or positions rejects anything past
    WMTP_MAX_SEQ_LEN (2^30) before any HIP call, and accepts the maximum itself."""
    lib = W.load()
    sh = shape()
    big, top = 2 ** 31 - 1, W.MAX_SEQ_LEN
    for n in (big, top + 1):
        assert lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(n), 1, 0, 0, 1, 0) == W.EINVAL
        assert lib.wmtp_draft_workspace_bytes(W.SINK_WINDOW, ctypes.byref(sh), lens(n), 1, 0, 4, 64, 0) == W.EINVAL
        assert lib.wmtp_verify_workspace_bytes(ctypes.byref(sh), 4, lens(n), 1, 0) == W.EINVAL
        kv = paged(mb=1 << 27)                                    # a table row long enough for any length
        assert draft(kv=kv, seq=(n,)) == W.EINVAL
        assert draft(mode=W.SINK_WINDOW, seq=(n,)) == W.EINVAL
        p = W.Partials()
        assert lib.wmtp_verify_attn(ctypes.byref(sh), FAKE, 4, ctypes.byref(kv), lens(n), 1, 0, FAKE, 1 << 40,
                                    ctypes.byref(p), None) == W.EINVAL
        assert lib.wmtp_ring_rollback(ctypes.byref(ring()), lens(n), 1, None) == W.EINVAL
        pos = lens(n - 1)
        assert lib.wmtp_ring_append(ctypes.byref(sh), ctypes.byref(ring()), FAKE, FAKE, pos, 1, 2, None) == W.EINVAL
        assert lib.wmtp_paged_append(ctypes.byref(sh), ctypes.byref(kv), FAKE, FAKE, pos, 1, 2, None) == W.EINVAL
    # the maximum itself plans
    assert lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(top), 1, 0, 0, 1, 0) > 0
    assert lib.wmtp_verify_workspace_bytes(ctypes.byref(sh), 4, lens(top), 1, 0) > 0


def test_binding_checks_buffers_before_the_call():
    """The binding passes raw pointers to the C ABI, so it checks sizes, dtypes and contiguity of the
    tensors first: a mis-sized buffer raises on the host instead of reaching a kernel."""
    sh = W.make_shape(16, 2, 256, torch.bfloat16, 1 / 16)
    p = W.Partials()
    p.batch, p.rows_per_seq, p.head_dim, p.total_splits = 2, 16, 256, 4
    with pytest.raises(ValueError, match="out"):
        W.combine(p, torch.empty((2, 15, 256)))                        # one row short
    with pytest.raises(ValueError, match="lse"):
        W.combine(p, torch.empty((2, 16, 256)), torch.empty((2, 17)))
    with pytest.raises(ValueError, match="dtype"):
        W.combine(p, torch.empty((2, 16, 256), dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        W.combine(p, torch.empty((2, 16, 256)))                        # right size, but host memory
    ws = torch.empty(1 << 12, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q"):
        W.draft_attn(W.FULL, sh, torch.empty((1, 8, 256), dtype=torch.bfloat16), [100], ws)
    with pytest.raises(ValueError, match="q"):
        W.verify_attn(sh, torch.empty((1, 3, 16, 256), dtype=torch.bfloat16), 4, W.Paged(), [100], ws)
    with pytest.raises(ValueError, match="contiguous"):
        W.draft_attn(W.FULL, sh, torch.empty((1, 256, 16), dtype=torch.bfloat16).transpose(1, 2), [100], ws)
    with pytest.raises(ValueError, match="k_new"):
        W.ring_append(sh, W.Ring(), torch.empty((1, 3, 2, 256)), torch.empty((1, 3, 2, 256)), [0])
    kr = torch.zeros((1, 2, 12, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="slots"):
        W.make_ring(kr, kr.clone(), torch.full((1, 12), -1, dtype=torch.int32), 4, 8, 1)   # 13 slots wanted
    with pytest.raises(ValueError, match="slot_pos"):
        W.make_ring(kr, kr.clone(), torch.full((1, 12), -1, dtype=torch.int64), 4, 8)
    with pytest.raises(ValueError, match="k, v"):
        W.make_ring(kr, torch.zeros((1, 2, 12, 128), dtype=torch.bfloat16), torch.full((1, 12), -1, dtype=torch.int32),
                    4, 8)


def test_descriptors_keep_their_tensors_alive():
    """A descriptor holds raw pointers; it must keep the tensors behind them alive, so that a
    block table or ring built inline is not freed (and its memory reused) while it is in use,
    and let them go with it."""
    import gc
    import weakref

    def pools():
        return torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)

    def table():
        return torch.zeros((1, 4), dtype=torch.int32)

    def tags():
        return torch.full((1, 12), -1, dtype=torch.int32)

    def ring_kv():
        return torch.zeros((1, 2, 12, 64), dtype=torch.bfloat16)

    builds = [
        lambda t: W.make_paged(t[0], t[1], t[2]),
        lambda t: W.make_paged_interleaved(t[0], t[1]),
        lambda t: W.make_ring(t[0], t[1], t[2], 4, 8),
        lambda t: W.with_policy(W.make_ring(t[0], t[1], t[2], 4, 8), [2], [8]),
    ]
    inputs = [
        lambda: (pools(), pools(), table()),
        lambda: (torch.zeros((4, 2, 2, 16, 64), dtype=torch.bfloat16), table()),
        lambda: (ring_kv(), ring_kv(), tags()),
        lambda: (ring_kv(), ring_kv(), tags()),
    ]
    for build, make_inputs in zip(builds, inputs):
        temporaries = make_inputs()
        refs = [weakref.ref(t) for t in temporaries]
        desc = build(temporaries)
        del temporaries
        gc.collect()
        assert all(r() is not None for r in refs)
        del desc
        gc.collect()
        assert all(r() is None for r in refs)



def test_noalloc_draft_checks_before_any_hip_call():
    """wmtp_draft_attn_noalloc runs every check of the draft and combine calls, and sizes its plan
    against the fixed scratch, before its first HIP call: each invalid call here returns on a
    machine without a GPU."""
    lib = W.load()
    sh = shape()
    kv, rg = paged(mb=1 << 17), ring()

    def call(mode=W.FULL | W.DRAFT_FAST_PV, q=FAKE, k_new=None, v_new=None, seq=(1000,), chunk=0, out=FAKE, lse=None,
             dt=W.F32, kvp=kv, rgp=rg):
        return lib.wmtp_draft_attn_noalloc(mode, ctypes.byref(sh), q, ctypes.byref(kvp) if kvp else None,
                                           ctypes.byref(rgp) if rgp else None, k_new, v_new, lens(*seq), len(seq),
                                           chunk, out, lse, dt, None)
    assert call(q=None) == W.EINVAL
    assert call(k_new=FAKE) == W.EINVAL                         # k_new without v_new
    assert call(out=None) == W.EINVAL
    assert call(out=FAKE_ODD) == W.EALIGN
    assert call(lse=FAKE + 2) == W.EALIGN
    assert call(dt=5) == W.EINVAL
    assert call(kvp=None) == W.EINVAL
    assert call(mode=W.SINK_WINDOW, rgp=None) == W.EINVAL
    assert call(seq=(2 ** 31 - 1,)) == W.EINVAL
    # 64-key splits over 1M keys: 16,384 splits x 16 rows x 1,028 bytes, past the 16 MiB scratch
    n = 1 << 20
    need = lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(n), 1, 64, 0, 1, 0)
    assert need > W.NOALLOC_SCRATCH_BYTES
    assert call(seq=(n,), chunk=64) == W.EWORKSPACE
    assert "scratch" in lib.wmtp_status_str(W.EWORKSPACE).decode()
    # the default splits at the same length fit
    assert lib.wmtp_draft_workspace_bytes(W.FULL, ctypes.byref(sh), lens(n), 1, 0, 0, 1, 0) <= W.NOALLOC_SCRATCH_BYTES
