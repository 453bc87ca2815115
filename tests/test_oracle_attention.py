"""Pins for the oracle's attention (no GPU).

The oracle is checked against (a) explicit triple loops with no max
subtraction, (b) torch's CPU float64 softmax / scaled_dot_product_attention
(library routines), and (c) closed forms.  GQA uses torch's repeat_interleave,
so a wrong query-head -> KV-head mapping fails here.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _brute(q, k, v, scale):
    """Explicit loops: exp of raw scores, no max subtraction (tiny inputs only)."""
    R, D = q.shape
    n = k.shape[0]
    o = np.zeros((R, v.shape[1]))
    lse = np.zeros(R)
    for r in range(R):
        e = []
        for t in range(n):
            s = 0.0
            for d in range(D):
                s += q[r, d] * k[t, d]
            e.append(math.exp(s * scale))
        tot = sum(e)
        for t in range(n):
            for d in range(v.shape[1]):
                o[r, d] += e[t] * v[t, d] / tot
        lse[r] = math.log(tot)
    return o, lse


@pytest.mark.parametrize("R,n,D", [(1, 1, 4), (3, 5, 8), (4, 17, 16), (8, 64, 16)])
def test_softmax_attention_equals_explicit_loops(R, n, D):
    rng = np.random.default_rng(R * 100 + n)
    q, k, v = _rand(rng, R, D), _rand(rng, n, D), _rand(rng, n, D)
    o, lse = O.softmax_attention(q, k, v, 1 / math.sqrt(D))
    ob, lb = _brute(q, k, v, 1 / math.sqrt(D))
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12


def _torch_gqa(q_hd, k_thd, v_thd, scale):
    """torch float64 reference: repeat each KV head G times (MHA), softmax, matmul."""
    Hq = q_hd.shape[0]
    Hk = k_thd.shape[1]
    G = Hq // Hk
    q = torch.from_numpy(q_hd)                               # [Hq][D]
    k = torch.from_numpy(k_thd).repeat_interleave(G, dim=1)  # [n][Hq][D]
    v = torch.from_numpy(v_thd).repeat_interleave(G, dim=1)
    s = torch.einsum("hd,nhd->hn", q, k) * scale
    o = torch.einsum("hn,nhd->hd", torch.softmax(s, dim=-1), v)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("Hq,Hk,n,D", [(4, 1, 33, 16), (8, 2, 50, 8), (16, 2, 40, 32), (6, 6, 9, 4)])
def test_draft_full_equals_torch_gqa(Hq, Hk, n, D):
    rng = np.random.default_rng(Hq * 7 + n)
    q = _rand(rng, Hq, D)
    k = _rand(rng, n, Hk, D, scale=0.5).astype(np.float32)
    v = _rand(rng, n, Hk, D, scale=0.5).astype(np.float32)
    src_k, src_v = O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32")
    o, lse = O.draft_attention(q, src_k, src_v, n, O.FULL, 0, 0, 1 / math.sqrt(D))
    ot, lt = _torch_gqa(q, k.astype(np.float64), v.astype(np.float64), 1 / math.sqrt(D))
    assert np.max(np.abs(o - ot)) < 1e-12
    assert np.max(np.abs(lse - lt)) < 1e-12


def test_draft_full_equals_torch_sdpa():
    rng = np.random.default_rng(5)
    Hq, Hk, n, D = 8, 2, 70, 16
    q = _rand(rng, Hq, D)
    k = _rand(rng, n, Hk, D).astype(np.float32)
    v = _rand(rng, n, Hk, D).astype(np.float32)
    o, _ = O.draft_attention(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), n, O.FULL, 0, 0, 0.3)
    G = Hq // Hk
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, 1).permute(1, 0, 2)  # [Hq][n][D]
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, 1).permute(1, 0, 2)
    qt = torch.from_numpy(q)[:, None, :]
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.3)[:, 0, :].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_closed_form_single_token():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 3, 8), _rand(rng, 1, 8), _rand(rng, 1, 8)
    o, lse = O.softmax_attention(q, k, v, 0.25)
    assert np.array_equal(o, np.repeat(v, 3, axis=0))
    assert np.allclose(lse, 0.25 * (q @ k[0]), atol=1e-15, rtol=0)


def test_closed_form_constant_values_and_identical_keys():
    rng = np.random.default_rng(2)
    n, D = 37, 8
    q = _rand(rng, 4, D)
    k = _rand(rng, n, D)
    v = np.tile(_rand(rng, 1, D), (n, 1))
    o, _ = O.softmax_attention(q, k, v, 0.5)
    assert np.max(np.abs(o - v[0])) < 1e-14
    k_same = np.tile(_rand(rng, 1, D), (n, 1))
    v2 = _rand(rng, n, D)
    o2, lse2 = O.softmax_attention(q, k_same, v2, 0.5)
    assert np.max(np.abs(o2 - v2.mean(axis=0))) < 1e-14
    assert np.max(np.abs(lse2 - (0.5 * (q @ k_same[0]) + math.log(n)))) < 1e-12


def test_empty_key_set():
    o, lse = O.softmax_attention(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_chunked_two_pass_equals_single_pass():
    rng = np.random.default_rng(3)
    n, Hk, D = 1000, 2, 16
    k = _rand(rng, n, Hk, D).astype(np.float32)
    v = _rand(rng, n, Hk, D).astype(np.float32)
    q = _rand(rng, 4, D)
    pos = np.arange(n)
    a = O.attention_over(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), pos, 1, 0.25, chunk=97)
    b = O.softmax_attention(q, k[:, 1].astype(np.float64), v[:, 1].astype(np.float64), 0.25)
    assert np.max(np.abs(a[0] - b[0])) < 1e-13 and np.max(np.abs(a[1] - b[1])) < 1e-12


def _causal_torch(q_thd, k_nhd, v_nhd, scale):
    """torch float64 reference for verify: explicit bottom-right causal mask."""
    T, Hq, D = q_thd.shape
    n, Hk, _ = k_nhd.shape
    G = Hq // Hk
    k = torch.from_numpy(k_nhd).repeat_interleave(G, 1)
    v = torch.from_numpy(v_nhd).repeat_interleave(G, 1)
    q = torch.from_numpy(q_thd)
    s = torch.einsum("thd,nhd->thn", q, k) * scale
    allowed = torch.arange(n)[None, :] <= (n - T + torch.arange(T))[:, None]   # [T][n]
    s = s.masked_fill(~allowed[:, None, :], float("-inf"))
    return torch.einsum("thn,nhd->thd", torch.softmax(s, -1), v).numpy(), torch.logsumexp(s, -1).numpy()


@pytest.mark.parametrize("T", [1, 2, 4])
def test_verify_equals_causal_torch(T):
    rng = np.random.default_rng(10 + T)
    n, Hq, Hk, D = 45, 8, 2, 16
    q = _rand(rng, T, Hq, D)
    k = _rand(rng, n, Hk, D).astype(np.float32)
    v = _rand(rng, n, Hk, D).astype(np.float32)
    o, lse = O.verify_attention(q, O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32"), n, 0.25)
    ot, lt = _causal_torch(q, k.astype(np.float64), v.astype(np.float64), 0.25)
    assert np.max(np.abs(o - ot)) < 1e-12 and np.max(np.abs(lse - lt)) < 1e-12


def test_verify_single_query_is_a_full_draft_step():
    rng = np.random.default_rng(4)
    n, Hq, Hk, D = 30, 4, 2, 8
    q = _rand(rng, 1, Hq, D)
    k = _rand(rng, n, Hk, D).astype(np.float32)
    v = _rand(rng, n, Hk, D).astype(np.float32)
    kk, vv = O.LogicalKV(k, "f32"), O.LogicalKV(v, "f32")
    o, lse = O.verify_attention(q, kk, vv, n, 0.3)
    od, ld = O.draft_attention(q[0], kk, vv, n, O.FULL, 0, 0, 0.3)
    assert np.array_equal(o[0], od) and np.array_equal(lse[0], ld)


def test_concat_source_appends_after_context():
    rng = np.random.default_rng(6)
    a = _rand(rng, 10, 2, 4).astype(np.float32)
    b = _rand(rng, 3, 2, 4).astype(np.float32)
    src = O.ConcatKV(O.LogicalKV(a, "f32"), O.LogicalKV(b, "f32"))
    allk = np.concatenate([a, b]).astype(np.float64)
    pos = np.array([12, 0, 9, 10, 11, 3])
    assert np.array_equal(src.rows(pos, 1), allk[pos, 1])
