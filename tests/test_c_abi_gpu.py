"""The C ABI from a plain C program, with no Python or torch in the call path.

tests/c_abi/decode_step.c (built by the build entry point into tests/c_abi/_bin/) reads
seeded inputs written here, runs one verify layer, one windowed draft step and one native
draft step (through the no-allocation call) on hipMalloc'd buffers with the library's C
calls only, and writes the outputs and three argument-error codes.  The outputs must match
the float64 oracle within the bf16 tolerance, and the error codes must be the documented ones.
The pool is filled with NaN wherever no context token is placed, so no kernel may depend on
rows it should not read.  The program runs as a child process (never an exec of this one).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_cases import TOL

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "_bin", "decode_step")
MAGIC = 0x574D5450
WMTP_EINVAL, WMTP_EALIGN, WMTP_EWORKSPACE = -1, -3, -4


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got.astype(np.float64) - ref).max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_decode_step_from_c(tmp_path):
    if not os.path.exists(BIN):
        raise RuntimeError(f"{BIN} is missing: run the build entry point (it builds the C program)")
    wl = synth.workload("draft_131k_bf16", window=256)
    Hq, Hk, D, S, Wn, R, tq, n0 = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.sink, wl.window, 2, 4, 1500
    seed = 61
    say("C ABI decode step", Hq, Hk, D, n0)
    k_ctx = synth.bf16_bits(synth.normal((n0, Hk, D), seed, "c_k_ctx", wl.kv_scale, "bf16"))
    v_ctx = synth.bf16_bits(synth.normal((n0, Hk, D), seed, "c_v_ctx", wl.kv_scale, "bf16"))
    q_v = synth.bf16_bits(synth.normal((tq, Hq, D), seed, "c_q_verify", 1.0, "bf16"))
    k_nv = synth.bf16_bits(synth.normal((tq, Hk, D), seed, "c_k_new_verify", wl.kv_scale, "bf16"))
    v_nv = synth.bf16_bits(synth.normal((tq, Hk, D), seed, "c_v_new_verify", wl.kv_scale, "bf16"))
    q_d = synth.bf16_bits(synth.normal((Hq, D), seed, "c_q_draft", 1.0, "bf16"))
    k_nd = synth.bf16_bits(synth.normal((Hk, D), seed, "c_k_new_draft", wl.kv_scale, "bf16"))
    v_nd = synth.bf16_bits(synth.normal((Hk, D), seed, "c_v_new_draft", wl.kv_scale, "bf16"))

    # K|V pool [blocks][H_kv][2][16][D] with a permuted block table; NaN (bf16 0x7fc0) elsewhere
    nb = synth.blocks_for(n0 + tq + 1, 16)
    bt, total = synth.block_table(seed, [nb], permuted=True, spare_blocks=2)
    pool = np.full((total, Hk, 2, 16, D), 0x7FC0, dtype=np.uint16)
    t = np.arange(n0)
    blk = bt[0, t // 16]
    pool[blk, :, 0, t % 16] = k_ctx
    pool[blk, :, 1, t % 16] = v_ctx

    header = np.array([MAGIC, Hq, Hk, D, tq, n0, total, bt.shape[1], S, Wn, R], dtype=np.int32)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(header.tobytes())
        f.write(np.float32(wl.scale).tobytes())
        for arr in (pool, bt[0].astype(np.int32), q_v, k_nv, v_nv, q_d, k_nd, v_nd, k_ctx, v_ctx):
            f.write(np.ascontiguousarray(arr).tobytes())
    r = subprocess.run([BIN, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, (r.returncode, r.stderr)

    raw = np.fromfile(outp, dtype=np.uint8)
    at = 0

    def take(count, dtype):
        nonlocal at
        n = count * np.dtype(dtype).itemsize
        x = raw[at:at + n].view(dtype)
        at += n
        return x

    out_v, lse_v = take(tq * Hq * D, np.float32).reshape(tq * Hq, D), take(tq * Hq, np.float32)
    out_w, lse_w = take(Hq * D, np.float32).reshape(Hq, D), take(Hq, np.float32)
    out_n, lse_n = take(Hq * D, np.float32).reshape(Hq, D), take(Hq, np.float32)
    errs = take(3, np.int32)
    assert at == raw.size
    assert list(errs) == [WMTP_EINVAL, WMTP_EALIGN, WMTP_EWORKSPACE], errs

    ctx_k, ctx_v = O.LogicalKV(k_ctx, "bf16", n0), O.LogicalKV(v_ctx, "bf16", n0)
    # verify: the t_q tokens appended at n0 .. n0 + t_q - 1
    sk = O.ConcatKV(ctx_k, O.LogicalKV(k_nv, "bf16"))
    sv = O.ConcatKV(ctx_v, O.LogicalKV(v_nv, "bf16"))
    o_ref, l_ref = O.verify_attention(O.to_f64(q_v, "bf16"), sk, sv, n0 + tq, wl.scale)
    ev = (max_err(out_v, o_ref.reshape(tq * Hq, D)), max_err(lse_v, l_ref.reshape(tq * Hq)))
    # windowed draft: the ring holds the context, the draft token at n0
    qd = O.to_f64(q_d, "bf16")
    sk = O.ConcatKV(ctx_k, O.LogicalKV(k_nd[None], "bf16"))
    sv = O.ConcatKV(ctx_v, O.LogicalKV(v_nd[None], "bf16"))
    o_ref, l_ref = O.draft_attention(qd, sk, sv, n0 + 1, O.SINK_WINDOW, S, Wn, wl.scale)
    ew = (max_err(out_w, o_ref), max_err(lse_w, l_ref))
    # native draft: the pool holds the context and the verify tokens, the draft token at n0 + t_q
    sk = O.ConcatKV(O.ConcatKV(ctx_k, O.LogicalKV(k_nv, "bf16")), O.LogicalKV(k_nd[None], "bf16"))
    sv = O.ConcatKV(O.ConcatKV(ctx_v, O.LogicalKV(v_nv, "bf16")), O.LogicalKV(v_nd[None], "bf16"))
    o_ref, l_ref = O.draft_attention(qd, sk, sv, n0 + tq + 1, O.FULL, S, Wn, wl.scale)
    en = (max_err(out_n, o_ref), max_err(lse_n, l_ref))
    say("errors verify / window / native", ev, ew, en)
    for e in (*ev, *ew, *en):
        assert e <= TOL["bf16"], (ev, ew, en)
