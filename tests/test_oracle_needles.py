"""Needle inputs make the million-key parity checks sensitive to the value rows a kernel reads.

With K, V ~ 0.5 N(0, 1), queries ~ N(0, 1) and scale 1/16 (the bf16 workloads), a
softmax over a million keys is nearly flat: every output element is an average
of about a million independent values, of order 1e-3.  A kernel that read half of
its value rows from the wrong blocks would still land within the 2e-3 max-abs
bar.  The needle recipe of `synth` (keys parallel to chosen query rows at seeded
positions, fresh values there) concentrates each row's softmax on a few dozen
known positions.  These CPU tests run the oracle at a million keys on both kinds
of input and show that the same wrong value reads that pass on flat inputs fail
by a wide margin on needle inputs: the full-size GPU checks can fail on V.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth

N = 1 << 20
D = 256
G = 8
PER_ROW = 32
SCALE = 1.0 / 16
TOL = 2e-3
BS = 16


class Remapped:
    """A K or V view that reads position src_of(p) wherever position p is asked for (a wrong address)."""

    def __init__(self, base, src_of):
        self.base, self.src_of, self.n, self.hk = base, src_of, base.n, base.hk

    def rows(self, positions, h):
        return self.base.rows(self.src_of(np.asarray(positions, dtype=np.int64)), h)


def swap_blocks(a, b):
    def src_of(p):
        blk = p // BS
        out = p.copy()
        out[blk == a] += (b - a) * BS
        out[blk == b] -= (b - a) * BS
        return out
    return src_of


def every_other_block_reads_the_next(p):
    """Half of the value rows come from the wrong block: even blocks read the following block."""
    out = p.copy()
    even = ((p // BS) % 2 == 0) & (p + BS < N)
    out[even] += BS
    return out


def make_inputs():
    k = synth.normal((N, 1, D), 11, "needle_pin_k", 0.5, "bf16")
    v = synth.normal((N, 1, D), 11, "needle_pin_v", 0.5, "bf16")
    q = synth.normal((G, D), 11, "needle_pin_q", 1.0, "bf16")
    flat = (synth.bf16_bits(k).copy(), synth.bf16_bits(v).copy())
    far = [3 * BS + 5, N - 7 * BS + 2]                         # one needle near each end of the context
    pos = synth.needle_positions(11, "pin", G * PER_ROW, 0, N, include=far)
    logits = synth.needle_logits(11, "pin", G * PER_ROW)
    kn = synth.needle_keys(q.repeat_interleave(PER_ROW, 0), logits, SCALE, "bf16")
    vn = synth.normal((G * PER_ROW, D), 11, "pin_v", 0.5, "bf16")
    k[torch.from_numpy(pos), 0] = kn
    v[torch.from_numpy(pos), 0] = vn
    needles = (synth.bf16_bits(k).copy(), synth.bf16_bits(v).copy())
    qf = O.to_f64(synth.bf16_bits(q), "bf16")
    return qf, flat, needles, pos, logits, far


@pytest.fixture(scope="module")
def inputs():
    return make_inputs()


def run(qf, kbits, vview_of):
    kv_k = O.LogicalKV(kbits, "bf16")
    return O.attention_over(qf, kv_k, vview_of, np.arange(N), 0, SCALE)


def test_needle_recipe(inputs):
    """Positions are distinct and in range, the forced ones first; every needle's scaled dot product
    with its query row lands on its target value (bf16 rounding of the key moves it by < 0.1)."""
    qf, _, (kb, _), pos, logits, far = inputs
    assert len(set(pos.tolist())) == len(pos) == G * PER_ROW
    assert pos.min() >= 0 and pos.max() < N and list(pos[:2]) == far
    keys = O.to_f64(kb[pos, 0], "bf16")
    rows = np.repeat(np.arange(G), PER_ROW)
    got = SCALE * np.einsum("jd,jd->j", qf[rows], keys)
    assert np.abs(got - logits.double().numpy()).max() < 0.1


def test_flat_inputs_cannot_see_half_of_the_values_read_wrong(inputs):
    """The weakness of the flat inputs: outputs of order 1e-3, and half the value rows from the wrong
    blocks still passes the 2e-3 bar."""
    qf, (kb, vb), _, _, _, _ = inputs
    vv = O.LogicalKV(vb, "bf16")
    o_ref, _ = run(qf, kb, vv)
    o_bad, _ = run(qf, kb, Remapped(vv, every_other_block_reads_the_next))
    assert np.abs(o_ref).max() < 3 * TOL
    assert np.abs(o_bad - o_ref).max() < TOL


def test_needle_inputs_fail_on_wrong_value_reads(inputs):
    """On needle inputs the outputs are of order 0.5, and each wrong value read the flat inputs let
    through, or a swap of two value blocks at the two ends of the context, moves them far past
    the 2e-3 bar."""
    qf, _, (kb, vb), pos, _, far = inputs
    vv = O.LogicalKV(vb, "bf16")
    o_ref, l_ref = run(qf, kb, vv)
    assert np.abs(o_ref).max() > 0.25
    assert l_ref.min() > 21.5 + np.log(PER_ROW) - 1.0          # the needles carry the mass
    o_half, _ = run(qf, kb, Remapped(vv, every_other_block_reads_the_next))
    assert np.abs(o_half - o_ref).max() > 25 * TOL
    o_swap, _ = run(qf, kb, Remapped(vv, swap_blocks(far[0] // BS, far[1] // BS)))
    assert np.abs(o_swap - o_ref).max() > 5 * TOL
