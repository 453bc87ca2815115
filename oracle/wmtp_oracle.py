"""Float64 CPU oracle for Windowed-MTP decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the HIP library: it has its own bfloat16 decoding, its own visible-set,
ring-slot and block-table arithmetic, and its own softmax.  Everything is plain
numpy in float64, written for readability, not speed.

Sources (the pages print no formulas or code; each function states the passage
it follows and the reading taken where the text is silent):

  [P1] "Does speculative decode still pay at 128K context?" (howtospark.com case
       study): Method (verify cycle = three draft forwards plus one batched
       verify), Findings (1 draft layer against 10 full-attention target layers,
       about 0.5 ms of draft cost per draft step), Limitations (the technique
       is a sliding window plus attention sink on the draft's attention).
  [P2] "Your Million-Token Pipeline Is Bleeding Speed You Don't Know You're
       Losing" (readpriors.com): What happened (the native draft reads the whole
       cache at every draft step; the windowed draft keeps a constant working
       set that leaves out about 99% of entries at 1M; Figure 3's cost-side ratio).
  [P3] "Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
       Context" (arxivlens.com summary): Abstract (gamma draft forwards per
       decode step, window plus sink on the draft only, full-context target
       verification, compact ring buffer).

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * a draft step appends its own new entry, then attends over it (causal decode);
  * the window holds the W most recent entries including the current one, the
    sinks are absolute positions 0..S-1, and the two sets are unioned;
  * the ring has S+W+R slots, slot(p) = p for p < S, else S + (p - S) mod (W+R),
    where R >= 0 headroom slots absorb drafted tokens that verification
    rejects (R >= gamma - 1 keeps every entry a later window needs);
  * rejected drafted tokens are forgotten by clearing the tags of positions at
    or past the accepted length; a re-append at the same position overwrites;
  * adaptive windows and dynamic sinks (named as future work) are per-sequence
    S_b <= S and W_b <= W + R read from the ring laid out for (S, W, R), so a
    sequence may change them between steps without moving any entry;
  * query head h reads KV head h // G (consecutive query heads share a KV head);
  * the softmax scale is 1/sqrt(D);
  * the paged pool is laid out [block][kv_head][block_offset][D], or, with K and
    V of a (block, head) side by side, [block][kv_head][K|V][block_offset][D]:
    (block, head) runs of block_size rows that lie run_rows rows apart.

Parity pins for every function live in tests/test_oracle_*.py; none of them
re-types a formula from this file.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

FULL = 0
SINK_WINDOW = 1

# --------------------------------------------------------------------------- numbers
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64.

    A bfloat16 value is, by definition, the upper 16 bits of an IEEE-754
    binary32 value; widening puts the pattern back in the upper half and zero
    in the lower half.  binary32 -> binary64 is exact.
    """
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):       # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of an input tensor given as f32 values or bf16 bits."""
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- windowing
def visible_positions(n: int, mode: int, sink: int = 0, window: int = 0) -> np.ndarray:
    """Positions a draft query at length n attends to (ascending).

    [P2 What happened; P3 Abstract]: the native draft reads the whole cache;
    the windowed draft reads the attention-sink tokens plus a sliding window of
    recent tokens.  Reading: sinks = positions 0..S-1, window = the W most
    recent positions n-W..n-1 (the current token included); the union is taken
    without double counting.
    """
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    if mode == FULL:
        return np.arange(n, dtype=np.int64)
    if mode != SINK_WINDOW:
        raise ValueError(mode)
    sinks = set(range(min(sink, n)))
    recent = set(range(max(0, n - window), n))
    return np.array(sorted(sinks | recent), dtype=np.int64)


def draft_entries_read(n: int, mode: int, sink: int = 0, window: int = 0) -> int:
    """Number of KV entries (per KV head) one draft step reads at length n."""
    return int(len(visible_positions(n, mode, sink, window)))


# --------------------------------------------------------------------------- ring
def ring_slot(p: int, sink: int, window: int, headroom: int = 0) -> int:
    """Slot of absolute position p in the compact ring of S + W + R slots.

    [P3 Abstract] names a compact ring buffer holding the draft's window but
    gives no layout; the one taken here: sinks occupy slots 0..S-1 in place, every
    later position cycles through the C = W + R slots S..S+C-1.  R >= 0 extra
    slots ("headroom") let drafted tokens that verification rejects be written
    without overwriting an entry that a later window still needs.
    """
    if p < 0:
        raise ValueError("negative position")
    if p < sink:
        return int(p)
    return int(sink + (p - sink) % (window + headroom))


def ring_append(tags: np.ndarray, pos: int, count: int, sink: int, window: int,
                headroom: int = 0) -> List[Tuple[int, int]]:
    """Apply an append of `count` tokens at positions pos..pos+count-1 to `tags`.

    tags[slot] holds the absolute position stored in the slot (-1 = empty).
    Returns the (token index, slot) writes in order.  A token is stored only if
    it survives the append: p < S, or p among the C = W + R most recent
    positions of this append.  That keeps an append of more than C tokens
    deterministic (no slot is written twice) and equal to appending the tokens
    one by one.
    """
    last = pos + count - 1
    cycle = window + headroom
    writes = []
    for i in range(count):
        p = pos + i
        if p < sink or p > last - cycle:
            s = ring_slot(p, sink, window, headroom)
            tags[s] = p
            writes.append((i, s))
    return writes


def ring_rollback(tags: np.ndarray, n: int) -> List[int]:
    """Forget every entry at a position >= n (drafted tokens that were not
    accepted): their tags become -1.  Returns the cleared slots."""
    cleared = [int(s) for s in np.nonzero(tags >= n)[0]]
    tags[tags >= n] = -1
    return cleared


def ring_expected_tags(n: int, sink: int, window: int, headroom: int = 0) -> np.ndarray:
    """Tag of every slot (-1 = empty) after positions 0..n-1 were appended in order."""
    tags = np.full(sink + window + headroom, -1, dtype=np.int64)
    for p in range(n):
        tags[ring_slot(p, sink, window, headroom)] = p
    return tags


def window_slot_positions(n: int, sink: int, window: int, headroom: int = 0) -> np.ndarray:
    """For each ring slot, the position it must hold for a query at length n (-1 if none).

    This is the sink_window visible set placed in ring order.
    """
    out = np.full(sink + window + headroom, -1, dtype=np.int64)
    for p in visible_positions(n, SINK_WINDOW, sink, window):
        out[ring_slot(int(p), sink, window, headroom)] = p
    return out


def ring_visible(tags: np.ndarray, n: int, sink: int, window: int) -> np.ndarray:
    """Per slot, the position a draft query at length n reads there (-1 = masked):
    the slot's tag if that position is in the sink_window visible set."""
    vis = set(int(p) for p in visible_positions(n, SINK_WINDOW, sink, window))
    return np.array([int(t) if int(t) in vis else -1 for t in tags], dtype=np.int64)


# --------------------------------------------------------------------------- paging
def paged_element_offset(block_table_row: Sequence[int], t: int, h: int, num_kv_heads: int,
                         block_size: int, head_dim: int, run_rows: Optional[int] = None) -> int:
    """Element offset of (token t, KV head h, d=0) in a paged pool.

    Reading of the layout: the pool is a sequence of (block, kv_head) runs of
    block_size token rows, run_rows rows apart (run_rows = block_size:
    pool[block][kv_head][block_offset][D]); the token's block is
    block_table_row[t // block_size] and its row in the run t % block_size.
    Plain Python integers, so offsets beyond 2**31 are exact.
    """
    run_rows = block_size if run_rows is None else int(run_rows)
    blk = int(block_table_row[t // block_size])
    off = t % block_size
    return ((blk * num_kv_heads + h) * run_rows + off) * head_dim


class LogicalKV:
    """K or V tokens in position order: array [n][H_kv][D] (f32 values or bf16 bits)."""

    def __init__(self, arr: np.ndarray, dtype: str, n: Optional[int] = None):
        self.arr, self.dtype = arr, dtype
        self.n = arr.shape[0] if n is None else int(n)
        self.hk = arr.shape[1]

    def rows(self, positions: np.ndarray, h: int) -> np.ndarray:
        return to_f64(self.arr[positions, h, :], self.dtype)


class PagedKV:
    """K or V of one sequence read through a block table from a paged pool.

    pool: [num_blocks][H_kv][block_size][D] (f32 values or bf16 bits), or the
    K|V pool [num_blocks][H_kv][2][block_size][D] with part = 0 (K) or 1 (V).
    Each position is resolved with `paged_element_offset` on a flat view.
    """

    def __init__(self, pool: np.ndarray, block_table_row: Sequence[int], block_size: int, dtype: str, n: int,
                 part: Optional[int] = None):
        self.flat = pool.reshape(-1)
        self.hk, self.d = pool.shape[1], pool.shape[-1]
        self.bt = [int(x) for x in block_table_row]
        self.bs, self.dtype, self.n = int(block_size), dtype, int(n)
        if pool.ndim == 5:                       # K|V runs: 2 * block_size rows apart, V after K
            assert part in (0, 1)
            self.run_rows, self.base = 2 * self.bs, part * self.bs * self.d
        else:
            self.run_rows, self.base = self.bs, 0

    def rows(self, positions: np.ndarray, h: int) -> np.ndarray:
        offs = np.fromiter((self.base + paged_element_offset(self.bt, int(t), h, self.hk, self.bs, self.d,
                                                             self.run_rows)
                            for t in positions), dtype=np.int64, count=len(positions))
        idx = offs[:, None] + np.arange(self.d, dtype=np.int64)[None, :]
        return to_f64(self.flat[idx], self.dtype)


class ConcatKV:
    """Positions 0..a.n-1 from `a`, then `b` (the tokens appended by this step)."""

    def __init__(self, a, b):
        self.a, self.b, self.n, self.hk = a, b, a.n + b.n, a.hk

    def rows(self, positions: np.ndarray, h: int) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        lo = positions < self.a.n
        parts = []
        if lo.any():
            parts.append((np.nonzero(lo)[0], self.a.rows(positions[lo], h)))
        if (~lo).any():
            parts.append((np.nonzero(~lo)[0], self.b.rows(positions[~lo] - self.a.n, h)))
        d = parts[0][1].shape[1]
        out = np.empty((len(positions), d))
        for idx, vals in parts:
            out[idx] = vals
        return out


# --------------------------------------------------------------------------- attention
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows q [R][D] over keys k [n][D], values v [n][D].

    s = scale * q k^T; o = softmax(s) v row by row; lse = log sum exp(s).
    The row maximum is subtracted before exponentiating (this changes no
    value, only the range).  n = 0 gives o = 0 and lse = -inf.
    """
    R, D = q.shape
    if k.shape[0] == 0:
        return np.zeros((R, v.shape[1])), np.full(R, -np.inf)
    s = (q @ k.T) * scale
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    l = w.sum(axis=1)
    o = (w @ v) / l[:, None]
    return o, m + np.log(l)


def attention_over(q: np.ndarray, kv_k, kv_v, positions: np.ndarray, h: int, scale: float,
                   chunk: int = 1 << 16) -> Tuple[np.ndarray, np.ndarray]:
    """softmax_attention over the listed positions of a (possibly huge) KV source.

    Two passes over the positions in chunks, only to bound memory: the first
    gathers every score and the row maximum, the second sums the weights and
    the weighted values.  Plain accumulation, no partial-softmax merging.
    """
    R = q.shape[0]
    n = len(positions)
    if n == 0:
        return np.zeros((R, q.shape[1])), np.full(R, -np.inf)
    if n <= chunk:
        return softmax_attention(q, kv_k.rows(positions, h), kv_v.rows(positions, h), scale)
    s = np.empty((R, n))
    for i in range(0, n, chunk):
        s[:, i:i + chunk] = (q @ kv_k.rows(positions[i:i + chunk], h).T) * scale
    m = s.max(axis=1)
    l = np.zeros(R)
    acc = np.zeros((R, q.shape[1]))
    for i in range(0, n, chunk):
        w = np.exp(s[:, i:i + chunk] - m[:, None])
        l += w.sum(axis=1)
        acc += w @ kv_v.rows(positions[i:i + chunk], h)
    return acc / l[:, None], m + np.log(l)


def draft_attention(q: np.ndarray, kv_k, kv_v, n: int, mode: int, sink: int, window: int,
                    scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One draft step of one sequence: q [H_q][D] (float64) at length n.

    [P2 What happened; P3 Abstract]: full mode attends to every cached entry,
    sink_window to the sinks plus the recent window.  Query head h uses KV head
    h // G.  Returns o [H_q][D] and lse [H_q] (natural log).
    """
    Hq, D = q.shape
    Hk = kv_k.hk
    G = Hq // Hk
    pos = visible_positions(n, mode, sink, window)
    o = np.empty((Hq, D))
    lse = np.empty(Hq)
    for h in range(Hk):
        oh, lh = attention_over(q[h * G:(h + 1) * G], kv_k, kv_v, pos, h, scale)
        o[h * G:(h + 1) * G] = oh
        lse[h * G:(h + 1) * G] = lh
    return o, lse


def verify_attention(q: np.ndarray, kv_k, kv_v, n: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Target verify attention of one sequence and one layer.

    q [T][H_q][D] are the T = gamma+1 query tokens at positions n-T..n-1 (their
    keys are already in the cache, so the cache length is n).  [P3 Abstract]:
    the target's attention stays over the full context.  Causal reading: query
    token i sees positions 0..n-T+i.  Returns o [T][H_q][D], lse [T][H_q].
    """
    T, Hq, D = q.shape
    o = np.empty((T, Hq, D))
    lse = np.empty((T, Hq))
    for i in range(T):
        o[i], lse[i] = draft_attention(q[i], kv_k, kv_v, n - T + i + 1, FULL, 0, 0, scale)
    return o, lse


# --------------------------------------------------------------------------- combine
def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Merge attention results over disjoint key sets into the result over their union.

    o_parts [P][R][D], lse_parts [P][R].  Each part's weight is its share of
    the total exponential mass: exp(lse_i - L), L = log sum_i exp(lse_i).
    Parts with lse = -inf (no keys) carry no mass and are skipped.
    """
    P, R, D = o_parts.shape
    o = np.zeros((R, D))
    lse = np.full(R, -np.inf)
    for r in range(R):
        live = [i for i in range(P) if np.isfinite(lse_parts[i, r])]
        if not live:
            continue
        m = max(lse_parts[i, r] for i in live)
        total = sum(math.exp(lse_parts[i, r] - m) for i in live)
        L = m + math.log(total)
        for i in live:
            o[r] += math.exp(lse_parts[i, r] - L) * o_parts[i, r]
        lse[r] = L
    return o, lse


# --------------------------------------------------------------------------- cost model
def step_kv_bytes(n0: int, gamma: int, target_layers: int, num_kv_heads: int, head_dim: int,
                  elem_bytes: int, mode: int, sink: int = 0, window: int = 0,
                  draft_layers: int = 1) -> int:
    """K+V bytes one decode step reads in its attention.

    [P1 Method] one verify cycle is gamma draft forwards plus one batched
    verify; [P1 Findings] the draft is one layer and the target re-reads its
    full-attention layers.  Draft step j (1-based) attends at length n0+j; the
    verify of each target layer reads n0+gamma+1 tokens (its own appended
    queries included).
    """
    per_tok = 2 * num_kv_heads * head_dim * elem_bytes
    draft = sum(draft_entries_read(n0 + j, mode, sink, window) for j in range(1, gamma + 1))
    verify = target_layers * (n0 + gamma + 1)
    return per_tok * (draft_layers * draft + verify)


# --------------------------------------------------------------------------- memory accounting
def memory_plan(num_kv_heads: int, head_dim: int, elem_bytes: int, target_layers: int, context: int,
                sink: int, window: int, headroom: int, budget_bytes: int, block_size: int = 16) -> dict:
    """KV memory of one sequence with a native or a windowed draft, and how many fit a budget.

    [P3 Abstract] the window leaves most of the draft's KV unread and a compact
    ring buffer turns that into capacity: the draft's full pool, which nothing
    reads any more, is freed (7.7-11.1% of total KV at 1M), room for one more
    concurrent 1M request.
    Reading: every full-attention layer, target or native draft, keeps a paged
    pool of ceil(context / block_size) blocks of K and V; one int32 block table
    per sequence serves all of them; the windowed draft keeps only its ring
    (S + W + R slots of K and V plus an int32 tag per slot).  The reclaimed
    share is a fraction of the sequence's KV, so a sequence must hold some:
    context >= 1, else ValueError.
    """
    if context < 1:
        raise ValueError("the reclaimed share is defined for a context of at least one token")
    blocks = -(-context // block_size)
    layer = blocks * block_size * num_kv_heads * head_dim * elem_bytes * 2
    table = blocks * 4
    ring = (sink + window + headroom) * (num_kv_heads * head_dim * elem_bytes * 2 + 4)
    target = target_layers * layer
    native = target + layer + table
    windowed = target + ring + table
    return {
        "layer_bytes": layer, "block_table_bytes": table, "ring_bytes": ring,
        "native_seq_bytes": native, "windowed_seq_bytes": windowed,
        "reclaimed_fraction": (native - windowed) / native,
        "native_sequences": budget_bytes // native,
        "windowed_sequences": budget_bytes // windowed,
    }

