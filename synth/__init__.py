"""Seeded synthetic inputs for Windowed-MTP decode attention.

This module only draws inputs: query, key and value tensors, paged-pool
contents, block tables and ring positions.  Both sides of every parity check
(the float64 oracle under ``oracle/`` and the HIP library) consume exactly the
tensors produced here.  No attention, softmax, windowing, ring-slot or paging
arithmetic lives in this module: resolving a position to a slot or an address
is done independently by each side.

Recipe (the pages fix none of it; they describe real prompts of 2K-131K tokens
and a 1M-token context):
  * values are N(0, 1) float32 samples, multiplied by a per-tensor scale (0.5
    for keys and values in the bf16 workloads), then rounded to bfloat16 with
    round-to-nearest-even where the workload is bf16;
  * every tensor has its own stream, derived from (seed, stream id), so adding a
    tensor never changes another one;
  * a block table is a seeded random permutation of the physical block ids,
    split into consecutive runs, one per sequence;
  * small cases are drawn on the CPU; the multi-GiB paged pools of the 1M-token
    workloads are drawn on the GPU with torch's counter-based generator;
  * "needles" give a long context structure a parity check can see: at seeded
    positions, keys parallel to chosen query rows (scaled so that the row's
    scaled dot product with its key is a seeded value in [21.5, 22.5]) and
    freshly drawn values.  Each such row's softmax then rests on its few dozen
    needles instead of spreading evenly over a million keys, so its output is
    of order one and changes if any of those value rows is read from the
    wrong place.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "stream_seed", "normal", "block_table",
    "blocks_for", "bf16_bits", "DraftCase", "draft_case", "VerifyCase", "verify_case",
    "needle_positions", "needle_logits", "needle_keys", "NEEDLE_LOGITS",
]


# --------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (sizes only, no arithmetic)."""
    name: str
    contexts: Tuple[int, ...]          # n0 per sequence, before the step's appends
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                          # "f32" or "bf16": q, k and v element type
    sink: int
    window: int
    gamma: int = 3
    kv_scale: float = 1.0               # keys and values are multiplied by this
    block_size: int = 16
    paged: bool = True                  # full-mode draft reads a paged pool
    permuted: bool = True               # block table is a random permutation
    chunk_tokens: int = 256             # split size of the split-K kernels
    target_layers: int = 0              # full-attention target layers verified per step
    windows: Tuple[int, ...] = ()       # extra window sizes swept (mixed batch)
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.contexts)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(self.head_dim) ** -0.5


WORKLOADS = {
    # 1 sequence, 1 layer, 4,096 tokens, 4 query heads on 1 KV head, d=64, fp32.
    "tiny_fp32_4k": Workload(
        "tiny_fp32_4k", (4096,), 4, 1, 64, "f32", sink=4, window=256,
        paged=False, permuted=False, chunk_tokens=256, seed=0),
    # 1 draft layer, 131,072 tokens, 16 query / 2 KV heads, d=256, bf16, K/V x 0.5.
    "draft_131k_bf16": Workload(
        "draft_131k_bf16", (131072,), 16, 2, 256, "bf16", sink=4, window=4096,
        kv_scale=0.5, paged=False, permuted=False, chunk_tokens=256, seed=1),
    # Paged pool at 1,048,576 tokens, 16-token blocks in a random permutation.
    "paged_1m_bf16": Workload(
        "paged_1m_bf16", (1048576,), 16, 2, 256, "bf16", sink=4, window=4096,
        kv_scale=0.5, chunk_tokens=256, seed=2),
    # Per-decode-step cost model at 1M: 10 verify layers + 1 draft layer x gamma.
    "step_1m_bf16": Workload(
        "step_1m_bf16", (1048576,), 16, 2, 256, "bf16", sink=4, window=4096,
        kv_scale=0.5, chunk_tokens=256, target_layers=10, seed=3),
    # 4 sequences of mixed length, paged, load-balanced split-K.
    "mixed_4seq_bf16": Workload(
        "mixed_4seq_bf16", (32768, 131072, 524288, 1048576), 16, 2, 256, "bf16",
        sink=4, window=4096, kv_scale=0.5, chunk_tokens=256,
        windows=(1024, 4096, 16384), seed=4),
}


def workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (e.g. smaller contexts)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


# --------------------------------------------------------------------------- generators
def stream_seed(seed: int, *stream) -> int:
    """A 63-bit seed for the named stream of a workload seed (stable across runs)."""
    h = hashlib.sha256(repr((int(seed),) + tuple(stream)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal(shape: Sequence[int], seed: int, stream, scale: float = 1.0,
           dtype: str = "f32", device: str = "cpu") -> torch.Tensor:
    """N(0,1) float32 samples times ``scale``, cast to ``dtype`` (bf16: RNE)."""
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, *(stream if isinstance(stream, tuple) else (stream,))))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(_torch_dtype(dtype))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bfloat16 tensor, as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def blocks_for(tokens: int, block_size: int) -> int:
    return -(-int(tokens) // int(block_size))


def block_table(seed: int, blocks_per_seq: Sequence[int], permuted: bool = True,
                spare_blocks: int = 0) -> Tuple[np.ndarray, int]:
    """A block table [batch][max_blocks] (int32) and the physical pool size.

    The physical ids 0..P-1 (P = sum(blocks_per_seq) + spare_blocks) are
    shuffled with a seeded permutation and handed out in consecutive runs,
    one run per sequence.  Unused tail entries of a row hold 0 (a valid id).
    """
    total = int(sum(blocks_per_seq)) + int(spare_blocks)
    if permuted:
        ids = np.random.default_rng(stream_seed(seed, "block_table")).permutation(total)
    else:
        ids = np.arange(total)
    width = max(1, max(blocks_per_seq))
    bt = np.zeros((len(blocks_per_seq), width), dtype=np.int32)
    at = 0
    for b, nb in enumerate(blocks_per_seq):
        bt[b, :nb] = ids[at:at + nb]
        at += nb
    return bt, total


# --------------------------------------------------------------------------- needles
NEEDLE_LOGITS = (21.5, 22.5)


def needle_positions(seed: int, stream, count: int, lo: int, hi: int,
                     include: Sequence[int] = ()) -> np.ndarray:
    """`count` distinct positions in [lo, hi): the `include` positions first (in order, duplicates
    dropped), then seeded uniform draws without replacement from the rest."""
    stream = stream if isinstance(stream, tuple) else (stream,)
    first = list(dict.fromkeys(int(p) for p in include))
    if len(first) > count or any(not lo <= p < hi for p in first) or count > hi - lo:
        raise ValueError("needle positions do not fit the range")
    rng = np.random.default_rng(stream_seed(seed, "needle_positions", *stream))
    taken = set(first)
    out = list(first)
    while len(out) < count:
        for p in rng.integers(lo, hi, size=2 * (count - len(out)) + 8):
            p = int(p)
            if p not in taken:
                taken.add(p)
                out.append(p)
                if len(out) == count:
                    break
    return np.asarray(out, dtype=np.int64)


def needle_logits(seed: int, stream, count: int) -> torch.Tensor:
    """Seeded target values of scale * q.k for `count` needles, uniform in NEEDLE_LOGITS (float32)."""
    stream = stream if isinstance(stream, tuple) else (stream,)
    g = torch.Generator()
    g.manual_seed(stream_seed(seed, "needle_logits", *stream))
    lo, hi = NEEDLE_LOGITS
    return lo + (hi - lo) * torch.rand(count, generator=g, dtype=torch.float32)


def needle_keys(q_rows: torch.Tensor, logits: torch.Tensor, scale: float, dtype: str) -> torch.Tensor:
    """Key rows parallel to query rows: row j is c_j * q_rows[j] with c_j = logits[j] / (scale |q_j|^2),
    so scale * q_j . key_j is logits[j] before the key is rounded to `dtype` (bf16: RNE)."""
    qf = q_rows.float()
    c = logits.to(qf.device).float() / (scale * (qf * qf).sum(dim=-1))
    return (c[:, None] * qf).to(_torch_dtype(dtype))


# --------------------------------------------------------------------------- cases
@dataclasses.dataclass
class DraftCase:
    """Inputs of gamma draft steps over one context.

    ``k_ctx``/``v_ctx`` hold the context tokens in position order,
    [batch][n0_max][H_kv][D] (only the first n0[b] rows of sequence b are
    meaningful).  Step j (0-based) appends ``k_new[j]``/``v_new[j]``
    ([batch][1][H_kv][D]) at position n0[b]+j and then queries with ``q[j]``
    ([batch][H_q][D]); the query attends over n0[b]+j+1 tokens.
    """
    wl: Workload
    n0: Tuple[int, ...]
    q: torch.Tensor
    k_ctx: torch.Tensor
    v_ctx: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor


def draft_case(wl: Workload, contexts: Optional[Sequence[int]] = None,
               device: str = "cpu", seed: Optional[int] = None) -> DraftCase:
    seed = wl.seed if seed is None else seed
    n0 = tuple(int(c) for c in (contexts if contexts is not None else wl.contexts))
    B, Hq, Hk, D, G = len(n0), wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma
    nmax = max(n0) if n0 else 0
    q = normal((G, B, Hq, D), seed, "q_draft", 1.0, wl.dtype, device)
    k_ctx = normal((B, nmax, Hk, D), seed, "k_ctx", wl.kv_scale, wl.dtype, device)
    v_ctx = normal((B, nmax, Hk, D), seed, "v_ctx", wl.kv_scale, wl.dtype, device)
    k_new = normal((G, B, 1, Hk, D), seed, "k_new", wl.kv_scale, wl.dtype, device)
    v_new = normal((G, B, 1, Hk, D), seed, "v_new", wl.kv_scale, wl.dtype, device)
    return DraftCase(wl, n0, q, k_ctx, v_ctx, k_new, v_new)


@dataclasses.dataclass
class VerifyCase:
    """Inputs of one target-layer verify: t_q query tokens appended at n0[b]..n0[b]+t_q-1.

    ``q`` is [batch][t_q][H_q][D]; ``k_new``/``v_new`` are [batch][t_q][H_kv][D].
    """
    wl: Workload
    n0: Tuple[int, ...]
    t_q: int
    q: torch.Tensor
    k_ctx: torch.Tensor
    v_ctx: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor


def verify_case(wl: Workload, contexts: Optional[Sequence[int]] = None, t_q: Optional[int] = None,
                device: str = "cpu", seed: Optional[int] = None, layer: int = 0) -> VerifyCase:
    seed = wl.seed if seed is None else seed
    n0 = tuple(int(c) for c in (contexts if contexts is not None else wl.contexts))
    t_q = wl.gamma + 1 if t_q is None else int(t_q)
    B, Hq, Hk, D = len(n0), wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    nmax = max(n0) if n0 else 0
    q = normal((B, t_q, Hq, D), seed, ("q_verify", layer), 1.0, wl.dtype, device)
    k_ctx = normal((B, nmax, Hk, D), seed, ("k_ctx_layer", layer), wl.kv_scale, wl.dtype, device)
    v_ctx = normal((B, nmax, Hk, D), seed, ("v_ctx_layer", layer), wl.kv_scale, wl.dtype, device)
    k_new = normal((B, t_q, Hk, D), seed, ("k_new_layer", layer), wl.kv_scale, wl.dtype, device)
    v_new = normal((B, t_q, Hk, D), seed, ("v_new_layer", layer), wl.kv_scale, wl.dtype, device)
    return VerifyCase(wl, n0, t_q, q, k_ctx, v_ctx, k_new, v_new)
