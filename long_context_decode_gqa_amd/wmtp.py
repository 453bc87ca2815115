"""Python binding of libwmtp (Windowed-MTP decode attention for gfx950).

Argument marshalling only: every function turns torch tensors (device memory)
and the current HIP stream into the raw pointers and sizes of the C ABI in
include/wmtp.h, calls it, and raises on a non-zero status.  No attention
arithmetic happens here.  If the built library is missing, loading fails
loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# WMTP_LIBRARY names another build of the same library (for instance the host-sanitizer variant of
# long_context_decode_gqa_amd.build --host-ubsan); unset, the in-tree build.
LIB_PATH = os.environ.get("WMTP_LIBRARY") or os.path.join(_PKG, "_lib", "libwmtp.so")

# ---------------------------------------------------------------- constants (wmtp.h)
OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, ELAUNCH = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
FULL, SINK_WINDOW = 0, 1
DRAFT_FAST_PV = 0x10
MAX_BATCH = 64
BLOCK_SIZE = 16
MAX_SEQ_LEN = 1 << 30
NOALLOC_SCRATCH_BYTES = 16 << 20
MAX_VERIFY_ROWS = 96


class WmtpError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


# ---------------------------------------------------------------- C structs
class Shape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class Paged(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("run_rows", ctypes.c_int32)]


class Ring(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("slot_pos", ctypes.c_void_p),
                ("sink", ctypes.c_int32), ("window", ctypes.c_int32), ("headroom", ctypes.c_int32),
                ("seq_sink", ctypes.c_void_p), ("seq_window", ctypes.c_void_p)]


class MemoryPlan(ctypes.Structure):
    _fields_ = [("layer_bytes", ctypes.c_int64), ("block_table_bytes", ctypes.c_int64),
                ("ring_bytes", ctypes.c_int64), ("native_seq_bytes", ctypes.c_int64),
                ("windowed_seq_bytes", ctypes.c_int64), ("reclaimed_fraction", ctypes.c_double),
                ("native_sequences", ctypes.c_int64), ("windowed_sequences", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Partials(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("rows_per_seq", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("total_splits", ctypes.c_int32), ("split_base", ctypes.c_int32 * (MAX_BATCH + 1))]


EXPORTS = (
    "wmtp_draft_workspace_bytes", "wmtp_verify_workspace_bytes", "wmtp_draft_attn", "wmtp_verify_attn",
    "wmtp_draft_attn_append", "wmtp_verify_attn_append", "wmtp_combine", "wmtp_ring_append", "wmtp_ring_rollback", "wmtp_paged_append", "wmtp_debug_resolve_paged",
    "wmtp_debug_resolve_ring", "wmtp_debug_window_positions", "wmtp_plan_memory", "wmtp_stream_read",
    "wmtp_stream_read_paged", "wmtp_status_str",
    "wmtp_version", "wmtp_draft_attn_noalloc",
)

_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libwmtp.so (built in-tree by long_context_decode_gqa_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libwmtp.so not found at {p}; run `python -m long_context_decode_gqa_amd.build` first")
    lib = ctypes.CDLL(p)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sp, pp, rp, tp = ctypes.POINTER(Shape), ctypes.POINTER(Paged), ctypes.POINTER(Ring), ctypes.POINTER(Partials)
    lib.wmtp_draft_workspace_bytes.argtypes = [I32, sp, P, I32, I32, I32, I32, I32]
    lib.wmtp_draft_workspace_bytes.restype = I64
    lib.wmtp_verify_workspace_bytes.argtypes = [sp, I32, P, I32, I32]
    lib.wmtp_verify_workspace_bytes.restype = I64
    lib.wmtp_draft_attn.argtypes = [I32, sp, P, pp, rp, P, I32, I32, P, SZ, tp, P]
    lib.wmtp_draft_attn.restype = ctypes.c_int
    lib.wmtp_verify_attn.argtypes = [sp, P, I32, pp, P, I32, I32, P, SZ, tp, P]
    lib.wmtp_verify_attn.restype = ctypes.c_int
    lib.wmtp_draft_attn_append.argtypes = [I32, sp, P, pp, rp, P, P, P, I32, I32, P, SZ, tp, P]
    lib.wmtp_draft_attn_append.restype = ctypes.c_int
    lib.wmtp_verify_attn_append.argtypes = [sp, P, I32, pp, P, P, P, I32, I32, P, SZ, tp, P]
    lib.wmtp_verify_attn_append.restype = ctypes.c_int
    lib.wmtp_combine.argtypes = [tp, P, P, I32, P]
    lib.wmtp_draft_attn_noalloc.argtypes = [I32, sp, P, pp, rp, P, P, P, I32, I32, P, P, I32, P]
    lib.wmtp_draft_attn_noalloc.restype = ctypes.c_int
    lib.wmtp_combine.restype = ctypes.c_int
    lib.wmtp_ring_append.argtypes = [sp, rp, P, P, P, I32, I32, P]
    lib.wmtp_ring_append.restype = ctypes.c_int
    lib.wmtp_paged_append.argtypes = [sp, pp, P, P, P, I32, I32, P]
    lib.wmtp_ring_rollback.argtypes = [rp, P, I32, P]
    lib.wmtp_ring_rollback.restype = ctypes.c_int
    lib.wmtp_paged_append.restype = ctypes.c_int
    lib.wmtp_debug_resolve_paged.argtypes = [pp, I32, I32, I32, I32, P, I32, P, P]
    lib.wmtp_debug_resolve_paged.restype = ctypes.c_int
    lib.wmtp_debug_resolve_ring.argtypes = [I32, I32, I32, P, I32, P, P]
    lib.wmtp_debug_resolve_ring.restype = ctypes.c_int
    lib.wmtp_debug_window_positions.argtypes = [I32, I32, I32, I32, P, P]
    lib.wmtp_debug_window_positions.restype = ctypes.c_int
    lib.wmtp_plan_memory.argtypes = [sp, I32, I64, I32, I32, I32, I64, ctypes.POINTER(MemoryPlan)]
    lib.wmtp_plan_memory.restype = ctypes.c_int
    lib.wmtp_stream_read.argtypes = [P, I64, P, I32, P]
    lib.wmtp_stream_read_paged.argtypes = [P, P, I64, P, I32, I32, P, I32, P]
    lib.wmtp_stream_read_paged.restype = ctypes.c_int
    lib.wmtp_stream_read.restype = ctypes.c_int
    lib.wmtp_status_str.argtypes = [ctypes.c_int]
    lib.wmtp_status_str.restype = ctypes.c_char_p
    lib.wmtp_version.argtypes = []
    lib.wmtp_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, st: int) -> int:
    if st < 0:
        raise WmtpError(fn, st, load().wmtp_status_str(int(st)).decode())
    return st


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _lens(xs: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])
    return arr


def dtype_code(dt: torch.dtype) -> int:
    return {torch.float32: F32, torch.bfloat16: BF16}[dt]


def _device_tensor(name: str, t: torch.Tensor, numel: int, dtypes, on_gpu: bool = True) -> None:
    """The C ABI sees a raw pointer only: check here that `t` is a contiguous device tensor of one of
    `dtypes` holding exactly `numel` elements, so a mis-sized buffer fails on the host.  on_gpu=False
    leaves the device check to the caller."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {tuple(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    if on_gpu and not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor, got device {t.device}")


def _shape_dtype(shape: Shape) -> torch.dtype:
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


def make_shape(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
               scale: Optional[float] = None) -> Shape:
    return Shape(num_q_heads, num_kv_heads, head_dim, head_dim ** -0.5 if scale is None else scale, dtype_code(dtype))


# The descriptors hold raw device pointers; each keeps a reference to the tensors it
# points into, so that a temporary (say a block table built inline) is not freed and
# its memory reused by torch's allocator while the descriptor is still in use.
def make_paged(k: torch.Tensor, v: torch.Tensor, block_table: torch.Tensor) -> Paged:
    """Separate pools k, v: [num_blocks][H_kv][16][D]; block_table: int32 [batch][max_blocks] (device).
    The descriptor keeps k, v and block_table alive."""
    assert block_table.dtype == torch.int32 and block_table.dim() == 2
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
    p = Paged(k.data_ptr(), v.data_ptr(), block_table.data_ptr(), BLOCK_SIZE, block_table.shape[1], k.shape[0],
              BLOCK_SIZE)
    p._tensors = (k, v, block_table)
    return p


def make_paged_interleaved(pool: torch.Tensor, block_table: torch.Tensor) -> Paged:
    """One pool [num_blocks][H_kv][2][16][D] holding K (index 0) and V (index 1) of each (block, head)
    as one contiguous run of 32 rows; k and v views are pool[:, :, 0] and pool[:, :, 1].  The
    descriptor keeps pool and block_table alive."""
    assert block_table.dtype == torch.int32 and block_table.dim() == 2
    assert pool.is_contiguous() and pool.dim() == 5 and pool.shape[2] == 2 and pool.shape[3] == BLOCK_SIZE
    p = Paged(pool[:, :, 0].data_ptr(), pool[:, :, 1].data_ptr(), block_table.data_ptr(), BLOCK_SIZE,
              block_table.shape[1], pool.shape[0], 2 * BLOCK_SIZE)
    p._tensors = (pool, block_table)
    return p


def make_ring(k: torch.Tensor, v: torch.Tensor, slot_pos: torch.Tensor, sink: int, window: int,
              headroom: int = 0) -> Ring:
    """k, v: [batch][H_kv][S+W+R][D]; slot_pos: int32 [batch][S+W+R] (device); R = headroom.  The
    descriptor keeps k, v and slot_pos alive."""
    slots = int(sink) + int(window) + int(headroom)
    if slot_pos.dtype != torch.int32 or slot_pos.dim() != 2 or not slot_pos.is_contiguous():
        raise ValueError("slot_pos: expected a contiguous int32 [batch][S+W+R] tensor")
    if k.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype or not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k, v: expected two contiguous [batch][H_kv][S+W+R][D] tensors of one dtype")
    if k.shape[2] != slots or tuple(slot_pos.shape) != (k.shape[0], slots):
        raise ValueError(f"ring of S+W+R = {slots} slots: k is {tuple(k.shape)}, slot_pos {tuple(slot_pos.shape)}")
    r = Ring(k.data_ptr(), v.data_ptr(), slot_pos.data_ptr(), int(sink), int(window), int(headroom), None, None)
    r._tensors = (k, v, slot_pos)
    return r


def with_policy(ring: Ring, seq_sink: Optional[Sequence[int]] = None,
                seq_window: Optional[Sequence[int]] = None) -> Ring:
    """A copy of `ring` whose draft queries use per-sequence sinks / windows (host arrays kept alive)."""
    r = Ring(ring.k, ring.v, ring.slot_pos, ring.sink, ring.window, ring.headroom, None, None)
    r._tensors = getattr(ring, "_tensors", None)
    if seq_sink is not None:
        r._seq_sink = _lens(seq_sink)
        r.seq_sink = ctypes.cast(r._seq_sink, ctypes.c_void_p)
    if seq_window is not None:
        r._seq_window = _lens(seq_window)
        r.seq_window = ctypes.cast(r._seq_window, ctypes.c_void_p)
    return r


# ---------------------------------------------------------------- planning
def draft_workspace_bytes(mode: int, shape: Shape, seq_lens: Sequence[int], chunk_tokens: int = 0,
                          sink: int = 0, window: int = 1, headroom: int = 0) -> int:
    return _check("wmtp_draft_workspace_bytes", load().wmtp_draft_workspace_bytes(
        mode, ctypes.byref(shape), ctypes.cast(_lens(seq_lens), ctypes.c_void_p), len(seq_lens), chunk_tokens,
        sink, window, headroom))


def verify_workspace_bytes(shape: Shape, t_q: int, seq_lens: Sequence[int], split_tokens: int = 0) -> int:
    return _check("wmtp_verify_workspace_bytes", load().wmtp_verify_workspace_bytes(
        ctypes.byref(shape), t_q, ctypes.cast(_lens(seq_lens), ctypes.c_void_p), len(seq_lens), split_tokens))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 buffer of at least nbytes (torch's allocator aligns to 512)."""
    return torch.empty(max(256, int(nbytes)), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- hot path
class Prepared:
    """One C-ABI call whose ctypes arguments were built once: calling it launches the same work again
    (same pointers, sizes and stream), with no argument marshalling on the host.  An attention call
    fills `parts` (the split partials it writes into its workspace) each time it runs."""

    def __init__(self, name: str, args: tuple, keep: tuple = (), parts: Optional["Partials"] = None):
        self.name, self.parts = name, parts
        self._fn, self._args, self._keep = getattr(load(), name), args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st < 0:
            _check(self.name, st)


def _attn_call(name: str, lead: tuple, seq_lens: Sequence[int], tail_before_ws: tuple, ws: torch.Tensor,
               stream, keep: tuple) -> Prepared:
    """Arguments of the four attention entry points: lead..., seq_lens_host, batch, split size, workspace,
    workspace bytes, parts, stream."""
    parts = Partials()
    parts._workspace = ws   # the partials live in ws: keep it alive with them
    lens = _lens(seq_lens)
    args = lead + (ctypes.cast(lens, ctypes.c_void_p), len(seq_lens)) + tail_before_ws + (
        ws.data_ptr(), ws.numel() * ws.element_size(), ctypes.byref(parts), _stream(stream))
    return Prepared(name, args, keep + (lens, ws), parts)


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def prepare_draft_attn(mode: int, shape: Shape, q: torch.Tensor, seq_lens: Sequence[int], ws: torch.Tensor,
                       paged: Optional[Paged] = None, ring: Optional[Ring] = None, chunk_tokens: int = 0,
                       stream=None) -> Prepared:
    _device_tensor("q", q, len(seq_lens) * shape.num_q_heads * shape.head_dim, (_shape_dtype(shape),))
    return _attn_call("wmtp_draft_attn", (mode, ctypes.byref(shape), q.data_ptr(), _ref(paged), _ref(ring)),
                      seq_lens, (chunk_tokens,), ws, stream, (shape, q, paged, ring))


def draft_attn(mode: int, shape: Shape, q: torch.Tensor, seq_lens: Sequence[int], ws: torch.Tensor,
               paged: Optional[Paged] = None, ring: Optional[Ring] = None, chunk_tokens: int = 0,
               stream=None) -> Partials:
    call = prepare_draft_attn(mode, shape, q, seq_lens, ws, paged, ring, chunk_tokens, stream)
    call()
    return call.parts


def prepare_verify_attn(shape: Shape, q: torch.Tensor, t_q: int, paged: Paged, seq_lens: Sequence[int],
                        ws: torch.Tensor, split_tokens: int = 0, stream=None) -> Prepared:
    _device_tensor("q", q, len(seq_lens) * t_q * shape.num_q_heads * shape.head_dim, (_shape_dtype(shape),))
    return _attn_call("wmtp_verify_attn", (ctypes.byref(shape), q.data_ptr(), t_q, _ref(paged)),
                      seq_lens, (split_tokens,), ws, stream, (shape, q, paged))


def verify_attn(shape: Shape, q: torch.Tensor, t_q: int, paged: Paged, seq_lens: Sequence[int], ws: torch.Tensor,
                split_tokens: int = 0, stream=None) -> Partials:
    call = prepare_verify_attn(shape, q, t_q, paged, seq_lens, ws, split_tokens, stream)
    call()
    return call.parts


def _new_tokens(shape: Shape, k_new: torch.Tensor, v_new: torch.Tensor, batch: int, t_new: int) -> None:
    """The fused calls read [batch][t_new][H_kv][D] from k_new and v_new: check that much is there."""
    want = batch * t_new * shape.num_kv_heads * shape.head_dim
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x.numel() != want or x.dtype != _shape_dtype(shape) or not x.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous [{batch}][{t_new}][{shape.num_kv_heads}]"
                             f"[{shape.head_dim}] tensor of the cache dtype, got {tuple(x.shape)} {x.dtype}")
        if not x.is_cuda:
            raise ValueError(f"{name}: expected a GPU tensor, got device {x.device}")


def prepare_draft_attn_append(mode: int, shape: Shape, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                              seq_lens: Sequence[int], ws: torch.Tensor, paged: Optional[Paged] = None,
                              ring: Optional[Ring] = None, chunk_tokens: int = 0, stream=None) -> Prepared:
    _device_tensor("q", q, len(seq_lens) * shape.num_q_heads * shape.head_dim, (_shape_dtype(shape),))
    _new_tokens(shape, k_new, v_new, len(seq_lens), 1)
    return _attn_call("wmtp_draft_attn_append",
                      (mode, ctypes.byref(shape), q.data_ptr(), _ref(paged), _ref(ring), k_new.data_ptr(),
                       v_new.data_ptr()), seq_lens, (chunk_tokens,), ws, stream, (shape, q, paged, ring, k_new, v_new))


def draft_attn_append(mode: int, shape: Shape, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      seq_lens: Sequence[int], ws: torch.Tensor, paged: Optional[Paged] = None,
                      ring: Optional[Ring] = None, chunk_tokens: int = 0, stream=None) -> Partials:
    """Append one token per sequence at position seq_lens[b] - 1 (paged or ring) and attend, in one launch."""
    call = prepare_draft_attn_append(mode, shape, q, k_new, v_new, seq_lens, ws, paged, ring, chunk_tokens, stream)
    call()
    return call.parts


def prepare_verify_attn_append(shape: Shape, q: torch.Tensor, t_q: int, paged: Paged, k_new: torch.Tensor,
                               v_new: torch.Tensor, seq_lens: Sequence[int], ws: torch.Tensor, split_tokens: int = 0,
                               stream=None) -> Prepared:
    _device_tensor("q", q, len(seq_lens) * t_q * shape.num_q_heads * shape.head_dim, (_shape_dtype(shape),))
    _new_tokens(shape, k_new, v_new, len(seq_lens), t_q)
    return _attn_call("wmtp_verify_attn_append",
                      (ctypes.byref(shape), q.data_ptr(), t_q, _ref(paged), k_new.data_ptr(), v_new.data_ptr()),
                      seq_lens, (split_tokens,), ws, stream, (shape, q, paged, k_new, v_new))


def verify_attn_append(shape: Shape, q: torch.Tensor, t_q: int, paged: Paged, k_new: torch.Tensor,
                       v_new: torch.Tensor, seq_lens: Sequence[int], ws: torch.Tensor, split_tokens: int = 0,
                       stream=None) -> Partials:
    """Append the t_q query tokens' K/V at positions seq_lens[b] - t_q .. seq_lens[b] - 1 and verify, in one launch."""
    call = prepare_verify_attn_append(shape, q, t_q, paged, k_new, v_new, seq_lens, ws, split_tokens, stream)
    call()
    return call.parts


def prepare_combine(parts: Partials, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> Prepared:
    """out: [batch][rows_per_seq][D] fp32 or bf16; lse: fp32 [batch][rows_per_seq] or None (device).  `parts`
    must already describe its partials (the attention call that fills it has run)."""
    rows = parts.batch * parts.rows_per_seq
    _device_tensor("out", out, rows * parts.head_dim, (torch.float32, torch.bfloat16), on_gpu=False)
    if lse is not None:
        _device_tensor("lse", lse, rows, (torch.float32,), on_gpu=False)
    for name, t in (("out", out), ("lse", lse)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: expected a GPU tensor, got device {t.device}")
    return Prepared("wmtp_combine", (ctypes.byref(parts), out.data_ptr(), _ptr(lse), dtype_code(out.dtype),
                                     _stream(stream)), (parts, out, lse))


def combine(parts: Partials, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """out: [batch][rows_per_seq][D] fp32 or bf16; lse: fp32 [batch][rows_per_seq] or None (device)."""
    prepare_combine(parts, out, lse, stream)()


def _append_call(name: str, shape: Shape, desc, k_new: torch.Tensor, v_new: torch.Tensor, pos: Sequence[int],
                 stream) -> Prepared:
    if k_new.dim() != 4:
        raise ValueError(f"k_new: expected [batch][t_new][H_kv][D], got shape {tuple(k_new.shape)}")
    _new_tokens(shape, k_new, v_new, len(pos), k_new.shape[1])
    lens = _lens(pos)
    return Prepared(name, (ctypes.byref(shape), ctypes.byref(desc), k_new.data_ptr(), v_new.data_ptr(),
                           ctypes.cast(lens, ctypes.c_void_p), len(pos), k_new.shape[1], _stream(stream)),
                    (shape, desc, k_new, v_new, lens))


def prepare_ring_append(shape: Shape, ring: Ring, k_new: torch.Tensor, v_new: torch.Tensor, pos: Sequence[int],
                        stream=None) -> Prepared:
    return _append_call("wmtp_ring_append", shape, ring, k_new, v_new, pos, stream)


def draft_attn_noalloc(mode: int, shape: Shape, q: torch.Tensor, seq_lens: Sequence[int], out: torch.Tensor,
                       lse: Optional[torch.Tensor] = None, paged: Optional[Paged] = None, ring: Optional[Ring] = None,
                       k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                       chunk_tokens: int = 0, stream=None) -> None:
    """A draft step (with the append inside when k_new / v_new are given) and its combine into out
    [batch][H_q][D] (fp32 or bf16) and lse [batch][H_q], using the library's fixed scratch: no
    workspace, and nothing allocated by the library."""
    batch = len(seq_lens)
    _device_tensor("q", q, batch * shape.num_q_heads * shape.head_dim, (_shape_dtype(shape),))
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new: give both or neither")
    if k_new is not None:
        _new_tokens(shape, k_new, v_new, batch, 1)
    rows = batch * shape.num_q_heads
    _device_tensor("out", out, rows * shape.head_dim, (torch.float32, torch.bfloat16))
    if lse is not None:
        _device_tensor("lse", lse, rows, (torch.float32,))
    lens = _lens(seq_lens)
    _check("wmtp_draft_attn_noalloc", load().wmtp_draft_attn_noalloc(
        mode, ctypes.byref(shape), q.data_ptr(), _ref(paged), _ref(ring), _ptr(k_new), _ptr(v_new),
        ctypes.cast(lens, ctypes.c_void_p), batch, chunk_tokens, out.data_ptr(), _ptr(lse), dtype_code(out.dtype),
        _stream(stream)))


def ring_append(shape: Shape, ring: Ring, k_new: torch.Tensor, v_new: torch.Tensor, pos: Sequence[int],
                stream=None) -> None:
    """k_new, v_new: [batch][t_new][H_kv][D]; pos[b]: absolute position of the first new token."""
    prepare_ring_append(shape, ring, k_new, v_new, pos, stream)()


def ring_rollback(ring: Ring, seq_lens: Sequence[int], stream=None) -> None:
    """Forget ring entries at positions >= seq_lens[b] (drafted tokens verification rejected)."""
    _check("wmtp_ring_rollback", load().wmtp_ring_rollback(
        ctypes.byref(ring), ctypes.cast(_lens(seq_lens), ctypes.c_void_p), len(seq_lens), _stream(stream)))


def prepare_paged_append(shape: Shape, paged: Paged, k_new: torch.Tensor, v_new: torch.Tensor, pos: Sequence[int],
                         stream=None) -> Prepared:
    return _append_call("wmtp_paged_append", shape, paged, k_new, v_new, pos, stream)


def paged_append(shape: Shape, paged: Paged, k_new: torch.Tensor, v_new: torch.Tensor, pos: Sequence[int],
                 stream=None) -> None:
    prepare_paged_append(shape, paged, k_new, v_new, pos, stream)()


# ---------------------------------------------------------------- index resolution hooks
def debug_resolve_paged(paged: Paged, num_kv_heads: int, head_dim: int, b: int, h: int,
                        positions: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(positions.numel(), dtype=torch.int64, device=positions.device)
    _check("wmtp_debug_resolve_paged", load().wmtp_debug_resolve_paged(
        ctypes.byref(paged), num_kv_heads, head_dim, b, h, positions.data_ptr(), positions.numel(), out.data_ptr(),
        _stream(stream)))
    return out


def debug_resolve_ring(sink: int, window: int, positions: torch.Tensor, headroom: int = 0,
                       stream=None) -> torch.Tensor:
    out = torch.empty(positions.numel(), dtype=torch.int32, device=positions.device)
    _check("wmtp_debug_resolve_ring", load().wmtp_debug_resolve_ring(
        sink, window, headroom, positions.data_ptr(), positions.numel(), out.data_ptr(), _stream(stream)))
    return out


def debug_window_positions(sink: int, window: int, n: int, device, headroom: int = 0, stream=None) -> torch.Tensor:
    out = torch.empty(sink + window + headroom, dtype=torch.int32, device=device)
    _check("wmtp_debug_window_positions", load().wmtp_debug_window_positions(
        sink, window, headroom, n, out.data_ptr(), _stream(stream)))
    return out


def plan_memory(shape: Shape, target_layers: int, context: int, sink: int, window: int, headroom: int,
                budget_bytes: int) -> dict:
    """KV bytes per sequence with a native or windowed draft, and sequences a budget admits (host only)."""
    out = MemoryPlan()
    _check("wmtp_plan_memory", load().wmtp_plan_memory(ctypes.byref(shape), target_layers, context, sink, window,
                                                       headroom, budget_bytes, ctypes.byref(out)))
    return out.as_dict()


def stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None) -> None:
    """Read all of `src` once (bandwidth probe); sink: int32/uint32 [workgroups * 256]."""
    _check("wmtp_stream_read", load().wmtp_stream_read(
        src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), workgroups, _stream(stream)))


def stream_read_paged(k: torch.Tensor, v: torch.Tensor, runs: torch.Tensor, run_bytes: int, sink: torch.Tensor,
                      workgroups: int, stream=None) -> None:
    """Read the listed runs of k and v in order (paged bandwidth probe); runs: device int32."""
    _check("wmtp_stream_read_paged", load().wmtp_stream_read_paged(
        k.data_ptr(), v.data_ptr(), k.numel() * k.element_size(), runs.data_ptr(), runs.numel(), run_bytes,
        sink.data_ptr(), workgroups, _stream(stream)))


def version() -> str:
    return load().wmtp_version().decode()
