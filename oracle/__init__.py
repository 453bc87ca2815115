"""Float64 CPU oracle for Windowed-MTP decode attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never imports, links or runs it.
"""
from .wmtp_oracle import *  # noqa: F401,F403
from .wmtp_oracle import (FULL, SINK_WINDOW, decode_bf16, to_f64, visible_positions,  # noqa: F401
                          draft_entries_read, ring_slot, ring_append, ring_rollback,
                          ring_expected_tags, window_slot_positions, ring_visible, paged_element_offset, LogicalKV, PagedKV,
                          ConcatKV, softmax_attention, attention_over, draft_attention,
                          verify_attention, lse_combine, step_kv_bytes, memory_plan)
