"""Windowed-MTP decode attention for AMD Instinct MI355X (gfx950).

`long_context_decode_gqa_amd.wmtp` binds the C ABI of libwmtp (include/wmtp.h);
`long_context_decode_gqa_amd.build` compiles it in-tree.  Importing the package
loads nothing; the library is loaded on first use.
"""
__all__ = ["wmtp", "build"]
