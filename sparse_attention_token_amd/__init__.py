"""HISA hierarchical indexer for token-level sparse attention, MI355X (gfx950) native.

The compute path is the C-ABI library ``libhisa.so`` (hand-written HIP kernels);
``sparse_attention_token_amd.hisa`` is the thin ctypes binding over it.  The
binding is imported lazily so that ``synth`` (seeded inputs) can be used on a
machine without the built library.
"""
__all__ = ["hisa", "synth"]
