"""libkvfuse: one transformer layer of RAG KV-cache fusion on MI355X (gfx950).

The compute path is the C-ABI library `libkvfuse.so` built from `csrc/`
(hand-written HIP kernels).  `kvfuse` is its thin ctypes binding and
`synth` the seeded synthetic-input generator.  Importing this package loads
nothing; `from rag_kv_cache_kvf_amd import kvfuse` loads the library and
fails loudly if it has not been built.
"""
__all__ = ["kvfuse", "synth"]
