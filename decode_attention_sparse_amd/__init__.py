"""Selected-cell INT8 decode attention for MI355X (gfx950).

Decode-time attention over a selected subset of KV cells held as INT8 K/V
pools behind a page table: a chunk pass (gather, INT8 dequant-dot, online
softmax, V accumulation into per-chunk partials) and a log-sum-exp merge
pass, both hand-written HIP kernels in libsda.so behind the C ABI of
include/sda.h.  The same library holds prompt (many-query, causal)
attention over the pools and the INT8 KV append that fills them.

    from decode_attention_sparse_amd import api      # ctypes binding (needs torch)
    from decode_attention_sparse_amd import inputs   # seeded synthetic inputs
"""
__all__ = ["api", "inputs", "build"]
