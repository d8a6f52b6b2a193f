"""MI355X-native MSA (MiniMax Sparse Attention) hot path.

The compute path is the C-ABI library ``libmsa.so`` (hand-written HIP kernels
for gfx950) declared in ``include/msa.h``; ``block_sparse_gqa_amd.msa`` is the
thin ctypes binding with the same entry-point names.  Importing this package
loads nothing; ``block_sparse_gqa_amd.msa`` loads the library on first use and
raises if it is missing.
"""
__all__ = ["synth", "msa"]
