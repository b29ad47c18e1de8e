"""MiniMax Sparse Attention (MSA) forward path for MI355X (gfx950).

The compute runs in ``libmsa.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/msa.h``); ``block_sparse_long_idx_amd.msa``
binds it with argument marshalling only.  ``synth`` draws seeded inputs.
"""
