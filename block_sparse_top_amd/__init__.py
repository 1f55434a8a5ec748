"""MI355X-native MiniMax Sparse Attention (MSA) forward path.

The compute lives in libmsa.so (HIP kernels for gfx950 behind the C ABI of
include/msa.h); `block_sparse_top_amd.msa` is its Python binding.
"""
