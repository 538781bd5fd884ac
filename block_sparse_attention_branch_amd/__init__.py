"""MI355X (gfx950) hot path of MiniMax Sparse Attention behind the libmsa C ABI.

``block_sparse_attention_branch_amd.msa`` is the ctypes binding; the kernels
live in ``csrc/`` and are built into ``libmsa.so`` by ``build.py``.
"""
from . import msa  # noqa: F401
from .msa import (  # noqa: F401
    MsaError,
    dense_prefill,
    index_topk,
    sparse_decode,
    sparse_prefill,
    workspace_size,
)
