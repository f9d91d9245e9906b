"""SOCKET soft-collision sparse-attention decode for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI declared in
include/socket_lsh.h (libsocket_lsh.so, built by soft_lsh_sparse_amd.build);
this package only marshals torch tensors into that ABI.
"""

from ._lib import SocketError, load  # noqa: F401
from .api import (  # noqa: F401
    bucket_probs,
    decode,
    decode_group_shared,
    decode_workspace_bytes,
    dense_attn,
    hard_bucket_table,
    hash_keys,
    score,
    sparse_attn,
    topk,
)

__version__ = "0.1.0"
