"""Shared-round verify step of LFM2 speculative decoding on MI355X (gfx950).

The computation lives in libasv.so (HIP kernels + the host table builder,
declared in include/asv.h). This package is its Python binding:

* ``seg_table_build``, ``table_upload``, ``shared_conv``, ``shared_attn``,
  ``attn_merge``, ``row_argmax``, ``shared_qk``, ``draft_ids``, ``markov_pick`` (and the
  helpers next to them) -- one function per C entry point, marshalling
  tensors and streams only;
* ``RoundBuffers`` -- device buffers of one round and the calls in order.

PyTorch provides device memory and streams; it does no arithmetic of the
method. Nothing here falls back to a CPU path: without libasv.so every call
raises.
"""

from ._lib import (  # noqa: F401
    ABI_VERSION, CONV_IN, HEAD_DIM, HIDDEN, KEY_BLOCK, KV_HEADS, MAX_KEYS, MAX_ROWS,
    PARTIAL_FLOATS, Q_HEADS, QKV_WIDTH, SYMBOLS, TILE_ROWS, AsvError, StreamDesc, TableInfo, abi_version,
    MARKOV_MAX_CHAINS, MARKOV_MAX_DEPTH, MARKOV_MAX_RANK, MarkovChain, attn_merge, draft_ids,
    lib, MARKOV_FORMS, markov_pack_w2, markov_pick, markov_workspace, partial_floats, row_argmax, row_argmax_noalloc, row_argmax_workspace, seg_table_build,
    shared_attn, shared_conv, shared_qk, strerror, table_arrays, table_upload,
)
from .runner import RoundBuffers  # noqa: F401
