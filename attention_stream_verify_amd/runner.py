"""Device buffers of one shared round, and the round's calls in order.

Plumbing only: it allocates with torch, builds and uploads the table through
the binding, and enqueues the library's calls on the current torch stream.
"""

import torch

from . import _lib


class RoundBuffers:
    """Buffers for a round over ``streams`` with the given per-layer inputs.

    conv_states: per conv layer, one bf16 [2][2048] tensor per stream
    k_caches, v_caches: per attention layer, one tensor per stream
    (layouts of include/asv.h). All tensors must live on ``device``.
    """

    def __init__(self, streams, conv_states, k_caches, v_caches, device="cuda", vocab=None,
                 full=False):
        self.streams = [tuple(int(v) for v in s) for s in streams]
        self.device = torch.device(device)
        self._keep = (conv_states, k_caches, v_caches)  # table addresses stay valid
        self.blob_host = None
        self.full = bool(full)
        info, blob = _lib.seg_table_build(self.streams, conv_states, k_caches, v_caches, full=full)
        pinned = torch.empty(int(info.blob_bytes), dtype=torch.uint8, pin_memory=True)
        info, _ = _lib.seg_table_build(self.streams, conv_states, k_caches, v_caches, blob=pinned,
                                       full=full)
        self.info = info
        self.blob_host = pinned
        self.blob = torch.empty(int(info.blob_bytes), dtype=torch.uint8, device=self.device)
        R = int(info.n_rows)
        self.R = R
        self.partials = torch.empty(_lib.partial_floats(info), dtype=torch.float32, device=self.device)
        self.y = torch.empty((R, _lib.HIDDEN), dtype=torch.int16, device=self.device)
        self.o = torch.empty((R, _lib.Q_HEADS, _lib.HEAD_DIM), dtype=torch.int16, device=self.device)
        self.q = torch.empty((R, _lib.Q_HEADS, _lib.HEAD_DIM), dtype=torch.int16, device=self.device)
        self.pick = torch.empty(R, dtype=torch.int32, device=self.device)
        self.flag = torch.empty(R, dtype=torch.uint8, device=self.device)
        self.vocab = vocab
        spans, r0 = [], 0
        for w, _, _ in self.streams:          # each stream's rows of the picks, in place
            spans.append((r0, r0, w))
            r0 += w
        self.spans = torch.tensor(spans, dtype=torch.int32, device=self.device).reshape(-1, 3)
        self.ids = torch.zeros(R, dtype=torch.int32, device=self.device)
        self.fail = torch.zeros(len(self.streams), dtype=torch.uint8, device=self.device)
        self.workspace = None
        if vocab is not None:
            nb = _lib.row_argmax_workspace(R, vocab)
            self.workspace = torch.empty(max(16, nb), dtype=torch.uint8, device=self.device)

    def upload(self):
        _lib.table_upload(self.blob_host, self.blob)

    def conv(self, layer, x, w, y=None):
        _lib.shared_conv(self.info, self.blob, layer, x, w, self.y if y is None else y)

    def qk(self, layer, qkv, q_gain, k_gain, theta, eps, q_out=None):
        """q and k head norm + RoPE into q_out (default self.q); k and v
        appended to the layer's caches."""
        _lib.shared_qk(self.info, self.blob, layer, qkv, q_gain, k_gain, theta, eps,
                       self.q if q_out is None else q_out)

    def attn(self, layer, q):
        _lib.shared_attn(self.info, self.blob, layer, q, self.partials)

    def merge(self, o=None):
        _lib.attn_merge(self.info, self.blob, self.partials, self.o if o is None else o)

    def argmax(self, logits, vocab=None, row_stride=None):
        vocab = self.vocab if vocab is None else vocab
        if self.workspace is None or self.workspace.numel() < _lib.row_argmax_workspace(self.R, vocab):
            self.workspace = torch.empty(max(16, _lib.row_argmax_workspace(self.R, vocab)),
                                         dtype=torch.uint8, device=self.device)
        stride = vocab if row_stride is None else row_stride
        _lib.row_argmax(logits, logits.shape[0], vocab, stride, self.pick, self.flag, self.workspace)

    def draft(self, vocab=None):
        """Gather the picks of every stream's rows into ids, with a fail flag
        per stream (asv_draft_ids)."""
        vocab = self.vocab if vocab is None else vocab
        _lib.draft_ids(self.spans, len(self.streams), self.pick, self.flag, self.R, vocab,
                       self.ids, self.R, self.fail)

    def partial_views(self):
        P = int(self.info.partial_count)
        po = self.partials[:P * _lib.HEAD_DIM].view(P, _lib.HEAD_DIM)
        pml = self.partials[P * _lib.HEAD_DIM:].view(P, 2)
        return po, pml
