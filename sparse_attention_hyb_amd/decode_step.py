"""One decode step of a hybrid attention layer, issued on two streams and capturable in a graph.

The step's work and what each part reads and writes:
  prep      hyb_q_norm_kv_insert: query RMSNorm + RoPE of the new tokens (writes q) and their
            window entries (writes the window pool at each sequence's position p); on C4 layers
            also hyb_compress of the new tokens' indexer-key rows into the indexer-key pool (an
            entry that a token completes at p is not visible at p, so the indexer never reads it);
  indexer   C4 layers: hyb_index_score_keys + hyb_topk_keys (reads the indexer keys, writes
            top-k) - independent of prep;
  attention hyb_attn_decode_compress: reads q, the window (entry p included) and the compressed
            pool; its combine launch also compresses the new token (the entry that token completes
            is not visible at p, so it cannot race with the attention's reads).
So prep runs on a side stream while the indexer runs on the main one, and the attention waits for
both ([vLLM] "vLLM side" list: multi-stream overlap of the indexer, the main-KV compression and the
window insertion). Every size and position the kernels need is on the device (sequence lengths,
token ranges, start positions), and no call allocates, clears memory with a memset or
synchronises, so the whole step can be captured once in a HIP graph and replayed. Streams keep
the default priority.
"""

from dataclasses import dataclass
from typing import Optional

import torch

from . import (hyb_attn_decode_compress, hyb_compress, hyb_index_score_keys, hyb_q_norm_kv_insert,
               hyb_topk_keys)


@dataclass
class DecodeStepBuffers:
    """Caller-owned device buffers of one decode step (batch B, one new token per sequence)."""

    q_raw: torch.Tensor        # [B, H, D] query before its norm and rotation
    kv_new: torch.Tensor       # [B, D] the new tokens' K=V rows (window insert and compressor)
    q: torch.Tensor            # [B, H, D] rotated query (written by prep)
    seq_lens: torch.Tensor     # int32 [B], the new token included
    cu: torch.Tensor           # int32 [B + 1] = 0, 1, .., B
    start: torch.Tensor        # int32 [B] = seq_lens - 1
    swa: object                # window pool (ratio 1)
    comp: object               # compressed pool (ratio 4: sparse, 128: dense)
    state: torch.Tensor        # compressor ring [B, ratio, D] in kv_new's dtype
    out: torch.Tensor          # [B, H, D]
    workspace: torch.Tensor    # attention workspace
    max_seq_len: int
    # C4 (sparse) layers only
    idx_q: Optional[torch.Tensor] = None
    idx_w: Optional[torch.Tensor] = None
    idx_pool: Optional[object] = None
    keys: Optional[torch.Tensor] = None
    hist: Optional[torch.Tensor] = None
    topk: Optional[torch.Tensor] = None
    k: int = 512
    idx_kv_new: Optional[torch.Tensor] = None   # [B, D_I] the new tokens' indexer-key rows
    idx_state: Optional[torch.Tensor] = None    # indexer-key compressor ring [B, 4, D_I]
    gate_logits: Optional[torch.Tensor] = None    # C128 softmax-gate pooling
    state_logits: Optional[torch.Tensor] = None
    rope_dim: int = 64
    rope_base: float = 10000.0
    eps: float = 1e-6


class DecodeStep:
    """Issues one decode step: prep on `side`, indexer then attention on the main stream."""

    def __init__(self, buf: DecodeStepBuffers, side: Optional[torch.cuda.Stream] = None):
        self.b = buf
        self.side = side if side is not None else torch.cuda.Stream()   # default priority
        self._fork = torch.cuda.Event()
        self._join = torch.cuda.Event()

    def _prep(self, stream):
        b = self.b
        hyb_q_norm_kv_insert(b.q_raw, b.kv_new, b.cu, b.start, 1, b.swa, q_out=b.q,
                             rope_dim=b.rope_dim, rope_base=b.rope_base, eps=b.eps, stream=stream)
        if b.idx_kv_new is not None:
            hyb_compress(b.idx_kv_new, b.cu, b.start, 1, b.idx_state, b.idx_pool, b.rope_dim,
                         rope_base=b.rope_base, eps=b.eps, stream=stream)

    def _indexer(self, stream):
        b = self.b
        L = b.max_seq_len
        hyb_index_score_keys(b.idx_q, b.idx_w, b.start, L - 1, b.idx_pool, b.keys, b.hist,
                             stream=stream)
        hyb_topk_keys(b.keys, b.hist, b.start, L - 1, b.k, b.topk, stream=stream)

    def _attention(self, stream):
        b = self.b
        sparse = b.topk is not None
        hyb_attn_decode_compress(b.q, b.seq_lens, b.max_seq_len, b.swa, b.comp, b.out, b.kv_new,
                                 b.cu, b.start, 1, b.state, b.comp,
                                 topk_idx=b.topk if sparse else None, k=b.k if sparse else 0,
                                 rope_dim=b.rope_dim, rope_base=b.rope_base, eps=b.eps,
                                 gate_logits=b.gate_logits, state_logits=b.state_logits,
                                 workspace=b.workspace, stream=stream)

    def run_serial(self, stream: Optional[torch.cuda.Stream] = None) -> None:
        """The same work, one call after another on one stream."""
        s = stream or torch.cuda.current_stream()
        self._prep(s)
        if self.b.topk is not None:
            self._indexer(s)
        self._attention(s)

    def run(self, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Prep on the side stream beside the indexer; the attention waits for both."""
        main = stream or torch.cuda.current_stream()
        self._fork.record(main)
        self.side.wait_event(self._fork)
        self._prep(self.side)
        self._join.record(self.side)
        if self.b.topk is not None:
            self._indexer(main)
        main.wait_event(self._join)
        self._attention(main)

    def capture(self) -> torch.cuda.CUDAGraph:
        """The two-stream step captured once; replay() re-issues it with the buffers' current
        contents (sequence lengths and positions included)."""
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        return g
