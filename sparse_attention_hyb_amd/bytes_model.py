"""Algorithmic bytes and flops of the hybrid attention step (what the method must move / compute;
no re-reads, no partials). Used by the benchmark to place measured times on the roofline.

Per-entry sizes: an attention entry is `dim` elements of the pool dtype (+ a 4-byte scale for
fp8); an indexer key is `idx_dim` elements (fp4: dim/2 bytes + dim/32 scale bytes).
"""

from __future__ import annotations

from dataclasses import dataclass

ELEM_BYTES = {"f32": 4.0, "bf16": 2.0, "fp8": 1.0, "fp4": 0.5}


def entry_bytes(dtype: str, dim: int) -> int:
    b = int(ELEM_BYTES[dtype] * dim)
    if dtype == "fp8":
        b += 4
    if dtype == "fp4":
        b += dim // 32
    return b


def window_start(p: int, window: int) -> int:
    return max(0, p - window + 1)


def n_visible(p: int, ratio: int, window: int) -> int:
    return -(-window_start(p, window) // ratio)


@dataclass
class StepBytes:
    indexer_keys: int = 0
    attn_entries: int = 0
    io: int = 0              # queries, outputs, indexer queries and weights, top-k indices
    compressor: int = 0

    @property
    def total(self) -> int:
        return self.indexer_keys + self.attn_entries + self.io + self.compressor


def decode_query_bytes(L: int, *, ratio: int, sparse: bool, n_heads: int = 64, dim: int = 512,
                       dtype: str = "bf16", q_bytes: int = 2, idx_heads: int = 64,
                       idx_dim: int = 128, idx_dtype: str = "bf16", k: int = 512,
                       window: int = 128) -> StepBytes:
    """Bytes one decode query token (context length L, query at p = L-1) must move."""
    p = L - 1
    nv = n_visible(p, ratio, window)
    n_win = p - window_start(p, window) + 1
    eb = entry_bytes(dtype, dim)
    sb = StepBytes()
    io = 2 * n_heads * dim * q_bytes                      # q in, out
    if sparse:
        sb.indexer_keys = nv * entry_bytes(idx_dtype, idx_dim)
        sb.attn_entries = (min(k, nv) + n_win) * eb
        io += idx_heads * idx_dim * q_bytes + idx_heads * 4 + k * 4
    else:
        sb.attn_entries = (nv + n_win) * eb
    sb.io = io
    return sb


def compress_decode_bytes(ratio: int, dim: int = 512, x_bytes: int = 2, out_dtype: str = "bf16",
                          completes: bool = True, gate: bool = False) -> int:
    """One new token per sequence. The state ring holds the raw tokens of the group in x's own
    storage type (x_bytes per element) and, with softmax-gate pooling, one float32 logit each.
    A completing group reads its r-1 earlier tokens from the ring and the new token and writes
    the entry; otherwise the new token is read and written to the ring."""
    lg = 4 if gate else 0
    if not completes:
        return 2 * (dim * x_bytes + lg)
    return (ratio - 1) * (dim * x_bytes + lg) + dim * x_bytes + lg + entry_bytes(out_dtype, dim)


def index_score_bytes(L: int, *, ratio: int = 4, idx_heads: int = 64, idx_dim: int = 128,
                      idx_dtype: str = "bf16", q_bytes: int = 2, window: int = 128) -> int:
    """The indexer's algorithmic traffic for one query: every visible key, its query and its head
    weights. The scores are an intermediate of the selection (a fused scorer and selector never
    writes them), so nothing written is counted; see handoff_bytes for what this library's
    scorer hands to its selector."""
    nv = n_visible(L - 1, ratio, window)
    return nv * entry_bytes(idx_dtype, idx_dim) + idx_heads * idx_dim * q_bytes + idx_heads * 4


def handoff_bytes(L: int, *, ratio: int = 4, window: int = 128) -> int:
    """What the scorer writes for the selector per query (not algorithmic): an 8-byte (key,
    index) pair per visible entry and a 1024-bin uint16 cumulative histogram per 1024 entries."""
    nv = n_visible(L - 1, ratio, window)
    return nv * 8 + (nv + 1023) // 1024 * 1024 * 2


def attention_flops(n_keys: int, n_heads: int = 64, dim: int = 512) -> int:
    """QK and PV: 2 * 2 * heads * dim flops per key."""
    return 4 * n_heads * dim * n_keys


def indexer_flops(n_keys: int, idx_heads: int = 64, idx_dim: int = 128) -> int:
    return 2 * idx_heads * idx_dim * n_keys


def prefill_flops(q_pos, *, k: int = 512, window: int = 128, n_heads: int = 64, dim: int = 512,
                  idx_heads: int = 64, idx_dim: int = 128, ratio: int = 4):
    """(indexer flops, attention flops) of a prefill chunk with the given query positions."""
    fi = fa = 0
    for p in q_pos:
        nv = n_visible(p, ratio, window)
        n_win = p - window_start(p, window) + 1
        fi += indexer_flops(nv, idx_heads, idx_dim)
        fa += attention_flops(min(k, nv) + n_win, n_heads, dim)
    return fi, fa


def kv_state_bytes(context: int, n_c4_layers: int, n_c128_layers: int, dim: int = 512,
                   idx_dim: int = 128, window: int = 128, elem: int = 2) -> int:
    """Whole-stack cache bytes at a context length: C4 layers hold context/4 entries plus
    context/4 indexer keys, C128 layers context/128 entries, every layer a window of raw entries."""
    c4 = n_c4_layers * (context // 4) * (dim + idx_dim) * elem
    c128 = n_c128_layers * (context // 128) * dim * elem
    swa = (n_c4_layers + n_c128_layers) * window * dim * elem
    return c4 + c128 + swa
