"""The hybrid attention step written out plainly in float64 (test infrastructure only).

Nothing here is blocked, fused or reordered: each function is one step of the method as the
pages state it (cited per function), taken in float64 on exactly the stored values (bf16 bit
patterns, fp8/fp4 codes with their scales). See ``oracle/__init__`` for the page list.

Notation: D = entry dim, r_d = RoPE dims, H = query heads, r = compression ratio (1 for raw
sliding-window entries, 4 for C4, 128 for C128), W = window (128), k = top-k (512), p = the
query's absolute 0-based position (= context length - 1 at decode).

Readings where the pages are silent (each also listed with its pin in the design notes):
  R1 visibility: the window is positions [max(0, p-W+1), p]; compressed entries 0..n_vis-1
     are visible with n_vis = ceil(window_start / r), i.e. every complete group that holds at
     least one position older than the window.
  R2 pooling: "mean" = arithmetic mean of the r raw tokens; "softmax gate" = softmax over one
     scalar logit per raw position, then the weighted sum.
  R3 order: pool -> RMSNorm over all D dims (eps, unit gain) -> RoPE at the group's last
     position g*r + r - 1.
  R4 RoPE: rotate adjacent pairs (D-r_d+2i, D-r_d+2i+1) by pos * base**(-2i/r_d).
  R5 softmax scale 1/sqrt(D); values equal keys (shared K=V); output gets RoPE(-p).
  R6 indexer: score_g = sum_h w_h * relu(q_h . k_g); top-k by (score desc, index asc) with
     -0 == +0; output ascending, padded with -1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_to_f64, round_to_bf16_bits, unpack_fp4_row

__all__ = [
    "BLOCK_POSITIONS",
    "OraclePool",
    "pool_entries",
    "logical_pool",
    "rope",
    "rmsnorm",
    "pool_tokens",
    "compressed_entry",
    "compress_stream",
    "pending_group",
    "swa_entries",
    "q_norm_rope",
    "window_start",
    "n_visible",
    "indexer_scores",
    "topk_select",
    "attend",
    "hybrid_query",
    "decode",
    "prefill",
    "default_scale",
]

# vLLM day-0 post, "vLLM side": one logical block covers 256 native positions for every
# compression rate, so a block holds 256 raw, 64 C4 or 2 C128 entries.
BLOCK_POSITIONS = 256


# --------------------------------------------------------------------------------------------
# Paged storage (vLLM day-0 post, "vLLM side": unified hybrid KV cache, 256-position blocks)
# --------------------------------------------------------------------------------------------
@dataclass
class OraclePool:
    """A paged pool as stored.

    data:  f32  -> float32 [num_blocks, 256 // ratio, dim]
           f64  -> float64, same shape (values kept unrounded)
           bf16 -> uint16 bit patterns, same shape
           fp8  -> uint8 E4M3 codes, same shape; scale float32 [num_blocks, 256 // ratio]
           fp4  -> uint8 packed pairs [num_blocks, 256 // ratio, dim // 2];
                   scale uint8 E8M0 [num_blocks, 256 // ratio, dim // 32]
    block_table: int32 [batch, max_blocks], logical block -> physical block, -1 = absent.
    """

    data: np.ndarray
    dtype: str
    dim: int
    ratio: int
    block_table: np.ndarray
    scale: Optional[np.ndarray] = None


def logical_pool(entries_per_seq, ratio: int, dtype: str = "f64") -> OraclePool:
    """Lay out per-sequence logical entry arrays [n_b, dim] as a pool with blocks in order.

    dtype "f64" keeps the values; "bf16" stores them rounded to bfloat16 (nearest-even).
    """
    per_block = BLOCK_POSITIONS // ratio
    dim = int(np.asarray(entries_per_seq[0]).shape[1])
    nblk = [max(1, -(-len(e) // per_block)) for e in entries_per_seq]
    total = sum(nblk)
    data = np.zeros((total, per_block, dim), np.float64)
    table = np.full((len(entries_per_seq), max(nblk)), -1, np.int32)
    nxt = 0
    for b, e in enumerate(entries_per_seq):
        e = np.asarray(e, np.float64)
        for lb in range(nblk[b]):
            table[b, lb] = nxt
            chunk = e[lb * per_block:(lb + 1) * per_block]
            data[nxt, :len(chunk)] = chunk
            nxt += 1
    if dtype == "bf16":
        return OraclePool(data=round_to_bf16_bits(data), dtype="bf16", dim=dim, ratio=ratio,
                          block_table=table)
    return OraclePool(data=data, dtype="f64", dim=dim, ratio=ratio, block_table=table)


def pool_entries(pool: OraclePool, seq: int, gs: Sequence[int]) -> np.ndarray:
    """Entries g of sequence ``seq`` as float64 [len(gs), dim].

    Entry g (of ratio r) lives in logical block floor(g*r/256) at slot g mod (256/r).
    """
    per_block = BLOCK_POSITIONS // pool.ratio
    out = np.empty((len(gs), pool.dim), dtype=np.float64)
    for n, g in enumerate(gs):
        lb, slot = divmod(int(g), per_block)
        phys = int(pool.block_table[seq, lb])
        if phys < 0:
            raise ValueError(f"entry {g} of sequence {seq} lies in an absent block")
        if pool.dtype in ("f32", "f64"):
            out[n] = pool.data[phys, slot].astype(np.float64)
        elif pool.dtype == "bf16":
            out[n] = bf16_bits_to_f64(pool.data[phys, slot])
        elif pool.dtype == "fp8":
            out[n] = e4m3fn_to_f64(pool.data[phys, slot]) * np.float64(pool.scale[phys, slot])
        elif pool.dtype == "fp4":
            out[n] = unpack_fp4_row(pool.data[phys, slot], pool.scale[phys, slot], pool.dim)
        else:
            raise ValueError(pool.dtype)
    return out


# --------------------------------------------------------------------------------------------
# Compressor: pool -> RMSNorm -> RoPE (vLLM day-0 post: "c4a / c128a KV compression" and the
# fused "compressor + RMSNorm + RoPE + cache insert" kernel; SGLang blog, "Shadow Radix":
# 4:1 and 128:1 compression with an in-progress state per compression layer)
# --------------------------------------------------------------------------------------------
def rope(x, pos, rope_dim: int, base: float) -> np.ndarray:
    """Reading R4. Rotates the last ``rope_dim`` dims of x in adjacent pairs.

    Pair i = (D - r_d + 2i, D - r_d + 2i + 1) turns by the angle pos * base**(-2i / r_d).
    ``pos`` may be a scalar or broadcast against x's leading dims. RoPE(x, -pos) undoes it
    (the output's inverse rotation in the "shared K/V + inverse RoPE" move).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return y
    dim = y.shape[-1]
    half = rope_dim // 2
    theta = np.power(np.float64(base), -2.0 * np.arange(half, dtype=np.float64) / rope_dim)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    a = y[..., dim - rope_dim + 0::2].copy()
    b = y[..., dim - rope_dim + 1::2].copy()
    y[..., dim - rope_dim + 0::2] = a * c - b * s
    y[..., dim - rope_dim + 1::2] = a * s + b * c
    return y


def rmsnorm(x, eps: float) -> np.ndarray:
    """Reading R3: x / sqrt(mean_d x_d^2 + eps) over all D dims, unit gain."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def pool_tokens(tokens, mode: str, logits=None) -> np.ndarray:
    """Reading R2: 'mean' = (1/r) sum_t x_t; 'gate' = sum_t softmax(logits)_t x_t."""
    t = np.asarray(tokens, dtype=np.float64)
    if mode == "mean":
        return t.sum(axis=0) / t.shape[0]
    if mode == "gate":
        z = np.asarray(logits, dtype=np.float64)
        e = np.exp(z - z.max())
        wts = e / e.sum()
        return (wts[:, None] * t).sum(axis=0)
    raise ValueError(mode)


def compressed_entry(tokens, logits, g: int, r: int, mode: str, rope_dim: int, base: float,
                     eps: float) -> np.ndarray:
    """Entry g = RoPE(RMSNorm(Pool(x_{gr..gr+r-1})), gr + r - 1) (readings R2, R3, R4)."""
    return rope(rmsnorm(pool_tokens(tokens, mode, logits), eps), g * r + r - 1, rope_dim, base)


def compress_stream(x, logits, r: int, mode: str, rope_dim: int, base: float,
                    eps: float) -> np.ndarray:
    """All complete-group entries of one sequence whose raw tokens are x[0..T) at positions 0..T-1.

    Returns float64 [T // r, D]; the trailing T mod r tokens form the in-progress group.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0] // r
    out = np.empty((n, x.shape[1]), dtype=np.float64)
    for g in range(n):
        lg = None if logits is None else np.asarray(logits, np.float64)[g * r:(g + 1) * r]
        out[g] = compressed_entry(x[g * r:(g + 1) * r], lg, g, r, mode, rope_dim, base, eps)
    return out


def pending_group(x, logits, r: int):
    """The in-progress compression state after positions 0..T-1: the raw tokens (and logits)
    of the incomplete last group, keyed by slot = position mod r (SGLang blog, "Shadow Radix":
    each compression layer keeps its in-progress compression state in a state pool)."""
    x = np.asarray(x, dtype=np.float64)
    t_total = x.shape[0]
    start = (t_total // r) * r
    slots = {t % r: x[t] for t in range(start, t_total)}
    lslots = None
    if logits is not None:
        lslots = {t % r: float(np.asarray(logits, np.float64)[t]) for t in range(start, t_total)}
    return slots, lslots


def swa_entries(x, positions, rope_dim: int, base: float) -> np.ndarray:
    """Raw sliding-window entries s_t = RoPE(x_t, t), no norm (the "KV RoPE + K insert" step)."""
    return rope(np.asarray(x, np.float64), np.asarray(positions, np.float64), rope_dim, base)


def q_norm_rope(q, positions, rope_dim: int, base: float, eps: float) -> np.ndarray:
    """Query preparation of the fused "Q-norm + KV RoPE + K insert" step (vLLM post, "vLLM side"
    list). Reading: each query head's row is RMS-normalised over its dim with unit gain (as the
    compressor's RMSNorm, reading R3), then rotated at its token's position (reading R4), which
    gives the rotated query the attention takes. q [T][H][D], positions [T]."""
    q = np.asarray(q, np.float64)
    pos = np.asarray(positions, np.float64)[:, None]
    return rope(rmsnorm(q, eps), pos, rope_dim, base)


# --------------------------------------------------------------------------------------------
# Visibility (reading R1): SGLang blog "Shadow Radix" - SWA over the newest 128 raw tokens plus
# C4 top-512 or C128 dense; vLLM post - "short sliding window for locality across compression
# boundaries".
# --------------------------------------------------------------------------------------------
def window_start(p: int, window: int) -> int:
    return max(0, p - window + 1)


def n_visible(p: int, r: int, window: int) -> int:
    """Number of compressed entries a query at position p attends to: ceil(window_start / r)."""
    ws = window_start(p, window)
    return -(-ws // r)


# --------------------------------------------------------------------------------------------
# Indexer + top-k (vLLM post: "DeepSeek Sparse Attention over compressed tokens"; SGLang blog:
# "C4 (top-512 sparse over 4:1 compressed KV)", "indexer top-k")
# --------------------------------------------------------------------------------------------
def indexer_scores(q_idx, w, keys) -> np.ndarray:
    """Reading R6: I_g = sum_h w_h * max(0, sum_d q_{h,d} k_{g,d}) for each key row g."""
    q = np.asarray(q_idx, dtype=np.float64)          # [H_I, D_I]
    kk = np.asarray(keys, dtype=np.float64)          # [n, D_I]
    wt = np.asarray(w, dtype=np.float64)             # [H_I]
    if kk.shape[0] == 0:
        return np.zeros(0, dtype=np.float64)
    dots = q @ kk.T                                  # [H_I, n]
    return (wt[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def topk_select(scores, k: int) -> np.ndarray:
    """Reading R6: the first min(k, n) indices under the order (score desc, index asc).

    Scores compare numerically, so -0.0 ties with +0.0. Returned ascending and padded to
    length k with -1.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = sorted(range(n), key=lambda g: (-s[g], g))
    chosen = sorted(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


# --------------------------------------------------------------------------------------------
# Attention core (vLLM post: "Shared K/V + inverse RoPE"; SGLang blog "Shadow Radix": SWA plus
# C4 top-512 sparse or C128 dense)
# --------------------------------------------------------------------------------------------
def attend(q, keys, scale: float):
    """Per head h: z_j = scale * q_h . kappa_j; softmax over j (max-subtracted); o_h = sum_j p_j kappa_j.

    Values are the keys themselves (one shared K=V head for all query heads).
    Returns (o [H, D], probabilities [H, n]).
    """
    q = np.asarray(q, dtype=np.float64)
    kk = np.asarray(keys, dtype=np.float64)
    z = scale * (q @ kk.T)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    pr = e / e.sum(axis=1, keepdims=True)
    return pr @ kk, pr


def hybrid_query(q, p: int, seq: int, swa: OraclePool, comp: OraclePool, window: int,
                 scale: float, rope_dim: int, base: float,
                 selected: Optional[Sequence[int]] = None) -> np.ndarray:
    """One query token at position p of sequence ``seq``.

    Keys = raw window entries at positions [window_start, p] from ``swa``, then compressed
    entries from ``comp``: the given ``selected`` indices (C4 top-k; -1 entries ignored) or,
    if None, all n_visible (C128 dense). Output = RoPE(attention output, -p).
    """
    ws = window_start(p, window)
    keys = [pool_entries(swa, seq, range(ws, p + 1))]
    if selected is None:
        gs = list(range(n_visible(p, comp.ratio, window)))
    else:
        gs = [int(g) for g in selected if int(g) >= 0]
    if gs:
        keys.append(pool_entries(comp, seq, gs))
    o, _ = attend(q, np.concatenate(keys, axis=0), scale)
    return rope(o, -p, rope_dim, base)


def decode(q, seq_lens, swa: OraclePool, comp: OraclePool, window: int, scale: float,
           rope_dim: int, base: float, idx=None, seqs: Optional[Sequence[int]] = None):
    """A decode step: one query per sequence at p = seq_lens[b] - 1.

    idx (sparse C4 layers) = dict(q=[B,H_I,D_I], w=[B,H_I], pool=OraclePool, k=int); when given
    the indexer scores the visible entries and its top-k selects them, otherwise all visible
    compressed entries are used. Returns (out [len(seqs), H, D] float64, topk or None).
    """
    seqs = range(len(seq_lens)) if seqs is None else seqs
    outs, sels = [], []
    for b in seqs:
        p = int(seq_lens[b]) - 1
        selected = None
        if idx is not None:
            nv = n_visible(p, idx["pool"].ratio, window)
            sc = indexer_scores(idx["q"][b], idx["w"][b], pool_entries(idx["pool"], b, range(nv)))
            selected = topk_select(sc, idx["k"])
            sels.append(selected)
        outs.append(hybrid_query(q[b], p, b, swa, comp, window, scale, rope_dim, base, selected))
    return np.stack(outs), (np.stack(sels) if idx is not None else None)


def prefill(q, q_seq, q_pos, swa: OraclePool, comp: OraclePool, window: int, scale: float,
            rope_dim: int, base: float, idx=None, rows: Optional[Sequence[int]] = None):
    """Chunked-prefill attention: query i of sequence q_seq[i] at position q_pos[i] attends to its
    own causal window and its own top-k among the compressed entries visible at q_pos[i].

    idx = dict(q=[n_q,H_I,D_I], w=[n_q,H_I], pool=OraclePool, k=int) or None (dense).
    """
    rows = range(len(q_pos)) if rows is None else rows
    outs, sels = [], []
    for i in rows:
        b, p = int(q_seq[i]), int(q_pos[i])
        selected = None
        if idx is not None:
            nv = n_visible(p, idx["pool"].ratio, window)
            sc = indexer_scores(idx["q"][i], idx["w"][i], pool_entries(idx["pool"], b, range(nv)))
            selected = topk_select(sc, idx["k"])
            sels.append(selected)
        outs.append(hybrid_query(q[i], p, b, swa, comp, window, scale, rope_dim, base, selected))
    return np.stack(outs), (np.stack(sels) if idx is not None else None)


def default_scale(dim: int) -> float:
    """Reading R5: 1/sqrt(D)."""
    return 1.0 / math.sqrt(dim)
