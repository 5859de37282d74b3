"""Seeded synthetic inputs for the hybrid attention step.

This module only draws random numbers, rounds them to their storage types, quantises stored
caches (fp8 E4M3 with a per-entry fp32 scale, fp4 E2M1 with a per-32-element E8M0 scale) and
lays them out in paged pools with seeded block permutations. It holds none of the method's
arithmetic (no pooling, normalisation, rotation, scoring, selection or attention), so the same
tensors can be handed both to the HIP library and to the float64 oracle.

Recipe (shapes follow the decode/prefill workloads the method is quoted on):
  * every value ~ N(0, 1), drawn in float32 from a torch.Generator seeded with
    ``stream_seed(workload_id, seed, stream)`` on the device that holds the tensor, then
    rounded to the storage dtype (round-to-nearest-even for bf16);
  * indexer head weights ~ N(0, 1) / sqrt(128); gate logits ~ N(0, 1);
  * paged pools: one logical block = 256 native positions (256 raw, 64 C4 or 2 C128 entries);
    physical block ids are a seeded permutation over all blocks a batch uses; blocks a step
    never touches are left absent (-1);
  * mixed-length batches: context lengths floor(exp(U(ln 4096, ln 2**20)));
  * quantised pools: fp8 scale = amax / 448 per entry; fp4 shared exponent
    floor(log2(amax)) - 2 per 32 elements (OCP MX rule), codes rounded to nearest-even with
    saturation.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

BLOCK_POSITIONS = 256
STORAGE = ("f32", "bf16", "fp8", "fp4")


def stream_seed(workload_id: int, seed: int, stream: int) -> int:
    return ((int(workload_id) * 1_000_003 + int(seed)) * 1_000_033 + int(stream)) % (2 ** 62)


def generator(workload_id: int, seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(stream_seed(workload_id, seed, stream))
    return g


def randn(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round float32 values to a plain storage dtype ('f32' or 'bf16')."""
    if dtype == "f32":
        return x.to(torch.float32).contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


# ------------------------------------------------------------------------------------------
# Quantisers for stored caches (data preparation only; the oracle decodes the codes itself)
# ------------------------------------------------------------------------------------------
def quantize_fp8_rows(x: torch.Tensor):
    """float32 [..., D] -> (uint8 E4M3 codes [..., D], float32 scale [...]) with scale = amax/448."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    v = (x / scale[..., None]).clamp(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


_E2M1_GRID_EVEN_FIRST = (0.0, 1.0, 2.0, 4.0, 0.5, 1.5, 3.0, 6.0)
_E2M1_CODE_OF = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def quantize_fp4_rows(x: torch.Tensor):
    """float32 [..., D] (D % 32 == 0) -> (uint8 packed [..., D/2], uint8 E8M0 [..., D/32]).

    Shared exponent e = floor(log2(amax)) - 2 per 32 elements (clamped to the E8M0 range),
    element code = nearest E2M1 value of x / 2**e (ties to the even mantissa, saturating at 6).
    Element 2j goes to the low nibble of byte j.
    """
    shp = x.shape
    d = shp[-1]
    assert d % 32 == 0
    xb = x.reshape(*shp[:-1], d // 32, 32)
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.zeros_like(amax))
    e = e.clamp(-127, 127)
    scale_code = (e + 127).to(torch.uint8)
    v = xb / torch.exp2(e)[..., None]
    grid = torch.tensor(_E2M1_GRID_EVEN_FIRST, dtype=torch.float32, device=x.device)
    mag_codes = torch.tensor([_E2M1_CODE_OF[g] for g in _E2M1_GRID_EVEN_FIRST],
                             dtype=torch.uint8, device=x.device)
    dist = (v.abs()[..., None] - grid).abs()
    pick = torch.argmin(dist, dim=-1)          # first minimum: even mantissa wins ties
    code = mag_codes[pick] | ((v < 0).to(torch.uint8) << 3)
    code = code.reshape(*shp[:-1], d)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), scale_code.reshape(*shp[:-1], d // 32).contiguous()


# ------------------------------------------------------------------------------------------
# Paged pools
# ------------------------------------------------------------------------------------------
@dataclass
class PagedTensors:
    """A paged pool as plain tensors.

    data  [num_blocks, 256 // ratio, dim] (f32 / bf16 / uint8 fp8 codes) or
          [num_blocks, 256 // ratio, dim // 2] (uint8 packed fp4)
    scale [num_blocks, 256 // ratio] float32 (fp8) / [num_blocks, 256 // ratio, dim // 32]
          uint8 E8M0 (fp4) / None
    block_table [batch, max_blocks] int32, -1 = absent.
    """

    data: torch.Tensor
    scale: Optional[torch.Tensor]
    block_table: torch.Tensor
    dtype: str
    dim: int
    ratio: int

    @property
    def num_blocks(self) -> int:
        return int(self.data.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def per_block(self) -> int:
        return BLOCK_POSITIONS // self.ratio

    def nbytes(self) -> int:
        n = self.data.numel() * self.data.element_size()
        if self.scale is not None:
            n += self.scale.numel() * self.scale.element_size()
        return n


def block_table(needed: Sequence[Sequence[int]], max_blocks: int, gen: torch.Generator,
                shuffle: bool = True):
    """Physical ids for the logical blocks each sequence needs.

    Returns (int32 [batch, max_blocks] on CPU, number of physical blocks). With ``shuffle`` the
    physical ids are a seeded permutation; otherwise they are assigned in order.
    """
    pairs = [(b, lb) for b, lbs in enumerate(needed) for lb in lbs]
    n = len(pairs)
    if shuffle:
        perm = torch.randperm(n, generator=gen, device=gen.device).cpu()
    else:
        perm = torch.arange(n)
    table = torch.full((len(needed), max_blocks), -1, dtype=torch.int32)
    for (b, lb), phys in zip(pairs, perm.tolist()):
        table[b, lb] = phys
    return table, n


def alloc_pool(dtype: str, dim: int, ratio: int, table: torch.Tensor, num_blocks: int,
               device) -> PagedTensors:
    per = BLOCK_POSITIONS // ratio
    if dtype == "f32":
        data = torch.zeros(num_blocks, per, dim, dtype=torch.float32, device=device)
        scale = None
    elif dtype == "bf16":
        data = torch.zeros(num_blocks, per, dim, dtype=torch.bfloat16, device=device)
        scale = None
    elif dtype == "fp8":
        data = torch.zeros(num_blocks, per, dim, dtype=torch.uint8, device=device)
        scale = torch.ones(num_blocks, per, dtype=torch.float32, device=device)
    elif dtype == "fp4":
        data = torch.zeros(num_blocks, per, dim // 2, dtype=torch.uint8, device=device)
        scale = torch.full((num_blocks, per, dim // 32), 127, dtype=torch.uint8, device=device)
    else:
        raise ValueError(dtype)
    return PagedTensors(data, scale, table.to(device), dtype, dim, ratio)


def fill_normal(pool: PagedTensors, gen: torch.Generator, chunk_blocks: int = 4096) -> None:
    """Fill every physical block with N(0,1) values in the pool's storage format."""
    dev = pool.data.device
    for b0 in range(0, pool.num_blocks, chunk_blocks):
        b1 = min(pool.num_blocks, b0 + chunk_blocks)
        x = randn((b1 - b0, pool.per_block, pool.dim), gen, dev)
        if pool.dtype in ("f32", "bf16"):
            pool.data[b0:b1] = to_storage(x, pool.dtype)
        elif pool.dtype == "fp8":
            c, s = quantize_fp8_rows(x)
            pool.data[b0:b1] = c
            pool.scale[b0:b1] = s
        else:
            c, s = quantize_fp4_rows(x)
            pool.data[b0:b1] = c
            pool.scale[b0:b1] = s


def make_pool(dtype: str, dim: int, ratio: int, needed, max_blocks: int, gen, device,
              fill: bool = True, shuffle: bool = True) -> PagedTensors:
    table, n = block_table(needed, max_blocks, gen, shuffle)
    pool = alloc_pool(dtype, dim, ratio, table, n, device)
    if fill:
        fill_normal(pool, gen)
    return pool


def blocks_for_positions(lo: int, hi: int) -> List[int]:
    """Logical blocks covering native positions [lo, hi)."""
    if hi <= lo:
        return []
    return list(range(lo // BLOCK_POSITIONS, (hi - 1) // BLOCK_POSITIONS + 1))


def blocks_for_entries(n_entries: int, ratio: int) -> List[int]:
    """Logical blocks holding compressed entries 0..n_entries-1 of ratio ``ratio``."""
    per = BLOCK_POSITIONS // ratio
    return list(range(0, -(-n_entries // per)))


# ------------------------------------------------------------------------------------------
# Workloads
# ------------------------------------------------------------------------------------------
@dataclass
class Decode:
    """One decode step over a batch: one query token per sequence at p = seq_len - 1."""

    name: str
    q: torch.Tensor                       # [B, H, D]
    seq_lens: torch.Tensor                # [B] int32 (device)
    seq_lens_host: List[int]
    swa: PagedTensors
    comp: PagedTensors
    idx_q: Optional[torch.Tensor] = None  # [B, H_I, D_I]
    idx_w: Optional[torch.Tensor] = None  # [B, H_I] float32
    idx_pool: Optional[PagedTensors] = None
    k: int = 512
    window: int = 128
    rope_dim: int = 64
    rope_base: float = 10000.0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens_host)


def _ints(x, device) -> torch.Tensor:
    return torch.tensor(list(x), dtype=torch.int32, device=device)


def sparse_decode(device, seed: int = 0, batch: int = 16, ctx=131072, n_heads: int = 64,
                  dim: int = 512, rope_dim: int = 64, idx_heads: int = 64, idx_dim: int = 128,
                  k: int = 512, window: int = 128, dtype: str = "bf16", idx_dtype: str = "bf16",
                  workload_id: int = 2, shuffle: bool = True, grow: int = 0) -> Decode:
    """C4 sparse decode: SWA window + indexer top-k over C4 entries (entries drawn directly).

    ``ctx`` is one context length for every sequence or a per-sequence list. ``grow`` > 0 sizes
    the pools (and block tables) for that many more tokens per sequence, for runs of several
    decode steps; the blocks the extra tokens reach hold drawn values until written.
    """
    lens = list(ctx) if isinstance(ctx, (list, tuple)) else [int(ctx)] * batch
    assert len(lens) == batch
    g = generator(workload_id, seed, 0, device)
    max_len = max(lens)
    qdt = "bf16" if dtype in ("bf16", "fp8") else dtype
    q = to_storage(randn((batch, n_heads, dim), g, device), qdt)
    idx_q = to_storage(randn((batch, idx_heads, idx_dim), g, device), qdt)
    idx_w = randn((batch, idx_heads), g, device) / math.sqrt(128.0)
    swa_need = [blocks_for_positions(max(0, L - window), L + grow) for L in lens]
    swa = make_pool(dtype, dim, 1, swa_need, -(-(max_len + grow) // BLOCK_POSITIONS),
                    generator(workload_id, seed, 1, device), device, shuffle=shuffle)
    c_need = [blocks_for_entries((L + grow) // 4, 4) for L in lens]
    mb = -(-(max_len + grow) // BLOCK_POSITIONS)
    comp = make_pool(dtype, dim, 4, c_need, mb, generator(workload_id, seed, 2, device), device,
                     shuffle=shuffle)
    idx_pool = make_pool(idx_dtype, idx_dim, 4, c_need, mb,
                         generator(workload_id, seed, 3, device), device, shuffle=shuffle)
    return Decode("c4_sparse_decode", q, _ints(lens, device), lens, swa, comp, idx_q, idx_w,
                  idx_pool, k=k, window=window, rope_dim=rope_dim)


def dense_decode(device, seed: int = 0, batch: int = 32, ctx=1 << 20, n_heads: int = 64,
                 dim: int = 512, rope_dim: int = 64, window: int = 128, dtype: str = "bf16",
                 workload_id: int = 3, fill_comp: bool = True, shuffle: bool = True) -> Decode:
    """C128 dense decode: SWA window + every visible C128 entry.

    With ``fill_comp`` the C128 entries are drawn directly; otherwise the pool is left zeroed
    for the caller to fill by compressing ``raw_chunk`` tokens.
    """
    lens = list(ctx) if isinstance(ctx, (list, tuple)) else [int(ctx)] * batch
    g = generator(workload_id, seed, 0, device)
    max_len = max(lens)
    qdt = "bf16" if dtype in ("bf16", "fp8") else dtype
    q = to_storage(randn((batch, n_heads, dim), g, device), qdt)
    mb = -(-max_len // BLOCK_POSITIONS)
    swa_need = [blocks_for_positions(max(0, L - window), L) for L in lens]
    swa = make_pool(dtype, dim, 1, swa_need, mb, generator(workload_id, seed, 1, device), device,
                    shuffle=shuffle)
    c_need = [blocks_for_entries(L // 128, 128) for L in lens]
    comp = make_pool(dtype, dim, 128, c_need, mb, generator(workload_id, seed, 2, device), device,
                     fill=fill_comp, shuffle=shuffle)
    return Decode("c128_dense_decode", q, _ints(lens, device), lens, swa, comp, k=0,
                  window=window, rope_dim=rope_dim)


RAW_CHUNK = 1 << 16


def raw_chunk(workload_id: int, seed: int, seq: int, chunk: int, dim: int, device,
              dtype: str = "bf16"):
    """Raw compressor input for tokens [chunk*65536, (chunk+1)*65536) of one sequence:
    (x [65536, dim] in ``dtype``, gate logits [65536] float32). Reproducible per (seq, chunk)."""
    g = generator(workload_id, seed, 1000 + seq * 4096 + chunk, device)
    x = to_storage(randn((RAW_CHUNK, dim), g, device), dtype)
    logits = randn((RAW_CHUNK,), g, device)
    return x, logits


def mixed_lengths(batch: int, gen: torch.Generator, lo: int = 4096, hi: int = 1 << 20):
    u = torch.rand(batch, generator=gen, device=gen.device, dtype=torch.float64).cpu()
    return [int(math.floor(math.exp(math.log(lo) + float(v) * (math.log(hi) - math.log(lo)))))
            for v in u]


@dataclass
class Prefill:
    """Chunked prefill of one sequence: prior entries drawn, new chunk of raw tokens."""

    q: torch.Tensor          # [n_q, H, D]
    q_seq: torch.Tensor      # [n_q] int32
    q_pos: torch.Tensor      # [n_q] int32
    q_pos_host: List[int]
    x_new: torch.Tensor      # [n_new, D] raw tokens of the new chunk
    gate_new: torch.Tensor   # [n_new] float32 gate logits
    swa: PagedTensors        # prior tail drawn; new positions to be inserted
    c4: PagedTensors         # prior entries drawn; new entries to be compressed into it
    c128: PagedTensors
    idx_q: torch.Tensor      # [n_q, H_I, D_I]
    idx_w: torch.Tensor      # [n_q, H_I]
    idx_pool: PagedTensors   # prior and new indexer keys, drawn directly
    prior: int
    n_new: int
    k: int = 512
    window: int = 128
    rope_dim: int = 64
    rope_base: float = 10000.0


def chunked_prefill(device, seed: int = 0, prior: int = 65536, n_new: int = 4096,
                    n_heads: int = 64, dim: int = 512, rope_dim: int = 64, idx_heads: int = 64,
                    idx_dim: int = 128, k: int = 512, window: int = 128, dtype: str = "bf16",
                    workload_id: int = 4) -> Prefill:
    g = generator(workload_id, seed, 0, device)
    total = prior + n_new
    mb = -(-total // BLOCK_POSITIONS)
    q = to_storage(randn((n_new, n_heads, dim), g, device), dtype)
    idx_q = to_storage(randn((n_new, idx_heads, idx_dim), g, device), dtype)
    idx_w = randn((n_new, idx_heads), g, device) / math.sqrt(128.0)
    x_new = to_storage(randn((n_new, dim), g, device), dtype)
    gate_new = randn((n_new,), g, device)
    pos = list(range(prior, total))
    swa = make_pool(dtype, dim, 1, [blocks_for_positions(max(0, prior - window), total)], mb,
                    generator(workload_id, seed, 1, device), device)
    c4 = make_pool(dtype, dim, 4, [blocks_for_entries(total // 4, 4)], mb,
                   generator(workload_id, seed, 2, device), device)
    c128 = make_pool(dtype, dim, 128, [blocks_for_entries(total // 128, 128)], mb,
                     generator(workload_id, seed, 3, device), device)
    idx_pool = make_pool(dtype, idx_dim, 4, [blocks_for_entries(total // 4, 4)], mb,
                         generator(workload_id, seed, 4, device), device)
    return Prefill(q, _ints([0] * n_new, device), _ints(pos, device), pos, x_new, gate_new, swa,
                   c4, c128, idx_q, idx_w, idx_pool, prior, n_new, k=k, window=window,
                   rope_dim=rope_dim)


@dataclass
class TinyDecode:
    """Tiny all-fp32 C4 decode built from raw tokens: x -> SWA entries and C4 entries."""

    x: torch.Tensor          # [T, D] raw tokens, positions 0..T-1
    q: torch.Tensor          # [1, H, D]
    idx_q: torch.Tensor      # [1, H_I, D_I]
    idx_w: torch.Tensor      # [1, H_I]
    idx_pool: PagedTensors   # drawn directly
    swa: PagedTensors        # empty, to be filled from x
    comp: PagedTensors       # empty, to be filled from x
    seq_lens: torch.Tensor
    seq_lens_host: List[int]
    k: int = 64
    window: int = 128
    rope_dim: int = 16
    rope_base: float = 10000.0


def tiny_decode(device, seed: int = 0, ctx: int = 1024, n_heads: int = 8, dim: int = 64,
                rope_dim: int = 16, idx_heads: int = 4, idx_dim: int = 32, k: int = 64,
                window: int = 128, workload_id: int = 1, shuffle: bool = True) -> TinyDecode:
    g = generator(workload_id, seed, 0, device)
    x = randn((ctx, dim), g, device)
    q = randn((1, n_heads, dim), g, device)
    idx_q = randn((1, idx_heads, idx_dim), g, device)
    idx_w = torch.ones(1, idx_heads, dtype=torch.float32, device=device)
    mb = -(-ctx // BLOCK_POSITIONS)
    need = [blocks_for_positions(0, ctx)]
    swa = make_pool("f32", dim, 1, need, mb, generator(workload_id, seed, 1, device), device,
                    fill=False, shuffle=shuffle)
    comp = make_pool("f32", dim, 4, [blocks_for_entries(ctx // 4, 4)], mb,
                     generator(workload_id, seed, 2, device), device, fill=False, shuffle=shuffle)
    idx_pool = make_pool("f32", idx_dim, 4, [blocks_for_entries(ctx // 4, 4)], mb,
                         generator(workload_id, seed, 3, device), device, shuffle=shuffle)
    return TinyDecode(x, q, idx_q, idx_w, idx_pool, swa, comp, _ints([ctx], device), [ctx], k=k,
                      window=window, rope_dim=rope_dim)


def quantized_mixed(device, seed: int = 0, batch: int = 64, n_heads: int = 64, dim: int = 512,
                    rope_dim: int = 64, idx_heads: int = 64, idx_dim: int = 128, k: int = 512,
                    window: int = 128, lens: Optional[Sequence[int]] = None,
                    workload_id: int = 5):
    """Mixed-length batch, fp8 attention caches, fp4 indexer cache: (C4 step, C128 step)."""
    g = generator(workload_id, seed, 0, device)
    if lens is None:
        lens = mixed_lengths(batch, g)
    c4 = sparse_decode(device, seed, batch, list(lens), n_heads, dim, rope_dim, idx_heads, idx_dim,
                       k, window, dtype="fp8", idx_dtype="fp4", workload_id=workload_id * 10 + 1)
    c128 = dense_decode(device, seed, batch, list(lens), n_heads, dim, rope_dim, window,
                        dtype="fp8", workload_id=workload_id * 10 + 2)
    c4.name, c128.name = "quant_c4_decode", "quant_c128_decode"
    return c4, c128


@dataclass
class MultiDecode:
    """Multi-query decode (the verify pass of speculative decoding): n_tok query tokens per
    sequence at the last n_tok positions of its context, in the prefill form (q_seq, q_pos). The
    pools already hold every position (the new tokens' raw window entries included); x_new holds
    the new tokens' raw values for the compressor."""

    q: torch.Tensor          # [B * n_tok, H, D], sequence-major
    q_seq: torch.Tensor      # [B * n_tok] int32
    q_pos: torch.Tensor      # [B * n_tok] int32
    q_pos_host: List[int]
    lens: List[int]
    n_tok: int
    swa: PagedTensors
    comp: PagedTensors
    idx_q: torch.Tensor      # [B * n_tok, H_I, D_I]
    idx_w: torch.Tensor      # [B * n_tok, H_I]
    idx_pool: PagedTensors
    x_new: torch.Tensor      # [B * n_tok, D] raw tokens at the query positions
    k: int = 512
    window: int = 128
    rope_dim: int = 64
    rope_base: float = 10000.0

    @property
    def n_q(self) -> int:
        return int(self.q.shape[0])


def multi_decode(device, seed: int = 0, batch: int = 16, ctx=131072, n_tok: int = 2,
                 n_heads: int = 64, dim: int = 512, rope_dim: int = 64, idx_heads: int = 64,
                 idx_dim: int = 128, k: int = 512, window: int = 128, dtype: str = "bf16",
                 workload_id: int = 6) -> MultiDecode:
    """C4 multi-query decode: the pools of a C4 sparse decode batch, n_tok queries per sequence."""
    base = sparse_decode(device, seed, batch, ctx, n_heads, dim, rope_dim, idx_heads, idx_dim, k,
                         window, dtype=dtype, workload_id=workload_id)
    lens = base.seq_lens_host
    g = generator(workload_id, seed, 5, device)
    n_q = batch * n_tok
    qdt = "bf16" if dtype in ("bf16", "fp8") else dtype
    q = to_storage(randn((n_q, n_heads, dim), g, device), qdt)
    idx_q = to_storage(randn((n_q, idx_heads, idx_dim), g, device), qdt)
    idx_w = randn((n_q, idx_heads), g, device) / math.sqrt(128.0)
    x_new = to_storage(randn((n_q, dim), g, device), qdt)
    seqs = [b for b in range(batch) for _ in range(n_tok)]
    pos = [lens[b] - n_tok + t for b in range(batch) for t in range(n_tok)]
    return MultiDecode(q, _ints(seqs, device), _ints(pos, device), pos, lens, n_tok, base.swa,
                       base.comp, idx_q, idx_w, base.idx_pool, x_new, k=k, window=window,
                       rope_dim=rope_dim)
