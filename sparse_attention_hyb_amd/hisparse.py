"""C4 pool offload with a device working set (HiSparse-style).

DeepSeek-V4 launch review (SGLang / Miles day-0 blog, section "HiSparse"): the C4 layer's whole
compressed KV cache lives in a pinned CPU mirror, the GPU keeps only a small buffer for the active
working set, and every step the coordinator brings in the pages the step misses from the CPU and
evicts inactive GPU pages by LRU; newly produced entries are backed up to the CPU mirror. The
indexer's top-k touches a small part of the compressed positions at each step, so most C4 entries
stay inactive. The C128 pool (dense: every entry is read) and the window pool (128 entries) stay
on the device.

Here a page is one logical block of the C4 pool (256 native positions = 64 entries). The working
set is a device pool of `slots` pages whose block table maps each sequence's logical blocks to
slots (-1 = not resident), so the attention kernels read it like any pool: the step runs
`hyb_attn_decode` with `pool()` as its compressed pool. The coordinator is host code: `admit` takes
the step's top-k rows (on the host), copies the missing pages from the mirror (asynchronous
host -> device copies on the given stream) and updates the block table; `write_back` copies pages
the step changed (the one that receives a new entry) back to the mirror.
"""

from dataclasses import dataclass
from typing import Iterable, List, Optional, Tuple

import numpy as np
import torch

from .workloads import BLOCK_POSITIONS, PagedTensors


@dataclass
class AdmitStats:
    pages: int      # distinct pages the step needs
    misses: int     # of those, copied from the mirror
    bytes: int      # bytes copied host -> device


class C4Offload:
    """Pinned host mirror of a C4 pool plus a device working set of `slots` pages (LRU)."""

    def __init__(self, mirror: PagedTensors, slots: int, device="cuda"):
        if mirror.ratio != 4:
            raise ValueError("the offload takes a C4 pool (ratio 4)")
        if mirror.scale is not None:
            raise ValueError("fp8 mirrors: not supported by this coordinator")
        self.mirror = mirror                              # data on the host (pinned), table on the host
        self.table = mirror.block_table.cpu().numpy()     # logical block -> mirror block
        self.per = BLOCK_POSITIONS // 4
        self.slots = int(slots)
        self.device = torch.device(device)
        shape = (self.slots,) + tuple(mirror.data.shape[1:])
        self.data = torch.zeros(shape, dtype=mirror.data.dtype, device=self.device)
        self.dev_table_host = np.full(self.table.shape, -1, dtype=np.int32)
        pin = self.device.type == "cuda"
        self._table_stage = torch.empty(self.table.shape, dtype=torch.int32, pin_memory=pin)
        self.dev_table = torch.full(self.table.shape, -1, dtype=torch.int32, device=self.device)
        self.owner: List[Optional[Tuple[int, int]]] = [None] * self.slots   # slot -> (seq, block)
        self.where = {}                                                       # (seq, block) -> slot
        self.stamp = np.zeros(self.slots, dtype=np.int64)
        self.clock = 0

    def pool(self) -> PagedTensors:
        """The working set as a pool for the attention entry points."""
        return PagedTensors(self.data, None, self.dev_table, self.mirror.dtype, self.mirror.dim, 4)

    def pages_of(self, topk_rows: np.ndarray) -> List[Tuple[int, int]]:
        """Distinct (sequence, logical block) pages that top-k rows [B, k] select (-1 ignored)."""
        need = set()
        for b, row in enumerate(np.asarray(topk_rows)):
            for lb in np.unique(row[row >= 0] // self.per):
                need.add((b, int(lb)))
        return sorted(need)

    def admit(self, topk_rows: np.ndarray, extra: Iterable[Tuple[int, int]] = (),
              stream: Optional[torch.cuda.Stream] = None) -> AdmitStats:
        """Make every page the rows select (and `extra` pages) resident; evict least recently used
        pages that this step does not need. Copies run on `stream` (the current one by default)
        before the block table update, so work queued after this call on that stream sees them."""
        need = sorted(set(self.pages_of(topk_rows)) | {(int(b), int(lb)) for b, lb in extra})
        if len(need) > self.slots:
            raise RuntimeError(f"step needs {len(need)} pages, working set holds {self.slots}")
        self.clock += 1
        needed = set(need)
        misses = [pg for pg in need if pg not in self.where]
        for pg in need:
            if pg in self.where:
                self.stamp[self.where[pg]] = self.clock
        free = [s for s in range(self.slots) if self.owner[s] is None]
        # eviction order: least recently used first, among pages this step does not need
        victims = sorted((s for s in range(self.slots)
                          if self.owner[s] is not None and self.owner[s] not in needed),
                         key=lambda s: self.stamp[s])
        nbytes = 0
        ctx = torch.cuda.stream(stream) if stream is not None else _nullctx()
        with ctx:
            for pg in misses:
                if free:
                    s = free.pop()
                else:
                    s = victims.pop(0)
                    old = self.owner[s]
                    del self.where[old]
                    self.dev_table_host[old] = -1
                b, lb = pg
                src = int(self.table[b, lb])
                if src < 0:
                    raise RuntimeError(f"page {pg} is not in the mirror")
                self.data[s].copy_(self.mirror.data[src], non_blocking=True)
                nbytes += self.data[s].numel() * self.data[s].element_size()
                self.owner[s] = pg
                self.where[pg] = s
                self.stamp[s] = self.clock
                self.dev_table_host[pg] = s
            self._table_stage.copy_(torch.from_numpy(self.dev_table_host))
            self.dev_table.copy_(self._table_stage, non_blocking=True)
        return AdmitStats(len(need), len(misses), nbytes)

    def write_back(self, pages: Iterable[Tuple[int, int]],
                   stream: Optional[torch.cuda.Stream] = None) -> None:
        """Copy resident pages (e.g. the one that received this step's new entry) to the mirror,
        asynchronously on `stream`."""
        ctx = torch.cuda.stream(stream) if stream is not None else _nullctx()
        with ctx:
            for pg in pages:
                s = self.where[(int(pg[0]), int(pg[1]))]
                self.mirror.data[int(self.table[pg])].copy_(self.data[s], non_blocking=True)


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False
