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
`hyb_attn_decode` with `pool()` as its compressed pool. Two coordinators, one per instance:
  * device (`device=True`): `admit_device` hands the step's top-k rows, still on the device, to
    `hyb_offload_admit`, which finds the missing pages, picks the victims and copies the pages in
    the step's stream (no host read-back, nothing on the host but the step counter);
    `write_back_device` backs each new entry up to the mirror with `hyb_offload_write_back`;
  * host: `admit` takes the rows on the host (a read-back), decides with numpy and copies the
    pages with one gather launch; `write_back` copies changed pages back.
Both follow one rule: the needed pages that miss, in ascending key order, take the least recently
used slots the step does not need (smallest stamp, then lowest slot), the i-th page the i-th of
those slots in slot order; so their tables and working sets agree step for step.
"""

from dataclasses import dataclass
from typing import Iterable, Optional, Tuple

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

    def __init__(self, mirror: PagedTensors, slots: int, device="cuda", device_admission: bool = False):
        if mirror.ratio != 4:
            raise ValueError("the offload takes a C4 pool (ratio 4)")
        if mirror.dtype not in ("bf16", "f32", "fp8"):
            raise ValueError(f"{mirror.dtype} C4 mirrors are not supported")
        self.mirror = mirror                              # data on the host (pinned), table on the host
        self.table = mirror.block_table.cpu().numpy()     # logical block -> mirror block
        self.per = BLOCK_POSITIONS // 4
        self.slots = int(slots)
        self.device = torch.device(device)
        shape = (self.slots,) + tuple(mirror.data.shape[1:])
        self.data = torch.zeros(shape, dtype=mirror.data.dtype, device=self.device)
        # fp8 pools: each page's per-entry scales travel with its codes
        self.scale = None if mirror.scale is None else torch.ones(
            (self.slots,) + tuple(mirror.scale.shape[1:]), dtype=mirror.scale.dtype, device=self.device)
        self.dev_table_host = np.full(self.table.shape, -1, dtype=np.int32)
        pin = self.device.type == "cuda"
        self._table_stage = torch.empty(self.table.shape, dtype=torch.int32, pin_memory=pin)
        self.dev_table = torch.full(self.table.shape, -1, dtype=torch.int32, device=self.device)
        # pages copied by one gather launch (hyb_gather_pages) when the mirror is pinned and the
        # working set is on the GPU; page lists staged through pinned memory
        self.one_launch = (pin and mirror.data.is_pinned() and mirror.data.is_contiguous() and
                           (mirror.scale is None or (mirror.scale.is_pinned() and mirror.scale.is_contiguous())))
        if self.one_launch:
            self._idx_stage = torch.empty((2, self.slots), dtype=torch.int32, pin_memory=True)
            self._idx_dev = torch.empty((2, self.slots), dtype=torch.int32, device=self.device)
        self.owner = np.full(self.slots, -1, dtype=np.int64)   # slot -> page key seq * max_blocks + block
        self.stamp = np.zeros(self.slots, dtype=np.int64)       # last step that needed the slot's page
        self.clock = 0
        self.device_admission = bool(device_admission)
        if self.device_admission:
            # the device coordinator's state: slot owners and stamps, the mirror's table, the
            # admission workspace (zero before the first call) and its per-step result
            from . import hyb_offload_workspace_bytes
            self.owner_dev = torch.full((self.slots,), -1, dtype=torch.int32, device=self.device)
            self.stamp_dev = torch.zeros(self.slots, dtype=torch.int32, device=self.device)
            self.mirror_table_dev = mirror.block_table.to(device=self.device, dtype=torch.int32).contiguous()
            nb = hyb_offload_workspace_bytes(self.table.shape[0], self.table.shape[1], self.slots)
            self._ws = torch.zeros(nb, dtype=torch.uint8, device=self.device)
            self.result = torch.zeros(2, dtype=torch.int32, device=self.device)

    @property
    def where(self) -> dict:
        """Resident pages: (sequence, logical block) -> slot."""
        mb = self.table.shape[1]
        return {(int(k // mb), int(k % mb)): int(s) for s, k in enumerate(self.owner) if k >= 0}

    def pool(self) -> PagedTensors:
        """The working set as a pool for the attention entry points."""
        return PagedTensors(self.data, self.scale, self.dev_table, self.mirror.dtype, self.mirror.dim, 4)

    def page_keys(self, topk_rows: np.ndarray) -> np.ndarray:
        """Sorted distinct page keys (sequence * max_blocks + logical block) that top-k rows
        [B, k] select (-1 entries ignored)."""
        rows = np.asarray(topk_rows, dtype=np.int64)
        seq = np.broadcast_to(np.arange(rows.shape[0])[:, None], rows.shape)
        sel = rows >= 0
        return np.unique(seq[sel] * self.table.shape[1] + rows[sel] // self.per)

    def admit(self, topk_rows: np.ndarray, extra: Iterable[Tuple[int, int]] = (),
              stream: Optional[torch.cuda.Stream] = None) -> AdmitStats:
        """Make every page the rows select (and `extra` pages) resident; evict least recently used
        pages that this step does not need. Copies run on `stream` (the current one by default)
        before the block table update, so work queued after this call on that stream sees them.
        Calls are ordered by the caller's read-back of each step's top-k rows (a host sync)."""
        mb = self.table.shape[1]
        need = self.page_keys(topk_rows)
        ext = [int(b) * mb + int(lb) for b, lb in extra]
        if ext:
            need = np.union1d(need, np.asarray(ext, dtype=np.int64))
        if need.size > self.slots:
            raise RuntimeError(f"step needs {need.size} pages, working set holds {self.slots}")
        self.clock += 1
        flat = self.dev_table_host.reshape(-1)
        cur = flat[need]
        hit = cur >= 0
        self.stamp[cur[hit]] = self.clock
        miss = need[~hit]
        free = np.flatnonzero(self.owner < 0)
        if miss.size > free.size:
            # least recently used first, among resident pages this step does not need
            keep = np.zeros(self.slots, dtype=bool)
            keep[cur[hit]] = True
            cand = np.flatnonzero((self.owner >= 0) & ~keep)
            victims = cand[np.argsort(self.stamp[cand], kind="stable")[:miss.size - free.size]]
            flat[self.owner[victims]] = -1
            self.owner[victims] = -1
            slots = np.concatenate([free, victims])
        else:
            slots = free[:miss.size]
        slots = np.sort(slots)   # the i-th missing page (ascending key) takes the i-th slot
        src = self.table.reshape(-1)[miss]
        if (src < 0).any():
            raise RuntimeError("a selected page is not in the mirror")
        page = self.data[0].numel() * self.data.element_size()
        if self.scale is not None:
            page += self.scale[0].numel() * self.scale.element_size()
        nbytes = page * int(miss.size)
        ctx = torch.cuda.stream(stream) if stream is not None else _nullctx()
        with ctx:
            if self.one_launch and miss.size:
                from . import hyb_gather_pages
                m = int(miss.size)
                self._idx_stage[0, :m].copy_(torch.from_numpy(src.astype(np.int32)))
                self._idx_stage[1, :m].copy_(torch.from_numpy(slots.astype(np.int32)))
                self._idx_dev[:, :m].copy_(self._idx_stage[:, :m], non_blocking=True)
                hyb_gather_pages(self.mirror.data, self.data, self._idx_dev[0, :m], self._idx_dev[1, :m],
                                 stream=stream)
                if self.scale is not None:
                    hyb_gather_pages(self.mirror.scale, self.scale, self._idx_dev[0, :m],
                                     self._idx_dev[1, :m], stream=stream)
            else:
                for sl, sb in zip(slots.tolist(), src.tolist()):
                    self.data[sl].copy_(self.mirror.data[sb], non_blocking=True)
                    if self.scale is not None:
                        self.scale[sl].copy_(self.mirror.scale[sb], non_blocking=True)
            self.owner[slots] = miss
            self.stamp[slots] = self.clock
            flat[miss] = slots
            self._table_stage.copy_(torch.from_numpy(self.dev_table_host))
            self.dev_table.copy_(self._table_stage, non_blocking=True)
        return AdmitStats(int(need.size), int(miss.size), nbytes)

    def admit_device(self, topk, extra=None, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Device coordinator: make every page the device rows topk [B, k] select (and the page
        keys in `extra`, an int32 device tensor) resident, in `stream` order, with no host
        read-back. self.result then holds (pages admitted, pages left out)."""
        from . import hyb_offload_admit
        if not self.device_admission:
            raise RuntimeError("this offload was built for host admission")
        self.clock += 1
        hyb_offload_admit(topk, self.dev_table, self.mirror_table_dev, self.owner_dev, self.stamp_dev,
                          self.clock, self.mirror.data, self.data, self._ws, self.result, extra=extra,
                          entries_per_page=self.per, mirror_scale_host=self.mirror.scale,
                          pool_scale=self.scale, stream=stream)

    def write_back_device(self, seq_lens, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Device coordinator: back up the entry each sequence completes at position
        seq_lens - 1 from its slot to the mirror (asynchronous to the host)."""
        from . import hyb_offload_write_back
        hyb_offload_write_back(seq_lens, 4, self.dev_table, self.mirror_table_dev, self.data,
                               self.mirror.data, entries_per_page=self.per, pool_scale=self.scale,
                               mirror_scale_host=self.mirror.scale, stream=stream)

    def write_back(self, pages: Iterable[Tuple[int, int]],
                   stream: Optional[torch.cuda.Stream] = None) -> None:
        """Copy resident pages (e.g. the one that received this step's new entry) to the mirror,
        asynchronously on `stream`."""
        ctx = torch.cuda.stream(stream) if stream is not None else _nullctx()
        with ctx:
            for b, lb in pages:
                s = int(self.dev_table_host[int(b), int(lb)])
                if s < 0:
                    raise RuntimeError(f"page {(b, lb)} is not resident")
                dst = int(self.table[int(b), int(lb)])
                self.mirror.data[dst].copy_(self.data[s], non_blocking=True)
                if self.scale is not None:
                    self.mirror.scale[dst].copy_(self.scale[s], non_blocking=True)


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False
