"""C4 offload (pinned host mirror + device working set): the attention over the working set equals
the attention over the device-resident pool bit for bit, step after step, while pages are
evicted and brought back, and sampled sequences match the float64 oracle (top-k and output)."""

import pytest
import torch

from sparse_attention_hyb_amd import workloads as W
from sparse_attention_hyb_amd.hisparse import C4Offload
from tests.conftest import to_f64, to_oracle_pool
from tests.parity_util import assert_abs_close, check_topk_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_c4_offload_equals_device_pool(gpu_lib, dtype):
    """Four sequences (20000, 50000, 131072 and 7000 tokens: 815 pages of 64 entries in all), a
    working set of 700 pages, and three decode steps whose indexer queries are drawn afresh, so
    each step selects about 600 pages, some of them evicted by the step before. fp8 pools bring
    each page's per-entry scales along."""
    hyb = gpu_lib
    from tests.test_gpu_parity import gpu_decode, gpu_topk, oracle_out, oracle_select
    lens = [20000, 50000, 131072, 7000]
    wl = W.sparse_decode(DEV, seed=6, batch=len(lens), ctx=lens, dtype=dtype)
    swa_o, comp_o, idx_o = to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), to_oracle_pool(wl.idx_pool)
    seqs = (1, 2)
    compared = 0
    mirror = W.PagedTensors(wl.comp.data.cpu().pin_memory(),
                            None if wl.comp.scale is None else wl.comp.scale.cpu().pin_memory(),
                            wl.comp.block_table.cpu(), wl.comp.dtype, wl.dim, 4)
    off = C4Offload(mirror, slots=700)
    g = W.generator(98, 0, 0, DEV)
    hits = 0
    for step in range(3):
        wl.idx_q = W.to_storage(W.randn(tuple(wl.idx_q.shape), g, DEV), "bf16")
        topk = gpu_topk(hyb, wl)
        st = off.admit(topk.cpu().numpy())
        assert st.pages <= 700
        hits += st.pages - st.misses
        want = gpu_decode(hyb, wl, topk)
        comp = wl.comp
        wl.comp = off.pool()
        got = gpu_decode(hyb, wl, topk)
        wl.comp = comp
        torch.cuda.synchronize()
        assert torch.equal(got, want), step
        # sampled sequences against the oracle: its own top-k and attention over its own pools
        # (the working set holds the pages of the GPU's selection, so the output is compared
        # where the two selections are equal; a near-tie swap is checked by the fp32 bound)
        sel = oracle_select(wl, idx_o, seqs)
        gt = topk.cpu().numpy()
        for b in seqs:
            check_topk_set(gt[b], sel[b][1], sel[b][0], sel[b][2], wl.k)
        same = [b for b in seqs if list(gt[b]) == list(sel[b][1])]
        if same:
            want_o = oracle_out(wl, swa_o, comp_o, same, {b: sel[b][1] for b in same})
            assert_abs_close(to_f64(got)[same], want_o)
            compared += len(same)
        # resident pages hold their mirror pages byte for byte (sampled)
        res = sorted(off.where.items())
        for (b, lb), s in res[::max(1, len(res) // 64)]:
            src = int(mirror.block_table[b, lb])
            assert torch.equal(off.data[s].cpu(), mirror.data[src]), (b, lb)
            if mirror.scale is not None:
                assert torch.equal(off.scale[s].cpu(), mirror.scale[src]), (b, lb)
    assert compared >= 3   # outputs were checked against the oracle in most steps
    assert off.one_launch   # the pinned mirror took the one-launch gather
    assert hits > 0   # later steps reuse resident pages


def test_gather_pages_refuses_pageable_memory(gpu_lib):
    """A host buffer that is not pinned has no device alias: the call fails on the host with
    HYB_EINVAL and launches nothing."""
    hyb = gpu_lib
    src = torch.zeros(4, 64, 16)                       # pageable
    dst = torch.zeros(4, 64, 16, device=DEV)
    idx = torch.arange(4, dtype=torch.int32, device=DEV)
    with pytest.raises(hyb.HybError) as e:
        hyb.hyb_gather_pages(src, dst, idx, idx)
    assert e.value.status == hyb.HYB_EINVAL
    torch.cuda.synchronize()
    assert torch.count_nonzero(dst) == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_device_admission_equals_host(gpu_lib, dtype):
    """The device coordinator (hyb_offload_admit: misses found, victims chosen and pages copied on
    the device, no read-back of the top-k) keeps the same block table, slot owners, stamps and
    resident pages as the host coordinator, step after step, with evictions; and the attention
    over its working set equals the attention over the resident pool bit for bit."""
    hyb = gpu_lib
    from tests.test_gpu_parity import gpu_decode, gpu_topk
    lens = [20000, 50000, 131072, 7000]
    wl = W.sparse_decode(DEV, seed=7, batch=len(lens), ctx=lens, dtype=dtype)
    mirror = W.PagedTensors(wl.comp.data.cpu().pin_memory(),
                            None if wl.comp.scale is None else wl.comp.scale.cpu().pin_memory(),
                            wl.comp.block_table.cpu(), wl.comp.dtype, wl.dim, 4)
    host = C4Offload(mirror, slots=700)
    dev = C4Offload(mirror, slots=700, device_admission=True)
    g = W.generator(97, 0, 0, DEV)
    evicted = 0
    for step in range(4):
        wl.idx_q = W.to_storage(W.randn(tuple(wl.idx_q.shape), g, DEV), "bf16")
        topk = gpu_topk(hyb, wl)
        st = host.admit(topk.cpu().numpy())
        dev.admit_device(topk)
        want = gpu_decode(hyb, wl, topk)
        comp = wl.comp
        wl.comp = dev.pool()
        got = gpu_decode(hyb, wl, topk)
        wl.comp = comp
        torch.cuda.synchronize()
        assert torch.equal(dev.dev_table, host.dev_table), step
        owner = dev.owner_dev.cpu().numpy()
        assert (owner == host.owner).all(), step
        assert (dev.stamp_dev.cpu().numpy() == host.stamp).all(), step
        res = dev.result.cpu().tolist()
        assert res == [st.misses, 0], (step, res, st)
        used = torch.from_numpy(owner >= 0)
        assert torch.equal(dev.data.cpu()[used], host.data.cpu()[used]), step
        if dev.scale is not None:
            assert torch.equal(dev.scale.cpu()[used], host.scale.cpu()[used]), step
        assert torch.equal(got, want), step
        evicted += int(step > 0 and st.misses > 0)
    assert evicted > 0   # later steps brought pages in over evicted ones


def test_device_write_back(gpu_lib):
    """hyb_offload_write_back copies the entry each sequence completes at its position from its
    resident slot to the mirror, and leaves sequences that complete none untouched."""
    hyb = gpu_lib
    lens = [20000, 50001, 8192]   # (p + 1) % 4 == 0 for sequences 0 and 2
    wl = W.sparse_decode(DEV, seed=8, batch=len(lens), ctx=lens)
    mirror = W.PagedTensors(wl.comp.data.cpu().pin_memory(), None, wl.comp.block_table.cpu(),
                            wl.comp.dtype, wl.dim, 4)
    before = mirror.data.clone()
    dev = C4Offload(mirror, slots=64, device_admission=True)
    mb = wl.comp.block_table.shape[1]
    keys = [b * mb + ((L // 4 - 1) if L % 4 == 0 else (L // 4)) // 64 for b, L in enumerate(lens)]
    extra = torch.tensor(keys, dtype=torch.int32, device=DEV)
    dev.admit_device(None, extra=extra)
    torch.cuda.synchronize()
    assert dev.result.cpu().tolist() == [3, 0]
    g = W.generator(96, 0, 0, DEV)
    rows = {}
    for b, L in enumerate(lens):
        lb = keys[b] - b * mb
        slot = int(dev.dev_table[b, lb])
        assert slot >= 0
        if L % 4 == 0:
            row = (L // 4 - 1) % 64
            new = W.to_storage(W.randn((wl.dim,), g, DEV), "bf16")
            dev.data[slot, row] = new
            rows[b] = (int(mirror.block_table[b, lb]), row, new.cpu())
    dev.write_back_device(wl.seq_lens)
    torch.cuda.synchronize()
    for b, (mp, row, new) in rows.items():
        assert torch.equal(mirror.data[mp, row], new), b
    changed = (mirror.data.view(torch.int16) != before.view(torch.int16)).any(dim=-1).nonzero().tolist()
    assert sorted(map(tuple, changed)) == sorted((mp, row) for mp, row, _ in rows.values())
