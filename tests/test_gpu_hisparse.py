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
