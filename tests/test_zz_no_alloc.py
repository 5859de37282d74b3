"""The allocation-free selector (hyb_index_topk_noalloc, scratch in the library's static per-GPU
array) against hyb_index_topk with a caller workspace: the same top-k rows bit for bit, on two
calls in a row, the second with a smaller input (so the array holds the first call's contents
when the second starts), and a sampled row against the float64 oracle."""

import pytest
import torch

import oracle as O
from sparse_attention_hyb_amd import workloads as W
from tests.conftest import to_f64, to_oracle_pool
from tests.parity_util import check_topk_set, topk_delta

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(hyb, wl):
    qpos = (wl.seq_lens - 1).contiguous()
    ref = torch.full((wl.batch, wl.k), -7, dtype=torch.int32, device=DEV)
    got = torch.full((wl.batch, wl.k), -9, dtype=torch.int32, device=DEV)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, qpos, wl.max_seq_len - 1, wl.idx_pool, wl.k, ref)
    hyb.hyb_index_topk_noalloc(wl.idx_q, wl.idx_w, qpos, wl.max_seq_len - 1, wl.idx_pool, wl.k, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_index_topk_equals_workspace_form(gpu_lib):
    hyb = gpu_lib
    big = W.sparse_decode(DEV, seed=3, batch=4, ctx=[40000, 131072, 9000, 70001])
    ref, got = _both(hyb, big)
    assert torch.equal(ref, got)
    # one row against the oracle (fp32-bound protocol on N(0,1) inputs)
    ip = to_oracle_pool(big.idx_pool)
    b, p = 2, big.seq_lens_host[2] - 1
    keys = O.pool_entries(ip, b, range(O.n_visible(p, 4, 128)))
    iq, iw = to_f64(big.idx_q)[b], big.idx_w[b].cpu().double().numpy()
    sc = O.indexer_scores(iq, iw, keys)
    check_topk_set(got[b].cpu().numpy(), O.topk_select(sc, big.k), sc, topk_delta(iq, iw, keys), big.k)
    # second call, smaller: 2 sequences, one shorter than k + the window (padded rows)
    small = W.sparse_decode(DEV, seed=4, batch=2, ctx=[5000, 2000])
    ref2, got2 = _both(hyb, small)
    assert torch.equal(ref2, got2)
    assert (got2[1] == -1).any()   # 468 visible entries < k = 512: padded
