"""hyb_set_error_word: kernels report block-table entries >= num_blocks in a caller's device word
and still treat them as absent; with the word unset nothing is written."""

import pytest
import torch

from sparse_attention_hyb_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32


def test_bad_page_ids_are_reported(gpu_lib):
    hyb = gpu_lib
    wl = W.sparse_decode(DEV, seed=41, batch=2, ctx=[9000, 20000])
    L = wl.max_seq_len
    word = torch.zeros(1, dtype=I32, device=DEV)
    topk = torch.empty(2, wl.k, dtype=I32, device=DEV)
    out = torch.empty_like(wl.q)
    ref_topk = torch.empty_like(topk)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.seq_lens - 1, L - 1, wl.idx_pool, wl.k, ref_topk)
    try:
        hyb.hyb_set_error_word(word)
        # clean tables: nothing reported
        hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.seq_lens - 1, L - 1, wl.idx_pool, wl.k, topk)
        hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out, topk_idx=topk, k=wl.k)
        torch.cuda.synchronize()
        assert int(word.item()) == 0
        assert torch.equal(topk, ref_topk)
        # an indexer-key block of sequence 1 points past the pool: reported, and its entries
        # score -inf (never chosen while enough other entries exist)
        bt = wl.idx_pool.block_table
        saved = bt[1, 3].item()
        bt[1, 3] = wl.idx_pool.data.shape[0] + 5
        hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.seq_lens - 1, L - 1, wl.idx_pool, wl.k, topk)
        torch.cuda.synchronize()
        assert int(word.item()) == hyb.ERR_BAD_PAGE
        per = 64   # C4 entries per block
        row = topk[1].cpu().numpy()
        assert not ((row >= 3 * per) & (row < 4 * per)).any()
        bt[1, 3] = saved
        # a window block of the attention's raw pool
        word.zero_()
        sbt = wl.swa.block_table
        lb = (wl.seq_lens_host[0] - 1) // 256
        saved = sbt[0, lb].item()
        sbt[0, lb] = wl.swa.data.shape[0] + 1
        hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out, topk_idx=ref_topk, k=wl.k)
        torch.cuda.synchronize()
        assert int(word.item()) == hyb.ERR_BAD_PAGE
        sbt[0, lb] = saved
        # detection off: nothing written
        word.zero_()
        hyb.hyb_set_error_word(None)
        bt[1, 3] = wl.idx_pool.data.shape[0] + 5
        hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.seq_lens - 1, L - 1, wl.idx_pool, wl.k, topk)
        torch.cuda.synchronize()
        assert int(word.item()) == 0
        bt[1, 3] = saved
    finally:
        hyb.hyb_set_error_word(None)


def test_decode_steps_report_nothing_on_clean_inputs(gpu_lib):
    """With the error word set, C4 and C128 decode steps over clean tables (mixed lengths, three
    calls each) leave it zero."""
    hyb = gpu_lib
    word = torch.zeros(1, dtype=I32, device=DEV)
    c4 = W.sparse_decode(DEV, seed=42, batch=11, ctx=[131072] * 6 + [9000, 20000, 3000, 70000, 65536])
    c128 = W.dense_decode(DEV, seed=43, batch=9, ctx=[1 << 20] * 4 + [5000, 300000, 40000, 2048, 131072])
    try:
        hyb.hyb_set_error_word(word)
        for _ in range(3):
            out = torch.empty_like(c4.q)
            hyb.hyb_decode_step(c4.q, c4.seq_lens, c4.max_seq_len, c4.swa, c4.comp, out, idx_q=c4.idx_q,
                                idx_w=c4.idx_w, idx_pool=c4.idx_pool, k=c4.k)
            out = torch.empty_like(c128.q)
            hyb.hyb_decode_step(c128.q, c128.seq_lens, c128.max_seq_len, c128.swa, c128.comp, out)
        torch.cuda.synchronize()
        assert int(word.item()) == 0
    finally:
        hyb.hyb_set_error_word(None)
