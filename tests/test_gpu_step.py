"""The decode step on two streams (query prep, window insert and indexer-key compression beside the
indexer) and as one captured HIP graph: both give the serial eager step's results bit for bit, a
replay follows new sequence lengths written to the device-side metadata, and sampled sequences
match the float64 oracle, which rebuilds every input the step derives (rotated query, window
entries, compressed entries and indexer keys) from the step's raw inputs itself."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle.formats import bf16_bits_to_f64, round_to_bf16_bits
from sparse_attention_hyb_amd import workloads as W
from sparse_attention_hyb_amd.decode_step import DecodeStep, DecodeStepBuffers
from tests.conftest import to_f64, to_oracle_pool
from tests.parity_util import assert_abs_close, check_topk_set, topk_delta

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32
RD, BASE, EPS = 64, 1e4, 1e-6


def _buffers(hyb, lens, seed, grow=0, idx_compress=False):
    wl = W.sparse_decode(DEV, seed=seed, batch=len(lens), ctx=lens, grow=grow)
    B, D = wl.batch, wl.dim
    L = wl.max_seq_len + grow
    g = W.generator(97, seed, 0, DEV)
    kshape, hshape = hyb.index_keys_shapes(B, L - 1)
    di = wl.idx_q.shape[2]
    return wl, DecodeStepBuffers(
        q_raw=W.to_storage(W.randn((B, 64, D), g, DEV) * 3.0, "bf16"),
        kv_new=W.to_storage(W.randn((B, D), g, DEV), "bf16"),
        q=torch.empty_like(wl.q), seq_lens=wl.seq_lens.clone(),
        cu=torch.arange(0, B + 1, dtype=I32, device=DEV), start=(wl.seq_lens - 1).contiguous(),
        swa=wl.swa, comp=wl.comp, state=W.to_storage(W.randn((B, 4, D), g, DEV), "bf16"),
        out=torch.empty_like(wl.q),
        workspace=torch.zeros(hyb.hyb_attn_decode_workspace_bytes(B, 64, D, L, 4, wl.k),
                              dtype=torch.uint8, device=DEV),
        max_seq_len=L, idx_q=wl.idx_q, idx_w=wl.idx_w, idx_pool=wl.idx_pool,
        keys=torch.empty(kshape, dtype=I32, device=DEV),
        hist=torch.empty(hshape, dtype=torch.int16, device=DEV),
        topk=torch.empty(B, wl.k, dtype=I32, device=DEV), k=wl.k,
        idx_kv_new=W.to_storage(W.randn((B, di), g, DEV), "bf16") if idx_compress else None,
        idx_state=W.to_storage(W.randn((B, 4, di), g, DEV), "bf16") if idx_compress else None)


def _results(b):
    return [t.clone() for t in (b.out, b.topk, b.q, b.swa.data, b.comp.data, b.state)]


def _reset(b, pools):
    """Pools and state as before the first step; outputs cleared (eagerly, between replays)."""
    b.swa.data.copy_(pools[0])
    b.comp.data.copy_(pools[1])
    b.state.copy_(pools[2])
    b.out.zero_()
    b.q.zero_()
    b.topk.fill_(-7)
    torch.cuda.synchronize()


def _equal(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------------------------------------ oracle side
def _bf16(x64):
    """float64 -> the float64 value of its nearest-even bfloat16."""
    return bf16_bits_to_f64(round_to_bf16_bits(np.asarray(x64, np.float64)))


def _set_entry(pool, b, g, value64):
    """Store value64 (rounded to bf16) as entry g of sequence b of a bf16 oracle pool."""
    lb, slot = divmod(int(g), O.BLOCK_POSITIONS // pool.ratio)
    pool.data[int(pool.block_table[b, lb]), slot] = round_to_bf16_bits(np.asarray(value64, np.float64))


def _check_step(hyb, buf, b, q64, p, swa_o, comp_o, idx_o, idx_q, idx_w):
    """Sequence b of the step just run: the GPU's top-k against the oracle's (fp32-bound protocol)
    and the GPU's output against the oracle's attention over the oracle's selection. Should a
    near-tie make the two selections differ, the GPU attention is re-run on the step's pools with
    the oracle's selection fed in, so that the output is compared in every case."""
    k = buf.k
    nv = O.n_visible(p, 4, 128)
    keys = O.pool_entries(idx_o, b, range(nv))
    sc = O.indexer_scores(idx_q, idx_w, keys)
    sel = O.topk_select(sc, k)
    got_topk = buf.topk[b].cpu().numpy()
    check_topk_set(got_topk, sel, sc, topk_delta(idx_q, idx_w, keys), k)
    want = O.hybrid_query(q64, p, b, swa_o, comp_o, 128, 1.0 / math.sqrt(q64.shape[-1]), RD, BASE,
                          sel)
    got = to_f64(buf.out[b])
    if [int(v) for v in got_topk] != [int(v) for v in sel]:
        feed = torch.full(tuple(buf.topk.shape), -1, dtype=I32)
        feed[b] = torch.from_numpy(np.asarray(sel, np.int32))
        out = torch.empty_like(buf.out)
        hyb.hyb_attn_decode(buf.q, buf.seq_lens, buf.max_seq_len, buf.swa, buf.comp, out,
                            topk_idx=feed.to(DEV), k=k)
        torch.cuda.synchronize()
        got = to_f64(out[b])
    assert_abs_close(got, want)


def test_decode_step_two_streams_and_graph(gpu_lib):
    hyb = gpu_lib
    wl, b = _buffers(hyb, [4096, 8191, 20000, 65535], seed=5)   # groups complete for 2 of 4
    pools = (b.swa.data.clone(), b.comp.data.clone(), b.state.clone())
    swa_o, comp_o, idx_o = to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), to_oracle_pool(wl.idx_pool)
    step = DecodeStep(b)
    _reset(b, pools)
    step.run_serial()
    torch.cuda.synchronize()
    want = _results(b)
    assert not torch.equal(want[4], pools[1])   # completed groups were compressed
    assert not torch.equal(want[3], pools[0])   # window entries were inserted
    # sampled sequences against the oracle: it rotates the raw query and inserts the new window
    # entry itself (from the step's raw inputs), then selects and attends
    q_raw, kv = to_f64(b.q_raw), to_f64(b.kv_new)
    iq, iw = to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy()
    for s in (0, 3):
        p = wl.seq_lens_host[s] - 1
        q64 = _bf16(O.q_norm_rope(q_raw[s][None], [p], RD, BASE, EPS)[0])
        _set_entry(swa_o, s, p, O.swa_entries(kv[s][None], [p], RD, BASE)[0])
        _check_step(hyb, b, s, q64, p, swa_o, comp_o, idx_o, iq[s], iw[s])
    _reset(b, pools)
    step.run()
    torch.cuda.synchronize()
    assert _equal(_results(b), want)
    graph = step.capture()
    for rep in range(3):
        _reset(b, pools)
        graph.replay()
        torch.cuda.synchronize()
        assert _equal(_results(b), want), rep
    # device-side metadata: two sequences move back by 3 and 1 tokens; replay = eager serial
    b.seq_lens[1:3] -= torch.tensor([3, 1], dtype=I32, device=DEV)
    b.start.copy_(b.seq_lens - 1)
    _reset(b, pools)
    step.run_serial()
    torch.cuda.synchronize()
    want2 = _results(b)
    assert not torch.equal(want2[0], want[0])
    _reset(b, pools)
    graph.replay()
    torch.cuda.synchronize()
    assert _equal(_results(b), want2)


def test_decode_steps_past_the_window_match_oracle(gpu_lib):
    """140 consecutive two-stream decode steps of three sequences (4093, 9000 and 20001 tokens at
    the start, so the compressor rings start at three different fill levels). Each step inserts
    its token's window entry, compresses its token into the C4 pool and its indexer-key row into
    the indexer-key pool, selects and attends. After 140 steps the window holds only entries the
    run inserted and the first groups the run completed have become visible, so the last step's
    top-k and output depend on what every earlier step wrote. The oracle rebuilds those entries
    from the raw inputs (drawn rings, the steps' tokens) and checks the pools and the last step."""
    hyb = gpu_lib
    lens0, n = [4093, 9000, 20001], 140
    wl, b = _buffers(hyb, lens0, seed=11, grow=n, idx_compress=True)
    B, D = wl.batch, wl.dim
    di = b.idx_kv_new.shape[1]
    swa_o, comp_o, idx_o = to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), to_oracle_pool(wl.idx_pool)
    g = W.generator(96, 0, 0, DEV)
    q_all = W.to_storage(W.randn((n, B, 64, D), g, DEV) * 3.0, "bf16")
    kv_all = W.to_storage(W.randn((n, B, D), g, DEV), "bf16")
    ikv_all = W.to_storage(W.randn((n, B, di), g, DEV), "bf16")
    ring0, iring0 = to_f64(b.state), to_f64(b.idx_state)
    lens = torch.tensor(lens0, dtype=I32, device=DEV)
    step = DecodeStep(b)
    for t in range(n):
        b.q_raw.copy_(q_all[t])
        b.kv_new.copy_(kv_all[t])
        b.idx_kv_new.copy_(ikv_all[t])
        b.seq_lens.copy_(lens + t)
        b.start.copy_(lens + t - 1)
        step.run()
    torch.cuda.synchronize()
    q64_all, kv64, ikv64 = to_f64(q_all), to_f64(kv_all), to_f64(ikv_all)
    iq, iw = to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy()
    swa_g, comp_g, idx_g = to_oracle_pool(b.swa), to_oracle_pool(b.comp), to_oracle_pool(b.idx_pool)
    for s in (0, 2):
        p0, pf = lens0[s] - 1, lens0[s] - 2 + n
        for t in range(n):
            _set_entry(swa_o, s, p0 + t, O.swa_entries(kv64[t, s][None], [p0 + t], RD, BASE)[0])
        # raw tokens by position: the drawn ring holds the in-progress group's first p0 % 4
        tok = {4 * (p0 // 4) + j: ring0[s, j] for j in range(p0 % 4)}
        itok = {4 * (p0 // 4) + j: iring0[s, j] for j in range(p0 % 4)}
        tok.update({p0 + t: kv64[t, s] for t in range(n)})
        itok.update({p0 + t: ikv64[t, s] for t in range(n)})
        groups = list(range(p0 // 4, (pf + 1) // 4))
        for gi in groups:
            ent = O.compressed_entry(np.stack([tok[4 * gi + j] for j in range(4)]), None, gi, 4,
                                     "mean", RD, BASE, EPS)
            ient = O.compressed_entry(np.stack([itok[4 * gi + j] for j in range(4)]), None, gi, 4,
                                      "mean", RD, BASE, EPS)
            _set_entry(comp_o, s, gi, ent)
            _set_entry(idx_o, s, gi, ient)
        # what the run wrote: window entries, compressed entries and indexer keys
        assert_abs_close(O.pool_entries(swa_g, s, range(p0, pf + 1)), O.pool_entries(swa_o, s, range(p0, pf + 1)))
        assert_abs_close(O.pool_entries(comp_g, s, groups), O.pool_entries(comp_o, s, groups))
        assert_abs_close(O.pool_entries(idx_g, s, groups), O.pool_entries(idx_o, s, groups))
        assert O.n_visible(pf, 4, 128) > groups[0] + 1   # the run's first groups are visible
        q64 = _bf16(O.q_norm_rope(q64_all[n - 1, s][None], [pf], RD, BASE, EPS)[0])
        _check_step(hyb, b, s, q64, pf, swa_o, comp_o, idx_o, iq[s], iw[s])
