"""hyb_decode_step: a whole decode step of a C4 layer (indexer, top-k, attention, the new tokens
compressed into the C4 pool and into the indexer-key pool) or of a C128 layer (attention, the new
tokens compressed with softmax gates) in one call. Its results equal the separate calls made one
after another, bit for bit (outputs, top-k rows, pools and compressor rings), and sampled
sequences match the float64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_hyb_amd import workloads as W
from tests.conftest import to_f64, to_oracle_pool
from tests.parity_util import assert_abs_close, check_topk_set, topk_delta

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32


def _rings(B, D, r, dtype, g):
    return W.to_storage(W.randn((B, r, D), g, DEV), "bf16" if dtype == torch.bfloat16 else "f32")


def _clone_pool(p):
    return W.PagedTensors(p.data.clone(), None if p.scale is None else p.scale.clone(),
                          p.block_table, p.dtype, p.dim, p.ratio)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_c4_decode_step_equals_separate_calls(gpu_lib, dtype):
    """Five sequences (two complete a group on this token), bf16 or fp8 attention pools (the
    compressor quantises its new entries into the fp8 pool as it stores them), bf16 indexer keys."""
    hyb = gpu_lib
    lens = [4096, 8191, 20000, 65535, 131072]
    wl = W.sparse_decode(DEV, seed=21, batch=len(lens), ctx=lens, dtype=dtype)
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    g = W.generator(95, 0, 0, DEV)
    x = W.to_storage(W.randn((B, D), g, DEV), "bf16")
    xi = W.to_storage(W.randn((B, 128), g, DEV), "bf16")
    ring, iring = _rings(B, D, 4, torch.bfloat16, g), _rings(B, 128, 4, torch.bfloat16, g)
    cu = torch.arange(0, B + 1, dtype=I32, device=DEV)
    start = (wl.seq_lens - 1).contiguous()
    comp0, idx0, ring0, iring0 = _clone_pool(wl.comp), _clone_pool(wl.idx_pool), ring.clone(), iring.clone()

    # separate calls
    topk_a = torch.full((B, wl.k), -7, dtype=I32, device=DEV)
    out_a = torch.empty_like(wl.q)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, start, L - 1, wl.idx_pool, wl.k, topk_a)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out_a, topk_idx=topk_a, k=wl.k)
    hyb.hyb_compress(x, cu, start, 1, ring, wl.comp, 64)
    hyb.hyb_compress(xi, cu, start, 1, iring, wl.idx_pool, 64)
    torch.cuda.synchronize()
    want = [t.clone() for t in (out_a, topk_a, wl.comp.data, wl.idx_pool.data, ring, iring)]
    want_scale = None if wl.comp.scale is None else wl.comp.scale.clone()

    # one step, from the same starting pools and rings
    wl.comp.data.copy_(comp0.data)
    if wl.comp.scale is not None:
        wl.comp.scale.copy_(comp0.scale)
    wl.idx_pool.data.copy_(idx0.data)
    ring.copy_(ring0)
    iring.copy_(iring0)
    topk_b = torch.full((B, wl.k), -9, dtype=I32, device=DEV)
    out_b = torch.empty_like(wl.q)
    calls = [hyb.compress_call(x, cu, start, 1, ring, wl.comp, 64),
             hyb.compress_call(xi, cu, start, 1, iring, wl.idx_pool, 64)]
    ws = torch.zeros(hyb.hyb_decode_step_workspace_bytes(B, 64, D, L, 4, wl.k), dtype=torch.uint8, device=DEV)
    hyb.hyb_decode_step(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out_b, idx_q=wl.idx_q, idx_w=wl.idx_w,
                        idx_pool=wl.idx_pool, k=wl.k, topk_out=topk_b, compress=calls, workspace=ws)
    torch.cuda.synchronize()
    got = [out_b, topk_b, wl.comp.data, wl.idx_pool.data, ring, iring]
    for n, (a, b) in enumerate(zip(want, got)):
        assert torch.equal(a, b), n
    if want_scale is not None:
        assert torch.equal(want_scale, wl.comp.scale)
    assert not torch.equal(want[2], comp0.data)   # groups were completed and stored

    # sampled sequences against the oracle (selection and attention over the pools as drawn)
    swa_o, comp_o, idx_o = to_oracle_pool(wl.swa), to_oracle_pool(comp0), to_oracle_pool(idx0)
    iq, iw, q = to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy(), to_f64(wl.q)
    for s in (1, 4):
        p = lens[s] - 1
        keys = O.pool_entries(idx_o, s, range(O.n_visible(p, 4, 128)))
        sc = O.indexer_scores(iq[s], iw[s], keys)
        sel = O.topk_select(sc, wl.k)
        check_topk_set(topk_b[s].cpu().numpy(), sel, sc, topk_delta(iq[s], iw[s], keys), wl.k)
        if list(topk_b[s].cpu().numpy()) == list(sel):
            o = O.hybrid_query(q[s], p, s, swa_o, comp_o, 128, 1 / math.sqrt(D), 64, 1e4, sel)
            assert_abs_close(to_f64(out_b[s]), o)


def test_c128_decode_step_equals_separate_calls(gpu_lib):
    """Four sequences of C128 dense decode (entries drawn), a softmax-gate compression of the new
    tokens (two of them complete a group)."""
    hyb = gpu_lib
    lens = [2048, 40959, 300000, 131072]
    wl = W.dense_decode(DEV, seed=22, batch=len(lens), ctx=lens)
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    g = W.generator(94, 0, 0, DEV)
    x = W.to_storage(W.randn((B, D), g, DEV), "bf16")
    lg = W.randn((B,), g, DEV)
    ring, rl = _rings(B, D, 128, torch.bfloat16, g), W.randn((B, 128), g, DEV)
    cu = torch.arange(0, B + 1, dtype=I32, device=DEV)
    start = (wl.seq_lens - 1).contiguous()
    comp0, ring0, rl0 = wl.comp.data.clone(), ring.clone(), rl.clone()
    out_a = torch.empty_like(wl.q)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out_a)
    hyb.hyb_compress(x, cu, start, 1, ring, wl.comp, 64, gate_logits=lg, state_logits=rl)
    torch.cuda.synchronize()
    want = [t.clone() for t in (out_a, wl.comp.data, ring, rl)]
    wl.comp.data.copy_(comp0)
    ring.copy_(ring0)
    rl.copy_(rl0)
    out_b = torch.empty_like(wl.q)
    calls = [hyb.compress_call(x, cu, start, 1, ring, wl.comp, 64, gate_logits=lg, state_logits=rl)]
    hyb.hyb_decode_step(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out_b, compress=calls)
    torch.cuda.synchronize()
    for n, (a, b) in enumerate(zip(want, [out_b, wl.comp.data, ring, rl])):
        assert torch.equal(a, b), n
    assert not torch.equal(want[1], comp0)
    swa_o = to_oracle_pool(wl.swa)
    comp_o = to_oracle_pool(W.PagedTensors(comp0, None, wl.comp.block_table, "bf16", D, 128))
    q = to_f64(wl.q)
    for s in (0, 2):
        o = O.hybrid_query(q[s], lens[s] - 1, s, swa_o, comp_o, 128, 1 / math.sqrt(D), 64, 1e4, None)
        assert_abs_close(to_f64(out_b[s]), o)


@pytest.mark.parametrize("lens", [[2048, 40959, 300000, 131072, 5000], [1 << 20] * 8])
def test_c128_step_repeatedly(gpu_lib, lens):
    """C128 steps over three calls with one workspace: the output equals hyb_attn_decode's bit for
    bit every time. Five mixed lengths (1 to 8 splits of the longest); eight 2^20-token queries
    (8 splits each, the benchmark's shape)."""
    hyb = gpu_lib
    wl = W.dense_decode(DEV, seed=23, batch=len(lens), ctx=lens)
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    want = torch.empty_like(wl.q)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, want)
    ws = torch.zeros(hyb.hyb_decode_step_workspace_bytes(B, 64, D, L, 128, 0), dtype=torch.uint8,
                     device=DEV)
    for call in range(3):
        out = torch.empty_like(wl.q)
        hyb.hyb_decode_step(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, want), call


def _step_no_compress(hyb, wl, topk, out, ws):
    hyb.hyb_decode_step(wl.q, wl.seq_lens, wl.max_seq_len, wl.swa, wl.comp, out, idx_q=wl.idx_q,
                        idx_w=wl.idx_w, idx_pool=wl.idx_pool, k=wl.k, topk_out=topk, workspace=ws)


@pytest.mark.parametrize("case", ["mixed", "long", "ties", "longest"])
def test_c4_step_selects_in_attention_repeatedly(gpu_lib, case):
    """The C4 step's attention workgroups select their rows from the indexer's hand-off. Over
    three calls with one workspace the rows equal hyb_index_topk's and the outputs
    hyb_attn_decode's bit for bit, and the workspace's leading zero block (per-row counts) is zero
    again after every call. Cases: mixed lengths including rows no longer than k; a 2^18-token row
    (64 parts of 64 prefetched pairs each, which a part's candidates can outrun); dyadic indexer
    values whose scores tie heavily; a 2^20-token row (256 parts: beyond the fused selection, so the
    step runs the selection kernel for that batch)."""
    hyb = gpu_lib
    lens = {"mixed": [700, 2100, 2200, 40000, 131072],
            "long": [262144, 150000],
            "ties": [3000, 70001, 131072],
            "longest": [1 << 20, 300000, 5000]}[case]
    wl = W.sparse_decode(DEV, seed=31, batch=len(lens), ctx=lens)
    if case == "ties":
        g = torch.Generator(device=DEV).manual_seed(12)
        vals = torch.tensor([0.0, 0.25, -0.25, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], device=DEV)
        wvals = torch.tensor([0.25, -0.25, 0.5, -0.5, 1.0, -1.0], device=DEV)
        wl.idx_q = vals[torch.randint(0, 9, wl.idx_q.shape, generator=g, device=DEV)].to(torch.bfloat16)
        wl.idx_w = wvals[torch.randint(0, 6, wl.idx_w.shape, generator=g, device=DEV)]
        wl.idx_pool.data = vals[torch.randint(0, 9, wl.idx_pool.data.shape, generator=g,
                                              device=DEV)].to(torch.bfloat16)
    B, L = wl.batch, wl.max_seq_len
    want_topk = torch.full((B, wl.k), -7, dtype=I32, device=DEV)
    want_out = torch.empty_like(wl.q)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.seq_lens - 1, L - 1, wl.idx_pool, wl.k, want_topk)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, L, wl.swa, wl.comp, want_out, topk_idx=want_topk, k=wl.k)
    ws = torch.zeros(hyb.hyb_decode_step_workspace_bytes(B, 64, wl.dim, L, 4, wl.k), dtype=torch.uint8,
                     device=DEV)
    zero = hyb.STEP_ZERO_BYTES
    for call in range(3):
        topk = torch.full((B, wl.k), -9, dtype=I32, device=DEV)
        out = torch.empty_like(wl.q)
        _step_no_compress(hyb, wl, topk, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(topk, want_topk), call
        assert torch.equal(out, want_out), call
        assert int(torch.count_nonzero(ws[:zero])) == 0, call
    short = [b for b, n in enumerate(lens) if O.n_visible(n - 1, 4, 128) <= wl.k]
    for b in short:   # rows no longer than k: every entry in order, then -1
        nv = O.n_visible(lens[b] - 1, 4, 128)
        assert list(topk[b].cpu().numpy()) == list(range(nv)) + [-1] * (wl.k - nv)


@pytest.mark.parametrize("layer", ["c4", "c4_fp8", "c128"])
def test_decode_step_with_prep_equals_separate_calls(gpu_lib, layer):
    """The step before the attention given to hyb_decode_step (query RMSNorm + RoPE of the new
    tokens into q, their window entries at p): on a C4 layer its waves ride at the end of the
    indexer's launch, on a C128 layer it is launched first. Output, top-k rows, rotated queries
    and window pool equal hyb_q_norm_kv_insert followed by the step, bit for bit, compressor calls
    included; the query rows equal the oracle's RMSNorm + RoPE, and a sampled C4 sequence's output
    the oracle's attention over the pools the prep wrote."""
    hyb = gpu_lib
    lens = [4096, 8191, 20000, 65535, 131072]
    dtype = "fp8" if layer == "c4_fp8" else "bf16"
    sparse = layer != "c128"
    wl = (W.sparse_decode(DEV, seed=41, batch=len(lens), ctx=lens, dtype=dtype) if sparse
          else W.dense_decode(DEV, seed=42, batch=len(lens), ctx=lens))
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    g = W.generator(96, 0, 0, DEV)
    q_raw = W.to_storage(W.randn((B, 64, D), g, DEV), "bf16")
    kv = W.to_storage(W.randn((B, D), g, DEV), "bf16")
    x = W.to_storage(W.randn((B, D), g, DEV), "bf16")
    ring = _rings(B, D, 4 if sparse else 128, torch.bfloat16, g)
    cu = torch.arange(0, B + 1, dtype=I32, device=DEV)
    start = (wl.seq_lens - 1).contiguous()
    swa0 = _clone_pool(wl.swa)
    comp0, ring0 = _clone_pool(wl.comp), ring.clone()
    ratio = 4 if sparse else 128

    def pools_back():
        wl.swa.data.copy_(swa0.data)
        if wl.swa.scale is not None:
            wl.swa.scale.copy_(swa0.scale)
        wl.comp.data.copy_(comp0.data)
        if wl.comp.scale is not None:
            wl.comp.scale.copy_(comp0.scale)
        ring.copy_(ring0)

    def run(q, out, topk, prep):
        calls = [hyb.compress_call(x, cu, start, 1, ring, wl.comp, 64)]
        ws = torch.zeros(hyb.hyb_decode_step_workspace_bytes(B, 64, D, L, ratio, wl.k if sparse else 0),
                         dtype=torch.uint8, device=DEV)
        if sparse:
            hyb.hyb_decode_step(q, wl.seq_lens, L, wl.swa, wl.comp, out, idx_q=wl.idx_q, idx_w=wl.idx_w,
                                idx_pool=wl.idx_pool, k=wl.k, topk_out=topk, compress=calls, workspace=ws,
                                prep=prep)
        else:
            hyb.hyb_decode_step(q, wl.seq_lens, L, wl.swa, wl.comp, out, compress=calls, workspace=ws,
                                prep=prep)

    # separate calls: the prep, then the step
    q_a = torch.empty_like(q_raw)
    out_a = torch.empty_like(q_raw)
    topk_a = torch.full((B, wl.k), -7, dtype=I32, device=DEV)
    hyb.hyb_q_norm_kv_insert(q_raw, kv, cu, start, 1, wl.swa, q_out=q_a)
    run(q_a, out_a, topk_a, None)
    torch.cuda.synchronize()
    want = [t.clone() for t in (q_a, out_a, topk_a, wl.swa.data, wl.comp.data, ring)]
    swa_prepped = _clone_pool(wl.swa)
    # one call with the prep
    pools_back()
    q_b = torch.full_like(q_raw, 3.0)
    out_b = torch.empty_like(q_raw)
    topk_b = torch.full((B, wl.k), -9, dtype=I32, device=DEV)
    run(q_b, out_b, topk_b, hyb.prep_call(q_raw, kv, cu, start, 1, wl.swa, q_out=q_b))
    torch.cuda.synchronize()
    got = [q_b, out_b, topk_b, wl.swa.data, wl.comp.data, ring]
    for n, (a, b) in enumerate(zip(want, got)):
        if not sparse and n == 2:
            continue   # no top-k on a C128 layer
        assert torch.equal(a, b), n
    if wl.swa.scale is not None:
        assert torch.equal(swa_prepped.scale, wl.swa.scale)
    assert not torch.equal(want[3], swa0.data)   # the window entries at p were written

    # the query rows against the oracle's RMSNorm + RoPE at each p
    qo = to_f64(q_b)
    for s in (0, 3):   # bf16 rows: within half a bf16 ulp of the float64 values
        want_q = O.q_norm_rope(to_f64(q_raw[s:s + 1]), [lens[s] - 1], 64, 1e4, 1e-6)[0]
        assert np.all(np.abs(qo[s] - want_q) <= 2.0 ** -8 * np.abs(want_q) + 1e-5)
    if sparse and dtype == "bf16":
        swa_o, comp_o, idx_o = to_oracle_pool(swa_prepped), to_oracle_pool(comp0), to_oracle_pool(wl.idx_pool)
        iq, iw = to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy()
        s = 2
        p = lens[s] - 1
        keys = O.pool_entries(idx_o, s, range(O.n_visible(p, 4, 128)))
        sc = O.indexer_scores(iq[s], iw[s], keys)
        sel = O.topk_select(sc, wl.k)
        check_topk_set(topk_b[s].cpu().numpy(), sel, sc, topk_delta(iq[s], iw[s], keys), wl.k)
        if list(topk_b[s].cpu().numpy()) == list(sel):
            o = O.hybrid_query(qo[s], p, s, swa_o, comp_o, 128, 1 / math.sqrt(D), 64, 1e4, sel)
            assert_abs_close(to_f64(out_b[s]), o)
