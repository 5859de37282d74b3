"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Small cases span several tiles and ragged tails and are compared element by element; the
full-size workloads (the launch configurations the benchmark times) are compared on sampled
sequences / query rows that the oracle recomputes one by one. Attention is checked twice: fed
the oracle's own top-k (so a near-tie in the selection cannot hide an attention error) and
chained after the GPU's own selection where that selection equals the oracle's.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_hyb_amd import workloads as W
from tests.conftest import to_f64, to_oracle_pool
from tests.parity_util import (assert_abs_close, assert_fp32_close, check_topk_set, topk_delta)

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32


def ints(v):
    return torch.tensor(list(v), dtype=I32, device=DEV)


def sync():
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- GPU step helpers
def gpu_topk(hyb, wl, qpos=None):
    qpos = wl.seq_lens - 1 if qpos is None else qpos
    out = torch.full((wl.batch, wl.k), -7, dtype=I32, device=DEV)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, qpos, wl.max_seq_len - 1, wl.idx_pool, wl.k, out,
                       window=wl.window)
    return out


def gpu_decode(hyb, wl, topk=None, out_dtype=None):
    out = torch.empty(wl.q.shape, dtype=out_dtype or wl.q.dtype, device=DEV)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, wl.max_seq_len, wl.swa, wl.comp, out, topk_idx=topk,
                        k=wl.k if topk is not None else 0, window=wl.window,
                        rope_dim=wl.rope_dim, rope_base=wl.rope_base)
    return out


# ------------------------------------------------------------------------------ oracle side
def oracle_select(wl, ipool, seqs):
    """Oracle scores, top-k and fp32 error bound per sampled sequence."""
    iq, iw = to_f64(wl.idx_q), wl.idx_w.detach().cpu().double().numpy()
    res = {}
    for b in seqs:
        p = wl.seq_lens_host[b] - 1
        nv = O.n_visible(p, ipool.ratio, wl.window)
        keys = O.pool_entries(ipool, b, range(nv))
        sc = O.indexer_scores(iq[b], iw[b], keys)
        res[b] = (sc, O.topk_select(sc, wl.k), topk_delta(iq[b], iw[b], keys))
    return res


def oracle_out(wl, swa, comp, seqs, selected=None):
    q = to_f64(wl.q)
    scale = 1.0 / math.sqrt(wl.dim)
    return np.stack([O.hybrid_query(q[b], wl.seq_lens_host[b] - 1, b, swa, comp, wl.window, scale,
                                    wl.rope_dim, wl.rope_base,
                                    None if selected is None else selected[b]) for b in seqs])


def check_sparse(hyb, wl, seqs, tol=2e-2):
    swa, comp, ipool = to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), to_oracle_pool(wl.idx_pool)
    sel = oracle_select(wl, ipool, seqs)
    got_topk = gpu_topk(hyb, wl)
    # attention fed the oracle's selection (rows of unsampled sequences: all -1 is also valid)
    feed = torch.full((wl.batch, wl.k), -1, dtype=I32)
    for b in seqs:
        feed[b] = torch.from_numpy(sel[b][1].astype(np.int32))
    feed = feed.to(DEV)
    out_fed = gpu_decode(hyb, wl, feed)
    out_chain = gpu_decode(hyb, wl, got_topk)
    sync()
    gt = got_topk.cpu().numpy()
    swaps = 0
    for b in seqs:
        swaps += check_topk_set(gt[b], sel[b][1], sel[b][0], sel[b][2], wl.k)
    want = oracle_out(wl, swa, comp, seqs, {b: sel[b][1] for b in seqs})
    cmp = assert_abs_close if wl.q.dtype == torch.bfloat16 else assert_fp32_close
    kw = dict(tol=tol) if cmp is assert_abs_close else {}
    cmp(to_f64(out_fed)[list(seqs)], want, **kw)
    same = [b for b in seqs if list(gt[b]) == list(sel[b][1])]
    if same:
        cmp(to_f64(out_chain)[same], want[[list(seqs).index(b) for b in same]], **kw)
    return swaps


# ===================================================================== tiny C4 decode, fp32
def test_tiny_c4_decode_fp32_from_raw_tokens(gpu_lib):
    """1 sequence of 1024 raw tokens, 8 heads x 64 dims, 16 RoPE dims, C4 by mean, 4 x 32
    indexer, top-64, window 128 - the whole chain in fp32 from raw tokens."""
    hyb = gpu_lib
    wl = W.tiny_decode(DEV, seed=0)
    T, D = wl.x.shape
    cu, st = ints([0, T]), ints([0])
    state = torch.zeros(1, 4, D, dtype=wl.x.dtype, device=DEV)   # ring in x's dtype
    hyb.hyb_swa_insert(wl.x, cu, st, T, wl.swa, wl.rope_dim)
    hyb.hyb_compress(wl.x, cu, st, T, state, wl.comp, wl.rope_dim, eps=1e-6)
    qpos = wl.seq_lens - 1
    topk = torch.full((1, wl.k), -7, dtype=I32, device=DEV)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, qpos, T - 1, wl.idx_pool, wl.k, topk)
    sync()
    x = to_f64(wl.x)
    ents = O.compress_stream(x, None, 4, "mean", wl.rope_dim, wl.rope_base, 1e-6)
    sw = O.swa_entries(x, np.arange(T), wl.rope_dim, wl.rope_base)
    assert_fp32_close(O.pool_entries(to_oracle_pool(wl.comp), 0, range(T // 4)), ents)
    assert_fp32_close(O.pool_entries(to_oracle_pool(wl.swa), 0, range(T)), sw)
    # oracle pools built from the oracle's own entries
    swa_o, comp_o = O.logical_pool([sw], 1), O.logical_pool([ents], 4)
    ipool = to_oracle_pool(wl.idx_pool)
    p = T - 1
    nv = O.n_visible(p, 4, 128)
    assert nv == 224
    keys = O.pool_entries(ipool, 0, range(nv))
    iq, iw = to_f64(wl.idx_q)[0], wl.idx_w.cpu().double().numpy()[0]
    sc = O.indexer_scores(iq, iw, keys)
    want_sel = O.topk_select(sc, wl.k)
    check_topk_set(topk.cpu().numpy()[0], want_sel, sc, topk_delta(iq, iw, keys), wl.k)
    scores = torch.full((1, 256), -5.0, device=DEV)
    hyb.hyb_index_score(wl.idx_q, wl.idx_w, qpos, T - 1, wl.idx_pool, scores)
    sync()
    got_sc = scores.cpu().double().numpy()[0]
    assert np.allclose(got_sc[:nv], sc, rtol=1e-5, atol=1e-5)
    assert (got_sc[nv:] == -5.0).all()   # entries beyond the visible range are not written
    out = torch.empty(1, 8, D, device=DEV)
    feed = torch.from_numpy(want_sel.astype(np.int32))[None].to(DEV)
    hyb.hyb_attn_decode(wl.q, wl.seq_lens, T, wl.swa, wl.comp, out, topk_idx=feed, k=wl.k,
                        rope_dim=wl.rope_dim)
    sync()
    want = O.hybrid_query(to_f64(wl.q)[0], p, 0, swa_o, comp_o, 128, 1 / 8.0, wl.rope_dim,
                          wl.rope_base, want_sel)
    assert_fp32_close(to_f64(out)[0], want)


# ============================================================================== compressor
@pytest.mark.parametrize("ratio,mode,dtype,D,rd,T", [
    (4, "mean", "f32", 64, 16, 1000), (128, "gate", "f32", 64, 16, 1500),
    (4, "gate", "bf16", 512, 64, 1000), (128, "mean", "bf16", 512, 64, 1500),
    # wider rows and other load shapes: 16-byte chunks with several per lane (1024, 2048, 520),
    # eight virtual waves above dim 1024 (1536), element pairs when a row is not a whole number
    # of 16-byte chunks (514)
    (128, "gate", "bf16", 1024, 64, 600), (4, "mean", "f32", 2048, 128, 300),
    (128, "mean", "f32", 1536, 64, 600), (4, "gate", "bf16", 514, 64, 300),
    (128, "mean", "bf16", 520, 32, 600)])
def test_compress_chunked_matches_oracle_and_state(gpu_lib, ratio, mode, dtype, D, rd, T):
    """Three sequences with different chunkings (token by token, ragged chunks, one shot):
    entries equal the oracle's; chunked output is bitwise equal to one-shot; the state ring holds
    exactly the in-progress group's raw tokens."""
    hyb = gpu_lib
    g = W.generator(90, ratio, 0, DEV)
    xs = [W.to_storage(W.randn((T, D), g, DEV), dtype) for _ in range(3)]
    lg = [W.randn((T,), g, DEV) for _ in range(3)]
    mb = -(-T // 256)
    pool_chunked = W.make_pool(dtype, D, ratio, [W.blocks_for_entries(T // ratio, ratio)] * 3, mb,
                               g, DEV, fill=False)
    pool_once = W.PagedTensors(torch.zeros_like(pool_chunked.data), None,
                               pool_chunked.block_table.clone(), dtype, D, ratio)
    state = torch.zeros(3, ratio, D, dtype=xs[0].dtype, device=DEV)   # ring in x's dtype
    st_l = torch.zeros(3, ratio, device=DEV)
    gate = (lambda c: torch.cat([lg[b][c[b][0]:c[b][1]] for b in range(3)])) if mode == "gate" else None
    cuts = [list(range(0, T + 1)),                              # token by token
            sorted({0, 1, 3, 130, 131, 517 % T, 900 % T, T}),    # ragged
            [0, T]]                                              # one shot
    n_steps = max(len(c) for c in cuts) - 1
    for s in range(n_steps):
        rng = [(c[s], c[s + 1]) if s + 1 < len(c) else (T, T) for c in cuts]
        x = torch.cat([xs[b][a:e] for b, (a, e) in enumerate(rng)])
        cu = ints([0] + list(np.cumsum([e - a for a, e in rng])))
        start = ints([a for a, _ in rng])
        hyb.hyb_compress(x, cu, start, max(e - a for a, e in rng), state, pool_chunked, rd, eps=1e-6,
                         gate_logits=gate(rng) if gate else None,
                         state_logits=st_l if gate else None)
    full = torch.cat(xs)
    st2, stl2 = torch.zeros_like(state), torch.zeros_like(st_l)
    hyb.hyb_compress(full, ints([0, T, 2 * T, 3 * T]), ints([0, 0, 0]), T, st2, pool_once, rd,
                     eps=1e-6, gate_logits=torch.cat(lg) if gate else None,
                     state_logits=stl2 if gate else None)
    sync()
    assert torch.equal(pool_chunked.data, pool_once.data)
    po = to_oracle_pool(pool_chunked)
    for b in range(3):
        x64 = to_f64(xs[b])
        l64 = lg[b].cpu().double().numpy() if gate else None
        want = O.compress_stream(x64, l64, ratio, mode, rd, 10000.0, 1e-6)
        got = O.pool_entries(po, b, range(T // ratio))
        if dtype == "f32":
            assert_fp32_close(got, want)
        else:
            assert_abs_close(got, want, tol=2e-2)
        slots, lslots = O.pending_group(x64, l64, ratio)
        for slot, row in slots.items():
            assert np.array_equal(state[b, slot].cpu().double().numpy(), row)
            assert np.array_equal(st2[b, slot].cpu().double().numpy(), row)
            if gate:
                assert st_l[b, slot].item() == lslots[slot]


# ======================================================================== C4 sparse decode
def test_c4_sparse_decode_small(gpu_lib):
    """bf16, 64 heads x 512, indexer 64 x 128: L = 1 (one key), 100 (pure window), 700 (all
    visible entries selected), 5000 and 33333 (real top-512 selection, ragged tiles)."""
    wl = W.sparse_decode(DEV, seed=1, batch=5, ctx=[1, 100, 700, 5000, 33333])
    check_sparse(gpu_lib, wl, range(5))


def test_c4_sparse_decode_full_size_sampled(gpu_lib):
    """Batch 16 x 131072 raw tokens (32768 C4 entries each), shuffled block tables, the bench's
    launch configuration; sequences 0, 7 and 15 recomputed by the oracle."""
    wl = W.sparse_decode(DEV, seed=0)
    swaps = check_sparse(gpu_lib, wl, [0, 7, 15])
    assert swaps <= 1


@pytest.mark.parametrize("k", [1024, 2048])
def test_c4_sparse_decode_large_k(gpu_lib, k):
    """Top-1024 and top-2048 (the largest k) through the indexer, the selector and the sparse
    attention (up to 2176 keys per query with the window), over L = 3000 (fewer visible entries
    than k), 40000 and 131072."""
    wl = W.sparse_decode(DEV, seed=8, batch=3, ctx=[3000, 40000, 131072], k=k)
    swaps = check_sparse(gpu_lib, wl, range(3))
    assert swaps <= 2


def test_exact_arithmetic_topk_is_bit_exact(gpu_lib):
    """Dyadic indexer inputs make every fp32 partial sum exact in any order, so the GPU scores
    equal the oracle's exactly and the top-k sets (with their many ties) must be identical."""
    hyb = gpu_lib
    wl = W.sparse_decode(DEV, seed=3, batch=3, ctx=[5000, 20000, 131072])
    g = torch.Generator(device=DEV).manual_seed(11)
    vals = torch.tensor([0.0, 0.25, -0.25, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], device=DEV)
    wvals = torch.tensor([0.25, -0.25, 0.5, -0.5, 1.0, -1.0], device=DEV)
    wl.idx_q = vals[torch.randint(0, 9, wl.idx_q.shape, generator=g, device=DEV)].to(torch.bfloat16)
    wl.idx_w = wvals[torch.randint(0, 6, wl.idx_w.shape, generator=g, device=DEV)]
    pdat = wl.idx_pool.data
    wl.idx_pool.data = vals[torch.randint(0, 9, pdat.shape, generator=g, device=DEV)].to(torch.bfloat16)
    ipool = to_oracle_pool(wl.idx_pool)
    sel = oracle_select(wl, ipool, range(3))
    got = gpu_topk(hyb, wl).cpu().numpy()
    scores = torch.zeros(3, wl.max_seq_len // 4 + 1, device=DEV)   # >= the visible C4 entries
    hyb.hyb_index_score(wl.idx_q, wl.idx_w, wl.seq_lens - 1, wl.max_seq_len - 1, wl.idx_pool, scores)
    sync()
    for b in range(3):
        sc = sel[b][0]
        assert np.array_equal(scores[b, :len(sc)].cpu().double().numpy(), sc)
        assert list(got[b]) == list(sel[b][1])
        assert len(np.unique(sc)) < len(sc)        # ties are present


def test_index_keys_halves_match_fused(gpu_lib):
    """hyb_index_score_keys + hyb_topk_keys select exactly what hyb_index_topk selects. The hand-off
    holds, per block of 1024 entries, every entry once as (order key of hyb_index_score's float,
    index), ordered by the keys' top 10 bits from high to low, and a cumulative count of those
    bits (bit-exact)."""
    hyb = gpu_lib
    wl = W.sparse_decode(DEV, seed=5, batch=4, ctx=[3000, 20000, 70001, 131072])
    qpos = wl.seq_lens - 1
    mp = wl.max_seq_len - 1
    kshape, hshape = hyb.index_keys_shapes(wl.batch, mp)
    keys = torch.empty(kshape, dtype=torch.int32, device=DEV)
    hist = torch.empty(hshape, dtype=torch.int16, device=DEV)
    hyb.hyb_index_score_keys(wl.idx_q, wl.idx_w, qpos, mp, wl.idx_pool, keys, hist)
    out = torch.full((wl.batch, wl.k), -7, dtype=I32, device=DEV)
    hyb.hyb_topk_keys(keys, hist, qpos, mp, wl.k, out)
    fused = gpu_topk(hyb, wl)
    scores = torch.zeros((wl.batch, kshape[1] // 2), device=DEV)
    hyb.hyb_index_score(wl.idx_q, wl.idx_w, qpos, mp, wl.idx_pool, scores)
    sync()
    assert torch.equal(out, fused)
    for b, L in enumerate(wl.seq_lens_host):
        nv = O.n_visible(L - 1, 4, wl.window)
        f = scores[b, :nv].cpu().numpy().view(np.uint32).astype(np.uint64)
        f = np.where(f == 0x80000000, 0, f)
        want = np.where(f & 0x80000000, (~f) & 0xFFFFFFFF, f | 0x80000000).astype(np.uint32)
        row = keys[b].cpu().numpy().view(np.uint32)
        nb = (nv + 1023) // 1024
        h = hist[b, :nb].cpu().numpy().view(np.uint16).astype(np.int64)
        for blk in range(nb):
            cnt = min(1024, nv - 1024 * blk)
            pr = row[2048 * blk: 2048 * blk + 2 * cnt].reshape(cnt, 2)
            idx = pr[:, 1].astype(np.int64)
            assert np.array_equal(np.sort(idx), np.arange(1024 * blk, 1024 * blk + cnt))
            assert np.array_equal(pr[:, 0], want[idx])
            top = (pr[:, 0] >> 22).astype(np.int64)
            assert np.all(np.diff(top) <= 0), "pairs not ordered by their top bits"
            cum = np.cumsum(np.bincount(top, minlength=1024)[::-1])[::-1]
            assert np.array_equal(cum, h[blk])


# ========================================================================= C128 dense decode
def test_c128_dense_decode_small(gpu_lib):
    wl = W.dense_decode(DEV, seed=1, batch=6, ctx=[1, 128, 129, 300, 20000, 70001])
    out = gpu_decode(gpu_lib, wl)
    sync()
    want = oracle_out(wl, to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), range(6))
    assert_abs_close(to_f64(out), want)


def test_c128_dense_decode_two_resolution_segments(gpu_lib):
    """One sequence of 2^24 + 2^17 tokens: 132096 visible C128 entries + the window are more keys
    than 64 splits of one 2048-key resolution segment hold, so every workgroup resolves and
    streams its keys in two segments (the online softmax carried across them)."""
    L = (1 << 24) + (1 << 17)
    wl = W.dense_decode(DEV, seed=9, batch=1, ctx=[L])
    out = gpu_decode(gpu_lib, wl)
    sync()
    want = oracle_out(wl, to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), range(1))
    assert_abs_close(to_f64(out), want)


def test_c128_dense_decode_skewed_lengths(gpu_lib):
    """One 2^20-token sequence among seventeen short ones (1 .. 5000 tokens): the balanced decode
    plan cuts the long query into many pieces and gives each short one a single piece. The long
    query, the shortest ones and one more are recomputed by the oracle."""
    lens = [1 << 20] + [4096] * 13 + [1, 200, 129, 5000]
    wl = W.dense_decode(DEV, seed=12, batch=len(lens), ctx=lens)
    out = gpu_decode(gpu_lib, wl)
    sync()
    seqs = [0, 5, 14, 15, 16, 17]
    want = oracle_out(wl, to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), seqs)
    assert_abs_close(to_f64(out)[seqs], want)


def test_c4_with_k_at_least_visible_equals_dense(gpu_lib):
    """With k >= n_vis the sparse path selects every visible entry, so it must equal the dense
    path over the same C4 pool (up to the order of fp32 partial sums)."""
    hyb = gpu_lib
    wl = W.sparse_decode(DEV, seed=4, batch=3, ctx=[600, 1000, 2100], k=512)
    topk = gpu_topk(hyb, wl)
    sparse = gpu_decode(hyb, wl, topk)
    dense = gpu_decode(hyb, wl, None)
    sync()
    t = topk.cpu().numpy()
    for b, L in enumerate(wl.seq_lens_host):
        nv = O.n_visible(L - 1, 4, 128)
        assert list(t[b][:nv]) == list(range(nv)) and (t[b][nv:] == -1).all()
    assert_abs_close(to_f64(sparse), to_f64(dense), tol=2e-3)


def test_c128_dense_from_raw_tokens_full_size_sampled(gpu_lib):
    """Batch 32 x 2^20 raw tokens compressed by softmax gates into 8192 C128 entries per
    sequence (chunks of 65536 tokens), then one dense decode step - the bench's configuration.
    For sequences 5 and 31 the oracle recomputes every C128 entry from the same raw tokens."""
    hyb = gpu_lib
    wl = W.dense_decode(DEV, seed=0, fill_comp=False)
    B, L, D = wl.batch, wl.seq_lens_host[0], wl.dim
    state = torch.zeros(B, 128, D, dtype=torch.bfloat16, device=DEV)   # ring in x's dtype
    st_l = torch.zeros(B, 128, device=DEV)
    n_chunks = L // W.RAW_CHUNK
    for c in range(n_chunks):
        xs, ls = zip(*[W.raw_chunk(3, 0, b, c, D, DEV) for b in range(B)])
        hyb.hyb_compress(torch.cat(xs), ints(range(0, (B + 1) * W.RAW_CHUNK, W.RAW_CHUNK)),
                         ints([c * W.RAW_CHUNK] * B), W.RAW_CHUNK, state, wl.comp, wl.rope_dim,
                         eps=1e-6, gate_logits=torch.cat(ls), state_logits=st_l)
    out = gpu_decode(hyb, wl)
    sync()
    swa = to_oracle_pool(wl.swa)
    seqs = [5, 31]
    ents = []
    for b in seqs:
        rows = []
        for c in range(n_chunks):
            x, lg = W.raw_chunk(3, 0, b, c, D, DEV)
            x64, l64 = to_f64(x), lg.cpu().double().numpy()
            for gl in range(W.RAW_CHUNK // 128):
                gg = c * (W.RAW_CHUNK // 128) + gl
                rows.append(O.compressed_entry(x64[gl * 128:(gl + 1) * 128],
                                               l64[gl * 128:(gl + 1) * 128], gg, 128, "gate",
                                               wl.rope_dim, wl.rope_base, 1e-6))
        ents.append(np.stack(rows))
    # stored-entry check (bf16 cache) on the sampled sequences
    pc = to_oracle_pool(wl.comp)
    for n, b in enumerate(seqs):
        assert_abs_close(O.pool_entries(pc, b, range(0, 8192, 97)), ents[n][::97], tol=2e-2)
    comp_o = O.logical_pool([ents[0] if b == 5 else ents[1] if b == 31 else ents[0][:1]
                             for b in range(B)], 128, dtype="bf16")
    want = oracle_out(wl, swa, comp_o, seqs)
    assert_abs_close(to_f64(out)[seqs], want)


# ===================================================================== chunked prefill
def test_prefill_from_raw_small(gpu_lib):
    """One sequence: 1000 prior raw tokens then a 300-token chunk (neither a multiple of 4 nor of
    128, so both compressors carry state across the chunk boundary); C4 top-64 and C128 dense
    prefill attention for every new query, all inputs from raw tokens and drawn indexer keys."""
    hyb = gpu_lib
    D, rd, H, T0, T1 = 512, 64, 64, 1000, 300
    T = T0 + T1
    g = W.generator(91, 0, 0, DEV)
    x = W.to_storage(W.randn((T, D), g, DEV), "bf16")
    lg = W.randn((T,), g, DEV)
    q = W.to_storage(W.randn((T1, H, D), g, DEV), "bf16")
    iq = W.to_storage(W.randn((T1, 64, 128), g, DEV), "bf16")
    iw = W.randn((T1, 64), g, DEV) / math.sqrt(128.0)
    mb = -(-T // 256)
    swa = W.make_pool("bf16", D, 1, [W.blocks_for_positions(0, T)], mb, g, DEV, fill=False)
    c4 = W.make_pool("bf16", D, 4, [W.blocks_for_entries(T // 4, 4)], mb, g, DEV, fill=False)
    c128 = W.make_pool("bf16", D, 128, [W.blocks_for_entries(T // 128, 128)], mb, g, DEV, fill=False)
    ip = W.make_pool("bf16", 128, 4, [W.blocks_for_entries(T // 4, 4)], mb, g, DEV)
    s4, s128, l128 = (torch.zeros(1, 4, D, dtype=x.dtype, device=DEV),
                      torch.zeros(1, 128, D, dtype=x.dtype, device=DEV), torch.zeros(1, 128, device=DEV))
    for a, e in ((0, T0), (T0, T)):
        cu, st = ints([0, e - a]), ints([a])
        hyb.hyb_swa_insert(x[a:e], cu, st, e - a, swa, rd)
        hyb.hyb_compress(x[a:e], cu, st, e - a, s4, c4, rd, eps=1e-6)
        hyb.hyb_compress(x[a:e], cu, st, e - a, s128, c128, rd, eps=1e-6, gate_logits=lg[a:e],
                         state_logits=l128)
    pos = torch.arange(T0, T, dtype=I32, device=DEV)
    qseq = torch.zeros(T1, dtype=I32, device=DEV)
    k = 64
    topk = torch.empty(T1, k, dtype=I32, device=DEV)
    hyb.hyb_index_topk(iq, iw, pos, T - 1, ip, k, topk, q_seq=qseq)
    out4 = torch.empty_like(q)
    out128 = torch.empty_like(q)
    hyb.hyb_attn_prefill(q, pos, T - 1, swa, c4, out4, topk_idx=topk, k=k, q_seq=qseq)
    hyb.hyb_attn_prefill(q, pos, T - 1, swa, c128, out128, q_seq=qseq)
    sync()
    x64, l64 = to_f64(x), lg.cpu().double().numpy()
    sw = O.logical_pool([O.swa_entries(x64, np.arange(T), rd, 1e4)], 1, dtype="bf16")
    e4 = O.logical_pool([O.compress_stream(x64, None, 4, "mean", rd, 1e4, 1e-6)], 4, dtype="bf16")
    e128 = O.logical_pool([O.compress_stream(x64, l64, 128, "gate", rd, 1e4, 1e-6)], 128,
                          dtype="bf16")
    ipo = to_oracle_pool(ip)
    qq, iq64, iw64 = to_f64(q), to_f64(iq), iw.cpu().double().numpy()
    tk = topk.cpu().numpy()
    rows = [0, 1, 57, 128, 200, 299]
    for i in rows:
        p = T0 + i
        nv = O.n_visible(p, 4, 128)
        keys = O.pool_entries(ipo, 0, range(nv))
        sc = O.indexer_scores(iq64[i], iw64[i], keys)
        sel = O.topk_select(sc, k)
        check_topk_set(tk[i], sel, sc, topk_delta(iq64[i], iw64[i], keys), k)
        scale = 1 / math.sqrt(D)
        if list(tk[i]) == list(sel):
            assert_abs_close(to_f64(out4)[i], O.hybrid_query(qq[i], p, 0, sw, e4, 128, scale, rd,
                                                             1e4, sel))
        assert_abs_close(to_f64(out128)[i], O.hybrid_query(qq[i], p, 0, sw, e128, 128, scale, rd,
                                                           1e4, None))


def test_prefill_full_size_sampled(gpu_lib):
    """65536 prior tokens + a 4096-token chunk, 4096 queries x 64 heads x 512, C4 top-512: the
    bench's prefill configuration. Rows 0, 1, 2047, 4095 recomputed by the oracle from the prior
    pools (copied before the chunk is inserted) and the chunk's raw tokens."""
    hyb = gpu_lib
    wl = W.chunked_prefill(DEV, seed=0)
    prior_swa, prior_c4 = to_oracle_pool(wl.swa), to_oracle_pool(wl.c4)
    D, rd, n = wl.q.shape[2], wl.rope_dim, wl.n_new
    cu, st = ints([0, n]), ints([wl.prior])
    hyb.hyb_swa_insert(wl.x_new, cu, st, n, wl.swa, rd)
    s4 = torch.zeros(1, 4, D, dtype=wl.x_new.dtype, device=DEV)
    s128 = torch.zeros(1, 128, D, dtype=wl.x_new.dtype, device=DEV)
    l128 = torch.zeros(1, 128, device=DEV)
    hyb.hyb_compress(wl.x_new, cu, st, n, s4, wl.c4, rd, eps=1e-6)
    hyb.hyb_compress(wl.x_new, cu, st, n, s128, wl.c128, rd, eps=1e-6, gate_logits=wl.gate_new,
                     state_logits=l128)
    max_pos = wl.prior + n - 1
    topk = torch.empty(n, wl.k, dtype=I32, device=DEV)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.q_pos, max_pos, wl.idx_pool, wl.k, topk, q_seq=wl.q_seq)
    out = torch.empty_like(wl.q)
    hyb.hyb_attn_prefill(wl.q, wl.q_pos, max_pos, wl.swa, wl.c4, out, topk_idx=topk, k=wl.k,
                         q_seq=wl.q_seq)
    sync()
    x64 = to_f64(wl.x_new)
    new_sw = O.swa_entries(x64, np.arange(wl.prior, wl.prior + n), rd, 1e4)
    new_c4 = [O.compressed_entry(x64[4 * j:4 * j + 4], None, wl.prior // 4 + j, 4, "mean", rd, 1e4,
                                 1e-6) for j in range(n // 4)]
    total = wl.prior + n
    sw_all = np.concatenate([np.zeros((wl.prior - 128, D)),
                             O.pool_entries(prior_swa, 0, range(wl.prior - 128, wl.prior)), new_sw])
    c4_all = np.concatenate([O.pool_entries(prior_c4, 0, range(wl.prior // 4)), np.stack(new_c4)])
    sw_o = O.logical_pool([sw_all], 1, dtype="bf16")
    c4_o = O.logical_pool([c4_all], 4, dtype="bf16")
    assert sw_all.shape[0] == total
    ipo = to_oracle_pool(wl.idx_pool)
    qq, iq64, iw64 = to_f64(wl.q), to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy()
    tk = topk.cpu().numpy()
    for i in (0, 1, 2047, 4095):
        p = wl.prior + i
        nv = O.n_visible(p, 4, 128)
        keys = O.pool_entries(ipo, 0, range(nv))
        sc = O.indexer_scores(iq64[i], iw64[i], keys)
        sel = O.topk_select(sc, wl.k)
        check_topk_set(tk[i], sel, sc, topk_delta(iq64[i], iw64[i], keys), wl.k)
        if list(tk[i]) == list(sel):
            want = O.hybrid_query(qq[i], p, 0, sw_o, c4_o, 128, 1 / math.sqrt(D), rd, 1e4, sel)
            assert_abs_close(to_f64(out)[i], want)


def test_prefill_indexer_mixed_sequences(gpu_lib):
    """Prefill queries of three sequences in one indexer launch of 283 queries (the last group of
    four is ragged): 37 of sequence 0, then 20 of sequences 1 and 2 interleaved query by query,
    then the rest of each. Groups of four then hold one, two or three sequences. Each sampled
    query's top-64 must equal that of a launch holding the query alone (the one-query kernel), and
    agree with the oracle's selection."""
    hyb = gpu_lib
    g = W.generator(92, 0, 0, DEV)
    lens, counts = [2003, 701, 4999], [37, 101, 145]
    rows = [(0, p) for p in range(lens[0] - counts[0], lens[0])]
    tail = [[(s, p) for p in range(lens[s] - counts[s], lens[s])] for s in (1, 2)]
    for j in range(20):
        rows += [tail[0][j], tail[1][j]]
    rows += tail[0][20:] + tail[1][20:]
    n = len(rows)
    assert n == 283
    mb = -(-max(lens) // 256)
    ip = W.make_pool("bf16", 128, 4, [W.blocks_for_entries(L // 4, 4) for L in lens], mb, g, DEV)
    iq = W.to_storage(W.randn((n, 64, 128), g, DEV), "bf16")
    iw = W.randn((n, 64), g, DEV) / math.sqrt(128.0)
    qseq, pos = ints([s for s, _ in rows]), ints([p for _, p in rows])
    max_pos, k = max(lens) - 1, 64
    topk = torch.empty(n, k, dtype=I32, device=DEV)
    hyb.hyb_index_topk(iq, iw, pos, max_pos, ip, k, topk, q_seq=qseq)
    sample = [0, 1, 35, 36, 37, 38, 39, 40, 76, 77, 78, 79, 120, 157, 158, 200, 279, 280, 281, 282]
    alone = torch.empty(len(sample), k, dtype=I32, device=DEV)
    for j, i in enumerate(sample):
        hyb.hyb_index_topk(iq[i:i + 1], iw[i:i + 1], pos[i:i + 1], max_pos, ip, k, alone[j:j + 1],
                           q_seq=qseq[i:i + 1])
    sync()
    tk, al = topk.cpu().numpy(), alone.cpu().numpy()
    for j, i in enumerate(sample):
        assert list(tk[i]) == list(al[j]), f"query {i} (sequence {rows[i][0]})"
    ipo = to_oracle_pool(ip)
    iq64, iw64 = to_f64(iq), iw.cpu().double().numpy()
    for i in (0, 36, 37, 38, 282):
        s, p = rows[i]
        keys = O.pool_entries(ipo, s, range(O.n_visible(p, 4, 128)))
        sc = O.indexer_scores(iq64[i], iw64[i], keys)
        check_topk_set(tk[i], O.topk_select(sc, k), sc, topk_delta(iq64[i], iw64[i], keys), k)


# ================================================================ quantised mixed-length decode
def _quant_check(hyb, c4, c128, seqs4, seqs128):
    check_sparse(hyb, c4, seqs4)
    out = gpu_decode(hyb, c128)
    sync()
    want = oracle_out(c128, to_oracle_pool(c128.swa), to_oracle_pool(c128.comp), seqs128)
    assert_abs_close(to_f64(out)[list(seqs128)], want)


def test_quantized_mixed_small(gpu_lib):
    """fp8 E4M3 attention caches (per-entry fp32 scale) and an fp4 E2M1 indexer cache (E8M0 per
    32): lengths 200 (window only), 4096, 10001, 50000."""
    c4, c128 = W.quantized_mixed(DEV, seed=1, batch=4, lens=[200, 4096, 10001, 50000])
    _quant_check(gpu_lib, c4, c128, range(4), range(4))


def test_quantized_mixed_full_size_sampled(gpu_lib):
    """Batch 64, lengths log-uniform in [4096, 2^20]: the bench's quantised configuration; the
    shortest and the longest sequences (and one more) recomputed by the oracle."""
    c4, c128 = W.quantized_mixed(DEV, seed=0)
    lens = c4.seq_lens_host
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    _quant_check(gpu_lib, c4, c128, pick, pick)


# =============================================================================== top-k alone
@pytest.mark.parametrize("n,k", [(0, 8), (5, 8), (8, 8), (9, 8), (1000, 64), (32736, 512),
                                 (300001, 512), (70000, 2048)])
def test_topk_alone_bit_exact(gpu_lib, n, k):
    """The selector alone on identical fp32 score rows: bit-exact against the oracle, with heavy
    ties (scores drawn from a small set, including -0.0 and +0.0). Row 3 holds about k/2 ones
    scattered among signed zeros: the k-th largest is a zero, only the lowest-indexed zeros are
    taken, and ones keep appearing after the last taken zero (their slots depend on the clamp
    min(remaining ties, ties before the slice))."""
    hyb = gpu_lib
    g = torch.Generator().manual_seed(n + k)
    rows = 4
    ld = max(n, 1) + 5
    choices = torch.tensor([-0.0, 0.0, 1.5, -2.25, 3.0, 1e-30, -1e30, 7.0])
    sc = torch.randn(rows, ld, generator=g)
    sc[1] = choices[torch.randint(0, 8, (ld,), generator=g)]
    sc[2, : ld // 2] = choices[torch.randint(0, 2, (ld // 2,), generator=g)]
    ones = torch.rand(ld, generator=g) < (k / 2) / max(n, 1)
    sc[3] = torch.where(ones, 1.0, choices[torch.randint(0, 2, (ld,), generator=g)])
    lens = [n, max(0, n - 3), n // 2, n]
    out = torch.full((rows, k), -7, dtype=I32, device=DEV)
    hyb.hyb_topk(sc.to(DEV), ints(lens), n, k, out)
    sync()
    o = out.cpu().numpy()
    for r in range(rows):
        want = O.topk_select(sc[r, :lens[r]].double().numpy(), k)
        assert list(o[r]) == list(want)


# =========================================================== block placement and determinism
def _permute_blocks(pool, seed):
    """Same logical contents, different physical placement (test plumbing: data movement)."""
    g = torch.Generator().manual_seed(seed)
    n = pool.num_blocks
    perm = torch.randperm(n, generator=g).to(DEV)
    data = torch.empty_like(pool.data)
    data[perm] = pool.data
    scale = None
    if pool.scale is not None:
        scale = torch.empty_like(pool.scale)
        scale[perm] = pool.scale
    bt = pool.block_table.clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(I32)
    return W.PagedTensors(data, scale, bt, pool.dtype, pool.dim, pool.ratio)


def test_block_placement_and_determinism(gpu_lib):
    hyb = gpu_lib
    wl = W.sparse_decode(DEV, seed=5, batch=4, ctx=[3000, 131072, 20000, 7])
    t1 = gpu_topk(hyb, wl)
    o1 = gpu_decode(hyb, wl, t1)
    t1b = gpu_topk(hyb, wl)
    o1b = gpu_decode(hyb, wl, t1b)
    wl.swa, wl.comp, wl.idx_pool = (_permute_blocks(wl.swa, 1), _permute_blocks(wl.comp, 2),
                                    _permute_blocks(wl.idx_pool, 3))
    t2 = gpu_topk(hyb, wl)
    o2 = gpu_decode(hyb, wl, t2)
    sync()
    assert torch.equal(t1, t1b) and torch.equal(o1, o1b)
    assert torch.equal(t1, t2) and torch.equal(o1, o2)


# ====================================================== attention with the compressor alongside
def _clone_pool(p):
    return W.PagedTensors(p.data.clone(), None if p.scale is None else p.scale.clone(),
                          p.block_table, p.dtype, p.dim, p.ratio)


_FUSED_CASES = ["c4_bf16", "c128_gate_bf16", "c4_f32x", "c4_unaligned_x", "c4_fp8out",
                "c128_gate_fp8out", "c4_fp8pool", "c128_gate_fp8pool"]


@pytest.mark.parametrize("case", _FUSED_CASES)
def test_attn_decode_compress_equals_two_calls(gpu_lib, case):
    """hyb_attn_decode_compress leaves exactly what hyb_attn_decode then hyb_compress leave: the
    attention output (bf16 rows, or fp8 rows and their scales), every pool byte, the state ring
    and its logits. The compressor runs beside the combine (bf16 / f32 x) or after it (x not
    16-byte aligned, or the pools are fp8 and the compressor quantises as it stores); sequences
    complete a group or only extend the ring."""
    hyb = gpu_lib
    g = W.generator(91, _FUSED_CASES.index(case), 0, DEV)
    fp8 = case.endswith("fp8out")
    if case.startswith("c4"):
        lens = [4096, 4097, 4098, 4099, 131072, 9000]
        wl = W.sparse_decode(DEV, seed=5, batch=len(lens), ctx=lens,
                             dtype="fp8" if case.endswith("fp8pool") else "bf16")
        topk = gpu_topk(hyb, wl)
        r, gate = 4, False
    else:
        lens = [2048, 5000, 65536, 131072]
        wl = W.dense_decode(DEV, seed=5, batch=len(lens), ctx=lens,
                            dtype="fp8" if case.endswith("fp8pool") else "bf16")
        topk, r, gate = None, 128, True
    B, D = wl.batch, wl.dim
    x = W.randn((B, D), g, DEV)
    if case == "c4_unaligned_x":
        buf = torch.zeros(B * D + 16, dtype=torch.bfloat16, device=DEV)
        x_use = buf[4:4 + B * D].view(B, D)          # 8-byte but not 16-byte aligned
        x_use.copy_(x.to(torch.bfloat16))
        assert x_use.data_ptr() % 16 != 0
    else:
        x_use = x if case == "c4_f32x" else W.to_storage(x, "bf16")
    cu = torch.arange(0, B + 1, dtype=I32, device=DEV)
    start = (wl.seq_lens - 1).contiguous()
    state = W.randn((B, r, D), g, DEV).to(x_use.dtype)   # ring in x's dtype
    st_l = W.randn((B, r), g, DEV) if gate else None
    gl = W.randn((B,), g, DEV) if gate else None
    runs = []
    for fused in (False, True):
        comp, swa = _clone_pool(wl.comp), wl.swa
        stt, stl = state.clone(), None if st_l is None else st_l.clone()
        out = torch.empty(wl.q.shape, dtype=torch.uint8 if fp8 else wl.q.dtype, device=DEV)
        sc = torch.empty(wl.q.shape[:2], dtype=torch.float32, device=DEV) if fp8 else None
        kw = dict(topk_idx=topk, k=wl.k if topk is not None else 0, window=wl.window,
                  rope_dim=wl.rope_dim, rope_base=wl.rope_base, out_scale=sc)
        if fused:
            hyb.hyb_attn_decode_compress(wl.q, wl.seq_lens, wl.max_seq_len, swa, comp, out, x_use,
                                         cu, start, 1, stt, comp, eps=1e-6, gate_logits=gl,
                                         state_logits=stl, **kw)
        else:
            hyb.hyb_attn_decode(wl.q, wl.seq_lens, wl.max_seq_len, swa, comp, out, **kw)
            hyb.hyb_compress(x_use, cu, start, 1, stt, comp, wl.rope_dim, wl.rope_base, eps=1e-6,
                             gate_logits=gl, state_logits=stl)
        runs.append((out, comp.data, stt, stl, sc, comp.scale))
    sync()
    (o0, c0, s0, l0, q0, e0), (o1, c1, s1, l1, q1, e1) = runs
    assert torch.equal(o0, o1)
    if e0 is not None:
        assert torch.equal(e0, e1)
    if fp8:
        assert torch.equal(q0, q1)
    assert torch.equal(c0, c1)
    assert torch.equal(s0, s1)
    if gate:
        assert torch.equal(l0, l1)
    # the call did write: every completed group's entry differs from the pool it started from
    for b, L in enumerate(lens):
        if L % r == 0:
            gidx = (L - 1) // r
            lb, slot = gidx // (256 // r), gidx % (256 // r)
            phys = int(wl.comp.block_table[b, lb])
            assert not torch.equal(c1[phys, slot], wl.comp.data[phys, slot])


# ============================================================ multi-query (speculative) decode
def _check_multi(hyb, wl, rows):
    """Indexer + top-k + attention of a multi-query decode batch through the prefill-form entry
    points; the oracle recomputes the sampled rows, fed its own selection and chained after the
    GPU's where the two agree."""
    max_pos = max(wl.q_pos_host)
    topk = torch.full((wl.n_q, wl.k), -7, dtype=I32, device=DEV)
    hyb.hyb_index_topk(wl.idx_q, wl.idx_w, wl.q_pos, max_pos, wl.idx_pool, wl.k, topk, q_seq=wl.q_seq)
    ipo, swa, comp = to_oracle_pool(wl.idx_pool), to_oracle_pool(wl.swa), to_oracle_pool(wl.comp)
    iq64, iw64 = to_f64(wl.idx_q), wl.idx_w.cpu().double().numpy()
    seqs = wl.q_seq.cpu().numpy()
    sel = {}
    for i in rows:
        p, b = wl.q_pos_host[i], int(seqs[i])
        keys = O.pool_entries(ipo, b, range(O.n_visible(p, 4, wl.window)))
        sc = O.indexer_scores(iq64[i], iw64[i], keys)
        sel[i] = (sc, O.topk_select(sc, wl.k), topk_delta(iq64[i], iw64[i], keys))
    feed = torch.full((wl.n_q, wl.k), -1, dtype=I32)
    for i in rows:
        feed[i] = torch.from_numpy(sel[i][1].astype(np.int32))
    feed = feed.to(DEV)
    out_fed, out_chain = torch.empty_like(wl.q), torch.empty_like(wl.q)
    for o, t in ((out_fed, feed), (out_chain, topk)):
        hyb.hyb_attn_prefill(wl.q, wl.q_pos, max_pos, wl.swa, wl.comp, o, topk_idx=t, k=wl.k,
                             q_seq=wl.q_seq, window=wl.window, rope_dim=wl.rope_dim,
                             rope_base=wl.rope_base)
    sync()
    gt = topk.cpu().numpy()
    q64 = to_f64(wl.q)
    scale = 1.0 / math.sqrt(wl.q.shape[2])
    for i in rows:
        check_topk_set(gt[i], sel[i][1], sel[i][0], sel[i][2], wl.k)
        want = O.hybrid_query(q64[i], wl.q_pos_host[i], int(seqs[i]), swa, comp, wl.window, scale,
                              wl.rope_dim, wl.rope_base, sel[i][1])
        assert_abs_close(to_f64(out_fed)[i], want)
        if list(gt[i]) == list(sel[i][1]):
            assert_abs_close(to_f64(out_chain)[i], want)


def test_multi_decode_small(gpu_lib):
    """Three sequences (3000, 9001, 20002 tokens), three query tokens each at the last three
    positions: every row against the oracle."""
    wl = W.multi_decode(DEV, seed=0, batch=3, ctx=[3000, 9001, 20002], n_tok=3)
    _check_multi(gpu_lib, wl, range(wl.n_q))


def test_multi_decode_full_size_sampled(gpu_lib):
    """16 sequences x 131072 tokens, two query tokens each (the C4 decode batch with one draft
    token): rows 0, 1, 17 and 31 against the oracle."""
    wl = W.multi_decode(DEV, seed=1, batch=16, ctx=131072, n_tok=2)
    _check_multi(gpu_lib, wl, (0, 1, 17, 31))


# ============================================================== graph capture of the decode step
def test_c4_decode_step_graph_replay(gpu_lib):
    """The C4 decode step (indexer halves, top-k, attention with the compressor beside the
    combine) captured in one HIP graph: no call allocates or clears memory, so every replay
    (outputs cleared eagerly in between) reproduces the eager step exactly."""
    hyb = gpu_lib
    lens = [4096, 8192, 20000, 65536]
    wl = W.sparse_decode(DEV, seed=3, batch=len(lens), ctx=lens)
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    g = W.generator(92, 0, 0, DEV)
    kshape, hshape = hyb.index_keys_shapes(B, L - 1)
    keys = torch.empty(kshape, dtype=I32, device=DEV)
    hist = torch.empty(hshape, dtype=torch.int16, device=DEV)
    topk = torch.empty(B, wl.k, dtype=I32, device=DEV)
    out = torch.empty_like(wl.q)
    ws = torch.zeros(hyb.hyb_attn_decode_workspace_bytes(B, 64, D, L, 4, wl.k), dtype=torch.uint8,
                     device=DEV)
    x_new = W.to_storage(W.randn((B, D), g, DEV), "bf16")
    cu = torch.arange(0, B + 1, dtype=I32, device=DEV)
    qpos = (wl.seq_lens - 1).contiguous()
    state = W.to_storage(W.randn((B, 4, D), g, DEV), "bf16")
    pool0, state0 = wl.comp.data.clone(), state.clone()

    def step():
        hyb.hyb_index_score_keys(wl.idx_q, wl.idx_w, qpos, L - 1, wl.idx_pool, keys, hist)
        hyb.hyb_topk_keys(keys, hist, qpos, L - 1, wl.k, topk)
        hyb.hyb_attn_decode_compress(wl.q, wl.seq_lens, L, wl.swa, wl.comp, out, x_new, cu, qpos, 1,
                                     state, wl.comp, topk_idx=topk, k=wl.k, workspace=ws)

    step()
    sync()
    want = (topk.clone(), out.clone(), wl.comp.data.clone(), state.clone())
    assert not torch.equal(want[2], pool0)   # the step completed groups (4096 % 4 == 0, ...)
    wl.comp.data.copy_(pool0)
    state.copy_(state0)
    graph = torch.cuda.CUDAGraph()
    sync()
    with torch.cuda.graph(graph):
        step()
    sync()
    for rep in range(3):
        topk.fill_(-7)
        out.zero_()
        wl.comp.data.copy_(pool0)
        state.copy_(state0)
        sync()
        graph.replay()
        sync()
        assert torch.equal(topk, want[0]), rep
        assert torch.equal(out, want[1]), rep
        assert torch.equal(wl.comp.data, want[2]), rep
        assert torch.equal(state, want[3]), rep
