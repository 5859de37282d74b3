"""Whole-step invariants of the oracle (CPU only).

These are the invariants the method's statement fixes: a context of at most 128 tokens is pure
sliding-window attention; C4 top-k with k >= the number of visible entries equals dense
attention over all of them; C128 equals dense attention (torch float64 SDPA) over the pooled
entries plus the window; physical block placement changes nothing; a single key returns itself.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O

B = O.BLOCK_POSITIONS


def make_pool(entries_per_seq, ratio, perm_seed=None):
    """float64 entry arrays per sequence -> float32 OraclePool (block ids permuted if seeded)."""
    per = B // ratio
    dim = entries_per_seq[0].shape[1]
    nblk = [-(-len(e) // per) for e in entries_per_seq]
    total = sum(nblk)
    ids = np.arange(total)
    if perm_seed is not None:
        ids = np.random.default_rng(perm_seed).permutation(total)
    data = np.zeros((total, per, dim), np.float32)
    table = np.full((len(entries_per_seq), max(nblk) + 1), -1, np.int32)
    c = 0
    for b, e in enumerate(entries_per_seq):
        for lb in range(nblk[b]):
            phys = ids[c]
            c += 1
            table[b, lb] = phys
            chunk = e[lb * per:(lb + 1) * per]
            data[phys, :len(chunk)] = chunk
    return O.OraclePool(data=data, dtype="f32", dim=dim, ratio=ratio, block_table=table)


def stored(x):
    return np.asarray(x, np.float32).astype(np.float64)


def sdpa64(q, keys, scale):
    qt = torch.from_numpy(q)[:, None, :]
    kt = torch.from_numpy(keys)[None].expand(q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)[:, 0].numpy()


RD, BASE, W, D, H = 16, 10000.0, 128, 64, 8
SCALE = 1 / math.sqrt(D)


def _raw(seed, T):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, D)), rng.standard_normal(T), rng.standard_normal((H, D))


@pytest.mark.parametrize("L", [1, 2, 77, 128])
def test_short_context_is_pure_swa(L):
    x, _, q = _raw(11, 300)
    swa = make_pool([stored(O.swa_entries(x[:L], np.arange(L), RD, BASE))], 1)
    junk = make_pool([np.full((64, D), 1e3)], 4)   # compressed pool must not be read
    out = O.hybrid_query(q, L - 1, 0, swa, junk, W, SCALE, RD, BASE)
    keys = O.pool_entries(swa, 0, range(L))
    want = O.rope(sdpa64(q, keys, SCALE), -(L - 1), RD, BASE)
    assert np.allclose(out, want, atol=1e-12)


def test_single_key_returns_raw_token():
    x, _, q = _raw(12, 4)
    swa = make_pool([stored(O.swa_entries(x[:1], [0], RD, BASE))], 1)
    comp = make_pool([np.zeros((1, D))], 4)
    out = O.hybrid_query(q, 0, 0, swa, comp, W, SCALE, RD, BASE)
    assert np.allclose(out, np.tile(stored(x[0]), (H, 1)), atol=1e-15)


def test_c128_is_dense_sdpa_over_pooled_entries_and_window():
    T = 1000
    x, lg, q = _raw(13, T)
    ents = stored(O.compress_stream(x, lg, 128, "gate", RD, BASE, 1e-6))
    comp = make_pool([ents], 128, perm_seed=1)
    swa = make_pool([stored(O.swa_entries(x, np.arange(T), RD, BASE))], 1, perm_seed=2)
    p = T - 1
    out = O.hybrid_query(q, p, 0, swa, comp, W, SCALE, RD, BASE)
    ws = p - W + 1
    nv = O.n_visible(p, 128, W)
    keys = np.concatenate([O.pool_entries(swa, 0, range(ws, p + 1)), ents[:nv]])
    want = O.rope(sdpa64(q, keys, SCALE), -p, RD, BASE)
    assert nv == 7
    assert np.allclose(out, want, atol=1e-12)


def test_c4_topk_with_large_k_equals_dense():
    T = 700
    x, _, q = _raw(14, T)
    rng = np.random.default_rng(15)
    ents = stored(O.compress_stream(x, None, 4, "mean", RD, BASE, 1e-6))
    comp = make_pool([ents], 4)
    swa = make_pool([stored(O.swa_entries(x, np.arange(T), RD, BASE))], 1)
    ikeys = make_pool([rng.standard_normal((T // 4, 32))], 4)
    iq, iw = rng.standard_normal((1, 4, 32)), np.ones((1, 4))
    lens = [T]
    nv = O.n_visible(T - 1, 4, W)
    dense, _ = O.decode(q[None], lens, swa, comp, W, SCALE, RD, BASE)
    for k in (nv, nv + 1, 4096):
        sparse, sel = O.decode(q[None], lens, swa, comp, W, SCALE, RD, BASE,
                               idx=dict(q=iq, w=iw, pool=ikeys, k=k))
        assert np.allclose(sparse, dense, atol=1e-13)
        assert sel[0][:nv].tolist() == list(range(nv)) and (sel[0][nv:] == -1).all()
    small, sel = O.decode(q[None], lens, swa, comp, W, SCALE, RD, BASE,
                          idx=dict(q=iq, w=iw, pool=ikeys, k=16))
    assert not np.allclose(small, dense, atol=1e-6)
    assert (np.diff(sel[0]) > 0).all()


def test_block_permutation_invariance():
    T = 900
    x, lg, q = _raw(16, T)
    ents = stored(O.compress_stream(x, lg, 4, "gate", RD, BASE, 1e-6))
    sw = stored(O.swa_entries(x, np.arange(T), RD, BASE))
    rng = np.random.default_rng(17)
    ik = rng.standard_normal((T // 4, 32))
    iq, iw = rng.standard_normal((1, 4, 32)), rng.standard_normal((1, 4))
    outs = []
    for seed in (None, 3, 4):
        comp, swa, ikp = make_pool([ents], 4, seed), make_pool([sw], 1, seed), make_pool([ik], 4, seed)
        o, s = O.decode(q[None], [T], swa, comp, W, SCALE, RD, BASE,
                        idx=dict(q=iq, w=iw, pool=ikp, k=64))
        outs.append((o, s))
    for o, s in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(s, outs[0][1])


def test_prefill_row_equals_decode_at_that_length():
    T = 600
    x, lg, _ = _raw(18, T)
    rng = np.random.default_rng(19)
    ents = stored(O.compress_stream(x, None, 4, "mean", RD, BASE, 1e-6))
    comp, swa = make_pool([ents], 4), make_pool([stored(O.swa_entries(x, np.arange(T), RD, BASE))], 1)
    ik = make_pool([rng.standard_normal((T // 4, 32))], 4)
    pos = [130, 250, 599]
    qs = rng.standard_normal((3, H, D))
    iq, iw = rng.standard_normal((3, 4, 32)), rng.standard_normal((3, 4))
    pf, psel = O.prefill(qs, [0, 0, 0], pos, swa, comp, W, SCALE, RD, BASE,
                         idx=dict(q=iq, w=iw, pool=ik, k=32))
    for i, p in enumerate(pos):
        d, dsel = O.decode(qs[i][None], [p + 1], swa, comp, W, SCALE, RD, BASE,
                           idx=dict(q=iq[i][None], w=iw[i][None], pool=ik, k=32))
        assert np.array_equal(pf[i], d[0]) and np.array_equal(psel[i], dsel[0])
