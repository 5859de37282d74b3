"""GPU parity of quantise-on-insert: window entries into an fp8 pool and compressed entries into
fp8 (attention cache) and fp4 (indexer keys) pools, through the C ABI, against the oracle's
encoders and entries.

Where the stored row is exactly the input (window insert without rotation) the codes and scales
must equal the oracle's encoder bit for bit. Where the row is computed (rotation, pooling and
normalisation in float32 against the oracle's float64), a code may differ from the oracle's
encoding of its own row only where that row lies within the float32 error of a rounding
boundary: the decoded values are checked against the oracle's entries to half a code step plus
that error, and the scales / shared exponents against the oracle's row maxima.
"""

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_hyb_amd import workloads as W
from tests.conftest import to_f64, to_oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32


def ints(v):
    return torch.tensor([int(a) for a in v], dtype=I32, device=DEV)


def stored(pt):
    """(data, scale, block table) of a pool on the host, as stored."""
    return pt.data.cpu().numpy(), pt.scale.cpu().numpy(), pt.block_table.cpu().numpy()


def raw_entry(host, ratio, seq, g):
    data, scale, table = host
    per = 256 // ratio
    phys = table[seq, g // per]
    return data[phys, g % per], scale[phys, g % per]


def e4m3_step(v):
    """Spacing of E4M3 values at magnitude |v| (subnormal spacing 2^-9 below 2^-6)."""
    return np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))), -6) - 3)


def check_fp8_rows(codes, scales, ref, err):
    """Rows stored as fp8 (codes [n, D], scales [n]) against the oracle's float64 rows `ref`,
    whose float32 computation may be off by `err` per element."""
    ref = np.asarray(ref, np.float64)
    amax = np.abs(ref).max(axis=1)
    s = scales.astype(np.float64)
    assert np.all(np.abs(s - amax / 448.0) <= (err + 1e-12) / 448.0 + 2.0 ** -23 * s)
    dec = O.e4m3fn_to_f64(codes) * s[:, None]
    bound = 0.5 * e4m3_step(ref / s[:, None]) * s[:, None] + 2 * err + 2.0 ** -23 * np.abs(ref)
    assert np.all(np.abs(dec - ref) <= bound)
    # codes differ from the oracle's own encoding only at near-ties
    want = np.stack([O.quantize_fp8_row(r.astype(np.float32))[0] for r in ref])
    assert np.mean(codes != want) < 0.01


# =================================================================== window insert, fp8 pool
@pytest.mark.parametrize("xdt,D", [("f32", 512), ("bf16", 512), ("f32", 96), ("bf16", 2048)])
def test_swa_insert_fp8_bit_exact(gpu_lib, xdt, D):
    """Without rotation (rope_dim 0) a window entry is the token itself, so the stored codes and
    scale must equal the oracle's fp8 row encoder bit for bit. Three sequences take 300 / 1 / 77
    new tokens from positions 0 / 1000 / 250 (crossing block boundaries); rows are N(0,1) values
    times 2^N(0, 13^2); one row is all zero and one holds exact E4M3 ties (its maximum is 448, so
    its scale is 1 and every quotient is the value itself)."""
    hyb = gpu_lib
    g = W.generator(93, D, 0, DEV)
    n_new, starts = [300, 1, 77], [0, 1000, 250]
    T = sum(n_new)
    x = W.randn((T, D), g, DEV) * torch.exp2(W.randn((T, 1), g, DEV) * 13.0)
    x[5] = 0.0
    pos = O.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    ties = ((pos[:-1] + pos[1:]) / 2)[:D - 1]
    ties = ties * np.where(np.arange(ties.size) % 2, -1.0, 1.0)
    x[7] = torch.tensor(np.concatenate([[448.0], ties, np.zeros(max(0, D - 1 - ties.size))])[:D],
                        dtype=torch.float32, device=DEV)
    x = W.to_storage(x, xdt)
    mb = (max(s + n for s, n in zip(starts, n_new)) + 255) // 256
    swa = W.make_pool("fp8", D, 1, [W.blocks_for_positions(s, s + n) for s, n in zip(starts, n_new)],
                      mb, g, DEV, fill=False)
    cu = np.cumsum([0] + n_new)
    hyb.hyb_swa_insert(x, ints(cu), ints(starts), max(n_new), swa, 0)
    torch.cuda.synchronize()
    xs = x.float().cpu().numpy()   # exact widening of the stored tokens
    host = stored(swa)
    for b in range(3):
        for i in range(n_new[b]):
            codes, sc = raw_entry(host, 1, b, starts[b] + i)
            want_c, want_s = O.quantize_fp8_row(xs[cu[b] + i])
            assert sc == want_s, (b, i)
            assert np.array_equal(codes, want_c), (b, i)


def test_swa_insert_fp8_rotated(gpu_lib):
    """With RoPE on the last 64 dims (bf16 tokens, dim 512, positions up to 2^20): decoded entries
    against the oracle's rotated entries."""
    hyb = gpu_lib
    g = W.generator(94, 0, 0, DEV)
    n_new, starts = [130, 64], [5, (1 << 20) - 64]
    T, D, rd = sum(n_new), 512, 64
    x = W.to_storage(W.randn((T, D), g, DEV), "bf16")
    mb = (max(s + n for s, n in zip(starts, n_new)) + 255) // 256
    swa = W.make_pool("fp8", D, 1, [W.blocks_for_positions(s, s + n) for s, n in zip(starts, n_new)],
                      mb, g, DEV, fill=False)
    cu = np.cumsum([0] + n_new)
    hyb.hyb_swa_insert(x, ints(cu), ints(starts), max(n_new), swa, rd)
    torch.cuda.synchronize()
    x64 = to_f64(x)
    host = stored(swa)
    for b in range(2):
        p = np.arange(starts[b], starts[b] + n_new[b])
        ref = O.swa_entries(x64[cu[b]:cu[b + 1]], p, rd, 1e4)
        rows = [raw_entry(host, 1, b, int(t)) for t in p]
        check_fp8_rows(np.stack([r[0] for r in rows]), np.array([r[1] for r in rows]), ref, 2e-5)


# ============================================================= compressor, fp8 and fp4 pools
def _compress_chunked_and_once(hyb, dtype, ratio, mode, xdt, D, rd, T, seed):
    """Three sequences compressed in ragged chunks and in one shot into two pools of `dtype`."""
    g = W.generator(95, seed, 0, DEV)
    xs = [W.to_storage(W.randn((T, D), g, DEV), xdt) for _ in range(3)]
    lg = [W.randn((T,), g, DEV) for _ in range(3)]
    mb = -(-T // 256)
    need = [W.blocks_for_entries(T // ratio, ratio)] * 3
    pc = W.make_pool(dtype, D, ratio, need, mb, g, DEV, fill=False)
    po = W.PagedTensors(pc.data.clone(), pc.scale.clone(), pc.block_table.clone(), dtype, D, ratio)
    gate = mode == "gate"
    state = torch.zeros(3, ratio, D, dtype=xs[0].dtype, device=DEV)
    st_l = torch.zeros(3, ratio, device=DEV)
    cuts = [sorted({0, 1, 3, 130, 131, 517 % T, 900 % T, T}), [0, 1, T], [0, T]]
    for s in range(max(len(c) for c in cuts) - 1):
        rng = [(c[s], c[s + 1]) if s + 1 < len(c) else (T, T) for c in cuts]
        x = torch.cat([xs[b][a:e] for b, (a, e) in enumerate(rng)])
        cu = ints([0] + list(np.cumsum([e - a for a, e in rng])))
        hyb.hyb_compress(x, cu, ints([a for a, _ in rng]), max(e - a for a, e in rng), state, pc, rd,
                         eps=1e-6, gate_logits=torch.cat([lg[b][a:e] for b, (a, e) in enumerate(rng)])
                         if gate else None, state_logits=st_l if gate else None)
    st2, stl2 = torch.zeros_like(state), torch.zeros_like(st_l)
    hyb.hyb_compress(torch.cat(xs), ints([0, T, 2 * T, 3 * T]), ints([0, 0, 0]), T, st2, po, rd,
                     eps=1e-6, gate_logits=torch.cat(lg) if gate else None,
                     state_logits=stl2 if gate else None)
    torch.cuda.synchronize()
    refs = [O.compress_stream(to_f64(xs[b]), lg[b].cpu().double().numpy() if gate else None,
                              ratio, mode, rd, 1e4, 1e-6) for b in range(3)]
    return pc, po, refs


@pytest.mark.parametrize("ratio,mode,xdt,D,rd,T", [
    (4, "mean", "bf16", 512, 64, 1000), (128, "gate", "bf16", 512, 64, 1500),
    (4, "gate", "f32", 256, 64, 600), (4, "mean", "bf16", 514, 64, 300)])
def test_compress_into_fp8_pool(gpu_lib, ratio, mode, xdt, D, rd, T):
    """Compressed entries quantised as they are stored (fp8 attention cache): chunked equals one
    shot byte for byte (codes and scales), and decoded entries match the oracle's."""
    pc, po, refs = _compress_chunked_and_once(gpu_lib, "fp8", ratio, mode, xdt, D, rd, T, ratio)
    assert torch.equal(pc.data, po.data) and torch.equal(pc.scale, po.scale)
    host = stored(pc)
    for b in range(3):
        n = T // ratio
        rows = [raw_entry(host, ratio, b, g) for g in range(n)]
        check_fp8_rows(np.stack([r[0] for r in rows]), np.array([r[1] for r in rows]), refs[b], 1e-5)


@pytest.mark.parametrize("ratio,mode,xdt,D,rd,T", [
    (4, "mean", "bf16", 128, 64, 1000), (4, "gate", "f32", 128, 64, 700),
    (128, "mean", "bf16", 256, 64, 600)])
def test_compress_into_fp4_pool(gpu_lib, ratio, mode, xdt, D, rd, T):
    """Compressed entries quantised to OCP MX fp4 as they are stored (indexer-key compression):
    chunked equals one shot byte for byte; each 32-value block's shared exponent is the oracle's
    (unless the block maximum lies within float32 error of a power of two) and decoded values lie
    within half an E2M1 step (or the saturation error above 6) of the oracle's entries."""
    pc, po, refs = _compress_chunked_and_once(gpu_lib, "fp4", ratio, mode, xdt, D, rd, T, 7 + ratio)
    assert torch.equal(pc.data, po.data) and torch.equal(pc.scale, po.scale)
    host = stored(pc)
    opool = to_oracle_pool(pc)
    err = 1e-5
    for b in range(3):
        n = T // ratio
        dec = O.pool_entries(opool, b, range(n))
        ref = refs[b]
        ex = np.stack([raw_entry(host, ratio, b, g)[1] for g in range(n)]).astype(np.int64) - 127
        amax = np.abs(ref).reshape(n, D // 32, 32).max(axis=2)
        want = np.vectorize(O.mx_exponent)(amax)
        near = np.abs(np.log2(amax) - np.round(np.log2(amax))) < 1e-5
        assert np.all((ex == want) | near)
        sc = np.repeat(np.exp2(ex.astype(np.float64)), 32, axis=1)
        v = np.abs(ref) / sc
        step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
        bound = (0.5 * step + np.maximum(v - 6.0, 0.0)) * sc + 2 * err
        assert np.all(np.abs(dec - ref) <= bound)


# ================================================== attention output: inverse RoPE + fp8 rows
def _check_fp8_output(codes, scales, out_bf16, want, tol):
    """fp8 output rows (codes [n, H, D], scales [n, H]) against (1) the same call's bf16 output:
    both come from one float32 row v, which bf16 rounds to within 2^-9 |v|, and (2) the oracle's
    output within the attention tolerance `tol`, each plus half an E4M3 step of the row's scale."""
    c = codes.cpu().numpy().reshape(-1, codes.shape[-1])
    s = scales.cpu().numpy().astype(np.float64).reshape(-1)
    b16 = to_f64(out_bf16).reshape(c.shape)
    amax = np.abs(b16).max(axis=1)
    assert np.all(np.abs(s * 448.0 - amax) <= 2.0 ** -8 * amax + 1e-30)
    dec = O.e4m3fn_to_f64(c) * s[:, None]
    half = 0.5 * e4m3_step(b16 / s[:, None]) * s[:, None]
    assert np.all(np.abs(dec - b16) <= half * 1.0001 + 2.0 ** -8 * np.abs(b16) + 1e-30)
    w = np.asarray(want, np.float64).reshape(-1, c.shape[1])
    assert np.all(np.abs(dec - w) <= 2 * half + tol)


def test_attention_fp8_output(gpu_lib):
    """C4 sparse decode (L = 1 .. 33333, top-512), C128 dense decode and the same C128 queries in
    the prefill form, each with a bf16 output and with an fp8 output (one scale per query and
    head) from otherwise identical calls."""
    hyb = gpu_lib
    from tests.test_gpu_parity import gpu_decode, gpu_topk, oracle_out
    from tests.parity_util import BF16_ABS
    c4 = W.sparse_decode(DEV, seed=1, batch=5, ctx=[1, 100, 700, 5000, 33333])
    c128 = W.dense_decode(DEV, seed=1, batch=6, ctx=[1, 128, 129, 300, 20000, 70001])
    for wl, sparse in ((c4, True), (c128, False)):
        topk = gpu_topk(hyb, wl) if sparse else None
        out = gpu_decode(hyb, wl, topk)
        codes = torch.empty(wl.q.shape, dtype=torch.uint8, device=DEV)
        sc = torch.empty(wl.q.shape[:2], dtype=torch.float32, device=DEV)
        hyb.hyb_attn_decode(wl.q, wl.seq_lens, wl.max_seq_len, wl.swa, wl.comp, codes,
                            topk_idx=topk, k=wl.k if sparse else 0, window=wl.window,
                            rope_dim=wl.rope_dim, rope_base=wl.rope_base, out_scale=sc)
        torch.cuda.synchronize()
        seqs = range(wl.batch)
        sel = {b: topk[b].cpu().numpy() for b in seqs} if sparse else None
        want = oracle_out(wl, to_oracle_pool(wl.swa), to_oracle_pool(wl.comp), seqs, sel)
        _check_fp8_output(codes, sc, out, want, BF16_ABS)
        if not sparse:
            # the prefill entry point, same queries (position seq_len - 1 of each sequence)
            pos = (wl.seq_lens - 1).contiguous()
            codes2, sc2 = torch.empty_like(codes), torch.empty_like(sc)
            hyb.hyb_attn_prefill(wl.q, pos, wl.max_seq_len - 1, wl.swa, wl.comp, codes2,
                                 window=wl.window, rope_dim=wl.rope_dim, rope_base=wl.rope_base,
                                 q_seq=torch.arange(wl.batch, dtype=I32, device=DEV), out_scale=sc2)
            torch.cuda.synchronize()
            assert torch.equal(codes2, codes) and torch.equal(sc2, sc)


# ====================================== fused step before the attention: Q-norm + KV RoPE + insert
@pytest.mark.parametrize("qdt,kvdt,pdt,D,H,rd", [
    ("bf16", "bf16", "bf16", 512, 64, 64), ("f32", "f32", "f32", 64, 8, 16),
    ("bf16", "f32", "fp8", 512, 64, 64), ("f32", "bf16", "bf16", 514, 3, 32)])
def test_q_norm_kv_insert(gpu_lib, qdt, kvdt, pdt, D, H, rd):
    """Three sequences (300 / 1 / 77 new tokens at positions 0 / 999_999 / 250): query rows
    against the oracle's RMSNorm + RoPE per head; the window entries equal hyb_swa_insert's bytes
    for the same tokens; the in-place form (q_out = q) writes the same rows."""
    hyb = gpu_lib
    g = W.generator(96, D, H, DEV)
    n_new, starts = [300, 1, 77], [0, 999_999, 250]
    T = sum(n_new)
    q = W.to_storage(W.randn((T, H, D), g, DEV) * torch.exp2(W.randn((T, H, 1), g, DEV) * 3), qdt)
    kv = W.to_storage(W.randn((T, D), g, DEV), kvdt)
    mb = (max(s + n for s, n in zip(starts, n_new)) + 255) // 256
    need = [W.blocks_for_positions(s, s + n) for s, n in zip(starts, n_new)]
    swa1 = W.make_pool(pdt, D, 1, need, mb, g, DEV, fill=False)
    swa2 = W.PagedTensors(swa1.data.clone(), None if swa1.scale is None else swa1.scale.clone(),
                          swa1.block_table.clone(), pdt, D, 1)
    cu, st = ints(np.cumsum([0] + n_new)), ints(starts)
    q_out = torch.empty_like(q)
    hyb.hyb_q_norm_kv_insert(q, kv, cu, st, max(n_new), swa1, q_out=q_out, rope_dim=rd, eps=1e-6)
    hyb.hyb_swa_insert(kv, cu, st, max(n_new), swa2, rd)
    q2 = q.clone()
    hyb.hyb_q_norm_kv_insert(q2, kv, cu, st, max(n_new), swa1, rope_dim=rd, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(swa1.data, swa2.data)
    if swa1.scale is not None:
        assert torch.equal(swa1.scale, swa2.scale)
    assert torch.equal(q2, q_out)
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, n_new)])
    want = O.q_norm_rope(to_f64(q), pos, rd, 1e4, 1e-6)
    got = to_f64(q_out)
    if qdt == "f32":
        assert np.all(np.abs(got - want) <= 4e-6 * (1.0 + np.abs(want)))
    else:
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-5)


# ================================== prefill over fp8 caches built by quantise-on-insert
def test_prefill_over_fp8_pools_built_from_raw_tokens(gpu_lib):
    """One sequence: 1000 prior raw tokens then a 300-token chunk, its window, C4 and C128 entries
    written into fp8 pools by the window insert and the compressors (quantised as stored), then C4
    top-64 and C128 dense prefill attention over those pools. The oracle attends over exactly the
    stored entries (decoded codes times scales) with the same selections."""
    hyb = gpu_lib
    from tests.parity_util import BF16_ABS
    D, rd, H, T0, T1, k = 512, 64, 64, 1000, 300, 64
    T = T0 + T1
    g = W.generator(99, 0, 0, DEV)
    x = W.to_storage(W.randn((T, D), g, DEV), "bf16")
    lg = W.randn((T,), g, DEV)
    q = W.to_storage(W.randn((T1, H, D), g, DEV), "bf16")
    iq = W.to_storage(W.randn((T1, 64, 128), g, DEV), "bf16")
    iw = W.randn((T1, 64), g, DEV) / 128 ** 0.5
    mb = -(-T // 256)
    swa = W.make_pool("fp8", D, 1, [W.blocks_for_positions(0, T)], mb, g, DEV, fill=False)
    c4 = W.make_pool("fp8", D, 4, [W.blocks_for_entries(T // 4, 4)], mb, g, DEV, fill=False)
    c128 = W.make_pool("fp8", D, 128, [W.blocks_for_entries(T // 128, 128)], mb, g, DEV, fill=False)
    ip = W.make_pool("bf16", 128, 4, [W.blocks_for_entries(T // 4, 4)], mb, g, DEV)
    s4 = torch.zeros(1, 4, D, dtype=x.dtype, device=DEV)
    s128 = torch.zeros(1, 128, D, dtype=x.dtype, device=DEV)
    l128 = torch.zeros(1, 128, device=DEV)
    for a, e in ((0, T0), (T0, T)):
        cu, st = ints([0, e - a]), ints([a])
        hyb.hyb_swa_insert(x[a:e], cu, st, e - a, swa, rd)
        hyb.hyb_compress(x[a:e], cu, st, e - a, s4, c4, rd, eps=1e-6)
        hyb.hyb_compress(x[a:e], cu, st, e - a, s128, c128, rd, eps=1e-6, gate_logits=lg[a:e],
                         state_logits=l128)
    pos = torch.arange(T0, T, dtype=I32, device=DEV)
    qseq = torch.zeros(T1, dtype=I32, device=DEV)
    topk = torch.empty(T1, k, dtype=I32, device=DEV)
    hyb.hyb_index_topk(iq, iw, pos, T - 1, ip, k, topk, q_seq=qseq)
    out4, out128 = torch.empty_like(q), torch.empty_like(q)
    hyb.hyb_attn_prefill(q, pos, T - 1, swa, c4, out4, topk_idx=topk, k=k, q_seq=qseq)
    hyb.hyb_attn_prefill(q, pos, T - 1, swa, c128, out128, q_seq=qseq)
    torch.cuda.synchronize()
    sw, p4, p128 = to_oracle_pool(swa), to_oracle_pool(c4), to_oracle_pool(c128)
    # the stored entries are the quantised oracle entries (checked against the float64 entries)
    ref4 = O.compress_stream(to_f64(x), None, 4, "mean", rd, 1e4, 1e-6)
    got4 = O.pool_entries(p4, 0, range(T // 4))
    assert np.all(np.abs(got4 - ref4) <= 0.5 * e4m3_step(ref4 / (np.abs(ref4).max(1, keepdims=True) / 448))
                  * (np.abs(ref4).max(1, keepdims=True) / 448) * 1.001 + 2e-5)
    qq, tk = to_f64(q), topk.cpu().numpy()
    for i in (0, 1, 57, 128, 200, 299):
        p = T0 + i
        want4 = O.hybrid_query(qq[i], p, 0, sw, p4, 128, D ** -0.5, rd, 1e4, tk[i])
        want128 = O.hybrid_query(qq[i], p, 0, sw, p128, 128, D ** -0.5, rd, 1e4, None)
        assert np.abs(to_f64(out4)[i] - want4).max() <= BF16_ABS, i
        assert np.abs(to_f64(out128)[i] - want128).max() <= BF16_ABS, i
