"""Pins for the oracle's per-step functions (CPU only).

Every check compares the oracle with something other than itself: hand-computed values,
closed forms, special cases that reduce to library routines (torch float64 SDPA) and brute
force over tiny inputs chosen so that a dropped term, a wrong sign or index, or a transposed
operand fails.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O


# ----------------------------------------------------------------------------------- RoPE
def test_rope_hand_example_pairs_and_frequencies():
    # D = 6, r_d = 4, base 100: dims 0,1 untouched; pair (2,3) turns by pos*1, pair (4,5) by
    # pos*100**(-2/4) = pos*0.1.
    x = np.array([5.0, -7.0, 1.0, 0.0, 0.0, 1.0])
    y = O.rope(x, 2.0, 4, 100.0)
    assert y[0] == 5.0 and y[1] == -7.0
    assert y[2] == pytest.approx(math.cos(2.0), abs=1e-15)
    assert y[3] == pytest.approx(math.sin(2.0), abs=1e-15)
    assert y[4] == pytest.approx(-math.sin(0.2), abs=1e-15)
    assert y[5] == pytest.approx(math.cos(0.2), abs=1e-15)


def test_rope_identity_inverse_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(O.rope(x, 0.0, 16, 10000.0), x)
    for pos in (1, 127, 131071, (1 << 20) - 1):
        y = O.rope(x, pos, 16, 10000.0)
        assert np.allclose(O.rope(y, -pos, 16, 10000.0), x, atol=1e-12)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        assert np.array_equal(y[:, :48], x[:, :48])


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    for m, n in ((3, 10), (1000, 17), (65536, 65537)):
        lhs = O.rope(q, m, 32, 10000.0) @ O.rope(k, n, 32, 10000.0)
        rhs = q @ O.rope(k, n - m, 32, 10000.0)
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


# -------------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form():
    y = O.rmsnorm(np.array([3.0, 4.0]), 0.0)
    assert np.allclose(y, np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=0, atol=1e-15)
    assert np.array_equal(O.rmsnorm(np.zeros(8), 1e-6), np.zeros(8))
    rng = np.random.default_rng(3)
    x = rng.standard_normal(512) * 0.01
    ms = np.mean(x * x)
    rms_out = math.sqrt(np.mean(O.rmsnorm(x, 1e-6) ** 2))
    assert rms_out == pytest.approx(1.0 / math.sqrt(1.0 + 1e-6 / ms), rel=1e-12)
    assert np.allclose(O.rmsnorm(7.0 * x, 0.0), O.rmsnorm(x, 0.0), atol=1e-13)


# -------------------------------------------------------------------------------- pooling
def test_pool_mean_and_gate():
    t = np.array([[1.0, 2.0], [3.0, 6.0], [5.0, 1.0], [7.0, 3.0]])
    assert np.allclose(O.pool_tokens(t, "mean"), [4.0, 3.0])
    # logits (0, ln 3): weights 1/4, 3/4
    t2 = np.array([[4.0, 0.0], [0.0, 8.0]])
    assert np.allclose(O.pool_tokens(t2, "gate", [0.0, math.log(3.0)]), [1.0, 6.0], atol=1e-14)
    assert np.allclose(O.pool_tokens(t, "gate", [0.3] * 4), O.pool_tokens(t, "mean"), atol=1e-14)
    dom = O.pool_tokens(t, "gate", [0.0, 0.0, 800.0, 0.0])
    assert np.allclose(dom, t[2], atol=1e-12)
    same = np.tile(np.array([[2.5, -1.0]]), (128, 1))
    rng = np.random.default_rng(4)
    assert np.allclose(O.pool_tokens(same, "gate", rng.standard_normal(128)), [2.5, -1.0],
                       atol=1e-13)


def test_compressed_entry_hand_example():
    # four identical tokens v = (1, 2, 2, 4): mean = v, rms = 2.5, RMSNorm (eps 0) = v / 2.5;
    # group g = 1 of ratio 4 ends at position 7, so the last pair turns by 7 rad (r_d = 2).
    v = np.array([1.0, 2.0, 2.0, 4.0])
    e = O.compressed_entry(np.tile(v, (4, 1)), None, 1, 4, "mean", 2, 10000.0, 0.0)
    a, b = 0.8, 1.6
    want = [0.4, 0.8, a * math.cos(7) - b * math.sin(7), a * math.sin(7) + b * math.cos(7)]
    assert np.allclose(e, want, atol=1e-15)


def test_compress_stream_prefix_and_pending():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((27, 16))
    lg = rng.standard_normal(27)
    full = O.compress_stream(x, lg, 4, "gate", 8, 10000.0, 1e-6)
    assert full.shape == (6, 16)
    part = O.compress_stream(x[:13], lg[:13], 4, "gate", 8, 10000.0, 1e-6)
    assert np.array_equal(part, full[:3])
    slots, lslots = O.pending_group(x, lg, 4)
    assert sorted(slots) == [0, 1, 2]
    assert np.array_equal(slots[2], x[26]) and lslots[0] == lg[24]


def test_compress_stream_hand_groups():
    """Three softmax-gate groups of ratio 2 built by hand, with a different logit pair in each
    group, plus one trailing token of an incomplete group. With r_d = 2 and theta_0 = 1 the last
    pair turns by the group-end position (1, 3, 5) in radians; eps = 0.
      group 0: logits (0, ln 3) -> weights (1/4, 3/4): pooled (1, 0, 0, 3), RMS sqrt(2.5)
      group 1: logits (ln 3, 0) -> weights (3/4, 1/4): pooled (0, 3, 1, 0), RMS sqrt(2.5)
      group 2: logits (5, 5)    -> weights (1/2, 1/2): pooled (1, 1, 1, 1), RMS 1
    A logits window taken at the wrong offset, a group rotated at the wrong position or a group
    built from the wrong tokens changes at least one entry."""
    x = np.array([[4.0, 0, 0, 0], [0, 0, 0, 4.0],
                  [0, 4.0, 0, 0], [0, 0, 4.0, 0],
                  [2.0, 2.0, 0, 0], [0, 0, 2.0, 2.0],
                  [9.0, -9.0, 9.0, 9.0]])
    lg = np.array([0.0, math.log(3.0), math.log(3.0), 0.0, 5.0, 5.0, -3.0])
    got = O.compress_stream(x, lg, 2, "gate", 2, 10000.0, 0.0)
    s25 = math.sqrt(2.5)
    want = np.array([
        [1 / s25, 0.0, -3 * math.sin(1.0) / s25, 3 * math.cos(1.0) / s25],
        [0.0, 3 / s25, math.cos(3.0) / s25, math.sin(3.0) / s25],
        [1.0, 1.0, math.cos(5.0) - math.sin(5.0), math.sin(5.0) + math.cos(5.0)],
    ])
    assert got.shape == (3, 4)
    assert np.allclose(got, want, rtol=0, atol=1e-14)
    # mean mode over the same tokens: group 1 pools to (0, 2, 2, 0), RMS sqrt(2)
    got_m = O.compress_stream(x, None, 2, "mean", 2, 10000.0, 0.0)
    r2 = math.sqrt(2.0)
    assert np.allclose(got_m[1], [0.0, r2, r2 * math.cos(3.0), r2 * math.sin(3.0)], rtol=0, atol=1e-14)


def test_logical_pool_layout_and_round_trip():
    """Entries of several sequences laid out block by block in sequence order: with ratio 4 a
    block holds 64 entries, so 150 entries take blocks 0, 1, 2 (the last one 22 entries, rest
    zero) and the next sequence starts at block 3; the table pads with -1. Reading every entry
    back through the paged address rule returns it unchanged (bf16: rounded to nearest even)."""
    rng = np.random.default_rng(12)
    e = [rng.standard_normal((150, 8)), rng.standard_normal((64, 8)), rng.standard_normal((1, 8))]
    pool = O.logical_pool(e, 4)
    assert pool.data.shape == (5, 64, 8)
    assert pool.block_table.tolist() == [[0, 1, 2], [3, -1, -1], [4, -1, -1]]
    assert np.array_equal(pool.data[1, 6], e[0][70])      # entry 70: block 1, slot 6
    assert np.array_equal(pool.data[2, 21], e[0][149])
    assert not pool.data[2, 22:].any() and not pool.data[4, 1:].any()
    for b, ent in enumerate(e):
        assert np.array_equal(O.pool_entries(pool, b, range(len(ent))), ent)
    # ratio 128: two entries per block
    p128 = O.logical_pool([e[0][:5]], 128)
    assert p128.data.shape == (3, 2, 8) and p128.block_table.tolist() == [[0, 1, 2]]
    assert np.array_equal(p128.data[2, 0], e[0][4])
    assert np.array_equal(O.pool_entries(p128, 0, [4, 0, 3]), e[0][[4, 0, 3]])
    # bf16 storage: the stored bit patterns are the nearest-even bf16 of each value
    vals = np.array([[1.0, 1.00390625, 1.01171875, -3.0e-3, 65504.0, 0.0, -0.0, 1e-40]])
    pb = O.logical_pool([vals], 1, dtype="bf16")
    # 1 + 2^-8 ties to 1 (even); 1 + 3 * 2^-8 ties up to 1 + 2^-6
    assert pb.data[0, 0, :3].tolist() == [0x3F80, 0x3F80, 0x3F82]
    back = O.pool_entries(pb, 0, [0])[0]
    assert back[0] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[4] == 65536.0


def test_swa_entries_are_rotated_tokens():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 8))
    s = O.swa_entries(x, [5, 6, 7], 8, 10000.0)
    for i, t in enumerate((5, 6, 7)):
        assert np.allclose(s[i], O.rope(x[i], t, 8, 10000.0), atol=0)
    assert np.allclose(np.linalg.norm(s, axis=1), np.linalg.norm(x, axis=1))


def test_q_norm_rope_hand_example_and_invariants():
    """Hand example: head rows (3, 4) and (0, 2) with no rotated dims normalise to (3, 4) / 3.5355..
    and (0, 1.4142..); with both dims rotated at position 1 (theta_0 = 1) the second row turns by
    one radian. Invariants at D = 512, r_d = 64: every head's norm is sqrt(D * ms / (ms + eps)) (the
    rotation keeps it), the unrotated dims equal the RMS-normalised row, and undoing the rotation
    gives the RMS-normalised row back."""
    q = np.array([[[3.0, 4.0], [0.0, 2.0]]])
    got = O.q_norm_rope(q, [0], 0, 1e4, 0.0)
    assert np.allclose(got[0, 0], [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    assert np.allclose(got[0, 1], [0.0, math.sqrt(2.0)], rtol=0, atol=1e-15)
    got = O.q_norm_rope(q, [1], 2, 1e4, 0.0)
    r2 = math.sqrt(2.0)
    assert np.allclose(got[0, 1], [-r2 * math.sin(1.0), r2 * math.cos(1.0)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 5, 512)) * 7.0
    pos = [0, 77, 1_000_000]
    eps = 1e-6
    got = O.q_norm_rope(q, pos, 64, 1e4, eps)
    ms = np.mean(q * q, axis=-1)
    assert np.allclose(np.linalg.norm(got, axis=-1), np.sqrt(512 * ms / (ms + eps)), rtol=1e-12)
    normed = q / np.sqrt(ms + eps)[..., None]
    assert np.allclose(got[..., :448], normed[..., :448], rtol=1e-14)
    back = O.rope(got, -np.asarray(pos, np.float64)[:, None], 64, 1e4)
    assert np.allclose(back, normed, rtol=0, atol=1e-9)


# ----------------------------------------------------------------------------- visibility
@pytest.mark.parametrize("p,r,want", [
    (0, 4, 0), (127, 4, 0), (128, 4, 1), (131, 4, 1), (132, 4, 2), (131071, 4, 32736),
    (127, 128, 0), (128, 128, 1), (255, 128, 1), (256, 128, 2), ((1 << 20) - 1, 128, 8191),
    (69631, 4, 17376), (65536, 4, 16353),
])
def test_n_visible_table(p, r, want):
    assert O.n_visible(p, r, 128) == want


def test_visibility_covers_every_older_position_exactly_once_groupwise():
    """Brute force: with n_vis visible groups, every raw position older than the window lies in
    a visible group, and every visible group holds at least one position older than the window
    (so the overlap with the window is < r positions)."""
    W = 16
    for r in (4, 8):
        for p in range(0, 80):
            ws = O.window_start(p, W)
            nv = O.n_visible(p, r, W)
            covered = set(range(nv * r))
            assert all(t in covered for t in range(ws))
            for g in range(nv):
                assert g * r < ws
            # visible groups are complete by the query position
            assert nv * r - 1 <= p


# -------------------------------------------------------------------------------- indexer
def test_indexer_hand_values():
    q = np.array([[1.0, 1.0], [2.0, 0.0]])
    w = np.array([-1.0, 0.5])
    keys = np.array([[1.0, 1.0],     # dots (2, 2)   -> -2 + 1 = -1
                     [-1.0, -2.0],   # dots (-3, -2) -> relu -> 0
                     [3.0, -4.0]])   # dots (-1, 6)  -> 0 + 3 = 3
    s = O.indexer_scores(q, w, keys)
    assert s.tolist() == [-1.0, 0.0, 3.0]


def test_indexer_brute_force_loops():
    rng = np.random.default_rng(7)
    q, w, keys = rng.standard_normal((3, 5)), rng.standard_normal(3), rng.standard_normal((9, 5))
    s = O.indexer_scores(q, w, keys)
    for g in range(9):
        tot = 0.0
        for h in range(3):
            d = sum(q[h, j] * keys[g, j] for j in range(5))
            tot += w[h] * (d if d > 0 else 0.0)
        assert s[g] == pytest.approx(tot, rel=1e-12, abs=1e-12)


# ---------------------------------------------------------------------------------- top-k
def _rank_rule(scores, k):
    """Independent characterisation: g is chosen iff fewer than k entries precede it in the
    order (score desc, index asc)."""
    n = len(scores)
    chosen = [g for g in range(n)
              if sum(1 for j in range(n) if scores[j] > scores[g]
                     or (scores[j] == scores[g] and j < g)) < k]
    return chosen


def test_topk_matches_rank_rule_with_many_ties():
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(0, 24))
        k = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, size=n).astype(np.float64) * 0.5
        got = O.topk_select(s, k)
        want = _rank_rule(s, k)
        assert got[:len(want)].tolist() == want
        assert (got[len(want):] == -1).all() and len(got) == k


def test_topk_exhaustive_small_sets():
    # every score vector over {0, 1, 2} of length 5, every k: brute force over subsets
    for s in itertools.product((0.0, 1.0, 2.0), repeat=5):
        for k in range(1, 7):
            got = [g for g in O.topk_select(np.array(s), k) if g >= 0]
            best = None
            for sub in itertools.combinations(range(5), min(k, 5)):
                key = (sorted((-s[g] for g in sub)), list(sub))
                if best is None or key < best[0]:
                    best = (key, list(sub))
            assert got == best[1]


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([-0.0, 0.0, -0.0, -1.0, 0.0])
    assert O.topk_select(s, 2).tolist() == [0, 1]
    assert O.topk_select(s, 4).tolist() == [0, 1, 2, 4]


def test_topk_degenerate():
    assert O.topk_select(np.zeros(0), 4).tolist() == [-1, -1, -1, -1]
    assert O.topk_select(np.array([3.0, 1.0]), 5).tolist() == [0, 1, -1, -1, -1]


# ------------------------------------------------------------------------------ attention
def _sdpa64(q, keys, scale):
    """torch float64 SDPA with one shared K=V head broadcast to every query head."""
    qt = torch.from_numpy(q)[:, None, :]                       # [H, 1, D]
    kt = torch.from_numpy(keys)[None].expand(q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)[:, 0].numpy()


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(9)
    q, keys = rng.standard_normal((6, 32)), rng.standard_normal((50, 32))
    o, pr = O.attend(q, keys, 1 / math.sqrt(32))
    assert np.allclose(o, _sdpa64(q, keys, 1 / math.sqrt(32)), atol=1e-12)
    assert np.allclose(pr.sum(axis=1), 1.0, atol=1e-14)


def test_attend_special_cases():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 8))
    one = rng.standard_normal((1, 8))
    o, _ = O.attend(q, one, 0.3)
    assert np.allclose(o, np.tile(one, (3, 1)), atol=0)
    two = np.array([[1.0] * 8, [3.0] * 8])
    o2, _ = O.attend(np.zeros((2, 8)), two, 1.0)   # equal scores -> average
    assert np.allclose(o2, 2.0)
    keys = rng.standard_normal((40, 8))
    o3, _ = O.attend(q * 5, keys, 1.0)              # each coordinate within the keys' hull
    assert (o3 <= keys.max(axis=0) + 1e-12).all() and (o3 >= keys.min(axis=0) - 1e-12).all()
    # scores far apart: the top key dominates (max-subtraction keeps this finite)
    big = np.array([[0.0] * 8, [1.0] * 8])
    o4, _ = O.attend(np.full((1, 8), 1e4), big, 1.0)
    assert np.allclose(o4, [[1.0] * 8])
