"""Host-side byte/flop model used by the benchmark, pinned to the page's KV accounting."""

import json
import os

from sparse_attention_hyb_amd import bytes_model as BM

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_c4_decode_bytes_per_query_token():
    sb = BM.decode_query_bytes(131072, ratio=4, sparse=True)
    assert sb.indexer_keys == 32736 * 256
    assert sb.attn_entries == (512 + 128) * 1024
    assert sb.io == 2 * 64 * 512 * 2 + 64 * 128 * 2 + 64 * 4 + 512 * 4
    assert sb.total == 9_185_536


def test_c128_decode_bytes_per_query_token():
    sb = BM.decode_query_bytes(1 << 20, ratio=128, sparse=False)
    assert sb.attn_entries == (8191 + 128) * 1024
    assert sb.total == 8_649_728


def test_quantised_entry_sizes():
    assert BM.entry_bytes("fp8", 512) == 516
    assert BM.entry_bytes("fp4", 128) == 68


def test_kv_accounting_reproduces_page_numbers():
    """The vLLM page's 1M-context numbers: 83.9 GiB for a V3.2-style 61-layer stack and 9.62 GiB
    for V4. 61 x (512 + 64 + 128) bf16 values per token reproduces the first exactly; a stack of 30
    C4 + 31 C128 layers of 512-dim bf16 entries with 128-dim bf16 indexer keys and a 128-token
    window reproduces the second (the layer split is a reading, not stated on the page)."""
    g = json.load(open(os.path.join(GOLD, "kv_accounting.json")))
    ctx = g["context_tokens"]
    v32 = g["v32_layers"] * (512 + 64 + 128) * g["bf16_bytes"] * ctx / 2 ** 30
    assert v32 == 83.875 and round(v32, 1) == g["v32_gib_printed"]
    v4 = BM.kv_state_bytes(ctx, 30, 31) / 2 ** 30
    assert round(v4, 2) == g["v4_gib_printed"]
    assert round(v32 / v4, 1) == g["ratio_printed"]


def test_prefill_flops_match_closed_form():
    fi, fa = BM.prefill_flops(range(65536, 65536 + 4096))
    # every query selects 512 C4 entries and sees a full 128-token window
    assert fa == 4096 * 4 * 64 * 512 * 640
    nv = sum(BM.n_visible(p, 4, 128) for p in range(65536, 65536 + 4096))
    assert fi == 2 * 64 * 128 * nv
    assert abs(fi / 1e9 - 1131.8) < 0.1 and abs(fa / 1e9 - 343.6) < 0.1


def test_page_constants_fixture():
    c = json.load(open(os.path.join(GOLD, "page_constants.json")))
    import oracle as O
    import sparse_attention_hyb_amd as hyb
    assert O.BLOCK_POSITIONS == hyb.BLOCK_POSITIONS == c["block_native_positions"]
    assert c["window_raw_tokens"] == 128 and c["topk"] == 512
    assert (c["c4_ratio"], c["c128_ratio"]) == (4, 128)


def test_compressor_and_indexer_bytes():
    """The compressor's ring holds raw tokens in x's storage type: a completing C128 group of bf16
    512-dim rows reads 127 ring rows and the new row (128 x 1 KiB) and writes one 1 KiB entry;
    softmax gates add a 4-byte logit per token. The indexer's algorithmic bytes at 128K are the
    32736 visible 256-byte keys, its 64 x 128 bf16 query and 64 float weights; the hand-off to the
    selector (8 bytes per entry + 2 KiB per 1024 entries) is counted apart."""
    assert BM.compress_decode_bytes(128) == 129 * 1024
    assert BM.compress_decode_bytes(128, gate=True) == 129 * 1024 + 128 * 4
    assert BM.compress_decode_bytes(4) == 5 * 1024
    assert BM.compress_decode_bytes(4, completes=False) == 2 * 1024
    assert BM.index_score_bytes(131072) == 32736 * 256 + 64 * 128 * 2 + 64 * 4
    assert BM.handoff_bytes(131072) == 32736 * 8 + 32 * 2048
