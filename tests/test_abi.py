"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and its host
validation returns the documented status before any HIP call (so fake device pointers are never
dereferenced)."""

import ctypes
import os
import re

import pytest

import sparse_attention_hyb_amd as hyb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000001000   # never dereferenced: every call below fails (or no-ops) in host checks


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hyb.LIB_PATH):
        pytest.skip("libhyb.so not built")
    return hyb.load()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^(?:int32_t|size_t|uint64_t|const char\*)\s+(hyb_\w+)\(", src, re.M))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 27
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(hyb.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert lib.hyb_abi_version() == hyb.ABI_VERSION == 5
    assert [lib.hyb_status_str(i).decode() for i in range(5)] == [
        "HYB_OK", "HYB_EINVAL", "HYB_ENOTSUP", "HYB_EWORKSPACE", "HYB_ELAUNCH"]


def pool(dtype=hyb.BF16, dim=512, ratio=4, scale=True, data=FAKE, reserved=0):
    return hyb.hyb_paged(data=data, scale=FAKE if scale else None, block_table=FAKE, dtype=dtype,
                         dim=dim, ratio=ratio, num_blocks=8, max_blocks=8, reserved=reserved)


def decode(lib, swa=None, comp=None, q_dtype=hyb.BF16, topk=None, k=0, window=128, ws=1 << 40,
           heads=64, scale=0.04, max_len=1000, rope_dim=64, q=FAKE, out_dtype=hyb.BF16,
           out_scale=None):
    swa = swa or pool(ratio=1)
    comp = comp or pool(ratio=128)
    return lib.hyb_attn_decode(q, q_dtype, FAKE, 4, heads, max_len, ctypes.byref(swa),
                               ctypes.byref(comp), topk, k, window, scale, rope_dim, 10000.0,
                               FAKE, out_dtype, out_scale, FAKE, ws, None)


@pytest.mark.parametrize("kw,code", [
    (dict(out_dtype=hyb.FP8_E4M3), hyb.HYB_EINVAL),                # fp8 output needs out_scale
    (dict(out_scale=FAKE), hyb.HYB_EINVAL),                        # out_scale only with fp8 output
    (dict(out_dtype=hyb.FP4_E2M1), hyb.HYB_ENOTSUP),
    (dict(out_dtype=hyb.FP8_E4M3, out_scale=FAKE, swa=pool(ratio=1, dim=4096),
          comp=pool(ratio=128, dim=4096)), hyb.HYB_ENOTSUP),      # fp8 output: dim <= 2048
    (dict(q=None), hyb.HYB_EINVAL),
    (dict(swa=pool(ratio=4)), hyb.HYB_EINVAL),                       # raw pool must be ratio 1
    (dict(comp=pool(ratio=1)), hyb.HYB_EINVAL),                      # compressed: 4 or 128
    (dict(comp=pool(ratio=128, dtype=hyb.F32)), hyb.HYB_EINVAL),     # pools share a dtype
    (dict(comp=pool(ratio=128, dim=256)), hyb.HYB_EINVAL),           # pools share a dim
    (dict(swa=pool(ratio=1, dtype=hyb.FP8_E4M3), comp=pool(ratio=128, dtype=hyb.FP8_E4M3),
          q_dtype=hyb.F32), hyb.HYB_ENOTSUP),                        # fp8 needs a bf16 query
    (dict(swa=pool(ratio=1, dtype=hyb.FP8_E4M3, scale=False),
          comp=pool(ratio=128, dtype=hyb.FP8_E4M3)), hyb.HYB_EINVAL),  # fp8 needs scales
    (dict(swa=pool(ratio=1, dtype=hyb.FP4_E2M1), comp=pool(ratio=128, dtype=hyb.FP4_E2M1)),
     hyb.HYB_ENOTSUP),
    (dict(topk=FAKE, k=0), hyb.HYB_EINVAL),
    (dict(topk=FAKE, k=hyb.KMAX + 1), hyb.HYB_EINVAL),
    (dict(window=0), hyb.HYB_EINVAL),
    (dict(scale=0.0), hyb.HYB_EINVAL),
    (dict(rope_dim=63), hyb.HYB_EINVAL),
    (dict(rope_dim=600), hyb.HYB_EINVAL),
    (dict(heads=0), hyb.HYB_EINVAL),
    (dict(ws=16), hyb.HYB_EWORKSPACE),
    (dict(swa=pool(ratio=1, dim=256), comp=pool(ratio=128, dim=256)), hyb.HYB_ENOTSUP),
    (dict(swa=pool(ratio=1, reserved=3)), hyb.HYB_EINVAL),
    (dict(swa=pool(ratio=1, data=None)), hyb.HYB_EINVAL),
])
def test_attn_decode_validation(lib, kw, code):
    assert decode(lib, **kw) == code
    assert lib.hyb_last_error().decode().startswith("hyb_attn_decode")


def test_attn_decode_compress_validation(lib):
    """The fused entry point checks the attention arguments, then the compressor's, before any
    launch (every case here fails in host code)."""
    out = pool(ratio=128)

    def call(swa=None, comp=None, ccall=True, mode=hyb.POOL_MEAN, o=out, rope=64, ws=1 << 40,
             eps=1e-6, state=FAKE):
        swa = swa or pool(ratio=1)
        comp = comp or pool(ratio=128)
        cc = hyb.hyb_compress_call(x=FAKE, x_dtype=hyb.BF16, gate_logits=None, cu_seqlens=FAKE,
                                   start_pos=FAKE, batch=4, max_new_tokens=1, state=state,
                                   state_logits=None, mode=mode, out=ctypes.pointer(o),
                                   rope_dim=rope, rope_base=1e4, eps=eps)
        return lib.hyb_attn_decode_compress(FAKE, hyb.BF16, FAKE, 4, 64, 1000, ctypes.byref(swa),
                                            ctypes.byref(comp), None, 0, 128, 0.04, 64, 1e4,
                                            FAKE, hyb.BF16, None, FAKE, ws,
                                            ctypes.byref(cc) if ccall else None, None)

    assert call(ccall=False) == hyb.HYB_EINVAL                        # compressor call required
    assert call(swa=pool(ratio=4)) == hyb.HYB_EINVAL                  # attention checked first
    assert call(ws=16) == hyb.HYB_EWORKSPACE
    assert call(state=None) == hyb.HYB_EINVAL
    assert call(mode=hyb.POOL_SOFTMAX_GATE) == hyb.HYB_EINVAL         # logits missing
    assert call(o=pool(ratio=1)) == hyb.HYB_EINVAL
    assert call(o=pool(ratio=128, dtype=hyb.FP8_E4M3, scale=False)) == hyb.HYB_EINVAL
    assert call(rope=3) == hyb.HYB_EINVAL
    assert call(eps=-1.0) == hyb.HYB_EINVAL
    assert lib.hyb_last_error().decode().startswith("hyb_attn_decode_compress")


def test_attn_workspace_sizes(lib):
    # C4 decode, 16 x 64 heads x 512 dims, 640 keys: 10 splits of 64 keys
    ws = lib.hyb_attn_decode_workspace_bytes(16, 64, 512, 131072, 4, 512, 128)
    assert ws == 16 * 10 * (512 * 64 + 2 * 64) * 4
    assert lib.hyb_attn_decode_workspace_bytes(0, 64, 512, 10, 4, 512, 128) == 0
    assert lib.hyb_attn_prefill_workspace_bytes(4096, 64, 512, 69631, 4, 512, 128) >= \
        4096 * (512 * 64 + 128) * 4


def test_prefill_validation(lib):
    s, c = pool(ratio=1), pool(ratio=4)
    st = lib.hyb_attn_prefill(FAKE, hyb.BF16, None, None, 4, 64, 100, ctypes.byref(s),
                              ctypes.byref(c), None, 0, 128, 0.04, 64, 1e4, FAKE, hyb.BF16,
                              None, FAKE, 1 << 40, None)
    assert st == hyb.HYB_EINVAL  # q_pos is required
    st = lib.hyb_attn_prefill(FAKE, hyb.BF16, None, FAKE, 0, 64, 100, ctypes.byref(s),
                              ctypes.byref(c), None, 0, 128, 0.04, 64, 1e4, FAKE, hyb.BF16,
                              None, None, 0, None)
    assert st == hyb.HYB_OK      # zero queries: nothing to do, nothing launched


def test_compress_validation(lib):
    out = pool(ratio=4)

    def call(x=FAKE, mode=hyb.POOL_MEAN, gate=None, st_logits=None, o=out, rope=64, batch=2,
             maxnew=4, eps=1e-6, x_dtype=hyb.BF16, state=FAKE):
        return lib.hyb_compress(x, x_dtype, gate, FAKE, FAKE, batch, maxnew, state, st_logits,
                                mode, ctypes.byref(o), rope, 1e4, eps, None)

    assert call(x=None) == hyb.HYB_EINVAL
    assert call(state=None) == hyb.HYB_EINVAL
    assert call(mode=7) == hyb.HYB_EINVAL
    assert call(mode=hyb.POOL_SOFTMAX_GATE) == hyb.HYB_EINVAL         # logits missing
    assert call(o=pool(ratio=1)) == hyb.HYB_EINVAL
    # quantised pools (fp8 entries, fp4 keys) need their scale arrays; fp4 rows whole blocks of 32
    assert call(o=pool(ratio=4, dtype=hyb.FP8_E4M3, scale=False)) == hyb.HYB_EINVAL
    assert call(o=pool(ratio=4, dtype=hyb.FP4_E2M1, scale=False)) == hyb.HYB_EINVAL
    assert call(o=pool(ratio=4, dim=80, dtype=hyb.FP4_E2M1)) == hyb.HYB_EINVAL
    assert call(o=pool(ratio=4, dim=4096)) == hyb.HYB_ENOTSUP
    assert call(rope=3) == hyb.HYB_EINVAL
    assert call(eps=-1.0) == hyb.HYB_EINVAL
    assert call(x_dtype=hyb.FP8_E4M3) == hyb.HYB_ENOTSUP
    assert call(batch=-1) == hyb.HYB_EINVAL
    assert call(batch=0) == hyb.HYB_OK
    assert call(maxnew=0) == hyb.HYB_OK
    s = pool(ratio=1)
    assert lib.hyb_swa_insert(FAKE, hyb.BF16, FAKE, FAKE, 2, 4, ctypes.byref(pool(ratio=4)), 64,
                              1e4, None) == hyb.HYB_EINVAL
    for bad, code in ((pool(ratio=1, dtype=hyb.FP4_E2M1), hyb.HYB_ENOTSUP),   # fp4 is for keys
                      (pool(ratio=1, dtype=hyb.FP8_E4M3, scale=False), hyb.HYB_EINVAL),
                      (pool(ratio=1, dtype=hyb.FP8_E4M3, dim=4096), hyb.HYB_ENOTSUP)):
        assert lib.hyb_swa_insert(FAKE, hyb.BF16, FAKE, FAKE, 2, 4, ctypes.byref(bad), 64, 1e4,
                                  None) == code
    assert lib.hyb_swa_insert(FAKE, hyb.BF16, FAKE, FAKE, 0, 4, ctypes.byref(s), 64, 1e4,
                              None) == hyb.HYB_OK


def test_index_validation(lib):
    ip = pool(ratio=4, dim=128)

    def call(k=512, ws=1 << 40, heads=64, q_dtype=hyb.BF16, p=ip, w=FAKE):
        return lib.hyb_index_topk(FAKE, q_dtype, w, None, FAKE, 16, heads, 131071, 128,
                                  ctypes.byref(p), k, FAKE, FAKE, ws, None)

    assert call(k=0) == hyb.HYB_EINVAL
    assert call(k=hyb.KMAX + 1) == hyb.HYB_EINVAL
    assert call(ws=100) == hyb.HYB_EWORKSPACE
    assert call(w=None) == hyb.HYB_EINVAL
    assert call(p=pool(ratio=1, dim=128)) == hyb.HYB_EINVAL
    assert call(p=pool(ratio=4, dim=100, dtype=hyb.FP4_E2M1)) == hyb.HYB_EINVAL
    assert call(p=pool(ratio=4, dim=128, dtype=hyb.FP8_E4M3)) == hyb.HYB_ENOTSUP
    assert call(heads=128, p=pool(ratio=4, dim=128, dtype=hyb.F32)) == hyb.HYB_ENOTSUP
    # hand-off pairs [16][32 x 1024] uint2, then the cumulative histograms [16][32][1024] uint16
    # a 1 MiB per-row histogram block (256 rows x 1024 bins x 4 B, zero between calls), then
    # per 1024-key part: bucketed (key, index) pairs and a cumulative uint16 histogram
    assert lib.hyb_index_topk_workspace_bytes(16, 131071, 128, 4) == \
        (1 << 20) + 16 * 32 * 1024 * 8 + 16 * 32 * 1024 * 2
    assert lib.hyb_topk(FAKE, 10, FAKE, 4, 20, 8, FAKE, None) == hyb.HYB_EINVAL   # ld < max_len
    assert lib.hyb_topk(FAKE, 20, FAKE, 4, 20, 0, FAKE, None) == hyb.HYB_EINVAL   # k = 0
    assert lib.hyb_topk(None, 20, FAKE, 4, 20, 8, FAKE, None) == hyb.HYB_EINVAL
    assert lib.hyb_index_score(FAKE, hyb.BF16, FAKE, None, FAKE, 16, 64, 131071, 128,
                               ctypes.byref(ip), FAKE, 100, None) == hyb.HYB_EINVAL  # ld too small


def test_index_keys_validation(lib):
    ip = pool(ratio=4, dim=128)

    def score(keys=FAKE, ld=65536, hist=FAKE, pld=32, p=ip):
        return lib.hyb_index_score_keys(FAKE, hyb.BF16, FAKE, None, FAKE, 16, 64, 131071, 128,
                                        ctypes.byref(p), keys, ld, hist, pld, None)

    def topk(keys=FAKE, ld=65536, hist=FAKE, pld=32, ratio=4, k=512, q_pos=FAKE):
        return lib.hyb_topk_keys(keys, ld, hist, pld, q_pos, 16, 131071, 128, ratio, k, FAKE, None)

    # 131071 - 127 = 130944 -> 32736 visible C4 entries -> 32 blocks of 1024
    assert score(keys=None) == hyb.HYB_EINVAL
    assert score(hist=None) == hyb.HYB_EINVAL
    assert score(ld=65535) == hyb.HYB_EINVAL   # below 2048 x part_ld
    assert score(ld=65537 + 2048) == hyb.HYB_EINVAL   # odd
    assert score(pld=31) == hyb.HYB_EINVAL
    assert score(pld=4097, ld=2048 * 4097) == hyb.HYB_EINVAL   # beyond the selector's parts
    assert score(p=pool(ratio=1, dim=128)) == hyb.HYB_EINVAL
    assert topk(keys=None) == hyb.HYB_EINVAL
    assert topk(q_pos=None) == hyb.HYB_EINVAL
    assert topk(ld=100) == hyb.HYB_EINVAL
    assert topk(pld=31) == hyb.HYB_EINVAL
    assert topk(ratio=8) == hyb.HYB_EINVAL
    assert topk(k=0) == hyb.HYB_EINVAL
    assert lib.hyb_last_error().decode().startswith("hyb_topk_keys")
    assert hyb.index_keys_shapes(16, 131071) == ((16, 65536), (16, 32, 1024))


def test_q_norm_kv_insert_validation(lib):
    def call(q=FAKE, q_dtype=hyb.BF16, heads=64, kv=FAKE, kv_dtype=hyb.BF16, batch=2, maxnew=4,
             q_out=FAKE, swa=None, rope=64, eps=1e-6):
        swa = swa or pool(ratio=1)
        return lib.hyb_q_norm_kv_insert(q, q_dtype, heads, kv, kv_dtype, FAKE, FAKE, batch, maxnew,
                                        q_out, ctypes.byref(swa), rope, 1e4, eps, None)

    assert call(q=None) == hyb.HYB_EINVAL
    assert call(q_out=None) == hyb.HYB_EINVAL
    assert call(kv=None) == hyb.HYB_EINVAL
    assert call(q_dtype=hyb.FP8_E4M3) == hyb.HYB_ENOTSUP
    assert call(kv_dtype=hyb.FP4_E2M1) == hyb.HYB_ENOTSUP
    assert call(heads=0) == hyb.HYB_EINVAL and call(heads=129) == hyb.HYB_EINVAL
    assert call(swa=pool(ratio=4)) == hyb.HYB_EINVAL                  # window pool: ratio 1
    assert call(swa=pool(ratio=1, dtype=hyb.FP4_E2M1)) == hyb.HYB_ENOTSUP
    assert call(swa=pool(ratio=1, dim=4096)) == hyb.HYB_ENOTSUP
    assert call(rope=3) == hyb.HYB_EINVAL
    assert call(eps=-1.0) == hyb.HYB_EINVAL
    assert call(batch=-1) == hyb.HYB_EINVAL
    assert call(eps=-1.0) == hyb.HYB_EINVAL
    assert lib.hyb_last_error().decode().startswith("hyb_q_norm_kv_insert")
    assert call(batch=0) == hyb.HYB_OK and call(maxnew=0) == hyb.HYB_OK


def test_gather_pages_validation(lib):
    def call(src=FAKE, dst=FAKE, sp=FAKE, dp=FAKE, n=4, page=65536, n_src=16, n_dst=8):
        return lib.hyb_gather_pages(src, n_src, dst, n_dst, sp, dp, n, page, None)

    assert call(src=None) == hyb.HYB_EINVAL and call(dp=None) == hyb.HYB_EINVAL
    assert call(n=-1) == hyb.HYB_EINVAL
    assert call(n_src=0) == hyb.HYB_EINVAL and call(n_dst=-3) == hyb.HYB_EINVAL
    assert call(page=0) == hyb.HYB_EINVAL and call(page=100) == hyb.HYB_EINVAL
    assert call(src=FAKE + 8) == hyb.HYB_EINVAL                      # not 16-byte aligned
    assert lib.hyb_last_error().decode().startswith("hyb_gather_pages")
    assert call(n=0) == hyb.HYB_OK


def test_gather_pages_binding_checks():
    """The binding refuses index tensors that are not 1-d int32 device tensors of one length and
    buffers that are not contiguous, before any library call (CPU tensors stand in here)."""
    import torch
    src = torch.zeros(4, 64, 16)
    dst = torch.zeros(4, 64, 16)
    i32 = torch.arange(4, dtype=torch.int32)
    with pytest.raises(TypeError, match="int32 device"):
        hyb.hyb_gather_pages(src, dst, i32, i32)               # host index tensors
    with pytest.raises(TypeError, match="int32 device"):
        hyb.hyb_gather_pages(src, dst, i32.long(), i32)
    with pytest.raises(TypeError, match="contiguous"):
        hyb.hyb_gather_pages(src.transpose(1, 2), dst, i32, i32)


@pytest.mark.parametrize("op", ["decode", "score", "topk"])
def test_window_smaller_than_ratio_is_refused(lib, op):
    """A window shorter than the compression ratio would make the group being filled visible."""
    if op == "decode":
        st = decode(lib, comp=pool(ratio=128), window=64)
    elif op == "score":
        ip = pool(dim=128, ratio=4)
        st = lib.hyb_index_score(FAKE, hyb.BF16, FAKE, None, FAKE, 2, 64, 1000, 2, ctypes.byref(ip),
                                 FAKE, 1024, None)
    else:
        st = lib.hyb_topk_keys(FAKE, 4096, FAKE, 2, FAKE, 2, 10000, 100, 128, 64, FAKE, None)
    assert st == hyb.HYB_EINVAL
    assert "window" in lib.hyb_last_error().decode()


def test_noalloc_index_topk_refuses_scratch_beyond_the_array(lib):
    """The allocation-free selector checks its scratch need against the static array on the host,
    before it looks up any device address: 100000 queries at 2^20 positions need far more."""
    ip = pool(dim=128, ratio=4)
    st = lib.hyb_index_topk_noalloc(FAKE, hyb.BF16, FAKE, None, FAKE, 100000, 64, 1 << 20, 128,
                                    ctypes.byref(ip), 512, FAKE, None)
    assert st == hyb.HYB_EINVAL
    assert "scratch" in lib.hyb_last_error().decode()
    need = lib.hyb_index_topk_workspace_bytes(16, (1 << 20) - 1, 128, 4)
    assert 0 < need <= hyb.NOALLOC_SCRATCH_BYTES
    # no queries: nothing to do, nothing looked up
    assert lib.hyb_index_topk_noalloc(FAKE, hyb.BF16, FAKE, None, FAKE, 0, 64, 1000, 128,
                                      ctypes.byref(ip), 512, FAKE, None) == hyb.HYB_OK


def test_decode_step_validation(lib):
    """hyb_decode_step checks on the host: a C4 layer needs the indexer query, a C128 layer none;
    at most two compressor calls; the workspace covers the step (selector rows, hand-off and
    attention partials)."""
    swa, c4, c128, ip = pool(ratio=1), pool(ratio=4), pool(ratio=128), pool(dim=128, ratio=4)

    def call(comp=c4, q_idx=FAKE, n_comp=0, ws=1 << 40, k=512, idx=ip, prep=None):
        return lib.hyb_decode_step(FAKE, hyb.BF16, FAKE, 4, 64, 100000, ctypes.byref(swa),
                                   ctypes.byref(comp), q_idx, hyb.BF16, FAKE, 64,
                                   ctypes.byref(idx) if idx is not None else None, k, None, 128,
                                   0.04, 64, 1e4, FAKE, hyb.BF16, None,
                                   ctypes.byref(prep) if prep is not None else None, None, n_comp,
                                   FAKE, ws, None)

    def prep(**kw):   # a query prep call in front of the step (hyb_q_norm_kv_insert's checks)
        a = dict(q=FAKE, q_dtype=hyb.BF16, n_heads=64, kv=FAKE, kv_dtype=hyb.BF16, cu_seqlens=FAKE,
                 start_pos=FAKE, batch=4, max_new_tokens=1, q_out=FAKE, swa=ctypes.pointer(swa),
                 rope_dim=64, rope_base=1e4, eps=1e-6)
        a.update(kw)
        return hyb.hyb_prep_call(**a)

    assert call(q_idx=None) == hyb.HYB_EINVAL                 # C4 without the indexer
    assert call(comp=c128) == hyb.HYB_EINVAL                  # C128 with an indexer query
    assert call(n_comp=3) == hyb.HYB_EINVAL
    assert call(n_comp=1) == hyb.HYB_EINVAL                   # compress NULL
    assert call(k=0) == hyb.HYB_EINVAL
    assert call(prep=prep(n_heads=0)) == hyb.HYB_EINVAL        # the prep is checked as its own call
    assert call(prep=prep(q_out=None)) == hyb.HYB_EINVAL
    assert call(prep=prep(eps=-1.0)) == hyb.HYB_EINVAL
    assert call(prep=prep(rope_dim=3)) == hyb.HYB_EINVAL
    assert lib.hyb_last_error().decode().startswith("hyb_decode_step")
    need = lib.hyb_decode_step_workspace_bytes(4, 64, 512, 100000, 4, 512, 128)
    # the step holds the indexer's hand-off (with its zero block) and the attention's partials
    assert need > lib.hyb_index_topk_workspace_bytes(4, 100000 - 1, 128, 4) + 4 * 5 * 64 * 512 * 2
    assert call(ws=need - 1) == hyb.HYB_EWORKSPACE
    assert lib.hyb_last_error().decode().startswith("hyb_decode_step")
    assert lib.hyb_decode_step_workspace_bytes(4, 64, 512, 100000, 128, 0, 128) == \
        lib.hyb_attn_decode_workspace_bytes(4, 64, 512, 100000, 128, 0, 128)


def test_error_word_needs_a_device():
    """hyb_set_error_word looks the current device up; with none it fails without side effects,
    and pools checked afterwards carry no error word (argument checks never query a device)."""
    lib = hyb.load()
    st = lib.hyb_set_error_word(None)
    if st == hyb.HYB_OK:
        pytest.skip("a GPU is present")
    assert st == hyb.HYB_ELAUNCH
    assert lib.hyb_last_error().decode().startswith("hyb_set_error_word")


def test_launch_logging_on_request(lib):
    """HYB_LOG=1 in the environment (read once per process) makes the entry points report what
    they launch on stderr; unset, they print nothing. A compressor call with no sequences checks
    its arguments and launches nothing, so this runs without a GPU (in fresh processes)."""
    import subprocess
    import sys
    code = ("import ctypes, sys; sys.path.insert(0, {root!r}); import sparse_attention_hyb_amd as hyb; "
            "from tests.test_abi import pool, FAKE; lib = hyb.load(); o = pool(ratio=4); "
            "sys.exit(lib.hyb_compress(FAKE, hyb.BF16, None, FAKE, FAKE, 0, 4, FAKE, None, "
            "hyb.POOL_MEAN, ctypes.byref(o), 64, 1e4, 1e-6, None))").format(root=ROOT)
    for value, expect in (("1", True), ("0", False), (None, False)):
        env = {k: v for k, v in os.environ.items() if k != "HYB_LOG"}
        if value is not None:
            env["HYB_LOG"] = value
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == hyb.HYB_OK, r.stderr
        logged = "[hyb] hyb_compress: 0 sequences x 4 new tokens: nothing to launch" in r.stderr
        assert logged == expect, (value, r.stderr)
