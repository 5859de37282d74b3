"""MI355X-native hybrid compressed/sparse + sliding-window attention.

Thin Python binding of the C ABI in ``include/hyb.h`` (libhyb.so, HIP kernels for gfx950).
Each function has the C entry point's name and only marshals arguments: torch tensors become
device pointers, pools become ``hyb_paged`` descriptors, the current torch stream is passed
through. Every step of the method runs in the library's kernels. Without the built library
every call raises: there is no fallback.

Pools are any object with the attributes ``data``, ``scale``, ``block_table`` (torch tensors),
``dtype`` ('f32' | 'bf16' | 'fp8' | 'fp4'), ``dim`` and ``ratio`` - e.g.
``sparse_attention_hyb_amd.workloads.PagedTensors``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhyb.so")

HYB_OK, HYB_EINVAL, HYB_ENOTSUP, HYB_EWORKSPACE, HYB_ELAUNCH = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3
ABI_VERSION = 5   # HYB_ABI_VERSION of include/hyb.h that these signatures follow
POOL_MEAN, POOL_SOFTMAX_GATE = 0, 1
BLOCK_POSITIONS = 256
KMAX = 2048
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp4": FP4_E2M1}

EXPORTS = (
    "hyb_abi_version", "hyb_status_str", "hyb_last_error", "hyb_set_error_word", "hyb_compress", "hyb_swa_insert",
    "hyb_q_norm_kv_insert", "hyb_gather_pages",
    "hyb_index_score", "hyb_topk", "hyb_index_score_keys", "hyb_topk_keys",
    "hyb_index_topk_workspace_bytes", "hyb_index_topk", "hyb_index_topk_noalloc",
    "hyb_attn_decode_workspace_bytes", "hyb_attn_decode", "hyb_attn_decode_compress",
    "hyb_attn_prefill_workspace_bytes", "hyb_attn_prefill",
    "hyb_decode_step_workspace_bytes", "hyb_decode_step",
    "hyb_probe_granule", "hyb_probe",
    "hyb_offload_workspace_bytes", "hyb_offload_admit", "hyb_offload_write_back",
)


class HybError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


class hyb_paged(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("ratio", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class hyb_compress_call(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("x_dtype", ctypes.c_int32),
        ("gate_logits", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("start_pos", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("max_new_tokens", ctypes.c_int32),
        ("state", ctypes.c_void_p),
        ("state_logits", ctypes.c_void_p),
        ("mode", ctypes.c_int32),
        ("out", ctypes.POINTER(hyb_paged)),
        ("rope_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("eps", ctypes.c_float),
    ]


class hyb_prep_call(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("kv", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("start_pos", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("max_new_tokens", ctypes.c_int32),
        ("q_out", ctypes.c_void_p),
        ("swa", ctypes.POINTER(hyb_paged)),
        ("rope_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("eps", ctypes.c_float),
    ]


_lib = None

_P, _I32, _I64, _SZ, _D, _F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                               ctypes.c_double, ctypes.c_float)
_PP = ctypes.POINTER(hyb_paged)
_SIGS = {
    "hyb_abi_version": (_I32, []),
    "hyb_set_error_word": (_I32, [_P]),
    "hyb_status_str": (ctypes.c_char_p, [_I32]),
    "hyb_last_error": (ctypes.c_char_p, []),
    "hyb_compress": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _P, _P, _I32, _PP, _I32, _D, _F, _P]),
    "hyb_swa_insert": (_I32, [_P, _I32, _P, _P, _I32, _I32, _PP, _I32, _D, _P]),
    "hyb_index_score": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _PP, _P, _I64, _P]),
    "hyb_topk": (_I32, [_P, _I64, _P, _I32, _I32, _I32, _P, _P]),
    "hyb_index_score_keys": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _PP, _P, _I64, _P,
                                    _I64, _P]),
    "hyb_topk_keys": (_I32, [_P, _I64, _P, _I64, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "hyb_index_topk_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "hyb_index_topk": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _PP, _I32, _P, _P, _SZ, _P]),
    "hyb_index_topk_noalloc": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _PP, _I32, _P, _P]),
    "hyb_q_norm_kv_insert": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _P, _PP, _I32, _D,
                                    _F, _P]),
    "hyb_gather_pages": (_I32, [_P, _I32, _P, _I32, _P, _P, _I32, _I64, _P]),
    "hyb_attn_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "hyb_attn_decode": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _PP, _PP, _P, _I32, _I32, _F, _I32,
                               _D, _P, _I32, _P, _P, _SZ, _P]),
    "hyb_attn_decode_compress": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _PP, _PP, _P, _I32, _I32, _F,
                                        _I32, _D, _P, _I32, _P, _P, _SZ,
                                        ctypes.POINTER(hyb_compress_call), _P]),
    "hyb_attn_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "hyb_attn_prefill": (_I32, [_P, _I32, _P, _P, _I32, _I32, _I32, _PP, _PP, _P, _I32, _I32, _F,
                                _I32, _D, _P, _I32, _P, _P, _SZ, _P]),
    "hyb_decode_step_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "hyb_decode_step": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _PP, _PP, _P, _I32, _P, _I32, _PP, _I32,
                               _P, _I32, _F, _I32, _D, _P, _I32, _P, ctypes.POINTER(hyb_prep_call),
                               ctypes.POINTER(hyb_compress_call), _I32, _P, _SZ, _P]),
    "hyb_probe_granule": (ctypes.c_uint64, [_I32, _I32]),
    "hyb_probe": (_I32, [_I32, _I32, _I32, _P, _P, ctypes.c_uint64, _P, _P, _I32, _I64, _P, _P]),
    "hyb_offload_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "hyb_offload_admit": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _P, _P, _I32, ctypes.c_uint32,
                                 _P, _I32, _P, _I64, _P, _P, _I64, _P, _SZ, _P, _P]),
    "hyb_offload_write_back": (_I32, [_P, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _I64, _P, _I32, _P, _P,
                                      _I64, _P]),
}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhyb.so (built by ``python -m sparse_attention_hyb_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libhyb.so is not built ({p}); run python -m sparse_attention_hyb_amd.build")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.hyb_abi_version() != ABI_VERSION:
        raise ImportError(f"{p} has ABI version {lib.hyb_abi_version()}, the binding expects {ABI_VERSION}")
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != HYB_OK:
        lib = load()
        raise HybError(status, lib.hyb_last_error().decode() or lib.hyb_status_str(status).decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _tdtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"tensor dtype {t.dtype} is not float32 or bfloat16")


def _odtype(out, out_scale) -> int:
    """Output dtype: FP8_E4M3 when a scale tensor is given (out holds the codes as uint8 or
    float8_e4m3fn), else that of `out`."""
    import torch
    if out_scale is None:
        return _tdtype(out)
    if out.dtype not in (torch.uint8, torch.float8_e4m3fn) or out_scale.dtype != torch.float32:
        raise TypeError("an fp8 output takes uint8 / float8_e4m3fn codes and float32 scales")
    return FP8_E4M3


def paged(pool) -> hyb_paged:
    """Pool object -> hyb_paged descriptor (keeps no reference: hold the tensors yourself)."""
    return hyb_paged(
        data=_ptr(pool.data), scale=_ptr(pool.scale), block_table=_ptr(pool.block_table),
        dtype=DTYPE_CODES[pool.dtype], dim=int(pool.dim), ratio=int(pool.ratio),
        num_blocks=int(pool.data.shape[0]), max_blocks=int(pool.block_table.shape[1]), reserved=0)


def _check_state(x, state) -> None:
    if state.dtype != x.dtype:
        raise TypeError(f"state ring dtype {state.dtype} must be x's dtype {x.dtype}")


def _empty_workspace(nbytes: int, device):
    """A workspace for one call: zeroed, as the attention entry points need their split counters
    zero before a workspace's first use (include/hyb.h)."""
    import torch
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------------
def hyb_abi_version() -> int:
    return load().hyb_abi_version()


ERR_BAD_PAGE = 1   # HYB_ERR_BAD_PAGE


def hyb_set_error_word(word) -> None:
    """Report block-table entries >= num_blocks into `word` (a one-element int32 tensor on the
    current device, zeroed by the caller), or stop reporting (None)."""
    _check(load().hyb_set_error_word(_ptr(word)))


def hyb_compress(x, cu_seqlens, start_pos, max_new_tokens: int, state, out_pool, rope_dim: int,
                 rope_base: float = 10000.0, eps: float = 1e-6, gate_logits=None,
                 state_logits=None, stream=None) -> None:
    """Compressor: see hyb_compress in include/hyb.h. Mean pooling unless gate_logits is given.
    The state ring holds raw tokens in x's dtype."""
    _check_state(x, state)
    mode = POOL_SOFTMAX_GATE if gate_logits is not None else POOL_MEAN
    d = paged(out_pool)
    _check(load().hyb_compress(_ptr(x), _tdtype(x), _ptr(gate_logits), _ptr(cu_seqlens),
                               _ptr(start_pos), int(start_pos.shape[0]), int(max_new_tokens),
                               _ptr(state), _ptr(state_logits), mode, ctypes.byref(d),
                               int(rope_dim), float(rope_base), float(eps), _stream(stream)))


def hyb_swa_insert(x, cu_seqlens, start_pos, max_new_tokens: int, swa_pool, rope_dim: int,
                   rope_base: float = 10000.0, stream=None) -> None:
    d = paged(swa_pool)
    _check(load().hyb_swa_insert(_ptr(x), _tdtype(x), _ptr(cu_seqlens), _ptr(start_pos),
                                 int(start_pos.shape[0]), int(max_new_tokens), ctypes.byref(d),
                                 int(rope_dim), float(rope_base), _stream(stream)))


def hyb_q_norm_kv_insert(q, kv, cu_seqlens, start_pos, max_new_tokens: int, swa_pool, q_out=None,
                         rope_dim: int = 64, rope_base: float = 10000.0, eps: float = 1e-6,
                         stream=None):
    """Query RMSNorm + RoPE and the window insert of the new tokens (see include/hyb.h). q_out
    defaults to q (in place). Returns q_out."""
    q_out = q if q_out is None else q_out
    if q_out.dtype != q.dtype or q_out.shape != q.shape:
        raise TypeError("q_out must have q's shape and dtype")
    d = paged(swa_pool)
    _check(load().hyb_q_norm_kv_insert(_ptr(q), _tdtype(q), int(q.shape[1]), _ptr(kv), _tdtype(kv),
                                       _ptr(cu_seqlens), _ptr(start_pos), int(start_pos.shape[0]),
                                       int(max_new_tokens), _ptr(q_out), ctypes.byref(d),
                                       int(rope_dim), float(rope_base), float(eps), _stream(stream)))
    return q_out


def hyb_gather_pages(src_host, dst, src_page, dst_page, stream=None) -> None:
    """Copy pages src_host[src_page[j]] -> dst[dst_page[j]] in one launch (see include/hyb.h).
    src_host: a contiguous pinned CPU tensor [pages, ...]; dst: a contiguous device tensor of the
    same page shape; src_page, dst_page: int32 device tensors of one length (indices outside the
    two tensors' page counts are skipped by the kernel)."""
    import torch
    if not (src_host.is_contiguous() and dst.is_contiguous()):
        raise TypeError("src_host and dst must be contiguous")
    for t in (src_page, dst_page):
        if t.dtype != torch.int32 or t.device.type != "cuda" or t.dim() != 1 or not t.is_contiguous():
            raise TypeError("src_page and dst_page must be contiguous 1-d int32 device tensors")
    if src_page.numel() != dst_page.numel():
        raise TypeError("src_page and dst_page differ in length")
    page = src_host[0].numel() * src_host.element_size()
    if dst[0].numel() * dst.element_size() != page:
        raise TypeError("src_host and dst pages differ in size")
    _check(load().hyb_gather_pages(_ptr(src_host), int(src_host.shape[0]), _ptr(dst),
                                   int(dst.shape[0]), _ptr(src_page), _ptr(dst_page),
                                   int(src_page.numel()), int(page), _stream(stream)))


def hyb_offload_workspace_bytes(batch: int, max_blocks: int, n_slots: int) -> int:
    return int(load().hyb_offload_workspace_bytes(int(batch), int(max_blocks), int(n_slots)))


def hyb_offload_admit(topk, dev_table, mirror_table, slot_owner, slot_stamp, step: int, mirror_host,
                      pool, workspace, result, extra=None, entries_per_page: int = 64,
                      mirror_scale_host=None, pool_scale=None, stream=None) -> None:
    """One step's working-set update of an offloaded C4 pool on the device (see include/hyb.h).
    topk [batch, k] int32 (device); dev_table / mirror_table [batch, max_blocks] int32 (device);
    slot_owner int32 / slot_stamp int32 (as uint32) [n_slots] (device); mirror_host: a contiguous
    pinned CPU tensor [pages, ...]; pool: a contiguous device tensor [n_slots, ...] of the same page
    shape; optional scale pages alike; workspace: uint8 device tensor, zero before its first use;
    result: int32 [2] device tensor (pages admitted, pages left out)."""
    if not (mirror_host.is_contiguous() and pool.is_contiguous()):
        raise TypeError("mirror_host and pool must be contiguous")
    page = mirror_host[0].numel() * mirror_host.element_size()
    if pool[0].numel() * pool.element_size() != page:
        raise TypeError("mirror_host and pool pages differ in size")
    spage = 0
    if mirror_scale_host is not None:
        spage = mirror_scale_host[0].numel() * mirror_scale_host.element_size()
    batch, k = (int(topk.shape[0]), int(topk.shape[1])) if topk is not None else (int(dev_table.shape[0]), 0)
    _check(load().hyb_offload_admit(
        _ptr(topk), batch, k, _ptr(extra), 0 if extra is None else int(extra.numel()),
        _ptr(dev_table), _ptr(mirror_table), int(dev_table.shape[1]), int(entries_per_page),
        _ptr(slot_owner), _ptr(slot_stamp), int(slot_owner.numel()), int(step), _ptr(mirror_host),
        int(mirror_host.shape[0]), _ptr(pool), int(page), _ptr(mirror_scale_host), _ptr(pool_scale),
        int(spage), _ptr(workspace), int(workspace.numel()), _ptr(result), _stream(stream)))


def hyb_offload_write_back(seq_lens, ratio: int, dev_table, mirror_table, pool, mirror_host,
                           entries_per_page: int = 64, pool_scale=None, mirror_scale_host=None,
                           stream=None) -> None:
    """Back up each sequence's newly completed entry from its resident slot to the pinned host
    mirror, on the device (see include/hyb.h)."""
    page = mirror_host[0].numel() * mirror_host.element_size()
    spage = 0 if mirror_scale_host is None else mirror_scale_host[0].numel() * mirror_scale_host.element_size()
    _check(load().hyb_offload_write_back(
        _ptr(seq_lens), int(seq_lens.numel()), int(ratio), _ptr(dev_table), _ptr(mirror_table),
        int(dev_table.shape[1]), int(entries_per_page), int(pool.shape[0]), _ptr(pool), int(page),
        _ptr(mirror_host), int(mirror_host.shape[0]), _ptr(pool_scale), _ptr(mirror_scale_host),
        int(spage), _stream(stream)))


def hyb_index_score(q_idx, w, q_pos, max_pos: int, idx_pool, scores, window: int = 128,
                    q_seq=None, stream=None) -> None:
    d = paged(idx_pool)
    _check(load().hyb_index_score(_ptr(q_idx), _tdtype(q_idx), _ptr(w), _ptr(q_seq), _ptr(q_pos),
                                  int(q_idx.shape[0]), int(q_idx.shape[1]), int(max_pos),
                                  int(window), ctypes.byref(d), _ptr(scores),
                                  int(scores.stride(0)), _stream(stream)))


def hyb_topk(scores, lengths, max_len: int, k: int, out_idx, stream=None) -> None:
    _check(load().hyb_topk(_ptr(scores), int(scores.stride(0)), _ptr(lengths),
                           int(scores.shape[0]), int(max_len), int(k), _ptr(out_idx),
                           _stream(stream)))


def index_keys_shapes(n_q: int, max_pos: int, window: int = 128, ratio: int = 4):
    """Shapes of the `keys` (uint32 as int32) and `part_hist` (uint16 as int16) buffers of
    hyb_index_score_keys / hyb_topk_keys: ([n_q, 2048 * parts], [n_q, parts, 1024])."""
    ws = max(0, max_pos - window + 1)                  # window start of the last position
    nv = max(1, (ws + ratio - 1) // ratio)             # compressed entries visible to it
    parts = (nv + 1023) // 1024
    return (n_q, 2048 * parts), (n_q, parts, 1024)


def hyb_index_score_keys(q_idx, w, q_pos, max_pos: int, idx_pool, keys, part_hist, window: int = 128,
                         q_seq=None, stream=None) -> None:
    d = paged(idx_pool)
    _check(load().hyb_index_score_keys(_ptr(q_idx), _tdtype(q_idx), _ptr(w), _ptr(q_seq), _ptr(q_pos),
                                       int(q_idx.shape[0]), int(q_idx.shape[1]), int(max_pos),
                                       int(window), ctypes.byref(d), _ptr(keys), int(keys.stride(0)),
                                       _ptr(part_hist), int(part_hist.shape[1]), _stream(stream)))


def hyb_topk_keys(keys, part_hist, q_pos, max_pos: int, k: int, out_idx, window: int = 128,
                  ratio: int = 4, stream=None) -> None:
    _check(load().hyb_topk_keys(_ptr(keys), int(keys.stride(0)), _ptr(part_hist),
                                int(part_hist.shape[1]), _ptr(q_pos), int(keys.shape[0]),
                                int(max_pos), int(window), int(ratio), int(k), _ptr(out_idx),
                                _stream(stream)))


def hyb_index_topk_workspace_bytes(n_q: int, max_pos: int, window: int, ratio: int) -> int:
    return int(load().hyb_index_topk_workspace_bytes(int(n_q), int(max_pos), int(window), int(ratio)))


def hyb_index_topk(q_idx, w, q_pos, max_pos: int, idx_pool, k: int, out_idx, window: int = 128,
                   q_seq=None, workspace=None, stream=None) -> None:
    n_q = int(q_idx.shape[0])
    need = hyb_index_topk_workspace_bytes(n_q, max_pos, window, idx_pool.ratio)
    if workspace is None:
        workspace = _empty_workspace(need, q_idx.device)
    d = paged(idx_pool)
    _check(load().hyb_index_topk(_ptr(q_idx), _tdtype(q_idx), _ptr(w), _ptr(q_seq), _ptr(q_pos),
                                 n_q, int(q_idx.shape[1]), int(max_pos), int(window),
                                 ctypes.byref(d), int(k), _ptr(out_idx), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20   # HYB_NOALLOC_SCRATCH_BYTES
STEP_ZERO_BYTES = (1 << 20) + 1024   # HYB_STEP_ZERO_BYTES: a C4 step workspace's leading zero block


def hyb_index_topk_noalloc(q_idx, w, q_pos, max_pos: int, idx_pool, k: int, out_idx,
                           window: int = 128, q_seq=None, stream=None) -> None:
    """hyb_index_topk with its scratch in the library's static per-GPU array (see include/hyb.h):
    nothing is allocated; calls overlapping on one GPU race."""
    d = paged(idx_pool)
    _check(load().hyb_index_topk_noalloc(_ptr(q_idx), _tdtype(q_idx), _ptr(w), _ptr(q_seq),
                                         _ptr(q_pos), int(q_idx.shape[0]), int(q_idx.shape[1]),
                                         int(max_pos), int(window), ctypes.byref(d), int(k),
                                         _ptr(out_idx), _stream(stream)))


def hyb_attn_decode_workspace_bytes(batch: int, n_heads: int, dim: int, max_seq_len: int,
                                    comp_ratio: int, k: int, window: int = 128) -> int:
    return int(load().hyb_attn_decode_workspace_bytes(int(batch), int(n_heads), int(dim),
                                                      int(max_seq_len), int(comp_ratio), int(k),
                                                      int(window)))


def hyb_attn_decode(q, seq_lens, max_seq_len: int, swa_pool, comp_pool, out, topk_idx=None,
                    k: int = 0, window: int = 128, softmax_scale: Optional[float] = None,
                    rope_dim: int = 64, rope_base: float = 10000.0, workspace=None,
                    out_scale=None, stream=None) -> None:
    b, h, dim = (int(s) for s in q.shape)
    if topk_idx is not None and not k:
        k = int(topk_idx.shape[1])
    scale = float(softmax_scale) if softmax_scale is not None else dim ** -0.5
    if workspace is None:
        need = hyb_attn_decode_workspace_bytes(b, h, dim, max_seq_len, comp_pool.ratio,
                                               k if topk_idx is not None else 0, window)
        workspace = _empty_workspace(need, q.device)
    ds, dc = paged(swa_pool), paged(comp_pool)
    _check(load().hyb_attn_decode(_ptr(q), _tdtype(q), _ptr(seq_lens), b, h, int(max_seq_len),
                                  ctypes.byref(ds), ctypes.byref(dc), _ptr(topk_idx), int(k),
                                  int(window), scale, int(rope_dim), float(rope_base), _ptr(out),
                                  _odtype(out, out_scale), _ptr(out_scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def hyb_attn_decode_compress(q, seq_lens, max_seq_len: int, swa_pool, comp_pool, out, x,
                             cu_seqlens, start_pos, max_new_tokens: int, state, out_pool,
                             topk_idx=None, k: int = 0, window: int = 128,
                             softmax_scale: Optional[float] = None, rope_dim: int = 64,
                             rope_base: float = 10000.0, eps: float = 1e-6, gate_logits=None,
                             state_logits=None, workspace=None, out_scale=None, stream=None) -> None:
    """hyb_attn_decode(q, ...) then hyb_compress(x, ...) in one call (see include/hyb.h); both
    use rope_dim and rope_base."""
    _check_state(x, state)
    b, h, dim = (int(s) for s in q.shape)
    if topk_idx is not None and not k:
        k = int(topk_idx.shape[1])
    scale = float(softmax_scale) if softmax_scale is not None else dim ** -0.5
    if workspace is None:
        need = hyb_attn_decode_workspace_bytes(b, h, dim, max_seq_len, comp_pool.ratio,
                                               k if topk_idx is not None else 0, window)
        workspace = _empty_workspace(need, q.device)
    ds, dc, do = paged(swa_pool), paged(comp_pool), paged(out_pool)
    call = hyb_compress_call(
        x=_ptr(x), x_dtype=_tdtype(x), gate_logits=_ptr(gate_logits), cu_seqlens=_ptr(cu_seqlens),
        start_pos=_ptr(start_pos), batch=int(start_pos.shape[0]), max_new_tokens=int(max_new_tokens),
        state=_ptr(state), state_logits=_ptr(state_logits),
        mode=POOL_SOFTMAX_GATE if gate_logits is not None else POOL_MEAN,
        out=ctypes.pointer(do), rope_dim=int(rope_dim), rope_base=float(rope_base), eps=float(eps))
    _check(load().hyb_attn_decode_compress(
        _ptr(q), _tdtype(q), _ptr(seq_lens), b, h, int(max_seq_len), ctypes.byref(ds),
        ctypes.byref(dc), _ptr(topk_idx), int(k), int(window), scale, int(rope_dim),
        float(rope_base), _ptr(out), _odtype(out, out_scale), _ptr(out_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(call), _stream(stream)))


def compress_call(x, cu_seqlens, start_pos, max_new_tokens: int, state, out_pool, rope_dim: int = 64,
                  rope_base: float = 10000.0, eps: float = 1e-6, gate_logits=None,
                  state_logits=None):
    """The arguments of one hyb_compress call as a hyb_compress_call struct (for the entry points
    that take compressor calls). Keep the returned object alive until the call is enqueued: it
    holds the pool descriptor."""
    _check_state(x, state)
    d = paged(out_pool)
    call = hyb_compress_call(
        x=_ptr(x), x_dtype=_tdtype(x), gate_logits=_ptr(gate_logits), cu_seqlens=_ptr(cu_seqlens),
        start_pos=_ptr(start_pos), batch=int(start_pos.shape[0]), max_new_tokens=int(max_new_tokens),
        state=_ptr(state), state_logits=_ptr(state_logits),
        mode=POOL_SOFTMAX_GATE if gate_logits is not None else POOL_MEAN,
        out=ctypes.pointer(d), rope_dim=int(rope_dim), rope_base=float(rope_base), eps=float(eps))
    call._keep = d
    return call


def prep_call(q, kv, cu_seqlens, start_pos, max_new_tokens: int, swa_pool, q_out=None,
              rope_dim: int = 64, rope_base: float = 10000.0, eps: float = 1e-6):
    """The arguments of one hyb_q_norm_kv_insert call as a hyb_prep_call struct (for
    hyb_decode_step's prep). q_out defaults to q. Keep the returned object alive until the call is
    enqueued: it holds the pool descriptor."""
    q_out = q if q_out is None else q_out
    if q_out.dtype != q.dtype or q_out.shape != q.shape:
        raise TypeError("q_out must have q's shape and dtype")
    d = paged(swa_pool)
    call = hyb_prep_call(
        q=_ptr(q), q_dtype=_tdtype(q), n_heads=int(q.shape[1]), kv=_ptr(kv), kv_dtype=_tdtype(kv),
        cu_seqlens=_ptr(cu_seqlens), start_pos=_ptr(start_pos), batch=int(start_pos.shape[0]),
        max_new_tokens=int(max_new_tokens), q_out=_ptr(q_out), swa=ctypes.pointer(d),
        rope_dim=int(rope_dim), rope_base=float(rope_base), eps=float(eps))
    call._keep = d
    return call


def hyb_decode_step_workspace_bytes(batch: int, n_heads: int, dim: int, max_seq_len: int,
                                    comp_ratio: int, k: int, window: int = 128) -> int:
    return int(load().hyb_decode_step_workspace_bytes(int(batch), int(n_heads), int(dim),
                                                      int(max_seq_len), int(comp_ratio), int(k),
                                                      int(window)))


def hyb_decode_step(q, seq_lens, max_seq_len: int, swa_pool, comp_pool, out, idx_q=None, idx_w=None,
                    idx_pool=None, k: int = 512, topk_out=None, compress=(), window: int = 128,
                    softmax_scale: Optional[float] = None, rope_dim: int = 64,
                    rope_base: float = 10000.0, workspace=None, out_scale=None, stream=None,
                    prep=None) -> None:
    """One decode step of a C4 layer (idx_q, idx_w, idx_pool given) or a C128 layer (none), with
    up to two compressor calls (compress_call(...) structs) and optionally the query prep and
    window insert in front (prep_call(...)); see include/hyb.h."""
    b, h, dim = (int(s) for s in q.shape)
    scale = float(softmax_scale) if softmax_scale is not None else dim ** -0.5
    if workspace is None:
        workspace = _empty_workspace(hyb_decode_step_workspace_bytes(b, h, dim, max_seq_len,
                                                                     comp_pool.ratio, k, window), q.device)
    calls = list(compress)
    arr = (hyb_compress_call * max(1, len(calls)))(*calls) if calls else None
    ds, dc = paged(swa_pool), paged(comp_pool)
    di = paged(idx_pool) if idx_pool is not None else None
    _check(load().hyb_decode_step(
        _ptr(q), _tdtype(q), _ptr(seq_lens), b, h, int(max_seq_len), ctypes.byref(ds), ctypes.byref(dc),
        _ptr(idx_q), _tdtype(idx_q) if idx_q is not None else BF16, _ptr(idx_w),
        int(idx_q.shape[1]) if idx_q is not None else 0, ctypes.byref(di) if di is not None else None,
        int(k), _ptr(topk_out), int(window), scale, int(rope_dim), float(rope_base), _ptr(out),
        _odtype(out, out_scale), _ptr(out_scale), ctypes.byref(prep) if prep is not None else None,
        arr, len(calls), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def hyb_attn_prefill_workspace_bytes(n_q: int, n_heads: int, dim: int, max_pos: int,
                                     comp_ratio: int, k: int, window: int = 128) -> int:
    return int(load().hyb_attn_prefill_workspace_bytes(int(n_q), int(n_heads), int(dim),
                                                       int(max_pos), int(comp_ratio), int(k),
                                                       int(window)))


def hyb_attn_prefill(q, q_pos, max_pos: int, swa_pool, comp_pool, out, topk_idx=None, k: int = 0,
                     q_seq=None, window: int = 128, softmax_scale: Optional[float] = None,
                     rope_dim: int = 64, rope_base: float = 10000.0, workspace=None,
                     out_scale=None, stream=None) -> None:
    n_q, h, dim = (int(s) for s in q.shape)
    if topk_idx is not None and not k:
        k = int(topk_idx.shape[1])
    scale = float(softmax_scale) if softmax_scale is not None else dim ** -0.5
    if workspace is None:
        need = hyb_attn_prefill_workspace_bytes(n_q, h, dim, max_pos, comp_pool.ratio,
                                                k if topk_idx is not None else 0, window)
        workspace = _empty_workspace(need, q.device)
    ds, dc = paged(swa_pool), paged(comp_pool)
    _check(load().hyb_attn_prefill(_ptr(q), _tdtype(q), _ptr(q_seq), _ptr(q_pos), n_q, h,
                                   int(max_pos), ctypes.byref(ds), ctypes.byref(dc),
                                   _ptr(topk_idx), int(k), int(window), scale, int(rope_dim),
                                   float(rope_base), _ptr(out), _odtype(out, out_scale), _ptr(out_scale), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


# ---------------------------------------------------------------------------------------------
# HBM bandwidth probe (include/hyb_probe.h): a measurement aid beside the attention step.
PROBE_READ, PROBE_READ_DYN, PROBE_READ_LDS, PROBE_READ_PAGES, PROBE_COPY = 0, 1, 2, 3, 4


def hyb_probe_granule(variant: int, unroll: int = 8) -> int:
    return int(load().hyb_probe_granule(int(variant), int(unroll)))


def hyb_probe(variant: int, src, n_workgroups: int, unroll: int = 8, dst=None, nbytes: int = 0,
              counter=None, pages=None, page_bytes: int = 0, trace=None, stream=None) -> None:
    """One probe launch (see include/hyb_probe.h). nbytes defaults to src's size."""
    nbytes = int(nbytes) or src.numel() * src.element_size()
    _check(load().hyb_probe(int(variant), int(unroll), int(n_workgroups), _ptr(src), _ptr(dst),
                            nbytes, _ptr(counter), _ptr(pages),
                            int(pages.numel()) if pages is not None else 0, int(page_bytes),
                            _ptr(trace), _stream(stream)))
