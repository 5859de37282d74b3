"""CPU float64 oracle for the hybrid compressed/sparse + sliding-window attention step.

TEST INFRASTRUCTURE ONLY. This package is the slow, plainly written specification that the
HIP library is checked against. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the C-ABI library and its
Python binding) never imports, calls or links anything here, and this package imports nothing
from the product: the two share no code. Inputs reach both sides from the seeded generators in
``sparse_attention_hyb_amd.workloads``, which hold no arithmetic of the method.

Sources (web pages; cited by title and section):
  * "Day-0 support for DeepSeek V4 Pro and Flash on vLLM" (vLLM's announcement, as mirrored on
    aiwiki.equalexperts.ai and as the vllm_project post on xfeed.redbud.ai): the "four moves"
    list (shared K/V + inverse RoPE, c4a/c128a compression, DeepSeek Sparse Attention over
    compressed tokens, short sliding window), the fp8 attention cache / fp4 indexer cache, and
    the "vLLM side" list (one logical block of 256 native positions for every compression
    rate; the fused compressor + RMSNorm + RoPE + cache-insert kernel).
  * "DeepSeek-V4 launch review" (SGLang/Miles day-0 blog in Japanese, winzheng.jp), section
    "Shadow Radix": every layer is SWA over the newest 128 raw tokens plus C4 (top-512 sparse
    over 4:1 compressed KV) or C128 (dense over 128:1 compressed KV); compression layers keep
    an in-progress compression state.
  * "DeepSeek-V4 auf NVIDIA Blackwell ..." (ki-news-radar.de): CSA / DSA / HCA naming.

Parity pins: every function here is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, special cases that reduce to library routines (torch float64 SDPA,
torch.float8_e4m3fn), hand-computed values and brute force. Functions or readings with no such
pin are marked "parity unpinned" in their docstrings.
"""

from .formats import (bf16_bits_to_f64, e2m1_to_f64, e4m3fn_to_f64, e8m0_to_f64,  # noqa: F401
                      encode_e2m1, encode_e4m3fn, f32_quotient, mx_exponent, quantize_fp4_row,
                      quantize_fp8_row, round_to_bf16_bits)
from .hyb_oracle import *  # noqa: F401,F403
