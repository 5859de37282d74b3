"""The decode step on two streams (query prep and window insert beside the indexer) and as one
captured HIP graph: both give the serial eager step's results bit for bit, and a replay follows
new sequence lengths written to the device-side metadata."""

import pytest
import torch

from sparse_attention_hyb_amd import workloads as W
from sparse_attention_hyb_amd.decode_step import DecodeStep, DecodeStepBuffers

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = torch.int32


def _buffers(hyb, lens, seed):
    wl = W.sparse_decode(DEV, seed=seed, batch=len(lens), ctx=lens)
    B, D, L = wl.batch, wl.dim, wl.max_seq_len
    g = W.generator(97, seed, 0, DEV)
    kshape, hshape = hyb.index_keys_shapes(B, L - 1)
    return DecodeStepBuffers(
        q_raw=W.to_storage(W.randn((B, 64, D), g, DEV) * 3.0, "bf16"),
        kv_new=W.to_storage(W.randn((B, D), g, DEV), "bf16"),
        q=torch.empty_like(wl.q), seq_lens=wl.seq_lens.clone(),
        cu=torch.arange(0, B + 1, dtype=I32, device=DEV), start=(wl.seq_lens - 1).contiguous(),
        swa=wl.swa, comp=wl.comp, state=W.to_storage(W.randn((B, 4, D), g, DEV), "bf16"),
        out=torch.empty_like(wl.q),
        workspace=torch.empty(hyb.hyb_attn_decode_workspace_bytes(B, 64, D, L, 4, wl.k),
                              dtype=torch.uint8, device=DEV),
        max_seq_len=L, idx_q=wl.idx_q, idx_w=wl.idx_w, idx_pool=wl.idx_pool,
        keys=torch.empty(kshape, dtype=I32, device=DEV),
        hist=torch.empty(hshape, dtype=torch.int16, device=DEV),
        topk=torch.empty(B, wl.k, dtype=I32, device=DEV), k=wl.k)


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


def test_decode_step_two_streams_and_graph(gpu_lib):
    hyb = gpu_lib
    b = _buffers(hyb, [4096, 8191, 20000, 65535], seed=5)   # groups complete for 2 of 4
    pools = (b.swa.data.clone(), b.comp.data.clone(), b.state.clone())
    step = DecodeStep(b)
    _reset(b, pools)
    step.run_serial()
    torch.cuda.synchronize()
    want = _results(b)
    assert not torch.equal(want[4], pools[1])   # completed groups were compressed
    assert not torch.equal(want[3], pools[0])   # window entries were inserted
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
