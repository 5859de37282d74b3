"""The C4 offload coordinator's bookkeeping on the CPU (host tensors stand in for the device):
LRU eviction among pages the step does not need, the block table of the working set, page
contents, the capacity error and write-back."""

import numpy as np
import pytest
import torch

from sparse_attention_hyb_amd.hisparse import C4Offload
from sparse_attention_hyb_amd.workloads import PagedTensors


def _mirror(n_seq=2, blocks=6, dim=8):
    data = torch.arange(n_seq * blocks * 64 * dim, dtype=torch.float32).reshape(n_seq * blocks, 64, dim)
    table = torch.arange(n_seq * blocks, dtype=torch.int32).reshape(n_seq, blocks).flip(1).contiguous()
    return PagedTensors(data, None, table, "f32", dim, 4)


def _rows(*pages_per_seq, n_seq=2, k=4):
    """Top-k rows selecting one entry in each listed logical block of each sequence."""
    rows = np.full((n_seq, k), -1, dtype=np.int64)
    for b, pages in enumerate(pages_per_seq):
        for j, lb in enumerate(pages):
            rows[b, j] = 64 * lb + 3 + j
    return rows


def test_lru_eviction_table_and_contents():
    m = _mirror()
    off = C4Offload(m, slots=3, device="cpu")
    st = off.admit(_rows([0, 1], []))                 # step 1: (0,0), (0,1)
    assert (st.pages, st.misses) == (2, 2)
    st = off.admit(_rows([1], [2]))                   # step 2: (0,1) hit, (1,2) miss
    assert (st.pages, st.misses) == (2, 1)
    slot_00 = off.where[(0, 0)]
    st = off.admit(_rows([], [5]))                    # step 3: (1,5) evicts LRU page (0,0)
    assert st.misses == 1 and (0, 0) not in off.where and off.where[(1, 5)] == slot_00
    assert off.dev_table_host[0, 0] == -1
    for (b, lb), s in off.where.items():
        assert off.dev_table_host[b, lb] == s
        assert torch.equal(off.data[s], m.data[int(m.block_table[b, lb])])
    assert torch.equal(off.dev_table, torch.from_numpy(off.dev_table_host))
    # a needed page is never evicted: (1,5) and (0,1) are needed, (1,2) (stamp 2) goes
    st = off.admit(_rows([1, 3], [5]))
    assert st.misses == 1 and (1, 2) not in off.where and {(0, 1), (0, 3), (1, 5)} == set(off.where)


def test_capacity_and_write_back():
    m = _mirror()
    off = C4Offload(m, slots=2, device="cpu")
    with pytest.raises(RuntimeError):
        off.admit(_rows([0, 1, 2], []))
    off.admit(_rows([4], []), extra=[(1, 0)])
    s = off.where[(0, 4)]
    off.data[s].fill_(-1.0)
    off.write_back([(0, 4)])
    assert torch.equal(m.data[int(m.block_table[0, 4])], torch.full((64, 8), -1.0))
