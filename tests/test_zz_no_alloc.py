"""The allocation-free fused decode entry against the fused entry with a
caller workspace: the same kernels run over the library's per-GPU scratch
array, so selections, outputs and log-sum-exp must be identical bit for bit.
Two calls in a row, the second on a smaller batch (the array keeps the
first call's contents), and the call changes no device memory use."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_attention_12_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "a GPU is required"
    from sparse_attention_12_amd import binding
    return binding


def _pair(B, w, check_memory):
    """(noalloc results, fused results) of one workload.  With check_memory,
    free device memory must be the same before and after the allocation-free
    call (the first call on a device is its one-time set-up: the runtime
    materialises the scratch array when its address is looked up)."""
    t = w.to_torch(DEV)
    batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)
    L = w.n_layers
    need = B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, w.k, L)
    assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
    res = []
    for noalloc in (False, True):
        outs = [torch.full((w.nq, 64, 512), float("nan"), device=DEV) for _ in range(L)]
        lses = [torch.full((w.nq, 64), float("nan"), device=DEV) for _ in range(L)]
        idx = torch.full((w.nq, w.k), -7, dtype=torch.int32, device=DEV)
        torch.cuda.synchronize()
        if noalloc:
            free0 = torch.cuda.mem_get_info()[0]
            B.dsa_mla_decode_fused_noalloc(batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau, lses,
                                           idx)
            torch.cuda.synchronize()
            if check_memory:
                assert torch.cuda.mem_get_info()[0] == free0, "the allocation-free call changed free device memory"
        else:
            ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
            B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau, lses, idx,
                                   ws)
            torch.cuda.synchronize()
        res.append([x.cpu() for x in outs + lses + [idx]])
    return res[1], res[0]


def test_noalloc_matches_fused_twice(B):
    # first: three sequences, one past 49,152 positions (the split top-k
    # path), two layers sharing the selection; second: a smaller batch; the
    # first call again (the array now holds the second call's contents)
    first = wl.make_decode([1500, 2600, 70000], "bf16", 2, seed=81)
    second = wl.make_decode([1200, 3000], "bf16", 1, seed=82)
    for i, w in enumerate((first, second, first)):
        got, ref = _pair(B, w, check_memory=i > 0)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"{w.name}: the allocation-free call differs from the fused call"
        idx = got[-1].numpy()
        for qi, n in enumerate(w.seq_len):
            assert int((idx[qi] >= 0).sum()) == min(2048, int(n))


def test_noalloc_rejects_batches_past_the_scratch(B):
    """A batch whose workspace exceeds the array is refused on the host."""
    nq, L = 64, 1 << 20
    need = B.dsa_mla_decode_fused_workspace_size(nq, L, 2048, 1)
    assert need > B.NOALLOC_SCRATCH_BYTES
    z = torch.zeros(nq, dtype=torch.int32, device=DEV)
    batch = B.Batch(z, z, torch.full((nq,), L, dtype=torch.int32, device=DEV), torch.zeros(nq, dtype=torch.int64,
                                                                                          device=DEV), L)
    # inputs are never read: the call is refused before anything runs
    dummy = torch.empty(1024, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(256, device=DEV)
    with pytest.raises(B.DsaError) as e:
        B.dsa_mla_decode_fused_noalloc(batch, dummy, out, dummy, 2048, [dummy[:576].view(1, 1, 576)],
                                       [dummy[:576].view(1, 576)], [out], 0.07)
    assert e.value.status == -5
