"""The debug build (libdsa_mla_debug.so: the kernels' checks compiled in)
on the GPU: its results equal the release build's bit for bit, valid calls
set no check bits, and the conditions the release build only guards (a
workspace's stale precounted histogram, selection entries outside the
candidates) are reported.  Every case here is a valid call or one the
kernels already handle (out-of-range selection entries are skipped)."""
import contextlib

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


@pytest.fixture(scope="module")
def dbg(B):
    return B.load_debug_library()


@contextlib.contextmanager
def using(B, library):
    saved = B.lib
    B.lib = library
    try:
        yield
    finally:
        B.lib = saved


def _fused(B, w, t, ws):
    outs = [torch.empty(w.nq, 64, 512, device=DEV) for _ in range(w.n_layers)]
    lses = [torch.empty(w.nq, 64, device=DEV) for _ in range(w.n_layers)]
    idx = torch.full((w.nq, w.k), -7, dtype=torch.int32, device=DEV)
    batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)
    B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau, lses, idx, ws)
    torch.cuda.synchronize()
    return idx.cpu(), [o.cpu() for o in outs], [x.cpu() for x in lses]


@pytest.mark.parametrize("lens", [[1500, 5000, 30000], [1500, 5000, 60000]],
                         ids=["row_topk", "split_topk"])
def test_debug_fused_decode(B, dbg, lens):
    """A workspace full of stale bytes: the first call recounts the stale
    histogram (reported), the second finds it cleared (nothing reported);
    selections and outputs equal the release build's."""
    w = wl.make_decode(lens, "bf16", n_layers=2, seed=61)
    t = w.to_torch(DEV)
    n = B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, w.k, w.n_layers)
    ref = _fused(B, w, t, torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV))
    B.debug_flags(True, dbg)  # start from a clear word
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    with using(B, dbg):
        first = _fused(B, w, t, ws)
        f1 = B.debug_flags(True, dbg)
        second = _fused(B, w, t, ws)
        f2 = B.debug_flags(True, dbg)
    assert f1 == B.DEBUG_BITS["hist_recount"], f"first call: flags {f1:#x}"
    assert f2 == 0, f"second call: flags {f2:#x}"
    for got in (first, second):
        assert torch.equal(got[0], ref[0])
        for a, b in zip(got[1] + got[2], ref[1] + ref[2]):
            assert torch.equal(a, b)


def test_debug_mla_selection_out_of_range(B, dbg):
    """Selection entries past the candidates or below -1 are skipped by both
    builds (same output) and reported by the debug build."""
    w = wl.make_decode([3000, 700], "bf16", n_layers=1, seed=62)
    t = w.to_torch(DEV)
    rng = np.random.default_rng(62)
    idx = np.full((w.nq, w.k), -1, np.int32)
    idx[0, :1500] = rng.choice(3000, 1500, replace=False)
    idx[1, :700] = np.arange(700)
    clean = torch.from_numpy(idx.copy()).to(DEV)
    idx[0, 1500:1510] = 3000 + np.arange(10)   # past the sequence
    idx[1, 700:705] = -5                        # below -1
    bad = torch.from_numpy(idx).to(DEV)
    batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)

    def attend(sel):
        out = torch.empty(w.nq, 64, 512, device=DEV)
        lse = torch.empty(w.nq, 64, device=DEV)
        B.mla_sparse_attend(batch, t["q"][0], t["kv"][0], sel, w.k, w.tau, out, lse)
        torch.cuda.synchronize()
        return out.cpu(), lse.cpu()

    ref = attend(clean)
    B.debug_flags(True, dbg)
    with using(B, dbg):
        got_clean = attend(clean)
        f_clean = B.debug_flags(True, dbg)
        got_bad = attend(bad)
        f_bad = B.debug_flags(True, dbg)
    assert f_clean == 0, f"valid selection: flags {f_clean:#x}"
    assert f_bad == B.DEBUG_BITS["idx_range"], f"out-of-range entries: flags {f_bad:#x}"
    for got in (got_clean, got_bad):
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_debug_topk_rows(B, dbg):
    """Engineered rows through the standalone top-k (its own histogram pass,
    the LDS candidate list and the all-equal streaming fallback): no check
    fires and the selections equal the release build's."""
    rng = np.random.default_rng(63)
    rows = [rng.integers(0, 50, 3000).astype(np.float32), np.zeros(20000, np.float32),
            rng.standard_normal(70001).astype(np.float32), rng.integers(0, 9, 60000).astype(np.float32)]
    lens = np.array([len(r) for r in rows], np.int32)
    L = int(lens.max())
    sc = np.zeros((len(rows), L), np.float32)
    for i, r in enumerate(rows):
        sc[i, :len(r)] = r
    scores = torch.from_numpy(sc).to(DEV)
    batch = B.Batch(torch.arange(len(rows), dtype=torch.int32, device=DEV), torch.from_numpy(lens - 1).to(DEV),
                    torch.from_numpy(lens).to(DEV), torch.zeros(len(rows), dtype=torch.int64, device=DEV), L)

    def topk():
        idx = torch.full((len(rows), 2048), -7, dtype=torch.int32, device=DEV)
        B.dsa_topk(batch, scores, 2048, idx)
        torch.cuda.synchronize()
        return idx.cpu()

    ref = topk()
    B.debug_flags(True, dbg)
    with using(B, dbg):
        got = topk()
        f = B.debug_flags(True, dbg)
    assert f == 0, f"flags {f:#x}"
    assert torch.equal(got, ref)
