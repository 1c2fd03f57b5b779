"""Parity at the five measured workloads' full sizes, run the way bench.py
runs them (the fused decode entry for decode batches; the three calls for
the prefill chunk), checked against the CPU oracle.

Decode workloads (single query, 64 x 32,768, the ragged 4-layer batch and
4 x 2^20): every query's selection, every layer's output and log-sum-exp.
The ragged batch holds the forced short sequences (1,024, 2,048 and 2,049
positions, where the read must equal dense attention).  The prefill chunk
(2,048 queries): one query per 32-query block, the first and the last of the
chunk among them, with its whole score row compared bit for bit, its
selection and its output.  Bars as in test_gpu_parity: scores and
selections bit-exact, outputs within 1e-4 (fp32) / 1e-2 (bf16) of max|ref|.

The FP8-indexer runs store the same integer draws in E4M3, so the oracle's
results (which take the widened values) are shared with the bf16 runs.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_12_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 1e-2}
PREFILL_SAMPLE = list(range(0, 2048, 32)) + [2047]   # one query per 32-query block, and the last

_REF = {}


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "a GPU is required"
    from sparse_attention_12_amd import binding
    return binding


def _run(B, w, score_rows=()):
    t = w.to_torch(DEV)
    batch = B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in range(w.n_layers)]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in range(w.n_layers)]
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device=DEV)
    rows = None
    if w.kind == "decode":
        B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau, lses, idx)
    else:
        scores = torch.full((w.nq, w.max_len), float("nan"), device=DEV)
        B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
        B.dsa_topk(batch, scores, w.k, idx)
        for l in range(w.n_layers):
            B.mla_sparse_attend(batch, t["q"][l], t["kv"][l], idx, w.k, w.tau, outs[l], lses[l])
        rows = scores[list(score_rows)].cpu().numpy()
        del scores
    torch.cuda.synchronize()
    del t
    return idx.cpu().numpy(), [o.cpu().numpy() for o in outs], [x.cpu().numpy() for x in lses], rows


def _reference(cfg, w, qi):
    """The oracle's read of query qi (cached per workload: the FP8-indexer
    run of a workload shares it)."""
    key = (cfg, qi)
    if key not in _REF:
        s = int(w.q_seq[qi])
        n = oracle.n_candidates(int(w.q_pos[qi]), int(w.seq_len[s]))
        scores = oracle.index_score(w.widen(w.qI[qi]), w.w[qi], w.widen(w.seq_rows(w.kI, s)[:n]))
        ref_idx, m = oracle.topk(scores, w.k)
        sel = ref_idx[:m]
        res = []
        for l in range(w.n_layers):
            rows = w.widen(w.seq_rows(w.kv[l], s)[sel])      # only the selected rows are widened
            res.append(oracle.mla_attend(w.widen(w.q[l][qi]), rows, np.arange(m, dtype=np.int32), w.tau))
        _REF[key] = (scores if w.kind == "prefill" else None, ref_idx, m, res)
    return _REF[key]


def _check_query(cfg, w, qi, idx, outs, lses, score_row=None):
    scores, ref_idx, m, res = _reference(cfg, w, qi)
    if score_row is not None:
        n = scores.shape[0]
        assert np.array_equal(score_row[:n].astype(np.float64), scores), f"query {qi}: scores differ"
        assert np.all(np.isnan(score_row[n:])), f"query {qi}: a column past its candidates was written"
    assert np.array_equal(idx[qi], ref_idx), f"query {qi}: selection differs"
    for l, (o, lse) in enumerate(res):
        err = np.abs(outs[l][qi].astype(np.float64) - o).max()
        assert err <= TOL[w.dtype] * np.abs(o).max(), f"query {qi} layer {l}: max|err| {err:.3e}"
        assert np.abs(lses[l][qi] - lse).max() <= (1e-4 if w.dtype == "f32" else 2e-3), f"query {qi} layer {l}: lse"
    return m


def _check_all(cfg, w, idx, outs, lses):
    for qi in range(w.nq):
        _check_query(cfg, w, qi, idx, outs, lses)


def test_config0_decode_fp32(B):
    w = wl.config(0)
    idx, outs, lses, _ = _run(B, w)
    assert _check_query(0, w, 0, idx, outs, lses) == 2048


def test_config1_decode_batch64(B):
    w = wl.config(1)
    idx, outs, lses, _ = _run(B, w)
    _check_all(1, w, idx, outs, lses)
    assert np.all(idx >= 0) and np.all(np.diff(idx, axis=1) > 0)


def test_config2_ragged_shared_selection(B):
    w = wl.config(2)
    assert list(w.seq_len[:3]) == [1024, 2048, 2049]
    idx, outs, lses, _ = _run(B, w)
    _check_all(2, w, idx, outs, lses)
    for qi in range(w.nq):
        assert int((idx[qi] >= 0).sum()) == min(2048, int(w.seq_len[qi]))
    # at or below 2,048 positions every position is kept
    assert np.array_equal(idx[0][:1024], np.arange(1024)) and np.all(idx[0][1024:] == -1)
    assert np.array_equal(idx[1], np.arange(2048))


def test_config3_causal_prefill(B):
    w = wl.config(3)
    idx, outs, lses, rows = _run(B, w, PREFILL_SAMPLE)
    for j, qi in enumerate(PREFILL_SAMPLE):
        _check_query(3, w, qi, idx, outs, lses, rows[j])
    # causality: no query selects a position after its own
    assert np.all(idx.max(axis=1) <= w.q_pos)


def test_config4_decode_1m(B):
    w = wl.config(4)
    idx, outs, lses, _ = _run(B, w)
    _check_all(4, w, idx, outs, lses)


DSA_MAX_LEN = 3728270   # include/dsa_mla.h: the longest sequence the library takes


def test_decode_at_the_longest_sequence(B):
    """One query over DSA_MAX_LEN positions, two layers: the MLA gathers
    address a sequence's bf16 rows with 32-bit byte offsets, and this length
    puts the last row's end 256 bytes below the 2^32 limit (3,728,270 x
    1,152 B = 4,294,967,040 B).  With 2,048 of 3.7 million positions kept,
    the selection reaches rows near the end.  Selection bit-exact, outputs and
    log-sum-exp to the bf16 bar."""
    w = wl.make_decode([DSA_MAX_LEN], "bf16", n_layers=2, seed=77, name="decode_b1_longest")
    assert DSA_MAX_LEN * 1152 < (1 << 32) <= (DSA_MAX_LEN + 1) * 1152
    idx, outs, lses, _ = _run(B, w)
    _check_query("longest", w, 0, idx, outs, lses)
    assert int(idx[0].max()) > DSA_MAX_LEN - 100000, "the selection should reach rows near the end"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_fp8_indexer(B, cfg):
    """The same workloads with the indexer's query and keys stored in FP8
    E4M3 (bench.py --index-dtype fp8): the integer draws are exact in E4M3,
    so scores, selections and outputs meet the same bars, query for query."""
    w = wl.config(cfg, "fp8")
    assert w.kI.dtype == np.uint8
    idx, outs, lses, rows = _run(B, w, PREFILL_SAMPLE if cfg == 3 else ())
    if cfg == 3:
        for j, qi in enumerate(PREFILL_SAMPLE):
            _check_query(cfg, w, qi, idx, outs, lses, rows[j])
    else:
        _check_all(cfg, w, idx, outs, lses)
