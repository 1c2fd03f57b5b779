"""GPU parity of every entry point against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.

Bars: selected index sets and (integer-input) indexer scores bit-exact;
attention output max|o - o_ref| <= 1e-4 max|o_ref| (fp32) or 1e-2 max|o_ref|
(bf16); log-sum-exp within 1e-4 (fp32) or 2e-3 (bf16) absolute.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_12_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 1e-2}
TAU_ = 1.0 / math.sqrt(192.0)
LSE_TOL = {"f32": 1e-4, "bf16": 2e-3}


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "a GPU is required"
    from sparse_attention_12_amd import binding
    return binding


def _batch(B, w, t):
    return B.Batch(t["q_seq"], t["q_pos"], t["seq_len"], t["seq_row0"], w.max_len)


def _assert_rel(got, ref, rel, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    assert err <= rel * scale, f"{what}: max|err| {err:.3e} > {rel} * {scale:.3e}"


def _oracle_scores(w, qi):
    s = int(w.q_seq[qi])
    n = oracle.n_candidates(int(w.q_pos[qi]), int(w.seq_len[s]))
    return oracle.index_score(w.widen(w.qI)[qi], w.w[qi], w.widen(w.seq_rows(w.kI, s))[:n])


# ----------------------------------------------------------------------------
# indexer
# ----------------------------------------------------------------------------

DECODE_LENS = [1, 31, 32, 33, 100, 2047, 2048, 2049, 4097, 9000, 16385]


@pytest.mark.parametrize("dtype,idt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "fp8")])
def test_index_score_decode_exact(B, dtype, idt):
    w = wl.make_decode(DECODE_LENS, dtype, 1, seed=21, index_dtype=idt)
    t = w.to_torch(DEV)
    ld = w.max_len + 5
    scores = torch.full((w.nq, ld), float("nan"), device=DEV)
    B.dsa_index_score(_batch(B, w, t), t["qI"], t["w"], t["kI"], scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for qi, n in enumerate(DECODE_LENS):
        ref = _oracle_scores(w, qi)
        assert np.array_equal(sc[qi, :n].astype(np.float64), ref), f"query {qi} (L={n})"
        assert np.all(np.isnan(sc[qi, n:])), f"query {qi}: columns beyond the candidates were written"


@pytest.mark.parametrize("idt", ["bf16", "fp8"])
def test_index_score_decode_many_queries(B, idt):
    """Over 1,024 decode queries: the one-workgroup-per-chunk grid (smaller
    batches cut the concatenated keys into equal ranges instead)."""
    rng = np.random.default_rng(22)
    lens = rng.integers(1, 1500, 1100).tolist()
    w = wl.make_decode(lens, "bf16", 1, seed=22, index_dtype=idt)
    t = w.to_torch(DEV)
    scores = torch.full((w.nq, w.max_len), float("nan"), device=DEV)
    B.dsa_index_score(_batch(B, w, t), t["qI"], t["w"], t["kI"], scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for qi in (0, 1, 517, 1023, 1024, 1099):
        n = lens[qi]
        assert np.array_equal(sc[qi, :n].astype(np.float64), _oracle_scores(w, qi)), f"query {qi} (L={n})"
    filled = ~np.isnan(sc)
    assert np.array_equal(filled.sum(axis=1), np.array(lens)), "every candidate scored, nothing else written"


@pytest.mark.parametrize("idt", ["bf16", "fp8"])
@pytest.mark.parametrize("cache,first,nq", [(3000, 2900, 70), (5000, 10, 64), (9000, 8960, 40),
                                            (30000, 29840, 160)])
def test_index_score_prefill_exact(B, cache, first, nq, idt):
    w = wl.make_prefill(cache, first, nq, "bf16", seed=22, index_dtype=idt)
    t = w.to_torch(DEV)
    scores = torch.full((w.nq, cache), float("nan"), device=DEV)
    B.dsa_index_score(_batch(B, w, t), t["qI"], t["w"], t["kI"], scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for qi in range(nq):
        n = min(first + qi + 1, cache)
        ref = _oracle_scores(w, qi)
        assert ref.shape[0] == n
        assert np.array_equal(sc[qi, :n].astype(np.float64), ref), f"query {qi}"
        assert np.all(np.isnan(sc[qi, n:]))


@pytest.mark.parametrize("idt", ["bf16", "fp8"])
@pytest.mark.parametrize("cache", [16384, 20480, 40960])
def test_index_score_prefill_key_chunks(B, cache, idt):
    """2,048 queries at the end of a cache of `cache` positions.  The
    prefill dispatch starts from 8,192-key chunks and halves them while the
    grid has fewer than 512 workgroups (64 query blocks here): 16,384
    positions give chunks of 2,048 (8 x 64 workgroups), 20,480 positions
    chunks of 2,048 (10 x 64) and 40,960 positions chunks of 4,096 (10 x 64),
    the lengths the FP8 kernel is instantiated for and the bf16 kernel takes
    at run time.  One query per 32-query block, the causal edge's first and
    last among them, has its whole score row compared bit for bit; columns
    past its candidates stay untouched; its selection equals the oracle's."""
    nq = 2048
    w = wl.make_prefill(cache, cache - nq, nq, "bf16", seed=48, index_dtype=idt)
    t = w.to_torch(DEV)
    batch = _batch(B, w, t)
    scores = torch.full((nq, cache), float("nan"), device=DEV)
    B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
    idx = torch.empty((nq, 2048), dtype=torch.int32, device=DEV)
    B.dsa_topk(batch, scores, 2048, idx)
    sample = list(range(0, nq, 32)) + [nq - 1]
    rows = scores[sample].cpu().numpy()
    idx_h = idx[sample].cpu().numpy()
    torch.cuda.synchronize()
    for j, qi in enumerate(sample):
        n = cache - nq + qi + 1
        ref = _oracle_scores(w, qi)
        assert ref.shape[0] == n
        assert np.array_equal(rows[j, :n].astype(np.float64), ref), f"query {qi}: scores"
        assert np.all(np.isnan(rows[j, n:])), f"query {qi}: a column past its candidates was written"
        ref_idx, _ = oracle.topk(ref, 2048)
        assert np.array_equal(idx_h[j], ref_idx), f"query {qi}: selection"


@pytest.mark.parametrize("idt", ["bf16", "fp8"])
@pytest.mark.parametrize("order", ["grouped", "interleaved"])
def test_index_score_prefill_several_sequences(B, idt, order):
    """A prefill batch over three sequences (50, 100 and 40 queries at the
    ends of 5,000-, 9,000- and 3,000-position caches) takes the blocked
    prefill kernels: grouped, the 32-query blocks straddle sequence
    boundaries; interleaved, every block holds queries of all three, and the
    key chunk is swept once per sequence.  Every score exact, columns past a
    query's candidates untouched."""
    rng = np.random.default_rng(47)
    lens = np.array([5000, 9000, 3000], np.int32)
    counts = [50, 100, 40]
    row0 = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    q_seq = np.concatenate([np.full(c, s, np.int32) for s, c in enumerate(counts)])
    q_pos = np.concatenate([np.arange(lens[s] - c, lens[s], dtype=np.int32) for s, c in enumerate(counts)])
    if order == "interleaved":
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
        perm = [starts[s] + k for k in range(max(counts)) for s in range(3) if k < counts[s]]
        q_seq, q_pos = q_seq[perm], q_pos[perm]
    else:
        q_seq[-1] = 3          # no such sequence: no candidates, its row untouched
    nq = len(q_seq)
    qI_i = rng.integers(-3, 4, size=(nq, 32, 128), dtype=np.int8)
    kI_i = rng.integers(-3, 4, size=(int(lens.sum()), 128), dtype=np.int8)
    w_ = rng.integers(1, 5, size=(nq, 32)).astype(np.float32)
    qI = wl._small_int_bits(qI_i, idt)
    kI = wl._small_int_bits(kI_i, idt)
    batch = B.Batch(torch.from_numpy(q_seq).to(DEV), torch.from_numpy(q_pos).to(DEV),
                    torch.from_numpy(lens).to(DEV), torch.from_numpy(row0).to(DEV), int(lens.max()))
    scores = torch.full((nq, int(lens.max())), float("nan"), device=DEV)
    dev = lambda a: torch.from_numpy(a).to(DEV).view(torch.bfloat16) if a.dtype == np.uint16 else \
        torch.from_numpy(a).to(DEV)
    B.dsa_index_score(batch, dev(qI), torch.from_numpy(w_).to(DEV), dev(kI), scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for qi in range(nq):
        s, n = int(q_seq[qi]), int(q_pos[qi]) + 1
        if s >= len(lens):
            assert np.all(np.isnan(sc[qi])), f"query {qi} of no sequence"
            continue
        keys = kI_i[row0[s]: row0[s] + n].astype(np.float32)
        ref = oracle.index_score(qI_i[qi].astype(np.float32), w_[qi], keys)
        assert np.array_equal(sc[qi, :n].astype(np.float64), ref), f"query {qi} (sequence {s})"
        assert np.all(np.isnan(sc[qi, n:]))


FINITE_E4M3 = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)


def _fp8_scores(B, lens, qI, kI, w_):
    """Indexer scores of one decode query per sequence from raw E4M3 bytes."""
    nq = len(lens)
    row0 = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    L = np.array(lens, np.int32)
    batch = B.Batch(torch.arange(nq, dtype=torch.int32, device=DEV), torch.from_numpy(L - 1).to(DEV),
                    torch.from_numpy(L).to(DEV), torch.from_numpy(row0).to(DEV), max(lens))
    scores = torch.full((nq, max(lens)), float("nan"), device=DEV)
    B.dsa_index_score(batch, torch.from_numpy(qI).to(DEV), torch.from_numpy(w_).to(DEV),
                      torch.from_numpy(kI).to(DEV), scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy().astype(np.float64), row0


def test_index_score_fp8_every_code_exact(B):
    """Every finite E4M3 code (subnormals, +-448, signed zeros) is read as the
    OCP encoding, bit-exact.  Query 0 has one-hot heads (+-1 at one element
    each) over keys drawn from all codes; query 1 has one-hot keys (+-1) under
    heads drawn from all codes.  With unit weights each score is a sum of 32
    E4M3 values, all multiples of 2^-9 below 32 x 448 < 2^14, so float32
    holds every partial sum exactly and the result must equal the oracle."""
    rng = np.random.default_rng(23)
    lens = [700, 1500]
    rows = sum(lens)
    qI = np.zeros((2, 32, 128), np.uint8)
    kI = rng.choice(FINITE_E4M3, size=(rows, 128))
    pick = rng.integers(0, 128, 32)
    qI[0, np.arange(32), pick] = rng.choice(np.array([0x38, 0xB8], np.uint8), 32)
    qI[1] = rng.choice(FINITE_E4M3, size=(32, 128))
    one = rng.integers(0, 128, lens[1])
    kI[lens[0]:] = 0
    kI[lens[0] + np.arange(lens[1]), one] = rng.choice(np.array([0x38, 0xB8], np.uint8), lens[1])
    w_ = np.ones((2, 32), np.float32)
    sc, row0 = _fp8_scores(B, lens, qI, kI, w_)
    qf, kf = wl.e4m3_bits_to_f32(qI), wl.e4m3_bits_to_f32(kI)
    # every code was exercised
    assert len(np.unique(kI[:lens[0]][:, pick])) == len(FINITE_E4M3)
    assert len(np.unique(qI[1])) == len(FINITE_E4M3)
    for qi, n in enumerate(lens):
        ref = oracle.index_score(qf[qi], w_[qi], kf[row0[qi]:row0[qi] + n])
        assert np.array_equal(sc[qi, :n], ref), f"query {qi}"


def test_index_score_fp8_full_range(B):
    """Random codes over the whole E4M3 range in q and k and normal weights.
    Products of two E4M3 values are exact, but the matrix core sums the 128
    products of a head at an internal precision that AMD does not specify bit
    by bit, so the bar is relative to the sum of absolute terms,
    sum_h |w_h| sum_i |q_hi k_i|: 2^-14 of it (fp32 rounding alone gives
    about 2^-17; a mis-read code or a dropped product is far larger).  The
    last query and its keys use only subnormals and the two lowest binades,
    where a flushed subnormal would exceed the bar."""
    rng = np.random.default_rng(24)
    lens = [3, 700, 2100, 500]
    rows = sum(lens)
    qI = rng.choice(FINITE_E4M3, size=(len(lens), 32, 128))
    kI = rng.choice(FINITE_E4M3, size=(rows, 128))
    tiny = FINITE_E4M3[(FINITE_E4M3 & 0x78) <= 0x10]
    qI[-1] = rng.choice(tiny, size=(32, 128))
    kI[rows - lens[-1]:] = rng.choice(tiny, size=(lens[-1], 128))
    w_ = rng.standard_normal((len(lens), 32)).astype(np.float32)
    sc, row0 = _fp8_scores(B, lens, qI, kI, w_)
    qf, kf = wl.e4m3_bits_to_f32(qI), wl.e4m3_bits_to_f32(kI)
    for qi, n in enumerate(lens):
        k = kf[row0[qi]:row0[qi] + n].astype(np.float64)
        ref = oracle.index_score(qf[qi], w_[qi], kf[row0[qi]:row0[qi] + n])
        mag = np.abs(w_[qi]).astype(np.float64) @ (np.abs(qf[qi]).astype(np.float64) @ np.abs(k.T))
        err = np.abs(sc[qi, :n] - ref)
        assert np.all(err <= 2.0 ** -14 * mag), f"query {qi}: worst {np.max(err / mag):.3e}"


# ----------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------


def _topk_gpu(B, rows, k, ld=None):
    """rows: list of float32 score arrays (one query per sequence)."""
    lens = np.array([len(r) for r in rows], np.int32)
    L = int(lens.max())
    ld = ld or L
    sc = np.zeros((len(rows), ld), np.float32)
    for i, r in enumerate(rows):
        sc[i, :len(r)] = r
    q_seq = torch.arange(len(rows), dtype=torch.int32, device=DEV)
    batch = B.Batch(q_seq, torch.from_numpy(lens - 1).to(DEV), torch.from_numpy(lens).to(DEV),
                    torch.zeros(len(rows), dtype=torch.int64, device=DEV), L)
    idx = torch.full((len(rows), k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((len(rows),), -7, dtype=torch.int32, device=DEV)
    ws_n = B.dsa_topk_workspace_size(len(rows), L, k)
    # a workspace full of stale bytes: the library clears what it relies on
    ws = torch.full((max(ws_n, 1),), 0xA5, dtype=torch.uint8, device=DEV) if ws_n else None
    B.dsa_topk(batch, torch.from_numpy(sc).to(DEV), k, idx, cnt, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("long_row", [False, True])
@pytest.mark.parametrize("k", [1, 5, 64, 2048])
def test_topk_engineered_rows(B, k, long_row):
    """long_row adds a 60,000-score row, which sends the batch down the
    split path (rows of at most 49,152 scores take one workgroup per row)."""
    rng = np.random.default_rng(23)
    rows = [
        rng.integers(0, 50, 3000).astype(np.float32),                 # heavy ties
        np.zeros(20000, np.float32),                                    # all equal, > LDS candidate cap
        rng.standard_normal(7777).astype(np.float32),                   # distinct
        np.where(rng.random(5000) < 0.5, 0.0, -0.0).astype(np.float32),  # signed zeros
        -np.abs(rng.standard_normal(4100)).astype(np.float32),          # all negative
        rng.integers(0, 3, 40000).astype(np.float32) * 1000.0,          # three huge tie groups
        rng.standard_normal(max(1, k - 3)).astype(np.float32),          # fewer candidates than k
        np.full(k, 5.0, np.float32),                                    # exactly k candidates
        # three keys one ulp apart: one 22-bit bin holds them all, so the
        # second 10-bit level must split them
        (np.float32(3.0) + rng.integers(0, 3, 9000).astype(np.float32) * np.spacing(np.float32(3.0))
         ).astype(np.float32),
    ]
    if long_row:
        rows.append(rng.integers(0, 9, 60000).astype(np.float32))
    idx, cnt = _topk_gpu(B, rows, k)
    for i, r in enumerate(rows):
        ref, m = oracle.topk(r.astype(np.float64), k)
        assert cnt[i] == m, f"row {i}"
        assert np.array_equal(idx[i], ref), f"row {i}: selection differs"


def test_topk_split_list_capacity(B):
    """Rows longer than 49,152 scores take the split path, whose final
    workgroup copies the threshold bin's candidates into LDS when they number
    at most 12,288 (the copy's largest case: 12 entries per thread, consecutive
    lanes on consecutive entries) and streams the row otherwise.  Threshold
    bins of exactly 12,287, 12,288 and 12,289 tied keys, spread over every
    chunk of a 70,000-score row, sit on either side of that capacity; the
    other scores lie below them."""
    rng = np.random.default_rng(57)
    n = 70000
    rows = []
    for j, tied in enumerate((12287, 12288, 12289)):
        row = rng.random(n).astype(np.float32)  # [0, 1): other first-level bins
        row[rng.choice(n, tied, replace=False)] = np.float32(2.0 + j)
        rows.append(row)
    idx, cnt = _topk_gpu(B, rows, 2048)
    for i, r in enumerate(rows):
        ref, m = oracle.topk(r.astype(np.float64), 2048)
        assert cnt[i] == m, f"row {i}"
        assert np.array_equal(idx[i], ref), f"row {i}: selection differs"


def test_topk_many_rows(B):
    """Batches of many rows take the one-workgroup-per-row path."""
    rng = np.random.default_rng(31)
    rows = []
    for i in range(300):
        kind = i % 5
        n = int(rng.integers(1, 9000))
        if kind == 0:
            rows.append(rng.integers(0, 40, n).astype(np.float32))
        elif kind == 1:
            rows.append(rng.standard_normal(n).astype(np.float32))
        elif kind == 2:
            rows.append(np.zeros(n if i != 2 else 20000, np.float32))
        elif kind == 3:
            rows.append(np.where(rng.random(n) < 0.5, 0.0, -0.0).astype(np.float32))
        else:
            rows.append((rng.integers(0, 3, n) * 7.0 - 5.0).astype(np.float32))
    idx, cnt = _topk_gpu(B, rows, 2048)
    for i, r in enumerate(rows):
        ref, m = oracle.topk(r.astype(np.float64), 2048)
        assert cnt[i] == m, f"row {i}"
        assert np.array_equal(idx[i], ref), f"row {i}: selection differs"


@pytest.mark.parametrize("nrows", [5, 290])
def test_topk_unaligned_rows(B, nrows):
    """Row strides that are not a multiple of four floats: every row but the
    first starts off a 16-byte boundary, so the vector passes take their
    scalar head and tail paths (few rows: split path, since some exceed
    49,152 scores; many: one per row)."""
    rng = np.random.default_rng(32 + nrows)
    rows = []
    for i in range(nrows):
        n = int(rng.integers(2049, 40001)) if i % 3 else int(rng.integers(1, 5000))
        if nrows < 256 and i == 1:
            n = 60001
        rows.append(rng.integers(0, 60, n).astype(np.float32) if i % 2 else rng.standard_normal(n).astype(np.float32))
    L = max(len(r) for r in rows)
    idx, cnt = _topk_gpu(B, rows, 2048, ld=L + 3)
    for i, r in enumerate(rows):
        ref, m = oracle.topk(r.astype(np.float64), 2048)
        assert cnt[i] == m, f"row {i}"
        assert np.array_equal(idx[i], ref), f"row {i}: selection differs"


def test_topk_many_long_rows(B):
    """Many rows, some longer than the 49,152 scores the per-row kernel keeps
    in registers: the rest of such a row is read from memory in both passes
    (row stride odd, so off 16-byte boundaries), including a long all-equal
    row that overflows the LDS candidate list."""
    rng = np.random.default_rng(41)
    rows = []
    for i in range(260):
        n = int(rng.integers(1, 4000))
        rows.append(rng.integers(0, 30, n).astype(np.float32) if i % 2 else rng.standard_normal(n).astype(np.float32))
    rows[3] = rng.integers(0, 9, 60001).astype(np.float32)          # remainder of 10,849 scores, heavy ties
    rows[4] = np.zeros(65536, np.float32)                            # all equal: streaming fallback
    rows[7] = rng.standard_normal(70001).astype(np.float32)          # distinct, longest
    rows[10] = rng.integers(0, 4, 49153).astype(np.float32) * 1e3    # one score past the registers
    L = max(len(r) for r in rows)
    idx, cnt = _topk_gpu(B, rows, 2048, ld=L + 1)
    for i, r in enumerate(rows):
        ref, m = oracle.topk(r.astype(np.float64), 2048)
        assert cnt[i] == m, f"row {i}"
        assert np.array_equal(idx[i], ref), f"row {i}: selection differs"


def test_topk_on_indexer_scores(B):
    w = wl.make_decode([2048, 2049, 5000, 33000], "bf16", 1, seed=24)
    t = w.to_torch(DEV)
    batch = _batch(B, w, t)
    scores = torch.empty((w.nq, w.max_len), device=DEV)
    B.dsa_index_score(batch, t["qI"], t["w"], t["kI"], scores)
    idx = torch.empty((w.nq, 2048), dtype=torch.int32, device=DEV)
    cnt = torch.empty((w.nq,), dtype=torch.int32, device=DEV)
    B.dsa_topk(batch, scores, 2048, idx, cnt)
    torch.cuda.synchronize()
    for qi in range(w.nq):
        ref, m = oracle.topk(_oracle_scores(w, qi), 2048)
        assert int(cnt[qi]) == m
        assert np.array_equal(idx[qi].cpu().numpy(), ref)


def test_topk_nonint_scores_property(B):
    """Real-valued indexer inputs: fp32 rounding may swap near-ties, so the
    check is that every kept position scores within a hair of the oracle's
    threshold and that the count is right."""
    rng = np.random.default_rng(25)
    L = 6000
    qI = rng.standard_normal((1, 32, 128)).astype(np.float32)
    wv = rng.uniform(0.5, 2.0, (1, 32)).astype(np.float32)
    kI = rng.standard_normal((L, 128)).astype(np.float32)
    batch = B.Batch(torch.zeros(1, dtype=torch.int32, device=DEV), torch.tensor([L - 1], dtype=torch.int32, device=DEV),
                    torch.tensor([L], dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int64, device=DEV), L)
    scores = torch.empty((1, L), device=DEV)
    B.dsa_index_score(batch, torch.from_numpy(qI).to(DEV), torch.from_numpy(wv).to(DEV),
                      torch.from_numpy(kI).to(DEV), scores)
    idx = torch.empty((1, 2048), dtype=torch.int32, device=DEV)
    B.dsa_topk(batch, scores, 2048, idx)
    ref_sc = oracle.index_score(qI[0], wv[0], kI)
    thr = np.sort(ref_sc)[::-1][2047]
    got = idx[0].cpu().numpy()
    assert np.all(got >= 0) and len(set(got.tolist())) == 2048 and np.all(np.diff(got) > 0)
    assert ref_sc[got].min() >= thr - 1e-4 * np.abs(ref_sc).max()


# ----------------------------------------------------------------------------
# sparse MLA
# ----------------------------------------------------------------------------


def _mla_case(B, dtype, lens, k, nq_pad=0, out_dtype=torch.float32, seed=26, rope=64):
    w = wl.make_decode(lens, dtype, 1, seed=seed, rope_dim=rope)
    t = w.to_torch(DEV)
    rng = np.random.default_rng(seed + 1)
    idx = np.full((w.nq, k), -1, np.int32)
    for qi, n in enumerate(lens):
        m = min(k, n)
        chosen = np.sort(rng.choice(n, m, replace=False))
        idx[qi, :m] = chosen
        if nq_pad and qi % 2 == 1 and m > 4:   # holes anywhere in the list are skipped
            idx[qi, 1:4] = -1
    out = torch.empty((w.nq, 64, 512), dtype=out_dtype, device=DEV)
    lse = torch.empty((w.nq, 64), device=DEV)
    ws_n = B.mla_sparse_attend_workspace_size(w.nq, k, 1)
    ws = torch.full((max(ws_n, 16),), 0xA5, dtype=torch.uint8, device=DEV)   # stale bytes
    runs = []
    for _ in range(2):   # the second call reuses the workspace the first left behind
        B.mla_sparse_attend(_batch(B, w, t), t["q"][0], t["kv"][0], torch.from_numpy(idx).to(DEV), k, w.tau,
                            out, lse, ws)
        runs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    # bitwise the same: the split merge does not depend on completion order
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    for qi in range(w.nq):
        sel = idx[qi][idx[qi] >= 0]
        r_o, r_l = oracle.mla_attend(w.widen(w.q[0])[qi], w.widen(w.seq_rows(w.kv[0], qi)), sel, w.tau)
        rel = TOL[dtype] if out_dtype == torch.float32 else 1e-2
        _assert_rel(o[qi], r_o, rel, f"query {qi} output")
        assert np.abs(l[qi] - r_l).max() <= LSE_TOL[dtype], f"query {qi} lse"


@pytest.mark.parametrize("rope", [64, 0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mla_split_path(B, dtype, rope):
    # few queries -> the selection is split across workgroups and merged;
    # rope 0: a layer without rotary encoding (512-wide rows)
    _mla_case(B, dtype, [5, 40, 2048, 3000, 70000], 2048, nq_pad=1, rope=rope)


@pytest.mark.parametrize("rope", [64, 0])
def test_mla_unsplit_path_bf16(B, rope):
    # enough queries that each runs in one workgroup
    lens = [2100 + 37 * i for i in range(520)]
    _mla_case(B, "bf16", lens[:520], 2048, seed=27, rope=rope)


@pytest.mark.parametrize("k", [1, 100, 2047])
def test_mla_small_k(B, k):
    _mla_case(B, "bf16", [50, 3000], k, seed=28)


def test_mla_bf16_output(B):
    _mla_case(B, "bf16", [3000, 4000], 2048, out_dtype=torch.bfloat16, seed=29)


# ----------------------------------------------------------------------------
# fused decode with a shared selection
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("dtype,idt,lens,layers,rope", [
    ("bf16", "bf16", [1024, 2048, 2049, 3333, 40000], 4, 64),
    ("f32", "f32", [700, 4096], 2, 64),
    ("bf16", "fp8", [1500, 2049, 9000], 2, 64),
    ("bf16", "bf16", [1500, 2049, 9000], 3, 0),
])
def test_fused_decode(B, dtype, idt, lens, layers, rope):
    w = wl.make_decode(lens, dtype, layers, seed=30, index_dtype=idt, rope_dim=rope)
    t = w.to_torch(DEV)
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in range(layers)]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in range(layers)]
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device=DEV)
    # stale workspace bytes must not matter (the call clears what it relies on)
    ws = torch.full((B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, w.k, layers),), 0xA5,
                    dtype=torch.uint8, device=DEV)
    B.dsa_mla_decode_fused(_batch(B, w, t), t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau,
                           lses, idx, ws)
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    # run again: results are deterministic
    B.dsa_mla_decode_fused(_batch(B, w, t), t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau,
                           lses, idx, ws)
    torch.cuda.synchronize()
    for a, b in zip(first, outs):
        assert torch.equal(a, b)
    idx_h = idx.cpu().numpy()
    for qi, n in enumerate(lens):
        r_idx, m, r_o, r_l = oracle.decode_query(
            w.widen(w.qI)[qi], w.w[qi], w.widen(w.seq_rows(w.kI, qi)), [w.widen(x)[qi] for x in w.q],
            [w.widen(w.seq_rows(x, qi)) for x in w.kv], n, w.k, w.tau)
        assert np.array_equal(idx_h[qi], r_idx), f"query {qi}: selection"
        for l in range(layers):
            _assert_rel(outs[l][qi].cpu().numpy(), r_o[l], TOL[dtype], f"query {qi} layer {l}")
            assert np.abs(lses[l][qi].cpu().numpy() - r_l[l]).max() <= LSE_TOL[dtype]


def test_fused_decode_padded_layout_and_shared_sequence(B):
    """Sequences stored out of order with gaps between them (seq_row0 is all
    the library uses to find rows), two queries on one sequence at
    different positions, and a selection size below 2,048."""
    rng = np.random.default_rng(35)
    lens = np.array([3000, 2500, 5000], np.int32)
    gap = 777
    row0 = np.array([2 * gap + 5000 + 2500, gap + 5000, 0], np.int64)   # reversed, with gaps
    rows = int(row0.max() + lens[0] + gap)
    q_seq = np.array([0, 1, 2, 0], np.int32)
    q_pos = np.array([2999, 2499, 4999, 2000], np.int32)
    k = 700
    qI = rng.integers(-3, 4, (4, 32, 128)).astype(np.float32)
    w_ = rng.integers(1, 5, (4, 32)).astype(np.float32)
    kI = rng.integers(-3, 4, (rows, 128)).astype(np.float32)
    layers = 2
    q = [wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(rng.standard_normal((4, 64, 576)).astype(np.float32)))
         for _ in range(layers)]
    kv = [wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(rng.standard_normal((rows, 576)).astype(np.float32)))
          for _ in range(layers)]
    bf = lambda a: torch.from_numpy(a).to(DEV).to(torch.bfloat16)
    batch = B.Batch(torch.from_numpy(q_seq).to(DEV), torch.from_numpy(q_pos).to(DEV), torch.from_numpy(lens).to(DEV),
                    torch.from_numpy(row0).to(DEV), int(lens.max()))
    outs = [torch.empty((4, 64, 512), device=DEV) for _ in range(layers)]
    lses = [torch.empty((4, 64), device=DEV) for _ in range(layers)]
    idx = torch.full((4, k), -7, dtype=torch.int32, device=DEV)
    B.dsa_mla_decode_fused(batch, bf(qI), torch.from_numpy(w_).to(DEV), bf(kI), k, [bf(x) for x in q],
                           [bf(x) for x in kv], outs, TAU_, lses, idx)
    torch.cuda.synchronize()
    for qi in range(4):
        s, n = int(q_seq[qi]), int(q_pos[qi]) + 1
        r0 = int(row0[s])
        r_idx, m, r_o, r_l = oracle.decode_query(qI[qi], w_[qi], kI[r0:r0 + lens[s]], [x[qi] for x in q],
                                                 [x[r0:r0 + lens[s]] for x in kv], n, k, TAU_)
        assert np.array_equal(idx[qi].cpu().numpy(), r_idx), f"query {qi}: selection"
        for l in range(layers):
            _assert_rel(outs[l][qi].cpu().numpy(), r_o[l], TOL["bf16"], f"query {qi} layer {l}")
            assert np.abs(lses[l][qi].cpu().numpy() - r_l[l]).max() <= LSE_TOL["bf16"]


def test_fused_decode_shared_cache(B):
    """Two layers of one fused call reading the same cache (pointer
    aliasing, as layers 39, 43, ... read layer 35's latent)."""
    w = wl.make_decode([1800, 5000], "bf16", 3, seed=31, rope_dim=0)
    t = w.to_torch(DEV)
    kvs = [t["kv"][0], t["kv"][0], t["kv"][2]]
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in range(3)]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in range(3)]
    B.dsa_mla_decode_fused(_batch(B, w, t), t["qI"], t["w"], t["kI"], w.k, t["q"], kvs, outs, w.tau, lses)
    torch.cuda.synchronize()
    for qi, n in enumerate([1800, 5000]):
        caches = [w.kv[0], w.kv[0], w.kv[2]]
        r_idx, m, r_o, r_l = oracle.decode_query(
            w.widen(w.qI)[qi], w.w[qi], w.widen(w.seq_rows(w.kI, qi)), [w.widen(x)[qi] for x in w.q],
            [w.widen(w.seq_rows(x, qi)) for x in caches], n, w.k, w.tau)
        for l in range(3):
            _assert_rel(outs[l][qi].cpu().numpy(), r_o[l], TOL["bf16"], f"query {qi} layer {l}")
            assert np.abs(lses[l][qi].cpu().numpy() - r_l[l]).max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("idt,n_layers", [("bf16", 72), ("fp8", 44)])
def test_decode_layers_schedule(B, idt, n_layers):
    """A decode step over Mistral Large 4's schedule (the library's plan):
    indexer layers select, reusing layers carry the selection, rotary-free
    layers read 512-wide rows, and from layer 39 those read layer 35's
    cache.  Every layer's output against the oracle's step over the
    oracle's own schedule."""
    plan = B.dsa_ml4_layer_plan(n_layers)
    oplan = oracle.layer_plan(n_layers)
    assert [(r, rope == 64, src) for r, rope, src in plan] == oplan
    lens = [1500, 2600]
    st = wl.make_layer_stack(lens, oplan, "bf16", seed=40, index_dtype=idt)
    w = st.base
    t = w.to_torch(DEV)
    d = st.to_torch(DEV)
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in plan]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in plan]
    idxs = [torch.full((w.nq, w.k), -7, dtype=torch.int32, device=DEV) if p[0] else None for p in plan]
    ws = torch.full((B.dsa_mla_decode_layers_workspace_size(w.nq, w.max_len, w.k, plan),), 0xA5,
                    dtype=torch.uint8, device=DEV)
    B.dsa_mla_decode_layers(_batch(B, w, t), plan, d["qI"], d["w"], d["kI"], w.k, d["q"], d["kv"], outs, w.tau,
                            lses, idxs, ws)
    torch.cuda.synchronize()
    for qi, n in enumerate(lens):
        rows = lambda a: None if a is None else w.widen(w.seq_rows(a, qi))
        r_idx, r_o, r_l = oracle.decode_layers(
            oplan, [None if a is None else w.widen(a)[qi] for a in st.qI],
            [None if a is None else a[qi] for a in st.w], [rows(a) for a in st.kI],
            [w.widen(a)[qi] for a in st.q], [rows(a) for a in st.kv], n, w.k, w.tau)
        for l, (runs, _, _) in enumerate(oplan):
            if runs:
                assert np.array_equal(idxs[l][qi].cpu().numpy(), r_idx[l]), f"query {qi} layer {l}: selection"
            _assert_rel(outs[l][qi].cpu().numpy(), r_o[l], TOL["bf16"], f"query {qi} layer {l}")
            assert np.abs(lses[l][qi].cpu().numpy() - r_l[l]).max() <= LSE_TOL["bf16"], f"query {qi} layer {l}"


def test_decode_layers_runs_of_four_and_three(B):
    """Runs of four and three layers over one shared cache at 32 queries:
    the three-layer run's launch takes more splits than the four-layer
    one's, and both fit the workspace the size query returns."""
    n = 7
    oplan = [(l in (0, 4), True, 0) for l in range(n)]
    plan = [(int(r), 64, src) for r, _, src in oplan]
    rng = np.random.default_rng(44)
    lens = [int(x) for x in rng.integers(2049, 2400, 32)]
    st = wl.make_layer_stack(lens, oplan, "bf16", seed=45)
    w = st.base
    t = w.to_torch(DEV)
    d = st.to_torch(DEV)
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in plan]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in plan]
    idxs = [torch.full((w.nq, w.k), -7, dtype=torch.int32, device=DEV) if r else None for r, _, _ in plan]
    ws = torch.full((B.dsa_mla_decode_layers_workspace_size(w.nq, w.max_len, w.k, plan),), 0xA5,
                    dtype=torch.uint8, device=DEV)
    B.dsa_mla_decode_layers(_batch(B, w, t), plan, d["qI"], d["w"], d["kI"], w.k, d["q"], d["kv"], outs, w.tau,
                            lses, idxs, ws)
    torch.cuda.synchronize()
    for qi in (0, 31):
        n_c = lens[qi]
        rows = lambda a: None if a is None else w.widen(w.seq_rows(a, qi))
        r_idx, r_o, r_l = oracle.decode_layers(
            oplan, [None if a is None else w.widen(a)[qi] for a in st.qI],
            [None if a is None else a[qi] for a in st.w], [rows(a) for a in st.kI],
            [w.widen(a)[qi] for a in st.q], [rows(a) for a in st.kv], n_c, w.k, w.tau)
        for l, (runs, _, _) in enumerate(oplan):
            if runs:
                assert np.array_equal(idxs[l][qi].cpu().numpy(), r_idx[l]), f"query {qi} layer {l}: selection"
            _assert_rel(outs[l][qi].cpu().numpy(), r_o[l], TOL["bf16"], f"query {qi} layer {l}")
            assert np.abs(lses[l][qi].cpu().numpy() - r_l[l]).max() <= LSE_TOL["bf16"], f"query {qi} layer {l}"


def test_fused_read_under_graph_capture(B):
    """The fused decode read captured in a graph (workspace passed in, so the
    capture allocates nothing): every replay, with eager work and
    synchronisations between replays, equals an eager call bit for bit --
    the library clears its scratch with its own kernels, never with a
    memset node."""
    w = wl.make_decode([1500, 2600, 70000], "bf16", 2, seed=46)
    t = w.to_torch(DEV)
    batch = _batch(B, w, t)
    ws = torch.empty(B.dsa_mla_decode_fused_workspace_size(w.nq, w.max_len, w.k, 2), dtype=torch.uint8, device=DEV)
    outs = [torch.empty((w.nq, 64, 512), device=DEV) for _ in range(2)]
    lses = [torch.empty((w.nq, 64), device=DEV) for _ in range(2)]
    idx = torch.empty((w.nq, w.k), dtype=torch.int32, device=DEV)
    call = lambda: B.dsa_mla_decode_fused(batch, t["qI"], t["w"], t["kI"], w.k, t["q"], t["kv"], outs, w.tau,
                                          lses, idx, ws)
    call()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs + lses + [idx]]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in outs + lses:
            x.fill_(float("nan"))
        idx.fill_(-7)
        ws.fill_(0xA5)                    # stale scratch before every replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs + lses + [idx], ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"


def _round_ref(x, dtype):
    """Bar for a value the kernel computes in float32 and stores in dtype:
    the oracle's float64 value within one rounding of dtype plus float32
    arithmetic."""
    x = np.asarray(x, np.float64)
    return (2.0 ** -8 if dtype == "bf16" else 2.0 ** -21) * np.abs(x) + 1e-6 * (np.abs(x).max() + 1e-30)


@pytest.mark.parametrize("dtype,rope,scaled,with_q", [
    ("bf16", 64, True, True), ("f32", 64, True, True), ("bf16", 64, False, False), ("bf16", 0, True, True),
])
def test_rope_append(B, dtype, rope, scaled, with_q):
    """Cache append and query preparation against oracle/rope.py: rows of
    the new tokens written, every other row untouched, queries scaled and
    rotated in place, positions from 0 to 2^20 - 1."""
    from oracle import rope as orope
    rng = np.random.default_rng(50)
    lens = np.array([1, 37, 4096, 70001, 1 << 20], np.int32)
    nq, W = len(lens), 512 + rope
    row0 = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    rows = int(lens.sum())
    q_pos = lens - 1
    q_pos[1] = 40          # past its sequence: this token is skipped
    alpha = (rng.standard_normal(32) * 0.3).astype(np.float32)
    freq = B.dsa_rope_frequencies(alpha)
    latent = rng.standard_normal((nq, 512)).astype(np.float32)
    rkey = rng.standard_normal((nq, 64)).astype(np.float32)
    qa = rng.standard_normal((nq, 64, W)).astype(np.float32)
    s_h = (rng.standard_normal(64) * 0.1).astype(np.float32) if scaled else None
    b_h = (1 + rng.standard_normal(64) * 0.1).astype(np.float32) if scaled else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sentinel = torch.full((rows, W), 7.0, dtype=tdt, device=DEV)
    kv = sentinel.clone()
    q_in = torch.from_numpy(qa).to(DEV).to(tdt)
    q_dev = q_in.clone() if with_q else None
    batch = B.Batch(torch.arange(nq, dtype=torch.int32, device=DEV), torch.from_numpy(q_pos).to(DEV),
                    torch.from_numpy(lens).to(DEV), torch.from_numpy(row0).to(DEV), int(lens.max()))
    dv = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    B.dsa_rope_append(batch, dv(freq) if rope else None, dv(latent), dv(rkey) if rope else None, kv, q_dev,
                      dv(s_h), dv(b_h))
    torch.cuda.synchronize()
    changed = torch.nonzero((kv != 7.0).any(dim=1)).flatten().cpu().numpy()
    q_h = None if q_dev is None else q_dev.float().cpu().numpy()
    qin_h = q_in.float().cpu().numpy()        # the query as stored before the call
    written = set()
    for qi in range(nq):
        t = int(q_pos[qi])
        if t >= lens[qi]:
            if q_h is not None:
                assert np.array_equal(q_h[qi], qin_h[qi]), "a skipped token's query was modified"
            continue
        r = int(row0[qi]) + t
        written.add(r)
        ref = orope.append_row(latent[qi], rkey[qi] if rope else None, t, freq)
        got = kv[r].float().cpu().numpy()
        assert np.all(np.abs(got - ref) <= _round_ref(ref, dtype)), f"token {qi}: cache row"
        if q_h is not None:
            ref_q = orope.prepare_query(qin_h[qi], t, freq, s_h, b_h)
            assert np.all(np.abs(q_h[qi] - ref_q) <= _round_ref(ref_q, dtype)), f"token {qi}: query"
    assert set(changed.tolist()) <= written, "a row other than the new tokens' was written"


def test_rope_append_prefill_chunk(B):
    """A chunk of 300 new tokens of one sequence (consecutive positions;
    batches of 256 or more tokens take one workgroup per token)."""
    from oracle import rope as orope
    rng = np.random.default_rng(51)
    L, nq, first = 5000, 300, 4700
    freq = B.dsa_rope_frequencies()
    latent = rng.standard_normal((nq, 512)).astype(np.float32)
    rkey = rng.standard_normal((nq, 64)).astype(np.float32)
    qa = rng.standard_normal((nq, 64, 576)).astype(np.float32)
    s_h = (rng.standard_normal(64) * 0.1).astype(np.float32)
    b_h = (1 + rng.standard_normal(64) * 0.1).astype(np.float32)
    kv = torch.full((L, 576), 7.0, dtype=torch.bfloat16, device=DEV)
    q_in = torch.from_numpy(qa).to(DEV).to(torch.bfloat16)
    q_dev = q_in.clone()
    batch = B.Batch(torch.zeros(nq, dtype=torch.int32, device=DEV),
                    torch.arange(first, first + nq, dtype=torch.int32, device=DEV),
                    torch.tensor([L], dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int64, device=DEV), L)
    dv = lambda a: torch.from_numpy(a).to(DEV)
    B.dsa_rope_append(batch, dv(freq), dv(latent), dv(rkey), kv, q_dev, dv(s_h), dv(b_h))
    torch.cuda.synchronize()
    kv_h = kv.float().cpu().numpy()
    q_h = q_dev.float().cpu().numpy()
    qin_h = q_in.float().cpu().numpy()
    for qi in range(0, nq, 37):
        t = first + qi
        ref = orope.append_row(latent[qi], rkey[qi], t, freq)
        assert np.all(np.abs(kv_h[t] - ref) <= _round_ref(ref, "bf16")), f"token {qi}: cache row"
        ref_q = orope.prepare_query(qin_h[qi], t, freq, s_h, b_h)
        assert np.all(np.abs(q_h[qi] - ref_q) <= _round_ref(ref_q, "bf16")), f"token {qi}: query"
    assert np.all(kv_h[:first] == 7.0)


def test_empty_batch_is_noop(B):
    z = torch.zeros(0, dtype=torch.int32, device=DEV)
    batch = B.Batch(z, z, torch.ones(1, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int64, device=DEV), 1)
    scores = torch.empty((0, 1), device=DEV)
    B.dsa_index_score(batch, torch.empty((0, 32, 128), dtype=torch.bfloat16, device=DEV),
                      torch.empty((0, 32), device=DEV), torch.empty((1, 128), dtype=torch.bfloat16, device=DEV),
                      scores, ld=1)
    torch.cuda.synchronize()
