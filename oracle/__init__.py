"""Plain CPU oracle of the DSA indexer -> top-2,048 -> sparse MLA read.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library
(``sparse_attention_12_amd``) never imports this package, and this package
imports nothing from it.

Arithmetic lives in ``dsa_oracle.c`` (IEEE double, one plain loop per sum in
the definitions); this module only marshals numpy arrays.  The definitions
follow the "Mistral Large 4" concept page, sections "What to keep", "Where to
look" and "Sparse attention"; the readings taken where that page lost its
display formula are stated in the C file's header.

The step just upstream of the read (rotary encoding with YaRN/LeRoPE
frequencies, per-head query scaling, cache append) is in ``oracle/rope.py``,
plain numpy in float64, pinned in tests/test_oracle_rope.py.

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself: a rank-count brute force for the selection, an ReLU sign identity
for the indexer, a library dense-attention routine for contexts of at most
2,048 positions, the page's closed form for the weight of a key that leads
by a logit gap, and the uniform-query mean.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

HI, DI, H, DC, DR, D = 32, 128, 64, 512, 64, 576

_lib = None


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c with gcc (-O2, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC,
               "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_index_score.argtypes = [f32p, f32p, f32p, ctypes.c_int64, f64p]
        lib.oracle_index_score.restype = None
        lib.oracle_topk.argtypes = [f64p, ctypes.c_int64, ctypes.c_int64, i32p]
        lib.oracle_topk.restype = ctypes.c_int64
        lib.oracle_mla_attend.argtypes = [f32p, f32p, i32p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_double, f64p, f64p]
        lib.oracle_mla_attend.restype = None
        lib.oracle_dims.argtypes = [i32p]
        lib.oracle_dims.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle expects float32 inputs (bf16 widened exactly), got {a.dtype}")
    return np.ascontiguousarray(a)


def dims() -> tuple:
    out = np.zeros(6, np.int32)
    _load().oracle_dims(_ptr(out, ctypes.c_int32))
    return tuple(int(x) for x in out)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads of the following oracle calls (timing only)."""
    _load().oracle_set_threads(int(n))


def index_score(qI, w, kI) -> np.ndarray:
    """Indexer scores of one query: qI [32,128], w [32], kI [n,128] -> float64 [n]."""
    qI, w, kI = _f32(qI), _f32(w), _f32(kI)
    assert qI.shape == (HI, DI) and w.shape == (HI,) and kI.ndim == 2 and kI.shape[1] == DI
    n = kI.shape[0]
    out = np.empty(n, np.float64)
    _load().oracle_index_score(_ptr(qI, ctypes.c_float), _ptr(w, ctypes.c_float),
                               _ptr(kI, ctypes.c_float), n, _ptr(out, ctypes.c_double))
    return out


def topk(scores, k: int):
    """Top-k of one score row: (idx int32 [k] ascending, -1 padded; count m)."""
    scores = np.ascontiguousarray(np.asarray(scores, np.float64))
    idx = np.empty(max(k, 1), np.int32)
    m = _load().oracle_topk(_ptr(scores, ctypes.c_double), scores.shape[0], k,
                            _ptr(idx, ctypes.c_int32))
    if m < 0:
        raise ValueError("oracle_topk: non-finite score or invalid argument")
    return idx[:k].copy(), int(m)


def mla_attend(q, kv, sel, tau: float):
    """Sparse MLA of one query: q [64,W], kv [rows,W], sel int32 [m] -> (o [64,512], lse [64]).

    W = 576 (512 latent + 64 rotary) or 512 for a layer without rotary
    encoding (every fourth layer on the concept page keeps the latent alone).
    """
    q, kv = _f32(q), _f32(kv)
    sel = np.ascontiguousarray(np.asarray(sel, np.int32))
    width = q.shape[-1]
    assert width in (D, DC) and q.shape == (H, width) and kv.ndim == 2 and kv.shape[1] == width
    if sel.size and sel.max() >= kv.shape[0]:
        raise IndexError("selected position outside the cache rows")
    o = np.empty((H, DC), np.float64)
    lse = np.empty(H, np.float64)
    _load().oracle_mla_attend(_ptr(q, ctypes.c_float), _ptr(kv, ctypes.c_float),
                              _ptr(sel, ctypes.c_int32), sel.shape[0], width - DC, float(tau),
                              _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, lse


def n_candidates(q_pos: int, seq_len: int) -> int:
    """Positions a query may select: its own and every earlier one, within the cache."""
    return max(0, min(int(q_pos) + 1, int(seq_len)))


def select_query(qI, w, kI_seq, n_cand: int, k: int):
    """Indexer scores over the first n_cand rows of a sequence, then top-k."""
    scores = index_score(qI, w, kI_seq[:n_cand])
    idx, m = topk(scores, k)
    return scores, idx, m


def decode_query(qI, w, kI_seq, q_layers, kv_layers, n_cand: int, k: int, tau: float):
    """One query through the whole read: one selection shared by every layer.

    q_layers: list of [64,576]; kv_layers: list of the sequence's [rows,576]
    caches (selection sharing, "Where to look" list on the concept page: a
    layer may reuse the selection of the most recent layer that ran its
    indexer).  Returns (idx, m, [o], [lse]).
    """
    _, idx, m = select_query(qI, w, kI_seq, n_cand, k)
    outs, lses = [], []
    for q, kv in zip(q_layers, kv_layers):
        o, lse = mla_attend(q, kv, idx[:m], tau)
        outs.append(o)
        lses.append(lse)
    return idx, m, outs, lses


# ----------------------------------------------------------------------------
# The model's layer schedule and one decode step over it
# ----------------------------------------------------------------------------

LAYERS = 72


def layer_plan(n_layers: int = LAYERS):
    """Per layer l < n_layers: (runs_indexer, rope, kv_source).

    Rules of the concept page's list of changes to the DeepSeek recipe,
    applied to the model's 18 groups of four consecutive layers:
      * every fourth layer has no rotary encoding: the last layer of each
        group (layers 3, 7, 11, ...);
      * from layer 39 on, those layers read layer 35's latent instead of
        keeping their own: the rotary-free layers of the groups after the
        one that ends at layer 35 (every layer that shares a cache is
        rotary-free, and so is layer 35);
      * 28 layers reuse the selection of the most recent layer that ran its
        indexer.  Which ones (reading of the summary page's DSA paragraph):
        in the groups from layer 16 on, the two middle layers reuse the
        selection of the group's first layer, and the first and last run
        their own indexer.
    """
    plan = []
    source_group = 35 // 4
    for g in range((n_layers + 3) // 4):
        for j in range(4):
            l = 4 * g + j
            if l >= n_layers:
                break
            rotary = j != 3
            reuses = g >= 4 and j in (1, 2)
            kv_source = 35 if (not rotary and g > source_group) else l
            plan.append((not reuses, rotary, kv_source))
    return plan


def decode_layers(plan, qI_l, w_l, kI_l, q_l, kv_l, n_cand: int, k: int, tau: float):
    """One query through the attention read of every layer of `plan`.

    A layer that runs its indexer selects from its own indexer query, head
    weights and keys (qI_l[l] [32,128], w_l[l] [32], kI_l[l] [rows,128]); a
    layer that reuses takes the selection of the most recent layer that ran
    its indexer.  Layer l attends with its query q_l[l] ([64,576], or
    [64,512] without rotary encoding) over the cache of layer
    plan[l].kv_source (kv_l[source] [rows,576 or 512]).
    Returns ([idx of each layer], [o], [lse]).
    """
    idx_l, outs, lses = [], [], []
    idx = m = None
    for l, (runs, rope, src) in enumerate(plan):
        if runs:
            _, idx, m = select_query(qI_l[l], w_l[l], kI_l[l], n_cand, k)
        if idx is None:
            raise ValueError("the first layer must run its indexer")
        o, lse = mla_attend(q_l[l], kv_l[src], idx[:m], tau)
        idx_l.append(idx)
        outs.append(o)
        lses.append(lse)
    return idx_l, outs, lses

