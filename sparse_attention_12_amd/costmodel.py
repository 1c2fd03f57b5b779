"""Cache and work arithmetic of the attention read, and the algorithmic
bytes/FLOP the benchmark divides by.

Two parts:

1. The model-wide arithmetic printed on the "Mistral Large 4" concept page
   (sections "Cache", "Sparse attention", "When does sparse attention pay?"
   and the 1M-token serving scenario), rebuilt from the layer rules the page
   states in its list of changes to the DeepSeek recipe:
     * every fourth layer (0-based layers 3, 7, 11, ...) has no rotary
       encoding (NoPE);
     * from layer 39 on, those NoPE layers read layer 35's latent instead of
       writing their own;
     * 28 of the 72 layers reuse the selection of the most recent layer that
       ran its indexer.  Which 28: the illustrated summary's DSA paragraph
       says that from layer 16 on the former sliding-window layers of each
       original four-layer group share one indexer, so in every group
       (16-19, 20-23, ...) the first layer runs it, the next two reuse it and
       the NoPE layer runs its own.
   The figures are counted from a census of layer kinds (rotary or not,
   owning its cache or not, running its indexer or not).  The tests pin
   every printed figure (35,712 values; 74.9 GB; 33x; 4.94e6 and 1.80e5
   multiply-adds; ~56,000 tokens; 3.5x/19x/26x; ~4%; 39%; 5.9 GB; 95%;
   ~1e17).

2. Per-workload algorithmic traffic of this library's hot path: bytes that
   must cross HBM at least once (inputs read once, final outputs written
   once) and the FLOP of the two contractions, with the per-position unit
   costs of the "Sparse attention" section: 32 x 128 multiply-adds per scored
   position and 64 x (512 + 64 + 512) per attended position.
"""
from __future__ import annotations

import collections
import functools

import numpy as np

LAYERS = 72
HEADS = 64
LATENT = 512
ROPE = 64
INDEXER_HEADS = 32
INDEXER_DIM = 128
TOPK = 2048
FIRST_SHARED_INDEXER_LAYER = 16
YOCO_SOURCE = 35


# Three facts describe a layer: whether it has rotary encoding, whose latent
# it reads, and whether it runs its own indexer.


def is_rope_layer(l: int) -> bool:
    """Layers 3, 7, 11, ... (every fourth, counting from one) are NoPE."""
    return l % 4 != 3


def kv_source(l: int) -> int:
    """The NoPE layers that come after layer 35 read its latent."""
    return YOCO_SOURCE if (not is_rope_layer(l) and l > YOCO_SOURCE) else l


def runs_indexer(l: int) -> bool:
    if l < FIRST_SHARED_INDEXER_LAYER:
        return True
    return (l - FIRST_SHARED_INDEXER_LAYER) % 4 in (0, 3)


@functools.lru_cache(maxsize=None)
def _census():
    """Number of layers of each kind (rotary, owns its cache, runs its indexer)."""
    return collections.Counter((is_rope_layer(l), kv_source(l) == l, runs_indexer(l)) for l in range(LAYERS))


def _layers(rope=None, owns=None, indexer=None) -> int:
    """Layers of the kinds that match every given fact."""
    return sum(n for (r, o, i), n in _census().items()
               if (rope is None or r == rope) and (owns is None or o == owns) and (indexer is None or i == indexer))


def row_values(rope: bool) -> int:
    """Values one position adds to a cache: the latent, plus the rotary key
    in a rotary layer."""
    return LATENT + (ROPE if rope else 0)


def indexer_layers() -> int:
    return _layers(indexer=True)


def cached_values_per_position() -> int:
    """Latent (+ rotary key) values stored per position across the model:
    one row per layer that owns its cache."""
    return sum(_layers(rope=r, owns=True) * row_values(r) for r in (True, False))


def values_saved_by_cache_sharing() -> int:
    """Values the layers that read another layer's cache would add."""
    return sum(_layers(rope=r, owns=False) * row_values(r) for r in (True, False))


def full_kv_values_per_position(head_k: int = 128, head_v: int = 128) -> int:
    return LAYERS * HEADS * (head_k + head_v)


def latent_cache_bytes(positions: int, bytes_per_value: int = 2) -> int:
    return cached_values_per_position() * bytes_per_value * positions


def attend_macs_per_position() -> int:
    """Model-wide multiply-adds per attended position: in each layer every
    head dots its query with the row (latent plus rotary key, if any) and
    adds the 512-value latent to its output."""
    return sum(_layers(rope=r) * HEADS * (row_values(r) + LATENT) for r in (True, False))


def score_macs_per_position() -> int:
    """Model-wide multiply-adds per scored position (indexer layers only)."""
    return indexer_layers() * INDEXER_HEADS * INDEXER_DIM


def dense_macs(t: int) -> int:
    """Dense MLA for one new token at context t: every position attended."""
    return attend_macs_per_position() * t


def sparse_macs(t: int) -> int:
    """The sparse read: at most TOPK attended positions, all t scored."""
    return attend_macs_per_position() * min(t, TOPK) + score_macs_per_position() * t


def indexer_crossover_tokens() -> float:
    """Context at which scoring t positions costs as much as attending TOPK."""
    return TOPK * attend_macs_per_position() / score_macs_per_position()


def sparse_gain(t: int) -> float:
    return dense_macs(t) / sparse_macs(t)


def short_prompt_overhead() -> float:
    """Extra work of the indexer when every position is attended anyway."""
    return score_macs_per_position() / attend_macs_per_position()


def selection_reuse_saving() -> float:
    return _layers(indexer=False) / LAYERS


def fp8_indexer_key_bytes(positions: int) -> int:
    return indexer_layers() * INDEXER_DIM * 1 * positions


def indexer_share(t: int) -> float:
    return score_macs_per_position() * t / sparse_macs(t)


def prefill_scoring_macs(t: int) -> float:
    return score_macs_per_position() * t * t / 2


# --------------------------------------------------------------------------
# per-workload algorithmic traffic of the hot path (one layer's read)
# --------------------------------------------------------------------------

SCORE_MACS = INDEXER_HEADS * INDEXER_DIM                # 4,096 per scored position
ATTEND_MACS = HEADS * (LATENT + ROPE + LATENT)          # 69,632 per attended position


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[dtype]


def path_traffic(seq_len, q_seq, q_pos, dtype: str, n_layers: int = 1, k: int = TOPK,
                 out_bytes: int = 4, index_dtype: str = "") -> dict:
    """Algorithmic bytes and FLOP of one pass of the read over a batch.

    dtype is the storage of the attention query and cache rows; index_dtype
    that of the indexer's query and keys ("" = dtype).

    Candidates of a query: its own position and every earlier one within the
    cache, n = min(q_pos + 1, seq_len).  Key rows and cache rows are counted
    once per sequence (the most any of its queries touches); scores, indices
    and split partials are intermediates and are reported apart.
    """
    seq_len = np.asarray(seq_len, np.int64)
    q_seq = np.asarray(q_seq, np.int64)
    q_pos = np.asarray(q_pos, np.int64)
    es = elem_bytes(dtype)
    ei = elem_bytes(index_dtype or dtype)
    nq = int(q_seq.shape[0])
    n_cand = np.maximum(0, np.minimum(q_pos + 1, seq_len[q_seq]))
    n_sel = np.minimum(n_cand, k)
    # unique rows each sequence exposes to its queries
    key_rows = np.zeros(seq_len.shape[0], np.int64)
    np.maximum.at(key_rows, q_seq, n_cand)
    row_d = LATENT + ROPE
    idx_q_bytes = nq * (INDEXER_HEADS * INDEXER_DIM * ei + INDEXER_HEADS * 4)
    indexer = dict(
        key_bytes=int(key_rows.sum()) * INDEXER_DIM * ei,
        q_bytes=idx_q_bytes,
        score_bytes=int(n_cand.sum()) * 4,
        flop=2 * SCORE_MACS * int(n_cand.sum()),
        positions=int(n_cand.sum()),
    )
    indexer["bytes"] = indexer["key_bytes"] + indexer["q_bytes"] + indexer["score_bytes"]
    topk = dict(bytes=int(n_cand.sum()) * 4 + nq * k * 4 + nq * 4)
    # unique cache rows a layer's read may touch: at most the selected rows
    # of each query, bounded by the sequence's candidates
    uniq_rows = 0
    for s in range(seq_len.shape[0]):
        mask = q_seq == s
        if mask.any():
            uniq_rows += min(int(n_sel[mask].sum()), int(key_rows[s]))
    mla_layer = dict(
        row_bytes_logical=int(n_sel.sum()) * row_d * es,
        row_bytes_unique=uniq_rows * row_d * es,
        q_bytes=nq * HEADS * row_d * es,
        out_bytes=nq * HEADS * (LATENT * out_bytes + 4),
        flop=2 * ATTEND_MACS * int(n_sel.sum()),
        positions=int(n_sel.sum()),
    )
    mla_layer["bytes"] = (mla_layer["row_bytes_unique"] + mla_layer["q_bytes"]
                          + mla_layer["out_bytes"])
    total_bytes = (indexer["key_bytes"] + indexer["q_bytes"]
                   + n_layers * mla_layer["bytes"])
    return dict(nq=nq, n_layers=n_layers, indexer=indexer, topk=topk, mla_layer=mla_layer,
                path_bytes=total_bytes,
                path_flop=indexer["flop"] + n_layers * mla_layer["flop"],
                intermediate_bytes=indexer["score_bytes"] + topk["bytes"])
