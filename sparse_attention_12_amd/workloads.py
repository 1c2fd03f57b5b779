"""Seeded synthetic inputs for the DSA indexer -> top-2,048 -> sparse MLA read.

This module holds no arithmetic of the method: it only draws arrays, stores
them in the requested precision and lays sequences out in the caches.  Both
the HIP path (tests, bench) and the CPU oracle (tests, bench CPU leg) take
their inputs from here.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):
  1. context lengths (ragged decode only),
  2. indexer queries qI [nq,32,128]: integers uniform in {-3..3},
  3. indexer head weights w [nq,32]: integers uniform in {1..4} (float32),
  4. indexer keys kI [rows,128]: integers uniform in {-3..3},
  5. per layer: MLA query q [nq,64,576] ~ N(0,1),
  6. per layer: cache rows kv [rows,576] ~ N(0,1) (512 latent then 64 rotary;
     with ``split_kv`` the latent block [rows,512] is drawn before the rotary
     block [rows,64] and the two are concatenated).
Normal draws are float32 and are rounded once to bf16 (round to nearest even)
when the workload is bf16; integer draws are exact in either precision.
Decode queries sit at the last position of their sequence.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

HI, DI, H, DC, DR, D = 32, 128, 64, 512, 64, 576
TOPK = 2048
TAU = 1.0 / math.sqrt(192.0)

# --------------------------------------------------------------------------
# bf16 storage helpers (format conversion only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        r = (c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = np.where(nan, (c >> np.uint32(16)) | np.uint32(0x40), r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _small_int_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Store small integers exactly as float32 or bf16 bits."""
    if dtype == "f32":
        return values.astype(np.float32)
    lut = f32_to_bf16_bits(np.arange(-128, 128, dtype=np.float32))
    return lut[values.astype(np.int16) + 128]


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "f32":
        return rng.standard_normal(n, dtype=np.float32).reshape(shape)
    out = np.empty(n, np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        m = min(step, n - s)
        out[s:s + m] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                 # "decode" or "prefill"
    dtype: str                # "f32" or "bf16" (storage of qI, kI, q, kv)
    n_layers: int
    seq_len: np.ndarray       # int32 [nseq]
    seq_row0: np.ndarray      # int64 [nseq]  first cache row of each sequence
    q_seq: np.ndarray         # int32 [nq]
    q_pos: np.ndarray         # int32 [nq]
    qI: np.ndarray            # [nq,32,128]  float32 or uint16 (bf16 bits)
    w: np.ndarray             # float32 [nq,32]
    kI: np.ndarray            # [rows,128]
    q: List[np.ndarray]       # per layer [nq,64,576]
    kv: List[np.ndarray]      # per layer [rows,576]
    k: int = TOPK
    tau: float = TAU
    seed: int = 0

    @property
    def nq(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def nseq(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def max_len(self) -> int:
        return int(self.seq_len.max()) if self.seq_len.size else 0

    @property
    def rows(self) -> int:
        return int(self.kI.shape[0])

    def widen(self, a: np.ndarray) -> np.ndarray:
        """float32 view of a stored array (exact for bf16)."""
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else np.ascontiguousarray(a, np.float32)

    def seq_rows(self, a: np.ndarray, s: int) -> np.ndarray:
        r0 = int(self.seq_row0[s])
        return a[r0:r0 + int(self.seq_len[s])]

    def to_torch(self, device):
        """Device tensors of every array (bf16 bits reinterpreted as torch.bfloat16)."""
        import torch

        def t(a):
            x = torch.from_numpy(np.ascontiguousarray(a))
            if a.dtype == np.uint16:
                x = x.view(torch.bfloat16)
            return x.to(device)

        return dict(
            seq_len=t(self.seq_len), seq_row0=t(self.seq_row0), q_seq=t(self.q_seq),
            q_pos=t(self.q_pos), qI=t(self.qI), w=t(self.w), kI=t(self.kI),
            q=[t(x) for x in self.q], kv=[t(x) for x in self.kv],
        )


def _layout(lens: np.ndarray):
    row0 = np.zeros(len(lens), np.int64)
    if len(lens) > 1:
        row0[1:] = np.cumsum(lens[:-1].astype(np.int64))
    return row0, int(np.sum(lens.astype(np.int64)))


def make_decode(lens, dtype: str = "bf16", n_layers: int = 1, seed: int = 0,
                name: Optional[str] = None, split_kv: bool = False,
                rng: Optional[np.random.Generator] = None) -> Workload:
    """Decode batch: one query per sequence, at its last position."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    nq = len(lens)
    row0, rows = _layout(lens)
    qI = _small_int_bits(rng.integers(-3, 4, size=(nq, HI, DI), dtype=np.int8), dtype)
    w = rng.integers(1, 5, size=(nq, HI), dtype=np.int8).astype(np.float32)
    kI = _small_int_bits(rng.integers(-3, 4, size=(rows, DI), dtype=np.int8), dtype)
    qs, kvs = [], []
    for _ in range(n_layers):
        qs.append(_normal(rng, (nq, H, D), dtype))
    for _ in range(n_layers):
        if split_kv:
            lat = _normal(rng, (rows, DC), dtype)
            rot = _normal(rng, (rows, DR), dtype)
            kvs.append(np.ascontiguousarray(np.concatenate([lat, rot], axis=1)))
        else:
            kvs.append(_normal(rng, (rows, D), dtype))
    return Workload(
        name=name or f"decode_b{nq}_{dtype}", kind="decode", dtype=dtype, n_layers=n_layers,
        seq_len=lens, seq_row0=row0, q_seq=np.arange(nq, dtype=np.int32),
        q_pos=(lens - 1).astype(np.int32), qI=qI, w=w, kI=kI, q=qs, kv=kvs, seed=seed)


def make_prefill(cache_len: int, first_pos: int, nq: int, dtype: str = "bf16",
                 seed: int = 0, name: Optional[str] = None) -> Workload:
    """Causal prefill chunk: nq consecutive queries of one sequence."""
    rng = np.random.default_rng(seed)
    lens = np.asarray([cache_len], np.int32)
    row0, rows = _layout(lens)
    qI = _small_int_bits(rng.integers(-3, 4, size=(nq, HI, DI), dtype=np.int8), dtype)
    w = rng.integers(1, 5, size=(nq, HI), dtype=np.int8).astype(np.float32)
    kI = _small_int_bits(rng.integers(-3, 4, size=(rows, DI), dtype=np.int8), dtype)
    q = _normal(rng, (nq, H, D), dtype)
    kv = _normal(rng, (rows, D), dtype)
    return Workload(
        name=name or f"prefill_{nq}q_{dtype}", kind="prefill", dtype=dtype, n_layers=1,
        seq_len=lens, seq_row0=row0, q_seq=np.zeros(nq, np.int32),
        q_pos=(first_pos + np.arange(nq)).astype(np.int32), qI=qI, w=w, kI=kI,
        q=[q], kv=[kv], seed=seed)


def ragged_lengths(rng: np.random.Generator, b: int, lo: int, hi: int, forced=(1024, 2048, 2049)):
    """Context lengths for the ragged decode batch.

    The first entries are forced to sit at, just below and just above the
    2,048-position selection size (so that the dense special case is always
    present); the rest are uniform integers in [lo, hi].
    """
    forced = [int(x) for x in forced][:b]
    rest = rng.integers(lo, hi + 1, size=b - len(forced)).astype(np.int32)
    return np.concatenate([np.asarray(forced, np.int32), rest])


# --------------------------------------------------------------------------
# the five workloads the path is measured and checked on
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "decode_b1_L4096_f32",
    1: "decode_b64_L32768_bf16",
    2: "ragged_decode_b16_L1024-131072_bf16_4layers_shared_selection",
    3: "causal_prefill_2048q_pos63488-65535_cache65536_bf16",
    4: "decode_b4_L1048576_bf16",
}


def config(i: int) -> Workload:
    seed = 1000 + i
    name = CONFIG_NAMES[i]
    if i == 0:
        return make_decode([4096], "f32", 1, seed, name, split_kv=True)
    if i == 1:
        return make_decode([32768] * 64, "bf16", 1, seed, name)
    if i == 2:
        rng = np.random.default_rng(seed)
        lens = ragged_lengths(rng, 16, 1024, 131072)
        return make_decode(lens, "bf16", 4, seed, name, rng=rng)
    if i == 3:
        return make_prefill(65536, 63488, 2048, "bf16", seed, name)
    if i == 4:
        return make_decode([1 << 20] * 4, "bf16", 1, seed, name)
    raise KeyError(i)
