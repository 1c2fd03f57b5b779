"""Seeded synthetic inputs for the DSA indexer -> top-2,048 -> sparse MLA read.

This module holds no arithmetic of the method: it only draws arrays, stores
them in the requested precision and lays sequences out in the caches.  Both
the HIP path (tests, bench) and the CPU oracle (tests, bench CPU leg) take
their inputs from here.

Recipe.  A workload's draws come from one ``Draws`` stream seeded with the
workload's seed: every array takes the next child of a
``numpy.random.SeedSequence``, in this order:
  1. context lengths (ragged decode only),
  2. indexer queries qI [nq,32,128]: integers uniform in {-3..3},
  3. indexer head weights w [nq,32]: integers uniform in {1..4} (float32),
  4. indexer keys kI [rows,128]: integers uniform in {-3..3},
  5. per layer: MLA query q [nq,64,576] ~ N(0,1),
  6. per layer: cache rows kv [rows,576] ~ N(0,1) (512 latent then 64 rotary;
     with ``split_kv`` the latent block [rows,512] is drawn before the rotary
     block [rows,64] and the two are concatenated).
An array is drawn in blocks of 2^22 elements, block b from the b-th child of
the array's seed, on a pool of threads; the values do not depend on the
number of threads.  Normal draws are float32 and are rounded once to bf16
(round to nearest even) when the workload is bf16; integer draws are exact in
either precision and also in FP8 E4M3, in which the indexer's qI and kI may
be stored (``index_dtype="fp8"``, as uint8 bit patterns).  Decode queries sit
at the last position of their sequence.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
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


# --------------------------------------------------------------------------
# FP8 E4M3 storage helpers (OCP 8-bit floating point, E4M3: exponent bias 7,
# no infinities, S.1111.111 is NaN, largest finite 448; format conversion only)
# --------------------------------------------------------------------------


def _e4m3_table() -> np.ndarray:
    b = np.arange(256, dtype=np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = sign * mag
    v[(b & 0x7F) == 0x7F] = np.nan
    return v.astype(np.float32)


E4M3_VALUES = _e4m3_table()


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen E4M3 bit patterns (uint8) to float32 exactly."""
    return E4M3_VALUES[np.ascontiguousarray(b, dtype=np.uint8)]


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to E4M3 (nearest, ties to even; magnitudes above 448
    saturate to 448, NaN gives 0x7F); returns uint8 bit patterns."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), 448.0)
    # quantum of the binade of a (subnormals share the quantum 2^-9)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    q = np.exp2(e - 3.0)
    r = np.round(a / q) * q                      # numpy rounds half to even
    r = np.minimum(r, 448.0)
    _, ex = np.frexp(r)
    e = ex - 1
    normal = r >= 2.0 ** -6
    field_e = np.where(normal, e + 7, 0)
    field_m = np.where(normal, r / np.exp2(np.where(normal, e, 0)) * 8.0 - 8.0, r * 512.0)
    bits = (field_e.astype(np.int64) << 3) | np.rint(field_m).astype(np.int64)
    bits = np.where(neg, bits | 0x80, bits)
    bits = np.where(nan, 0x7F, bits)
    return bits.astype(np.uint8)


def _small_int_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Store small integers exactly as float32, bf16 bits or E4M3 bits."""
    if dtype == "f32":
        return values.astype(np.float32)
    if dtype == "fp8":
        assert int(np.abs(values).max(initial=0)) <= 16, "integers above 16 are not exact in E4M3"
        lut = f32_to_e4m3_bits(np.arange(-128, 128, dtype=np.float32))
    else:
        lut = f32_to_bf16_bits(np.arange(-128, 128, dtype=np.float32))
    return lut[values.astype(np.int16) + 128]


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------

BLOCK = 1 << 22
_POOL = None


def _pool() -> cf.ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


class Draws:
    """A seeded stream of arrays.  Each call takes the next child of the
    stream's SeedSequence; the array is filled in blocks of BLOCK elements,
    block b from the b-th child of that seed, in parallel."""

    def __init__(self, seed: int):
        self._ss = np.random.SeedSequence(int(seed))

    def _fill(self, n: int, out: np.ndarray, draw) -> None:
        seeds = self._ss.spawn(1)[0].spawn(max(1, -(-n // BLOCK)))

        def one(b):
            lo = b * BLOCK
            hi = min(n, lo + BLOCK)
            if hi > lo:
                draw(np.random.default_rng(seeds[b]), out[lo:hi])

        list(_pool().map(one, range(len(seeds))))

    def integers(self, lo: int, hi: int, shape, dtype=np.int8) -> np.ndarray:
        """Integers uniform in [lo, hi) (int8 unless dtype says otherwise)."""
        n = int(np.prod(shape))
        out = np.empty(n, dtype)
        self._fill(n, out, lambda g, o: o.__setitem__(slice(None), g.integers(lo, hi, size=o.size, dtype=dtype)))
        return out.reshape(shape)

    def normal(self, shape, dtype: str) -> np.ndarray:
        """N(0,1) float32 draws; for dtype "bf16" rounded once to bf16 bits."""
        n = int(np.prod(shape))
        if dtype == "f32":
            out = np.empty(n, np.float32)
            self._fill(n, out, lambda g, o: g.standard_normal(size=o.size, dtype=np.float32, out=o))
        else:
            out = np.empty(n, np.uint16)
            self._fill(n, out, lambda g, o: o.__setitem__(
                slice(None), f32_to_bf16_bits(g.standard_normal(size=o.size, dtype=np.float32))))
        return out.reshape(shape)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                 # "decode" or "prefill"
    dtype: str                # "f32" or "bf16" (storage of q, kv; and of qI, kI
                              # unless index_dtype says otherwise)
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
    index_dtype: str = ""     # storage of qI, kI: "f32", "bf16" or "fp8" ("" = dtype)

    def __post_init__(self):
        if not self.index_dtype:
            self.index_dtype = self.dtype

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
        """float32 view of a stored array (exact for bf16 and E4M3 bits)."""
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        if a.dtype == np.uint8:
            return e4m3_bits_to_f32(a)
        return np.ascontiguousarray(a, np.float32)

    def seq_rows(self, a: np.ndarray, s: int) -> np.ndarray:
        r0 = int(self.seq_row0[s])
        return a[r0:r0 + int(self.seq_len[s])]

    def to_torch(self, device):
        """Device tensors of every array (bf16 bits reinterpreted as torch.bfloat16;
        E4M3 bits stay torch.uint8, which the binding passes as FP8 E4M3)."""
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
                draws: Optional[Draws] = None,
                index_dtype: Optional[str] = None, rope_dim: int = DR) -> Workload:
    """Decode batch: one query per sequence, at its last position.  With
    rope_dim=0 the layers have no rotary part: q [nq,64,512], kv [rows,512]."""
    dr = draws if draws is not None else Draws(seed)
    idt = index_dtype or dtype
    lens = np.asarray(lens, np.int32)
    nq = len(lens)
    row0, rows = _layout(lens)
    qI = _small_int_bits(dr.integers(-3, 4, (nq, HI, DI)), idt)
    w = dr.integers(1, 5, (nq, HI)).astype(np.float32)
    kI = _small_int_bits(dr.integers(-3, 4, (rows, DI)), idt)
    width = DC + rope_dim
    qs, kvs = [], []
    for _ in range(n_layers):
        qs.append(dr.normal((nq, H, width), dtype))
    for _ in range(n_layers):
        if split_kv and rope_dim:
            lat = dr.normal((rows, DC), dtype)
            rot = dr.normal((rows, rope_dim), dtype)
            kvs.append(np.ascontiguousarray(np.concatenate([lat, rot], axis=1)))
        else:
            kvs.append(dr.normal((rows, width), dtype))
    return Workload(
        name=name or f"decode_b{nq}_{dtype}", kind="decode", dtype=dtype, n_layers=n_layers,
        seq_len=lens, seq_row0=row0, q_seq=np.arange(nq, dtype=np.int32),
        q_pos=(lens - 1).astype(np.int32), qI=qI, w=w, kI=kI, q=qs, kv=kvs, seed=seed,
        index_dtype=idt)


def make_prefill(cache_len: int, first_pos: int, nq: int, dtype: str = "bf16",
                 seed: int = 0, name: Optional[str] = None,
                 index_dtype: Optional[str] = None) -> Workload:
    """Causal prefill chunk: nq consecutive queries of one sequence."""
    dr = Draws(seed)
    idt = index_dtype or dtype
    lens = np.asarray([cache_len], np.int32)
    row0, rows = _layout(lens)
    qI = _small_int_bits(dr.integers(-3, 4, (nq, HI, DI)), idt)
    w = dr.integers(1, 5, (nq, HI)).astype(np.float32)
    kI = _small_int_bits(dr.integers(-3, 4, (rows, DI)), idt)
    q = dr.normal((nq, H, D), dtype)
    kv = dr.normal((rows, D), dtype)
    return Workload(
        name=name or f"prefill_{nq}q_{dtype}", kind="prefill", dtype=dtype, n_layers=1,
        seq_len=lens, seq_row0=row0, q_seq=np.zeros(nq, np.int32),
        q_pos=(first_pos + np.arange(nq)).astype(np.int32), qI=qI, w=w, kI=kI,
        q=[q], kv=[kv], seed=seed, index_dtype=idt)


@dataclasses.dataclass
class LayerStack:
    """Inputs of a decode step over a stack of layers under a schedule
    (plan: list of (runs_indexer, rope, kv_source)).  Arrays a layer does not
    own are None: indexer inputs of reusing layers, caches of layers that
    read another layer's cache."""
    base: Workload            # batch layout (lengths, rows, positions); its own arrays unused
    plan: list
    qI: List[Optional[np.ndarray]]
    w: List[Optional[np.ndarray]]
    kI: List[Optional[np.ndarray]]
    q: List[np.ndarray]
    kv: List[Optional[np.ndarray]]

    def to_torch(self, device):
        import torch

        def t(a):
            if a is None:
                return None
            x = torch.from_numpy(np.ascontiguousarray(a))
            if a.dtype == np.uint16:
                x = x.view(torch.bfloat16)
            return x.to(device)

        return dict(qI=[t(a) for a in self.qI], w=[t(a) for a in self.w], kI=[t(a) for a in self.kI],
                    q=[t(a) for a in self.q], kv=[t(a) for a in self.kv])


def make_layer_stack(lens, plan, dtype: str = "bf16", seed: int = 0,
                     index_dtype: Optional[str] = None) -> LayerStack:
    """Decode batch over the layers of `plan`: per layer, in layer order,
    the indexer inputs (qI, w, kI) if it runs its indexer, its query (512 +
    64 wide, or 512 without rotary part), its cache if it owns one."""
    dr = Draws(seed)
    idt = index_dtype or dtype
    base = make_decode(lens, dtype, 0, seed, "layer_stack", draws=Draws(seed + 1), index_dtype=idt)
    nq, rows = base.nq, base.rows
    qI, w, kI, q, kv = [], [], [], [], []
    for l, (runs, rope, src) in enumerate(plan):
        width = DC + (DR if rope else 0)
        if runs:
            qI.append(_small_int_bits(dr.integers(-3, 4, (nq, HI, DI)), idt))
            w.append(dr.integers(1, 5, (nq, HI)).astype(np.float32))
            kI.append(_small_int_bits(dr.integers(-3, 4, (rows, DI)), idt))
        else:
            qI.append(None)
            w.append(None)
            kI.append(None)
        q.append(dr.normal((nq, H, width), dtype))
        kv.append(dr.normal((rows, width), dtype) if src == l else None)
    return LayerStack(base=base, plan=list(plan), qI=qI, w=w, kI=kI, q=q, kv=kv)


def ragged_lengths(draws: Draws, b: int, lo: int, hi: int, forced=(1024, 2048, 2049)):
    """Context lengths for the ragged decode batch.

    The first entries are forced to sit at, just below and just above the
    2,048-position selection size (so that the dense special case is always
    present); the rest are uniform integers in [lo, hi].
    """
    forced = [int(x) for x in forced][:b]
    rest = draws.integers(lo, hi + 1, (b - len(forced),), np.int32)
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


def config(i: int, index_dtype: Optional[str] = None) -> Workload:
    """Workload i; index_dtype="fp8" stores its indexer inputs in E4M3 (the
    same integer draws, so scores and selections are unchanged)."""
    seed = 1000 + i
    name = CONFIG_NAMES[i]
    if index_dtype == "fp8":
        name = name + "_fp8index"
    if i == 0:
        return make_decode([4096], "f32", 1, seed, name, split_kv=True, index_dtype=index_dtype)
    if i == 1:
        return make_decode([32768] * 64, "bf16", 1, seed, name, index_dtype=index_dtype)
    if i == 2:
        dr = Draws(seed)
        lens = ragged_lengths(dr, 16, 1024, 131072)
        return make_decode(lens, "bf16", 4, seed, name, draws=dr, index_dtype=index_dtype)
    if i == 3:
        return make_prefill(65536, 63488, 2048, "bf16", seed, name, index_dtype=index_dtype)
    if i == 4:
        return make_decode([1 << 20] * 4, "bf16", 1, seed, name, index_dtype=index_dtype)
    raise KeyError(i)
