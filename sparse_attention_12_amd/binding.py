"""Thin ctypes binding of libdsa_mla.so (C ABI in include/dsa_mla.h).

Argument marshalling only: torch tensors are passed as device pointers on the
caller's current stream; every step of the read runs in the HIP kernels.
There is no fallback: if the library is missing or fails to load, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_mla.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
INDEX_HEADS, INDEX_DIM, HEADS, LATENT, ROPE, ROW, TOPK_MAX = 32, 128, 64, 512, 64, 576, 2048

EXPORTS = [
    "dsa_abi_version", "dsa_status_string", "dsa_last_error", "dsa_index_score",
    "dsa_topk_workspace_size", "dsa_topk", "mla_sparse_attend_workspace_size",
    "mla_sparse_attend", "dsa_mla_decode_fused_workspace_size", "dsa_mla_decode_fused",
    "dsa_ml4_layer_plan", "dsa_mla_decode_layers_workspace_size", "dsa_mla_decode_layers",
    "dsa_rope_frequencies", "dsa_rope_append", "dsa_mla_decode_fused_noalloc", "dsa_debug_flags",
]
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_mla_debug.so")
DEBUG_BITS = {"idx_range": 1, "topk_slot": 2, "list": 4, "score_col": 8, "hist_recount": 16, "gather_row": 32}
NOALLOC_SCRATCH_BYTES = 128 << 20
ML4_LAYERS = 72


class LayerPlan(ctypes.Structure):
    """One layer of a schedule: whether it runs its indexer, its rotary
    width (64 or 0) and the layer whose cache it reads."""
    _fields_ = [("runs_indexer", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("kv_source", ctypes.c_int32)]


class DsaBatch(ctypes.Structure):
    _fields_ = [
        ("nq", ctypes.c_int32), ("nseq", ctypes.c_int32), ("max_len", ctypes.c_int32),
        ("q_seq", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p), ("seq_row0", ctypes.c_void_p),
    ]


def _load(path: str = None) -> ctypes.CDLL:
    """The library at path (default: the release build), its prototypes set."""
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    bp = ctypes.POINTER(DsaBatch)
    lib.dsa_abi_version.restype = i32
    lib.dsa_status_string.argtypes = [i32]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_score.argtypes = [bp, i32, vp, vp, vp, vp, i64, vp]
    lib.dsa_index_score.restype = i32
    lib.dsa_topk_workspace_size.argtypes = [i32, i32, i32]
    lib.dsa_topk_workspace_size.restype = sz
    lib.dsa_topk.argtypes = [bp, vp, i64, i32, vp, vp, vp, sz, vp]
    lib.dsa_topk.restype = i32
    lib.mla_sparse_attend_workspace_size.argtypes = [i32, i32, i32]
    lib.mla_sparse_attend_workspace_size.restype = sz
    lib.mla_sparse_attend.argtypes = [bp, i32, i32, vp, vp, vp, i32, ctypes.c_float, vp, i32, vp, vp, sz, vp]
    lib.mla_sparse_attend.restype = i32
    lib.dsa_mla_decode_fused_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_mla_decode_fused_workspace_size.restype = sz
    lib.dsa_mla_decode_fused.argtypes = [bp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, i32,
                                         ctypes.c_float, vp, vp, sz, vp]
    lib.dsa_mla_decode_fused.restype = i32
    lib.dsa_mla_decode_fused_noalloc.argtypes = [bp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, i32,
                                                 ctypes.c_float, vp, vp]
    lib.dsa_mla_decode_fused_noalloc.restype = i32
    pp = ctypes.POINTER(LayerPlan)
    lib.dsa_ml4_layer_plan.argtypes = [i32, pp]
    lib.dsa_ml4_layer_plan.restype = i32
    lib.dsa_mla_decode_layers_workspace_size.argtypes = [i32, i32, i32, i32, pp]
    lib.dsa_mla_decode_layers_workspace_size.restype = sz
    lib.dsa_mla_decode_layers.argtypes = [bp, i32, pp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, i32,
                                          ctypes.c_float, vp, vp, sz, vp]
    lib.dsa_mla_decode_layers.restype = i32
    lib.dsa_rope_frequencies.argtypes = [vp, vp]
    lib.dsa_rope_frequencies.restype = i32
    lib.dsa_rope_append.argtypes = [bp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dsa_rope_append.restype = i32
    lib.dsa_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    lib.dsa_debug_flags.restype = i32
    return lib


lib = _load()


def load_debug_library() -> ctypes.CDLL:
    """The debug build (kernel checks compiled in), with the same prototypes.
    Calls go to it while it is assigned to this module's `lib`."""
    return _load(DEBUG_LIB_PATH)


def debug_flags(reset: bool = True, library=None) -> int:
    """Union of the debug checks' bits set since the last reset (DEBUG_BITS);
    waits for the device.  Raises DsaError on a release build."""
    L = library or lib
    v = ctypes.c_uint32(0)
    st = L.dsa_debug_flags(ctypes.byref(v), 1 if reset else 0)
    if st != 0:
        raise DsaError(st, "dsa_debug_flags")
    return int(v.value)


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.dsa_last_error().decode() or lib.dsa_status_string(status).decode()
        super().__init__(f"{where}: {lib.dsa_status_string(status).decode()} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise DsaError(status, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_FP8_TYPES = tuple(getattr(torch, n) for n in ("float8_e4m3fn",) if hasattr(torch, n))


def _dt(t: torch.Tensor) -> int:
    """Library dtype code of a tensor.  FP8 E4M3 (OCP) inputs of the indexer
    may come as torch.float8_e4m3fn or as their uint8 bit patterns."""
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.uint8 or t.dtype in _FP8_TYPES:
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(ws, nbytes: int, like: torch.Tensor):
    """The caller's workspace, or a fresh torch allocation of the size the
    library asked for (PyTorch is the device-memory provider)."""
    if ws is not None or nbytes == 0:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Batch:
    """Queries over sequences: device index arrays plus the host sizes."""

    def __init__(self, q_seq, q_pos, seq_len, seq_row0, max_len: int):
        self.q_seq = q_seq.to(torch.int32).contiguous()
        self.q_pos = q_pos.to(torch.int32).contiguous()
        self.seq_len = seq_len.to(torch.int32).contiguous()
        self.seq_row0 = seq_row0.to(torch.int64).contiguous()
        self.nq = int(self.q_seq.shape[0])
        self.nseq = int(self.seq_len.shape[0])
        self.max_len = int(max_len)
        self._s = DsaBatch(self.nq, self.nseq, self.max_len, self.q_seq.data_ptr(),
                           self.q_pos.data_ptr(), self.seq_len.data_ptr(), self.seq_row0.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self._s)


def abi_version() -> int:
    return int(lib.dsa_abi_version())


def dsa_index_score(batch: Batch, q_idx, w_idx, k_idx, scores, ld: Optional[int] = None, stream=None):
    ld = scores.shape[-1] if ld is None else ld
    _check(lib.dsa_index_score(batch.ref, _dt(q_idx), _p(q_idx), _p(w_idx), _p(k_idx), _p(scores),
                               ld, _stream(stream)), "dsa_index_score")
    return scores


def dsa_topk_workspace_size(nq: int, max_len: int, k: int) -> int:
    return int(lib.dsa_topk_workspace_size(nq, max_len, k))


def dsa_topk(batch: Batch, scores, k: int, idx, count=None, ws=None, ld: Optional[int] = None,
             stream=None):
    ld = scores.shape[-1] if ld is None else ld
    ws = _workspace(ws, dsa_topk_workspace_size(batch.nq, batch.max_len, k), scores)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsa_topk(batch.ref, _p(scores), ld, k, _p(idx), _p(count), _p(ws), wsb, _stream(stream)),
           "dsa_topk")
    return idx


def mla_sparse_attend_workspace_size(nq: int, k: int, n_layers: int = 1) -> int:
    return int(lib.mla_sparse_attend_workspace_size(nq, k, n_layers))


def _rope(q, kv=None) -> int:
    """Rotary width of a layer from its query's row width (576 or 512)."""
    rope = int(q.shape[-1]) - LATENT
    if kv is not None and int(kv.shape[-1]) != int(q.shape[-1]):
        raise ValueError(f"query rows are {q.shape[-1]} wide but cache rows {kv.shape[-1]}")
    return rope


def mla_sparse_attend(batch: Batch, q, kv, idx, k: int, scale: float, out, lse=None, ws=None,
                      stream=None):
    ws = _workspace(ws, mla_sparse_attend_workspace_size(batch.nq, k, 1), q)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mla_sparse_attend(batch.ref, _dt(q), _rope(q, kv), _p(q), _p(kv), _p(idx), k, scale, _p(out),
                                 _dt(out), _p(lse), _p(ws), wsb, _stream(stream)), "mla_sparse_attend")
    return out


def dsa_mla_decode_fused_workspace_size(nq: int, max_len: int, k: int, n_layers: int) -> int:
    return int(lib.dsa_mla_decode_fused_workspace_size(nq, max_len, k, n_layers))


def dsa_mla_decode_fused(batch: Batch, q_idx, w_idx, k_idx, k: int, q_l: Sequence, kv_l: Sequence,
                         out_l: Sequence, scale: float, lse_l: Optional[Sequence] = None,
                         idx_out=None, ws=None, stream=None):
    n = len(q_l)
    arr = ctypes.c_void_p * n
    qa = arr(*[t.data_ptr() for t in q_l])
    kva = arr(*[t.data_ptr() for t in kv_l])
    oa = arr(*[t.data_ptr() for t in out_l])
    la = None if lse_l is None else arr(*[(0 if t is None else t.data_ptr()) for t in lse_l])
    ws = _workspace(ws, dsa_mla_decode_fused_workspace_size(batch.nq, batch.max_len, k, n), q_idx)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    cv = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    _check(lib.dsa_mla_decode_fused(batch.ref, _dt(q_idx), _p(q_idx), _p(w_idx), _p(k_idx), k, n,
                                    _dt(q_l[0]), _rope(q_l[0], kv_l[0]), cv(qa), cv(kva), cv(oa), cv(la),
                                    _dt(out_l[0]), scale, _p(idx_out),
                                    _p(ws), wsb, _stream(stream)), "dsa_mla_decode_fused")
    return out_l


def dsa_mla_decode_fused_noalloc(batch: Batch, q_idx, w_idx, k_idx, k: int, q_l: Sequence, kv_l: Sequence,
                                 out_l: Sequence, scale: float, lse_l: Optional[Sequence] = None, idx_out=None,
                                 stream=None):
    """The fused decode read in the library's own per-GPU scratch array (no
    workspace, nothing allocated)."""
    n = len(q_l)
    arr = ctypes.c_void_p * n
    qa = arr(*[t.data_ptr() for t in q_l])
    kva = arr(*[t.data_ptr() for t in kv_l])
    oa = arr(*[t.data_ptr() for t in out_l])
    la = None if lse_l is None else arr(*[(0 if t is None else t.data_ptr()) for t in lse_l])
    cv = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    _check(lib.dsa_mla_decode_fused_noalloc(batch.ref, _dt(q_idx), _p(q_idx), _p(w_idx), _p(k_idx), k, n,
                                            _dt(q_l[0]), _rope(q_l[0], kv_l[0]), cv(qa), cv(kva), cv(oa), cv(la),
                                            _dt(out_l[0]), scale, _p(idx_out), _stream(stream)),
           "dsa_mla_decode_fused_noalloc")
    return out_l


def _plan_array(plan):
    arr = (LayerPlan * len(plan))()
    for i, p in enumerate(plan):
        arr[i] = LayerPlan(int(p[0]), int(p[1]), int(p[2]))
    return arr


def dsa_ml4_layer_plan(n_layers: int = ML4_LAYERS):
    """Mistral Large 4's schedule as a list of (runs_indexer, rope_dim, kv_source)."""
    arr = (LayerPlan * max(n_layers, 1))()
    _check(lib.dsa_ml4_layer_plan(n_layers, arr), "dsa_ml4_layer_plan")
    return [(bool(p.runs_indexer), int(p.rope_dim), int(p.kv_source)) for p in arr[:n_layers]]


def dsa_mla_decode_layers_workspace_size(nq: int, max_len: int, k: int, plan) -> int:
    return int(lib.dsa_mla_decode_layers_workspace_size(nq, max_len, k, len(plan), _plan_array(plan)))


def dsa_mla_decode_layers(batch: Batch, plan, qI_l: Sequence, w_l: Sequence, kI_l: Sequence, k: int,
                          q_l: Sequence, kv_l: Sequence, out_l: Sequence, scale: float,
                          lse_l: Optional[Sequence] = None, idx_l: Optional[Sequence] = None, ws=None,
                          stream=None):
    """Decode read over a stack of layers under `plan` (list of
    (runs_indexer, rope_dim, kv_source)).  Per-layer sequences may hold None
    where the library does not read the entry (indexer inputs of reusing
    layers, caches of layers that read another layer's cache)."""
    n = len(plan)
    arr = ctypes.c_void_p * n
    tab = lambda ts: arr(*[(0 if t is None else t.data_ptr()) for t in ts])
    first = next(t for t in qI_l if t is not None)
    ws = _workspace(ws, dsa_mla_decode_layers_workspace_size(batch.nq, batch.max_len, k, plan), first)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    cv = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    tabs = [tab(qI_l), tab(w_l), tab(kI_l), tab(q_l), tab(kv_l), tab(out_l)]
    la = None if lse_l is None else tab(lse_l)
    ia = None if idx_l is None else tab(idx_l)
    _check(lib.dsa_mla_decode_layers(batch.ref, n, _plan_array(plan), _dt(first), cv(tabs[0]), cv(tabs[1]),
                                     cv(tabs[2]), k, _dt(q_l[0]), cv(tabs[3]), cv(tabs[4]), cv(tabs[5]), cv(la),
                                     _dt(out_l[0]), scale, cv(ia), _p(ws), wsb, _stream(stream)),
           "dsa_mla_decode_layers")
    return out_l


def dsa_rope_frequencies(alpha=None):
    """Rotary frequencies (radians per position) of the 32 pairs, YaRN-blended
    and multiplied by e^alpha (host; returns a float64 numpy array)."""
    import numpy as np
    out = np.zeros(ROPE // 2, np.float64)
    a = None if alpha is None else np.ascontiguousarray(alpha, np.float32)
    _check(lib.dsa_rope_frequencies(None if a is None else a.ctypes.data_as(ctypes.c_void_p),
                                    out.ctypes.data_as(ctypes.c_void_p)), "dsa_rope_frequencies")
    return out


def dsa_rope_append(batch: Batch, freq, latent, rope_key, kv, q_attn=None, ssmax_s=None, ssmax_b=None,
                    stream=None):
    """Write each new token's cache row (latent, rotated rotary key) and
    scale/rotate its attention query in place.  freq: device float64 [32]
    (None for rotary-free layers); the rotary width comes from kv's rows."""
    rope = int(kv.shape[-1]) - LATENT
    _check(lib.dsa_rope_append(batch.ref, _dt(kv), rope, _p(freq), _p(latent), _p(rope_key), _p(kv), _p(q_attn),
                               _p(ssmax_s), _p(ssmax_b), _stream(stream)), "dsa_rope_append")
    return kv

