"""CPU oracle for the multi-LoRA shrink/expand path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU product path never imports it and shares no
code with it.

Two independent implementations live here:

* ``liblora_oracle.so`` (``lora_oracle.cpp``): fp64 per-token loops, threaded
  over tokens; the reference the GPU path is compared against.
* ``bruteforce``: exact rational arithmetic (``fractions.Fraction``) for tiny
  inputs, used to pin the fp64 oracle.

What is computed follows vLLM PR #13096 "[V1] LoRA - Add triton kernels for V1"
(summary and "Why do we need a new set of kernels": shrink and expand over an
ungrouped batch whose kernels know each token's LoRA id) and the MLC-LLM issue
"[Tracking] Multi-LoRA Serving" (Overview: Punica's segment vector and the
per-request low-rank multiplication):

    buf[s, t, :r] = scale * x[t, :] @ A_s[l]^T
    y[t, off_s : off_s + n_s] += buf[s, t, :] @ B_s[l]^T,   l = map[t] (skip l = -1)
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

import numpy as np

from .build import LIB, build  # noqa: F401

_lib = None

_I32P = ctypes.POINTER(ctypes.c_int32)
_U16P = ctypes.POINTER(ctypes.c_uint16)
_F64P = ctypes.POINTER(ctypes.c_double)


def configure(L):
    """Declare the C signatures on a loaded oracle library and return it."""
    L.oracle_round_bf16.argtypes = [ctypes.c_double]
    L.oracle_round_bf16.restype = ctypes.c_uint16
    L.oracle_widen_bf16.argtypes = [ctypes.c_uint16]
    L.oracle_widen_bf16.restype = ctypes.c_double
    L.oracle_default_threads.argtypes = []
    L.oracle_default_threads.restype = ctypes.c_int
    L.oracle_prepare_metadata.argtypes = [_I32P, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P,
                                          _I32P, _I32P, _I32P]
    L.oracle_prepare_metadata.restype = ctypes.c_int
    L.oracle_shrink.argtypes = [_U16P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                ctypes.POINTER(_U16P), ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_double, _I32P, ctypes.c_int32, _F64P, ctypes.c_int32]
    L.oracle_shrink.restype = ctypes.c_int
    L.oracle_expand.argtypes = [_F64P, ctypes.POINTER(_U16P), _I32P, ctypes.c_int32,
                                ctypes.c_int32, _U16P, ctypes.c_int64, _I32P, ctypes.c_int32,
                                ctypes.c_int32, _F64P, _U16P, ctypes.c_int32]
    L.oracle_expand.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = configure(ctypes.CDLL(LIB))
    return _lib


def _p(a: np.ndarray, ptype):
    return a.ctypes.data_as(ptype)


def default_threads() -> int:
    return int(lib().oracle_default_threads())


def round_bf16(v: float) -> int:
    """Nearest bfloat16 bit pattern to a double, ties to even (one rounding)."""
    return int(lib().oracle_round_bf16(float(v)))


def round_bf16_array(a: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda v: lib().oracle_round_bf16(float(v)), otypes=[np.uint16])
    return f(np.asarray(a, dtype=np.float64))


def prepare_metadata(mapping: np.ndarray, max_loras: int) -> Dict[str, np.ndarray]:
    m = np.ascontiguousarray(mapping, dtype=np.int32)
    T = int(m.shape[0])
    out = dict(
        sorted_token_ids=np.zeros(T, dtype=np.int32),
        active_lora_ids=np.zeros(max_loras, dtype=np.int32),
        num_tokens_per_lora=np.zeros(max_loras, dtype=np.int32),
        lora_token_start=np.zeros(max_loras, dtype=np.int32),
        num_active=np.zeros(1, dtype=np.int32),
    )
    rc = lib().oracle_prepare_metadata(
        _p(m, _I32P) if T else None, T, max_loras,
        _p(out["sorted_token_ids"], _I32P) if T else None,
        _p(out["active_lora_ids"], _I32P), _p(out["num_tokens_per_lora"], _I32P),
        _p(out["lora_token_start"], _I32P), _p(out["num_active"], _I32P))
    if rc != 0:
        raise ValueError("oracle_prepare_metadata: invalid argument")
    return out


TILE = 16  # positions per tile of the padded grouped order


def prepare_tiles(mapping: np.ndarray, max_loras: int) -> Dict[str, np.ndarray]:
    """The padded grouped order the kernels read tiles of: for the k-th
    adapter present (ascending id), its tokens in batch order from position
    P_k = round_up(S_k + (TILE - 1) * k, TILE), S_k being the number of tokens of the
    adapters before it; -1 everywhere else below num_tiles * TILE.  Returns
    tile_token_ids [num_tiles * TILE], tile_lora [num_tiles] (the adapter of
    each tile, -1 for a tile of -1 entries) and num_tiles [1].

    A layout of this library's own (the pages fix only the grouping itself:
    vLLM PR #13096, "Why do we need a new set of kernels"); written out here
    from its definition, adapter by adapter, independently of the sort above.
    """
    m = np.asarray(mapping, dtype=np.int64).reshape(-1)
    ids = np.where((m >= -1) & (m < max_loras), m, -1)
    runs = []  # (start position, adapter, tokens)
    s_k = 0
    for k, l in enumerate(sorted(set(int(v) for v in ids if v >= 0))):
        toks = [t for t in range(ids.shape[0]) if ids[t] == l] if ids.shape[0] <= 4096 \
            else np.nonzero(ids == l)[0].tolist()
        p_k = -(-(s_k + (TILE - 1) * k) // TILE) * TILE
        runs.append((p_k, l, toks))
        s_k += len(toks)
    end = runs[-1][0] + len(runs[-1][2]) if runs else 0
    num_tiles = -(-end // TILE)
    tile_token_ids = np.full(num_tiles * TILE, -1, dtype=np.int32)
    tile_lora = np.full(num_tiles, -1, dtype=np.int32)
    for p_k, l, toks in runs:
        tile_token_ids[p_k:p_k + len(toks)] = toks
        tile_lora[p_k // TILE:-(-(p_k + len(toks)) // TILE)] = l
    return dict(tile_token_ids=tile_token_ids, tile_lora=tile_lora,
                num_tiles=np.array([num_tiles], dtype=np.int32))


def count_runs(mapping: np.ndarray, max_loras: int) -> np.ndarray:
    """num_runs [1]: the number of maximal runs of consecutive tokens (batch
    order) that share one adapter id >= 0, after ids outside [-1, max_loras)
    are read as -1.  Tokens without an adapter belong to no run and separate
    the runs around them.

    This is the batch's segment count in the sense of the MLC-LLM issue's
    Overview (Punica's segment vector: consecutive rows multiplied by the same
    adapter) for the batch as given, before any grouping.  Written from that
    definition, token by token.
    """
    m = np.asarray(mapping, dtype=np.int64).reshape(-1)
    ids = [int(v) if -1 <= v < max_loras else -1 for v in m.tolist()]
    runs = 0
    prev = -1
    for l in ids:
        if l >= 0 and l != prev:
            runs += 1
        prev = l
    return np.array([runs], dtype=np.int32)


def shrink(x: np.ndarray, lora_a: List[np.ndarray], mapping: np.ndarray, max_loras: int,
           rank: int, scale: float, num_threads: int = 0) -> np.ndarray:
    """fp64 buf [S, T, rank]; rows of tokens without an adapter stay NaN."""
    m = np.ascontiguousarray(mapping, dtype=np.int32)
    T = int(m.shape[0])
    x = np.ascontiguousarray(x, dtype=np.uint16)
    hidden = int(x.shape[1])
    S = len(lora_a)
    mats = [np.ascontiguousarray(a, dtype=np.uint16) for a in lora_a]
    for a in mats:
        assert a.shape[1:] == (rank, hidden) and a.shape[0] >= max_loras
    ptrs = (_U16P * S)(*[_p(a, _U16P) for a in mats])
    buf = np.full((S, T, rank), np.nan, dtype=np.float64)
    rc = lib().oracle_shrink(_p(x, _U16P), hidden, T, hidden, ptrs, S, rank, float(scale),
                             _p(m, _I32P), max_loras, _p(buf, _F64P), num_threads)
    if rc != 0:
        raise ValueError("oracle_shrink: invalid argument")
    return buf


def expand(buf: np.ndarray, lora_b: List[np.ndarray], y0: np.ndarray, mapping: np.ndarray,
           max_loras: int, rank: int, num_threads: int = 0):
    """Return (y64 float64 [T, ldy], y_bf16 uint16 [T, ldy])."""
    m = np.ascontiguousarray(mapping, dtype=np.int32)
    T = int(m.shape[0])
    S = len(lora_b)
    mats = [np.ascontiguousarray(b, dtype=np.uint16) for b in lora_b]
    sizes = np.array([b.shape[1] for b in mats], dtype=np.int32)
    for b in mats:
        assert b.shape[2] == rank and b.shape[0] >= max_loras
    y0 = np.ascontiguousarray(y0[:T], dtype=np.uint16)
    ldy = int(y0.shape[1])
    buf = np.ascontiguousarray(buf, dtype=np.float64)
    assert buf.shape == (S, T, rank)
    ptrs = (_U16P * S)(*[_p(b, _U16P) for b in mats])
    y64 = np.zeros((T, ldy), dtype=np.float64)
    yb = np.zeros((T, ldy), dtype=np.uint16)
    rc = lib().oracle_expand(_p(buf, _F64P), ptrs, _p(sizes, _I32P), S, rank, _p(y0, _U16P), ldy,
                             _p(m, _I32P), T, max_loras, _p(y64, _F64P), _p(yb, _U16P),
                             num_threads)
    if rc != 0:
        raise ValueError("oracle_expand: invalid argument")
    return y64, yb


def run_step(w, num_threads: int = 0) -> Dict[str, np.ndarray]:
    """Metadata, shrink and expand of one workload (``workloads.Workload``)."""
    T = w.num_tokens
    meta = prepare_metadata(w.mapping, w.max_loras)
    # the GPU path multiplies by a float32 scale; the oracle uses that same value
    scale = float(np.float32(w.scale))
    buf = shrink(w.x[:T], w.lora_a, w.mapping, w.max_loras, w.rank, scale, num_threads)
    y64, yb = expand(buf, w.lora_b, w.y0[:T], w.mapping, w.max_loras, w.rank, num_threads)
    out = dict(meta)
    out.update(buf=buf, y64=y64, y_bf16=yb)
    return out
