"""MI355X (gfx950) multi-LoRA shrink/expand: Python binding of liblora_mi355x.so.

The functions below carry the names of the C entry points declared in
``include/lora_mi355x.h`` and only marshal arguments: tensors become device
pointers, the current (or given) torch stream becomes the ``hipStream_t``.
Every step of the path runs in the library's HIP kernels; there is no other
implementation to fall back to, and importing this module fails if the
library has not been built.

torch is imported first so that the library binds to the HIP runtime torch
has already loaded (same soname), keeping one runtime per process.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (must precede loading the library, see above)

__all__ = [
    "LIB_PATH", "LoraError", "LoraMeta", "lib", "lora_prepare_metadata", "lora_shrink",
    "lora_prepare_and_shrink", "lora_fused_step", "lora_fused_step_workspace_bytes",
    "lora_fused_step_launches",
    "lora_fused_step_static", "lora_prepare_metadata_grouped", "ExpandConfig",
    "fused_step_workspace",
    "lora_shrink_default_splits", "lora_expand",
    "lora_status_string",
    "LORA_MAX_LORAS", "LORA_MAX_SLICES", "LORA_MAX_SPLITS", "SUPPORTED_RANKS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora_mi355x.so")

LORA_OK = 0
LORA_ERR_INVALID_ARGUMENT = 1
LORA_ERR_UNSUPPORTED = 2
LORA_ERR_LAUNCH = 3
LORA_MAX_LORAS = 256
LORA_MAX_SLICES = 4
LORA_MAX_SPLITS = 64
SUPPORTED_RANKS = (8, 16, 32, 64)


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {lora_status_string(status)} ({status})")
        self.status = status


class _MetaStruct(ctypes.Structure):
    _fields_ = [("sorted_token_ids", ctypes.c_void_p), ("active_lora_ids", ctypes.c_void_p),
                ("num_tokens_per_lora", ctypes.c_void_p), ("lora_token_start", ctypes.c_void_p),
                ("num_active", ctypes.c_void_p), ("tile_token_ids", ctypes.c_void_p),
                ("tile_lora", ctypes.c_void_p), ("num_tiles", ctypes.c_void_p),
                ("num_runs", ctypes.c_void_p)]

class ExpandConfig(ctypes.Structure):
    """lora_expand_config_t: launch choices of lora_expand (0 / -1: the
    library's rule).  Any valid setting gives the same bits."""
    _fields_ = [("chunks_per_range", ctypes.c_int32), ("range_fastest", ctypes.c_int32),
                ("workgroups_per_cu", ctypes.c_int32)]

    def __init__(self, chunks_per_range: int = 0, range_fastest: int = -1,
                 workgroups_per_cu: int = 0):
        super().__init__(int(chunks_per_range), int(range_fastest), int(workgroups_per_cu))

    def as_dict(self):
        return {"chunks_per_range": self.chunks_per_range, "range_fastest": self.range_fastest,
                "workgroups_per_cu": self.workgroups_per_cu}


class _StepOptions(ctypes.Structure):
    _fields_ = [("wait_polls", ctypes.c_int32), ("expand", ExpandConfig),
                ("start_delay_ns", ctypes.c_int32), ("part_sums", ctypes.c_int32),
                ("batch_order_shrink", ctypes.c_int32), ("y_delay_ns", ctypes.c_int32)]


def _expand_config(config, lora_b=None, num_splits=None, meta=None) -> Optional[ExpandConfig]:
    """None: the library's rules; "table": the measured choices for the call's
    shape in segmented_rank_gemm_amd/tuning_table.json (the rules if the table
    does not have it); an ExpandConfig or a dict of its fields."""
    if config is None or isinstance(config, ExpandConfig):
        return config
    if isinstance(config, str):
        if config != "table":
            raise ValueError(f"expand config {config!r}: expected 'table', None or ExpandConfig")
        from .tuning import expand_config_for
        return expand_config_for(lora_b, num_splits, meta)
    return ExpandConfig(**config)


def _start_delay(start_delay_ns, lora_b=None, num_splits=None, meta=None,
                 name="start_delay_ns") -> Optional[int]:
    """None: the library's default; "table": the measured choice for the call's
    shape in segmented_rank_gemm_amd/tuning_table.json (the default if the
    table does not have it); else nanoseconds."""
    if isinstance(start_delay_ns, str):
        if start_delay_ns != "table":
            raise ValueError(f"{name} {start_delay_ns!r}: expected 'table', None or ns")
        from .tuning import start_delay_for
        return start_delay_for(lora_b, num_splits, meta, name)
    return None if start_delay_ns is None else int(start_delay_ns)


def _table_flag(value, name, lora_b, num_splits, meta) -> bool:
    """A yes/no launch choice: a bool, or "table" for the table's choice for
    the call's shape (no when the table has none)."""
    if isinstance(value, str):
        if value != "table":
            raise ValueError(f"{name} {value!r}: expected 'table' or a bool")
        from .tuning import flag_for
        return flag_for(name, lora_b, num_splits, meta)
    return bool(value)


def _step_options(wait_polls, expand_config, start_delay_ns=None, lora_b=None, num_splits=None,
                  meta=None, part_sums=False, batch_order_shrink=False, y_delay_ns=None):
    cfg = _expand_config(expand_config, lora_b, num_splits, meta)
    delay = _start_delay(start_delay_ns, lora_b, num_splits, meta)
    y_delay = _start_delay(y_delay_ns, lora_b, num_splits, meta, "y_delay_ns")
    sums = _table_flag(part_sums, "part_sums", lora_b, num_splits, meta)
    batch = _table_flag(batch_order_shrink, "batch_order_shrink", lora_b, num_splits, meta)
    if (wait_polls is None and cfg is None and delay is None and y_delay is None and not sums
            and not batch):
        return None
    cfg = cfg or ExpandConfig()
    return ctypes.byref(_StepOptions(-1 if wait_polls is None else int(wait_polls), cfg,
                                     -1 if delay is None else delay, int(sums), int(batch),
                                     -1 if y_delay is None else y_delay))


TILE = 16  # positions per tile of the padded grouped order (LORA_TILE)


def max_tiles(max_tokens: int, max_loras: int) -> int:
    """LORA_MAX_TILES: tiles the padded grouped order may use."""
    return (int(max_tokens) + TILE - 1) // TILE + int(max_loras) + 1


_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python segmented_rank_gemm_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        MP = ctypes.POINTER(_MetaStruct)
        L.lora_status_string.argtypes = [ctypes.c_int]
        L.lora_status_string.restype = ctypes.c_char_p
        L.lora_prepare_metadata.argtypes = [_VP, _I32, _I32, _I32, MP, _VP]
        L.lora_prepare_metadata.restype = ctypes.c_int
        L.lora_prepare_metadata_grouped.argtypes = [_VP, _I32, _I32, _I32, MP, _VP]
        L.lora_prepare_metadata_grouped.restype = ctypes.c_int
        L.lora_shrink_default_splits.argtypes = [_I32, _I32, _I32, _I32, _I32]
        L.lora_shrink_default_splits.restype = _I32
        L.lora_shrink.argtypes = [_VP, _I64, _I32, ctypes.POINTER(_VP), _I32, _I32, ctypes.c_float,
                                  _VP, _I32, MP, _I32, _I32, _VP]
        L.lora_shrink.restype = ctypes.c_int
        L.lora_prepare_and_shrink.argtypes = [_VP, _I32, _VP, _I64, _I32, ctypes.POINTER(_VP), _I32,
                                              _I32, ctypes.c_float, _VP, _I32, MP, _I32, _I32, _VP]
        L.lora_prepare_and_shrink.restype = ctypes.c_int
        L.lora_expand.argtypes = [_VP, _I32, ctypes.POINTER(_VP), ctypes.POINTER(_I32), _I32, _I32,
                                  _VP, _I64, MP, _I32, _I32, ctypes.POINTER(ExpandConfig), _VP]
        L.lora_expand.restype = ctypes.c_int
        L.lora_fused_step_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
        L.lora_fused_step_workspace_bytes.restype = _I64
        L.lora_fused_step_launches.argtypes = [_I32, _I32, _I32, _I32]
        L.lora_fused_step_launches.restype = _I32
        L.lora_fused_step.argtypes = [_VP, _I32, _VP, _I64, _I32, ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), ctypes.POINTER(_I32), _I32, _I32,
                                      ctypes.c_float, _VP, _I32, _VP, _I64, MP, _VP, _I64,
                                      ctypes.POINTER(_StepOptions), _I32, _I32, _VP]
        L.lora_fused_step.restype = ctypes.c_int
        L.lora_fused_step_static.argtypes = [_VP, _I32, _VP, _I64, _I32, ctypes.POINTER(_VP),
                                             ctypes.POINTER(_VP), ctypes.POINTER(_I32), _I32, _I32,
                                             ctypes.c_float, _VP, _I32, _VP, _I64, MP,
                                             ctypes.POINTER(_StepOptions), _I32, _I32, _VP]
        L.lora_fused_step_static.restype = ctypes.c_int
        _lib = L
    return _lib


lib()  # fail at import, loudly, if the native library is absent


def lora_status_string(status: int) -> str:
    return lib().lora_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != LORA_OK:
        raise LoraError(fn, status)


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev_ptr(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return int(t.data_ptr())


class LoraMeta:
    """Device buffers of one batch's grouping (the ``lora_meta_t`` outputs).

    Allocated once for a (max_tokens, max_loras) pair and reused for every
    batch, as static buffers that a captured graph keeps pointing at.
    """

    def __init__(self, max_tokens: int, max_loras: int, device="cuda"):
        self.max_tokens = int(max_tokens)
        self.max_loras = int(max_loras)
        opts = dict(dtype=torch.int32, device=device)
        self.sorted_token_ids = torch.empty(self.max_tokens, **opts)
        self.active_lora_ids = torch.empty(self.max_loras, **opts)
        self.num_tokens_per_lora = torch.empty(self.max_loras, **opts)
        self.lora_token_start = torch.empty(self.max_loras, **opts)
        self.num_active = torch.empty(1, **opts)
        nt = max_tiles(max_tokens, max_loras)
        self.tile_token_ids = torch.empty(nt * TILE, **opts)
        self.tile_lora = torch.empty(nt, **opts)
        self.num_tiles = torch.empty(1, **opts)
        self.num_runs = torch.empty(1, **opts)
        self._struct = _MetaStruct(*(int(t.data_ptr()) for t in self.tensors()))

    def tensors(self):
        return (self.sorted_token_ids, self.active_lora_ids, self.num_tokens_per_lora,
                self.lora_token_start, self.num_active, self.tile_token_ids, self.tile_lora,
                self.num_tiles, self.num_runs)

    @property
    def struct_ref(self):
        return ctypes.byref(self._struct)


def _mapping_ptr(token_lora_mapping: torch.Tensor, num_tokens: int) -> int:
    """Device address of the token -> adapter map (0 for an empty batch)."""
    if not num_tokens:
        return 0
    ptr = _dev_ptr(token_lora_mapping, torch.int32, "token_lora_mapping")
    if token_lora_mapping.dim() != 1 or not token_lora_mapping.is_contiguous():
        raise ValueError("token_lora_mapping must be a contiguous 1-D tensor")
    if token_lora_mapping.numel() < num_tokens:
        raise ValueError("token_lora_mapping is shorter than num_tokens")
    return ptr


def lora_prepare_metadata(token_lora_mapping: torch.Tensor, num_tokens: int, meta: LoraMeta,
                          stream: Optional[torch.cuda.Stream] = None) -> None:
    ptr = _mapping_ptr(token_lora_mapping, num_tokens)
    _check("lora_prepare_metadata", lib().lora_prepare_metadata(
        ptr, int(num_tokens), meta.max_tokens, meta.max_loras, meta.struct_ref,
        _stream_handle(stream)))


def lora_prepare_metadata_grouped(token_lora_mapping: torch.Tensor, num_tokens: int,
                                  meta: LoraMeta,
                                  stream: Optional[torch.cuda.Stream] = None) -> None:
    """lora_prepare_metadata for a batch already grouped by adapter (one pass;
    an ungrouped batch gets the same outputs, more slowly)."""
    ptr = _mapping_ptr(token_lora_mapping, num_tokens)
    _check("lora_prepare_metadata_grouped", lib().lora_prepare_metadata_grouped(
        ptr, int(num_tokens), meta.max_tokens, meta.max_loras, meta.struct_ref,
        _stream_handle(stream)))


def lora_shrink_default_splits(hidden: int, max_tokens: int, max_loras: int, num_slices: int,
                               rank: int) -> int:
    return int(lib().lora_shrink_default_splits(hidden, max_tokens, max_loras, num_slices, rank))


def _shrink_args(x: torch.Tensor, lora_a: Sequence[torch.Tensor], buf: torch.Tensor,
                 num_splits: int, meta: LoraMeta):
    S = len(lora_a)
    if S < 1:
        raise ValueError("lora_a must hold at least one slice")
    if lora_a[0].dim() != 3:
        raise ValueError("lora_a[s] must be [max_loras, rank, hidden]")
    _, rank, hidden = lora_a[0].shape
    if (x.dim() != 2 or x.stride(1) != 1 or x.shape[0] < meta.max_tokens
            or x.shape[1] < hidden):
        raise ValueError("x must be [>=max_tokens, >=hidden] with unit column stride")
    if tuple(buf.shape) != (num_splits, S, meta.max_tokens, rank) or not buf.is_contiguous():
        raise ValueError("buf must be contiguous [num_splits, S, max_tokens, rank]")
    for a in lora_a:
        if tuple(a.shape) != (meta.max_loras, rank, hidden) or not a.is_contiguous():
            raise ValueError("lora_a[s] must be contiguous [max_loras, rank, hidden]")
    aptrs = (_VP * S)(*[_dev_ptr(a, torch.bfloat16, "lora_a") for a in lora_a])
    return S, int(rank), int(hidden), aptrs


def lora_shrink(x: torch.Tensor, lora_a: Sequence[torch.Tensor], scale: float, buf: torch.Tensor,
                num_splits: int, meta: LoraMeta,
                stream: Optional[torch.cuda.Stream] = None) -> None:
    """x: bf16 [max_tokens, >=hidden] (row stride x.stride(0)); lora_a[s]: bf16
    [max_loras, rank, hidden]; buf: fp32 [num_splits, S, max_tokens, rank]."""
    S, rank, hidden, aptrs = _shrink_args(x, lora_a, buf, num_splits, meta)
    _check("lora_shrink", lib().lora_shrink(
        _dev_ptr(x, torch.bfloat16, "x"), int(x.stride(0)), hidden, aptrs, S, rank,
        float(scale), _dev_ptr(buf, torch.float32, "buf"), int(num_splits), meta.struct_ref,
        meta.max_tokens, meta.max_loras, _stream_handle(stream)))


def lora_prepare_and_shrink(token_lora_mapping: torch.Tensor, num_tokens: int, x: torch.Tensor,
                            lora_a: Sequence[torch.Tensor], scale: float, buf: torch.Tensor,
                            num_splits: int, meta: LoraMeta,
                            stream: Optional[torch.cuda.Stream] = None) -> None:
    """lora_prepare_metadata then lora_shrink on the same batch (one launch up to
    512 token slots); arguments as for those two."""
    ptr = _mapping_ptr(token_lora_mapping, num_tokens)
    S, rank, hidden, aptrs = _shrink_args(x, lora_a, buf, num_splits, meta)
    _check("lora_prepare_and_shrink", lib().lora_prepare_and_shrink(
        ptr, int(num_tokens), _dev_ptr(x, torch.bfloat16, "x"), int(x.stride(0)), hidden, aptrs,
        S, rank, float(scale), _dev_ptr(buf, torch.float32, "buf"), int(num_splits),
        meta.struct_ref, meta.max_tokens, meta.max_loras, _stream_handle(stream)))


def _expand_args(buf: torch.Tensor, num_splits: int, lora_b: Sequence[torch.Tensor],
                 y: torch.Tensor, meta: LoraMeta):
    S = len(lora_b)
    if S < 1:
        raise ValueError("lora_b must hold at least one slice")
    if lora_b[0].dim() != 3:
        raise ValueError("lora_b[s] must be [max_loras, n_s, rank]")
    rank = int(lora_b[0].shape[2])
    sizes = [int(b.shape[1]) for b in lora_b]
    if tuple(buf.shape) != (num_splits, S, meta.max_tokens, rank) or not buf.is_contiguous():
        raise ValueError("buf must be contiguous [num_splits, S, max_tokens, rank]")
    if y.dim() != 2 or y.stride(1) != 1 or y.shape[0] < meta.max_tokens or y.shape[1] < sum(sizes):
        raise ValueError("y must be [>=max_tokens, >=sum(n_s)] with unit column stride")
    for b, n in zip(lora_b, sizes):
        if tuple(b.shape) != (meta.max_loras, n, rank) or not b.is_contiguous():
            raise ValueError("lora_b[s] must be contiguous [max_loras, n_s, rank]")
    bptrs = (_VP * S)(*[_dev_ptr(b, torch.bfloat16, "lora_b") for b in lora_b])
    nsz = (_I32 * S)(*sizes)
    return S, rank, bptrs, nsz


def lora_fused_step_workspace_bytes(max_tokens: int, max_loras: int, num_slices: int,
                                    rank: int) -> int:
    """Bytes of zero-filled workspace lora_fused_step needs for these sizes
    (0: none)."""
    return int(lib().lora_fused_step_workspace_bytes(max_tokens, max_loras, num_slices, rank))


def lora_fused_step_launches(max_tokens: int, max_loras: int, num_slices: int, rank: int) -> int:
    """1: lora_fused_step runs these sizes in one launch; 2: as
    lora_prepare_and_shrink then lora_expand; 0: sizes it rejects."""
    return int(lib().lora_fused_step_launches(max_tokens, max_loras, num_slices, rank))


def fused_step_workspace(max_tokens: int, max_loras: int, num_slices: int, rank: int,
                         device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled workspace for lora_fused_step (None when none is needed).
    torch's allocations are 256-byte aligned."""
    n = lora_fused_step_workspace_bytes(max_tokens, max_loras, num_slices, rank)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def lora_fused_step(token_lora_mapping: torch.Tensor, num_tokens: int, x: torch.Tensor,
                    lora_a: Sequence[torch.Tensor], lora_b: Sequence[torch.Tensor], scale: float,
                    buf: torch.Tensor, num_splits: int, y: torch.Tensor, meta: LoraMeta,
                    workspace: Optional[torch.Tensor], wait_polls: Optional[int] = None,
                    stream: Optional[torch.cuda.Stream] = None, expand_config="table",
                    start_delay_ns="table", part_sums="table",
                    batch_order_shrink="table", y_delay_ns="table") -> None:
    """Metadata, shrink and expand of one batch (one launch where the sizes
    allow); arguments as for lora_prepare_and_shrink and lora_expand, plus the
    zero-filled workspace of fused_step_workspace (reused call after call).
    start_delay_ns, y_delay_ns: the one-launch path's expand hold-offs before
    its B and its y loads (timing only; None: the library's defaults);
    part_sums: large rank-32/64 batches, the shrink sums the parts for the
    expand (same bits); batch_order_shrink: large batches, the shrink in batch
    order beside the metadata in one launch (same bits).  "table": the
    table's choice for the shape (off when the table has none)."""
    ptr = _mapping_ptr(token_lora_mapping, num_tokens)
    S, rank, hidden, aptrs = _shrink_args(x, lora_a, buf, num_splits, meta)
    Sb, rank_b, bptrs, nsz = _expand_args(buf, num_splits, lora_b, y, meta)
    if Sb != S or rank_b != rank:
        raise ValueError("lora_a and lora_b disagree on slices or rank")
    wptr, wbytes = 0, 0
    if workspace is not None:
        wptr, wbytes = _flat_dev_bytes(workspace, "workspace")
    opts = _step_options(wait_polls, expand_config, start_delay_ns, lora_b, num_splits, meta,
                         part_sums, batch_order_shrink, y_delay_ns)
    _check("lora_fused_step", lib().lora_fused_step(
        ptr, int(num_tokens), _dev_ptr(x, torch.bfloat16, "x"), int(x.stride(0)), hidden, aptrs,
        bptrs, nsz, S, rank, float(scale), _dev_ptr(buf, torch.float32, "buf"), int(num_splits),
        _dev_ptr(y, torch.bfloat16, "y"), int(y.stride(0)), meta.struct_ref, wptr, int(wbytes),
        opts, meta.max_tokens, meta.max_loras, _stream_handle(stream)))


def lora_fused_step_static(token_lora_mapping: torch.Tensor, num_tokens: int, x: torch.Tensor,
                           lora_a: Sequence[torch.Tensor], lora_b: Sequence[torch.Tensor],
                           scale: float, buf: torch.Tensor, num_splits: int, y: torch.Tensor,
                           meta: LoraMeta, wait_polls: Optional[int] = None,
                           stream: Optional[torch.cuda.Stream] = None, expand_config="table",
                           start_delay_ns="table", batch_order_shrink="table",
                           y_delay_ns="table") -> None:
    """lora_fused_step with the library's own counter array instead of a
    workspace (nothing is allocated; calls that overlap on one GPU race).
    No part sums (they need a workspace); the other launch choices as for
    lora_fused_step."""
    ptr = _mapping_ptr(token_lora_mapping, num_tokens)
    S, rank, hidden, aptrs = _shrink_args(x, lora_a, buf, num_splits, meta)
    Sb, rank_b, bptrs, nsz = _expand_args(buf, num_splits, lora_b, y, meta)
    if Sb != S or rank_b != rank:
        raise ValueError("lora_a and lora_b disagree on slices or rank")
    opts = _step_options(wait_polls, expand_config, start_delay_ns, lora_b, num_splits, meta,
                         False, batch_order_shrink, y_delay_ns)
    _check("lora_fused_step_static", lib().lora_fused_step_static(
        ptr, int(num_tokens), _dev_ptr(x, torch.bfloat16, "x"), int(x.stride(0)), hidden, aptrs,
        bptrs, nsz, S, rank, float(scale), _dev_ptr(buf, torch.float32, "buf"), int(num_splits),
        _dev_ptr(y, torch.bfloat16, "y"), int(y.stride(0)), meta.struct_ref, opts, meta.max_tokens,
        meta.max_loras, _stream_handle(stream)))


def lora_expand(buf: torch.Tensor, num_splits: int, lora_b: Sequence[torch.Tensor], y: torch.Tensor,
                meta: LoraMeta, stream: Optional[torch.cuda.Stream] = None,
                config="table") -> None:
    """buf: fp32 [num_splits, S, max_tokens, rank]; lora_b[s]: bf16 [max_loras, n_s, rank];
    y: bf16 [>=max_tokens, >=sum(n_s)] (row stride y.stride(0)), updated in place."""
    S, rank, bptrs, nsz = _expand_args(buf, num_splits, lora_b, y, meta)
    _check("lora_expand", lib().lora_expand(
        _dev_ptr(buf, torch.float32, "buf"), int(num_splits), bptrs, nsz, S, rank,
        _dev_ptr(y, torch.bfloat16, "y"), int(y.stride(0)), meta.struct_ref, meta.max_tokens,
        meta.max_loras, _cfg_ref(_expand_config(config, lora_b, num_splits, meta)),
        _stream_handle(stream)))


def _cfg_ref(cfg):
    return None if cfg is None else ctypes.byref(cfg)


def _flat_dev_bytes(t: torch.Tensor, name: str):
    """Device address and byte size of a contiguous device tensor (any dtype)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return int(t.data_ptr()), t.numel() * t.element_size()

