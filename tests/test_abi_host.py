"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects invalid arguments before
enqueuing anything.  No call here reaches the HIP runtime."""

import ctypes
import os
import re

import pytest

import segmented_rank_gemm_amd as srg
from segmented_rank_gemm_amd import measure

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")

FAKE = 0x10000  # a 16-byte aligned non-null address that is never dereferenced


def _declared(header="lora_mi355x.h"):
    text = open(os.path.join(INCLUDE, header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["lora_prepare_metadata", "lora_shrink", "lora_expand", "lora_status_string",
              "lora_prepare_and_shrink", "lora_fused_step", "lora_fused_step_static",
              "lora_fused_step_workspace_bytes", "lora_fused_step_launches",
              "lora_prepare_metadata_grouped", "lora_shrink_default_splits"]:
        assert n in names
    # the measurement aids are not part of the path's interface
    assert "lora_stream_copy" not in names and "lora_stream_update" not in names
    assert set(_declared("lora_measure.h")) == {"lora_stream_copy", "lora_stream_update"}


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(srg.LIB_PATH)
    for n in _declared():
        assert hasattr(L, n), n
    M = ctypes.CDLL(measure.MEASURE_LIB_PATH)
    for n in _declared("lora_measure.h"):
        assert hasattr(M, n), n
    assert not hasattr(L, "lora_stream_copy")


def test_status_strings():
    assert srg.lora_status_string(0) == "LORA_OK"
    assert srg.lora_status_string(1) == "LORA_ERR_INVALID_ARGUMENT"
    assert srg.lora_status_string(2) == "LORA_ERR_UNSUPPORTED"
    assert srg.lora_status_string(3) == "LORA_ERR_LAUNCH"
    assert srg.lora_status_string(99) == "LORA_ERR_UNKNOWN"


def _meta(**null):
    fields = dict(sorted_token_ids=FAKE, active_lora_ids=FAKE, num_tokens_per_lora=FAKE,
                  lora_token_start=FAKE, num_active=FAKE, tile_token_ids=FAKE, tile_lora=FAKE,
                  num_tiles=FAKE, num_runs=FAKE)
    fields.update(null)
    return ctypes.byref(srg._MetaStruct(**fields))


def _ptrs(n, value=FAKE):
    return (ctypes.c_void_p * n)(*([value] * n))


@pytest.mark.parametrize("num_tokens,max_tokens,max_loras,meta", [
    (-1, 16, 4, None), (17, 16, 4, None), (4, 0, 4, None), (4, 16, 0, None), (4, 16, 257, None),
    (4, 1 << 25, 4, None), (4, 16, 4, dict(num_active=None)), (4, 16, 4, dict(sorted_token_ids=None)),
    (4, 16, 4, dict(tile_token_ids=None)), (4, 16, 4, dict(tile_lora=None)),
    (4, 16, 4, dict(num_tiles=None)), (4, 16, 4, dict(num_runs=None)),
])
def test_prepare_metadata_rejects(num_tokens, max_tokens, max_loras, meta):
    m = _meta(**(meta or {}))
    assert srg.lib().lora_prepare_metadata(FAKE, num_tokens, max_tokens, max_loras, m, None) == 1


def test_prepare_metadata_rejects_null_mapping_with_tokens():
    assert srg.lib().lora_prepare_metadata(None, 3, 16, 4, _meta(), None) == 1


SHRINK_OK = dict(x=FAKE, ldx=4096, hidden=4096, a=3, S=3, rank=8, scale=1.0, buf=FAKE, splits=4,
                 maxT=256, L=4)


def _shrink(**kw):
    a = dict(SHRINK_OK)
    a.update(kw)
    aptr = a["a"] if not isinstance(a["a"], int) else _ptrs(a["a"])
    return srg.lib().lora_shrink(a["x"], a["ldx"], a["hidden"], aptr, a["S"], a["rank"],
                                 a["scale"], a["buf"], a["splits"], _meta(), a["maxT"], a["L"],
                                 None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(x=FAKE + 2), 1), (dict(buf=FAKE + 4), 1), (dict(hidden=4092), 1),
    (dict(hidden=0), 1), (dict(ldx=4000), 1), (dict(ldx=4100), 1), (dict(S=0), 1), (dict(S=5), 1),
    (dict(splits=0), 1), (dict(splits=65), 1), (dict(rank=0), 1), (dict(rank=65), 1),
    (dict(maxT=0), 1), (dict(L=300), 1), (dict(a=_ptrs(3, None)), 1),
    (dict(a=_ptrs(3, FAKE + 8)), 1), (dict(hidden=1 << 17, ldx=1 << 17), 1),
    (dict(rank=12), 2), (dict(rank=4), 2), (dict(rank=128 // 2 - 1), 2),
])
def test_shrink_rejects(kw, status):
    assert _shrink(**kw) == status


def _prep_shrink(mapping=FAKE, T=4, maxT=256, meta=None, **kw):
    a = dict(SHRINK_OK)
    a.update(kw)
    a["maxT"] = maxT
    aptr = a["a"] if not isinstance(a["a"], int) else _ptrs(a["a"])
    return srg.lib().lora_prepare_and_shrink(mapping, T, a["x"], a["ldx"], a["hidden"], aptr,
                                             a["S"], a["rank"], a["scale"], a["buf"],
                                             a["splits"], _meta(**(meta or {})), a["maxT"],
                                             a["L"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), 1), (dict(T=257), 1), (dict(mapping=None), 1), (dict(maxT=0, T=0), 1),
    (dict(meta=dict(num_runs=None)), 1), (dict(meta=dict(tile_lora=None)), 1), (dict(L=0), 1),
    (dict(L=257), 1), (dict(x=None), 1), (dict(buf=FAKE + 4), 1), (dict(hidden=4092), 1),
    (dict(splits=0), 1), (dict(S=5), 1), (dict(a=_ptrs(3, None)), 1), (dict(rank=12), 2),
])
def test_prepare_and_shrink_rejects(kw, status):
    assert _prep_shrink(**kw) == status


EXPAND_OK = dict(buf=FAKE, splits=4, b=3, sizes=(4096, 4096, 4096), S=3, rank=8, y=FAKE,
                 ldy=12288, maxT=256, L=4)


def _expand(**kw):
    a = dict(EXPAND_OK)
    a.update(kw)
    bptr = a["b"] if not isinstance(a["b"], int) else _ptrs(a["b"])
    sizes = (ctypes.c_int32 * len(a["sizes"]))(*a["sizes"]) if a["sizes"] is not None else None
    cfg = a.get("config")
    cfg = ctypes.byref(srg.ExpandConfig(*cfg)) if cfg is not None else None
    return srg.lib().lora_expand(a["buf"], a["splits"], bptr, sizes, a["S"], a["rank"], a["y"],
                                 a["ldy"], _meta(), a["maxT"], a["L"], cfg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(buf=None), 1), (dict(y=None), 1), (dict(y=FAKE + 2), 1), (dict(sizes=None), 1),
    (dict(sizes=(4096, 4096, 4092)), 1), (dict(sizes=(4096, 0, 4096)), 1), (dict(ldy=12280), 1),
    (dict(ldy=12290), 1), (dict(S=0), 1), (dict(S=5), 1), (dict(splits=0), 1),
    (dict(b=_ptrs(3, None)), 1), (dict(rank=80), 1), (dict(rank=24), 2),
    # launch choices out of range
    (dict(config=(-1, -1, 0)), 1), (dict(config=(65, -1, 0)), 1), (dict(config=(0, 2, 0)), 1),
    (dict(config=(0, -2, 0)), 1), (dict(config=(0, -1, 17)), 1), (dict(config=(0, -1, -1)), 1),
    (dict(rank=32, config=(17, -1, 0)), 1),
    # in range, but an unsupported rank still refuses
    (dict(rank=24, config=(4, 1, 2)), 2),
])
def test_expand_rejects(kw, status):
    assert _expand(**kw) == status


def test_stream_copy_rejects():
    L = measure.measure_lib()
    assert L.lora_stream_copy(None, FAKE, 64, None) == 1
    assert L.lora_stream_copy(FAKE, FAKE + 4096, 20, None) == 1
    assert L.lora_stream_copy(FAKE, FAKE + 32, 64, None) == 1  # overlap
    assert L.lora_stream_copy(FAKE, FAKE + 4096, 0, None) == 1
    assert L.lora_stream_update(None, 64, None) == 1
    assert L.lora_stream_update(FAKE + 8, 64, None) == 1
    assert L.lora_stream_update(FAKE, 24, None) == 1


def test_default_splits_is_pure_and_in_range():
    f = srg.lora_shrink_default_splits
    assert f(4096, 256, 4, 3, 8) == f(4096, 256, 4, 3, 8)
    for args in [(4096, 256, 4, 3, 8), (4096, 8192, 4, 2, 16), (11008, 2048, 16, 1, 64),
                 (8192, 4096, 64, 3, 32), (256, 16, 2, 1, 8), (8, 1, 1, 1, 8)]:
        v = f(*args)
        assert 1 <= v <= srg.LORA_MAX_SPLITS, args
    assert f(0, 256, 4, 3, 8) == 0
    assert f(4096, 256, 4, 9, 8) == 0


def test_binding_rejects_host_tensors():
    import torch
    meta_like = type("M", (), {"max_tokens": 4, "max_loras": 2})()
    with pytest.raises((TypeError, ValueError)):
        srg.lora_shrink(torch.zeros(4, 8, dtype=torch.bfloat16),
                        [torch.zeros(2, 8, 8, dtype=torch.bfloat16)], 1.0,
                        torch.zeros(1, 1, 4, 8), 1, meta_like)


def test_tuning_candidates():
    from segmented_rank_gemm_amd.tuning import candidate_splits
    for hidden, maxT, L, S, r in [(4096, 256, 4, 3, 8), (11008, 2048, 16, 1, 64), (128, 16, 2, 1, 8),
                                  (256, 16, 2, 1, 8), (8192, 4096, 64, 3, 32), (65536, 1, 1, 4, 16)]:
        c = candidate_splits(hidden, maxT, L, S, r)
        d = srg.lora_shrink_default_splits(hidden, maxT, L, S, r)
        chunks = -(-hidden // 64)
        assert c == sorted(set(c)) and c[0] == 1
        assert d in c
        assert all(1 <= v <= srg.LORA_MAX_SPLITS for v in c)
        assert all(v <= chunks for v in c if v != d)


# ------------------------------------------------------------ lora_fused_step

def test_fused_step_workspace_bytes():
    # one 256-byte counter line per 16-token tile inside the one-launch domain, else none
    assert srg.lora_fused_step_workspace_bytes(256, 4, 3, 8) == 16 * 256
    assert srg.lora_fused_step_workspace_bytes(1, 1, 1, 8) == 256
    assert srg.lora_fused_step_workspace_bytes(512, 8, 2, 8) == 32 * 256
    assert srg.lora_fused_step_workspace_bytes(513, 4, 3, 8) == 0      # too many token slots
    assert srg.lora_fused_step_workspace_bytes(256, 16, 1, 8) == 0     # max_loras * rank > 64
    assert srg.lora_fused_step_workspace_bytes(256, 4, 3, 32) == 0     # rank 32
    assert srg.lora_fused_step_workspace_bytes(256, 4, 4, 16) == 16 * 256  # 4*4*16 = 256 outputs
    assert srg.lora_fused_step_workspace_bytes(256, 4, 4, 16) > 0
    # large batches at rank 32/64: arrival counters (64 bytes per 64-token tile
    # and output group, rounded to 256) and the summed plane S * max_tokens * r
    assert srg.lora_fused_step_workspace_bytes(1024, 16, 1, 64) == 32 * 64 + 1024 * 64 * 4
    assert srg.lora_fused_step_workspace_bytes(4096, 64, 3, 32) == 128 * 64 + 3 * 4096 * 32 * 4
    assert srg.lora_fused_step_workspace_bytes(600, 2, 3, 64) == 12 * 2 * 64 + 3 * 600 * 64 * 4
    assert srg.lora_fused_step_workspace_bytes(4096, 4, 2, 16) == 0     # rank 16: no sums
    assert srg.lora_fused_step_workspace_bytes(0, 4, 3, 8) == 0         # invalid sizes
    assert srg.lora_fused_step_workspace_bytes(256, 4, 5, 8) == 0


def _fused(workspace=FAKE, workspace_bytes=1 << 20, options=None, **kw):
    a = dict(map=FAKE, T=200, x=FAKE, ldx=4096, hidden=4096, S=3, rank=8, scale=1.0, buf=FAKE,
             splits=16, y=FAKE, ldy=12288, maxT=256, L=4, meta=_meta(), n=4096)
    a.update(kw)
    sizes = (ctypes.c_int32 * a["S"])(*([a["n"]] * a["S"]))
    return srg.lib().lora_fused_step(
        a["map"], a["T"], a["x"], a["ldx"], a["hidden"], _ptrs(a["S"]), _ptrs(a["S"]), sizes,
        a["S"], a["rank"], a["scale"], a["buf"], a["splits"], a["y"], a["ldy"], a["meta"],
        workspace, workspace_bytes, options, a["maxT"], a["L"], None)


@pytest.mark.parametrize("kw", [
    dict(workspace=None), dict(workspace=FAKE + 16), dict(workspace_bytes=16 * 256 - 1),
    dict(T=257), dict(T=-1), dict(map=None), dict(meta=_meta(num_runs=None)), dict(x=None),
    dict(y=None), dict(buf=FAKE + 4), dict(ldy=4096), dict(n=12), dict(splits=0), dict(S=0),
    dict(hidden=12),
])
def test_fused_step_rejects(kw):
    assert _fused(**kw) == 1


def test_fused_step_rejects_long_start_delay():
    # lora_step_options_t: wait_polls, then the three ints of the expand's
    # config, then start_delay_ns, part_sums, batch_order_shrink and y_delay_ns
    O = srg._StepOptions
    assert (O.wait_polls.offset, O.expand.offset, O.start_delay_ns.offset,
            O.part_sums.offset, O.batch_order_shrink.offset, O.y_delay_ns.offset) == (
                0, 4, 16, 20, 24, 28)
    assert ctypes.sizeof(O) == 32
    assert _fused(options=ctypes.byref(O(-1, srg.ExpandConfig(), 100001, 0, 0, -1))) == 1
    assert _fused(options=ctypes.byref(O(-1, srg.ExpandConfig(), -1, 0, 0, 100001))) == 1


def test_step_options_carry_both_hold_offs():
    # the binding's options: explicit hold-offs reach their fields; defaults
    # everywhere mean no options struct at all
    r = srg._step_options(None, None, 2000, None, None, None, False, False, 600)
    o = r._obj
    assert (o.wait_polls, o.start_delay_ns, o.part_sums, o.batch_order_shrink, o.y_delay_ns) == (
        -1, 2000, 0, 0, 600)
    o = srg._step_options(7, None, None, y_delay_ns=None)._obj
    assert (o.wait_polls, o.start_delay_ns, o.y_delay_ns) == (7, -1, -1)
    assert srg._step_options(None, None, None) is None


def test_fused_step_rejects_unsupported_rank():
    # rank 12: valid range, no kernel for it (checked before anything is enqueued)
    assert _fused(rank=12) == 2


def test_fused_step_static_rejects_before_any_lookup():
    # invalid arguments are refused before the library looks up its array
    a = dict(map=FAKE, T=200, x=FAKE, ldx=4096, hidden=4096, S=3, rank=8, buf=FAKE, splits=16,
             y=FAKE, ldy=12288, maxT=256, L=4)
    sizes = (ctypes.c_int32 * 3)(4096, 4096, 4096)
    f = srg.lib().lora_fused_step_static
    assert f(a["map"], 300, a["x"], a["ldx"], a["hidden"], _ptrs(3), _ptrs(3), sizes, 3, 8, 1.0,
             a["buf"], 16, a["y"], a["ldy"], _meta(), None, 256, 4, None) == 1   # T > max_tokens
    assert f(a["map"], 200, a["x"], a["ldx"], a["hidden"], _ptrs(3), _ptrs(3), sizes, 3, 12, 1.0,
             a["buf"], 16, a["y"], a["ldy"], _meta(), None, 256, 4, None) == 2   # rank 12
    assert f(None, 200, a["x"], a["ldx"], a["hidden"], _ptrs(3), _ptrs(3), sizes, 3, 8, 1.0,
             a["buf"], 16, a["y"], a["ldy"], _meta(), None, 256, 4, None) == 1   # no map


@pytest.mark.parametrize("num_tokens,max_tokens,max_loras,meta", [
    (-1, 16, 4, None), (17, 16, 4, None), (4, 16, 257, None), (4, 16, 4, dict(num_runs=None)),
])
def test_prepare_metadata_grouped_rejects(num_tokens, max_tokens, max_loras, meta):
    m = _meta(**(meta or {}))
    assert srg.lib().lora_prepare_metadata_grouped(FAKE, num_tokens, max_tokens, max_loras, m,
                                                   None) == 1
    assert srg.lib().lora_prepare_metadata_grouped(None, 3, 16, 4, _meta(), None) == 1
