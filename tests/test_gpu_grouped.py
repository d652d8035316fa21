"""lora_prepare_metadata_grouped against the oracle and against
lora_prepare_metadata, bit for bit: on batches grouped by adapter (its one-pass
path) and on batches that are not (detected on the device, the general code in
the same launch)."""

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_amd as srg
from tests import gpu_harness as H
from workloads import WORKLOADS, make_fuzz_mapping, make_mapping

pytestmark = pytest.mark.gpu


def _run(fn, mapping, T, maxT, L):
    meta = srg.LoraMeta(maxT, L)
    meta.sorted_token_ids.fill_(-7)
    for t in meta.tensors()[1:]:
        t.fill_(-99)
    m = torch.from_numpy(np.ascontiguousarray(mapping, dtype=np.int32)).cuda()
    fn(m, T, meta)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in zip(H.META_KEYS, meta.tensors())}


def _check(mapping, maxT, L):
    T = len(mapping)
    got = _run(srg.lora_prepare_metadata_grouped, mapping, T, maxT, L)
    H.check_meta(got, oracle.prepare_metadata(mapping, L), T, maxT, mapping=mapping, L=L)
    ref = _run(srg.lora_prepare_metadata, mapping, T, maxT, L)
    nt = int(ref["num_tiles"][0])
    for k in H.META_KEYS:
        a, b = got[k], ref[k]
        if k == "tile_token_ids":
            a, b = a[:16 * nt], b[:16 * nt]
        elif k == "tile_lora":
            a, b = a[:nt], b[:nt]
        assert np.array_equal(a, b), k


def _grouped(ids, rng, order="ascending"):
    """The same multiset of ids, each group contiguous: runs in ascending id
    order, or in a random order of the groups."""
    ids = np.asarray(ids, dtype=np.int64)
    keys = np.unique(ids)
    if order == "shuffled":
        keys = rng.permutation(keys)
    return np.concatenate([ids[ids == k] for k in keys]) if ids.size else ids


@pytest.mark.parametrize("cfg", range(len(WORKLOADS)))
@pytest.mark.parametrize("order", ["ascending", "shuffled"])
def test_grouped_batches_of_the_workloads(cfg, order):
    # each workload's adapter map, regrouped the way a V0 scheduler would
    L = WORKLOADS[cfg]["max_loras"]
    rng = np.random.default_rng(cfg)
    m = make_mapping(cfg)
    ids = np.where((m >= -1) & (m < L), m, -1)
    _check(_grouped(ids, rng, order), len(ids) + 5, L)


@pytest.mark.parametrize("T,maxT,L,kind", [
    (0, 16, 4, "empty"), (1, 1, 1, "one"), (64, 64, 2, "all_none"), (100, 128, 3, "single"),
    (8191, 8192, 5, "runs"), (8192, 8192, 5, "runs"), (8193, 9000, 5, "runs"),  # block edges
    (20000, 20000, 256, "runs"), (1 << 20, (1 << 20) + 3, 256, "runs"),
    (5000, 5000, 64, "extreme"),  # out-of-range ids: part of the no-adapter group
])
def test_grouped_edge_cases(T, maxT, L, kind):
    rng = np.random.default_rng(T + L)
    if kind in ("empty", "one", "all_none", "single"):
        m = {"empty": np.zeros(0), "one": np.array([0]), "all_none": np.full(T, -1),
             "single": np.full(T, L - 1)}[kind]
    else:
        raw = make_fuzz_mapping(rng, T, L, "wild" if kind == "runs" else "extreme")
        ids = np.where((raw >= -1) & (raw < L), raw, -1)
        # keep the raw values (out-of-range ones too) but order them by group
        order = np.argsort(ids, kind="stable")
        m = raw[order]
    _check(np.asarray(m, dtype=np.int64), maxT, L)


@pytest.mark.parametrize("cfg", range(len(WORKLOADS)))
def test_ungrouped_batches_fall_back(cfg):
    # the workloads' own maps are not grouped: same outputs through the fallback
    m = make_mapping(cfg)
    _check(m, len(m) + 3, WORKLOADS[cfg]["max_loras"])


@pytest.mark.parametrize("T,L,kind", [(300, 4, "wild"), (4096, 64, "runs"), (9000, 7, "wild"),
                                      (777, 255, "single"), (3000, 16, "extreme")])
def test_ungrouped_fuzz_falls_back(T, L, kind):
    rng = np.random.default_rng(T * 3 + L)
    _check(make_fuzz_mapping(rng, T, L, kind), T + 1, L)


def test_one_group_split_late():
    # grouped except for one group that reappears at the very end, in a second
    # block of the map: the duplicate run is found after the first block
    L = 6
    m = np.concatenate([np.full(5000, 2), np.full(4000, 0), np.full(300, -1), np.full(10, 2)])
    _check(m, len(m), L)
    # exactly one more run than groups
    m2 = np.array([0, 1, 0, 1, 2, -1], dtype=np.int64)
    _check(m2, 8, 3)
