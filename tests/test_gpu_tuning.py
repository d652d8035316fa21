"""Every entry of the measured launch-choice table gives parity: the table's
part count and expand choices on a batch of the entry's shape, through
lora_fused_step, against the oracle."""

import numpy as np
import pytest
import torch

import segmented_rank_gemm_amd as srg
from segmented_rank_gemm_amd.tuning import load_table
from tests import gpu_harness as H
from workloads import make_custom_workload

pytestmark = pytest.mark.gpu

TABLE = load_table()


@pytest.mark.parametrize("key", sorted(TABLE))
def test_table_entry_parity(key):
    e = TABLE[key]
    sh = e["shape"]
    T = sh["max_tokens"]
    print(f"[table] {key} splits={e['num_splits']} expand={e['expand']}", flush=True)
    rng = np.random.default_rng(len(key))
    mapping = rng.integers(-1, sh["max_loras"], size=T)
    w = make_custom_workload(len(key), T, sh["hidden"], sh["slices"], sh["rank"], sh["max_loras"],
                             1.0, mapping)
    d = H.upload(w, num_splits=e["num_splits"])
    ws = srg.fused_step_workspace(T, sh["max_loras"], len(sh["slices"]), sh["rank"])
    srg.lora_fused_step(d.mapping, T, d.x, d.lora_a, d.lora_b, 1.0, d.buf, d.num_splits, d.y,
                        d.meta, ws, expand_config=srg.ExpandConfig(**e["expand"]))
    torch.cuda.synchronize()
    H.full_check(w, d)
    # the binding's default takes the same choices from the table
    assert srg._expand_config("table", d.lora_b, d.num_splits, d.meta).as_dict() == e["expand"]


@pytest.mark.parametrize("T,hidden,slices,rank,L,splits,configs", [
    (3000, 1024, [1000, 256], 16, 4, 4, [(1, 0, 1), (3, 1, 2), (8, 0, 3), (2, 1, 8)]),
    (300, 512, [512, 128], 8, 3, 2, [(1, 0, 0), (5, 1, 2), (8, 1, 8)]),
    (2500, 2048, [1024], 64, 9, 6, [(2, 1, 1), (5, 0, 2), (16, 1, 3)]),
    (1800, 1024, [640, 128, 128], 32, 12, 3, [(3, 0, 1), (7, 1, 3), (16, 0, 2)]),
])
def test_expand_configs_same_bits(T, hidden, slices, rank, L, splits, configs):
    """lora_expand's launch choices (range length, unit order, workgroups per
    CU) change no bit of y: each setting against the library's rules on the
    same parts, and the rules against the oracle."""
    rng = np.random.default_rng(T + rank)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T + 2, T, hidden, slices, rank, L, 0.75, mapping)
    d = H.upload(w, num_splits=splits)
    srg.lora_prepare_and_shrink(d.mapping, T, d.x, d.lora_a, float(w.scale), d.buf, splits, d.meta)
    y0 = d.y.clone()
    srg.lora_expand(d.buf, splits, d.lora_b, d.y, d.meta, config=None)
    torch.cuda.synchronize()
    ref = H.from_dev_bf16(d.y)
    H.full_check(w, d)
    for cpr, order, wpc in configs:
        d.y.copy_(y0)
        srg.lora_expand(d.buf, splits, d.lora_b, d.y, d.meta,
                        config=srg.ExpandConfig(cpr, order, wpc))
        torch.cuda.synchronize()
        assert np.array_equal(ref, H.from_dev_bf16(d.y)), (cpr, order, wpc)
