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
