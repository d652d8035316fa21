"""The committed launch-choice table (no GPU needed): it covers the benchmark's
four workloads, its keys are the shapes it describes, every choice is inside
the range the C ABI accepts, and plan() hands it out."""

import segmented_rank_gemm_amd as srg
from segmented_rank_gemm_amd.tuning import load_table, plan, shape_key
from workloads import WORKLOADS, make_workload


def test_table_covers_the_benchmark_workloads():
    table = load_table()
    for c in range(1, len(WORKLOADS)):
        cfg = WORKLOADS[c]
        key = shape_key(cfg["hidden"], cfg["num_tokens"], cfg["max_loras"], cfg["slices"],
                        cfg["rank"])
        assert key in table, key
        p = plan(cfg["hidden"], cfg["num_tokens"], cfg["max_loras"], cfg["slices"], cfg["rank"])
        assert p["source"] == "table" and p["num_splits"] == table[key]["num_splits"]


def test_table_entries_are_valid():
    for key, e in load_table().items():
        sh = e["shape"]
        assert key == shape_key(sh["hidden"], sh["max_tokens"], sh["max_loras"], sh["slices"],
                                sh["rank"])
        assert 1 <= e["num_splits"] <= srg.LORA_MAX_SPLITS
        x = e["expand"]
        max_cpr = 16 if sh["rank"] >= 32 else 64
        assert 0 <= x["chunks_per_range"] <= max_cpr
        assert x["range_fastest"] in (-1, 0, 1)
        assert 0 <= x["workgroups_per_cu"] <= 16
        # hold-offs: the library's default (None) or inside what the ABI accepts
        for k in ("start_delay_ns", "y_delay_ns"):
            assert e[k] is None or 0 <= e[k] <= 100000, (key, k)
        # the measured choice is no slower than the rule it replaces
        assert e["step_us"] <= e["rule"]["step_us"] + 1e-9


def test_plan_falls_back_to_the_rule():
    p = plan(4096, 300, 4, [4096], 8)  # a shape the table does not hold
    assert p["source"] == "size rule" and p["expand"] is None
    assert p["num_splits"] == srg.lora_shrink_default_splits(4096, 300, 4, 1, 8)
    assert make_workload(1).max_tokens == WORKLOADS[1]["num_tokens"]
