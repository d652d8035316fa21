"""Write tests/golden/tiny_exact.json from the exact-rational brute force.

The values come only from ``oracle.bruteforce`` (exact arithmetic) on inputs
drawn by the seeded generator; no GPU result is ever stored here.
Run: python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import bruteforce as bf  # noqa: E402
from workloads import make_custom_workload  # noqa: E402

SPEC = dict(seed=41, num_tokens=5, hidden=8, slices=[8, 4], rank=2, max_loras=3, scale=1.25,
            mapping=[2, -1, 0, 2, 1])


def main():
    s = SPEC
    w = make_custom_workload(s["seed"], s["num_tokens"], s["hidden"], s["slices"], s["rank"],
                             s["max_loras"], s["scale"], np.array(s["mapping"]))
    meta = bf.metadata(w.mapping, w.max_loras)
    buf, y = bf.lora_exact(w.mapping, w.x, w.lora_a, w.lora_b, w.y0, w.max_loras, w.rank,
                           float(np.float32(w.scale)))
    out = dict(s)
    out["_source"] = ("oracle.bruteforce exact rationals on workloads.make_custom_workload "
                      "inputs; written by tests/golden/make_golden.py")
    out["sorted_token_ids"] = meta["sorted_token_ids"]
    out["y_exact"] = [[str(v) for v in row] for row in y]
    out["y_bf16"] = [[bf.fraction_to_bf16(v) for v in row] for row in y]
    with open(os.path.join(HERE, "tiny_exact.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
