"""Writes the stored oracle outputs under tests/golden/.  Calls only the CPU oracle and the
seeded input generator; nothing from the GPU path.

    python tests/golden/make_golden.py
"""
import json
import pathlib
import sys

HERE = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(HERE.parent.parent))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    wl = workloads.workload("tiny_f32")
    inp = workloads.make_inputs(wl, seed=0)
    y = oracle.ss2d_forward(*[inp[k] for k in ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds",
                                              "dt_bias")], threads=1)
    meta = {
        "what": "float64 oracle output y (B, D, H, W) of the four-route SS2D forward "
                "operator on the seeded tiny workload; a regression anchor for the oracle, "
                "not a value printed by the pages (they print no worked example)",
        "workload": wl.name,
        "seed": 0,
        "shape": list(y.shape),
        "y": [float(v) for v in y.reshape(-1)],
    }
    (HERE / "tiny_f32.json").write_text(json.dumps(meta, indent=0) + "\n")


if __name__ == "__main__":
    main()
