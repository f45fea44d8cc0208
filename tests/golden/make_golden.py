"""Write the stored values derived from the oracle (run on the CPU; calls only
oracle/ and the input generators).

fp4_global_scale.json: the global scale of the 16384 x 7168 FP4 workload,
gs = fp32(448 * 6 / max|y|) with max|y| taken by the float64 oracle over the
whole tensor (the calibration step a deployment would run once).  The FP4
page takes gs as an input and describes it as lifting per-block scales into
the E4M3 range; with this gs the largest block scale is exactly 448.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

NAME = "rmsnorm_fp4_bf16_16384x7168"


def main():
    t0 = time.time()
    inp = workloads.make(NAME)
    w = inp["workload"]
    amax = oracle.absmax(workloads.bits(inp["x"]), workloads.bits(inp["gamma"]), in_dtype=w.in_dtype,
                         eps=w.eps, weight_offset=w.weight_offset)
    gs = float(np.float32(448.0 * 6.0 / amax))
    out = {"workload": NAME, "seed": 0, "global_amax": amax, "global_scale": gs,
           "definition": "gs = fp32(448 * 6 / max|y|), max over the whole tensor, float64 oracle"}
    with open(os.path.join(HERE, "fp4_global_scale.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out), f"({time.time() - t0:.1f} s)")


if __name__ == "__main__":
    main()
