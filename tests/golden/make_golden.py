"""Write the stored values derived from the oracle (run on the CPU; calls only
oracle/ and the input generators).

fp4_global_scale.json: the global scale of each FP4 workload with E4M3 block
scales, gs = fp32(448 * 6 / max|y|) with max|y| taken by the float64 oracle
over the whole tensor (the calibration step a deployment would run once; for
the residual workload y is the normalized pre-norm sum).  The FP4 page takes
gs as an input and describes it as lifting per-block scales into the E4M3
range; with this gs the largest block scale is exactly 448.  Workloads that
share an input tensor share the value.
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

CHUNK = 1024  # rows per oracle call for the residual workload (bounds memory)


def global_amax(w) -> float:
    inp = workloads.make(w)
    x, g = workloads.bits(inp["x"]), workloads.bits(inp["gamma"])
    kw = dict(in_dtype=w.in_dtype, eps=w.eps, weight_offset=w.weight_offset)
    if inp["residual"] is None:
        return oracle.absmax(x, g, **kw)
    r = workloads.bits(inp["residual"])
    return max(float(np.abs(oracle.rmsnorm_y(x[i:i + CHUNK], g, residual=r[i:i + CHUNK], **kw)["y"]).max())
               for i in range(0, w.rows, CHUNK))


def main():
    t0 = time.time()
    scales = {}
    for name, w in workloads.WORKLOADS.items():
        if not w.fp4 or w.fp4_scale != "e4m3":
            continue
        amax = global_amax(w)
        scales[name] = {"global_amax": amax, "global_scale": float(np.float32(448.0 * 6.0 / amax))}
    out = {"seed": 0, "definition": "gs = fp32(448 * 6 / max|y|), max over the whole tensor, float64 oracle",
           "workloads": scales}
    with open(os.path.join(HERE, "fp4_global_scale.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out), f"({time.time() - t0:.1f} s)")


if __name__ == "__main__":
    main()
