"""Write tests/golden/digests.json: SHA-256 digests of each workload's
generated inputs and of the oracle's output for them.

Calls only ``workloads`` (input generation) and ``oracle`` (the expected
output); nothing from the HIP path. Run from the repository root:

    python tests/golden/make_digests.py
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def input_digest(xs, ss) -> str:
    h = hashlib.sha256()
    for x in xs:
        h.update(np.ascontiguousarray(x).tobytes())
    for s in ss:
        h.update(np.ascontiguousarray(s).tobytes())
    return h.hexdigest()


def output_digest(out) -> str:
    return hashlib.sha256(np.ascontiguousarray(out).tobytes()).hexdigest()


def main():
    result = {
        "about": "SHA-256 of each workload's inputs (x slices of ranks 0..W-1, then their scale slices, raw bytes) "
                 "and of the oracle's output (float32 or bf16 bit patterns, little-endian, row-major). "
                 "Written by tests/golden/make_digests.py from workloads.generate and oracle.reduce_scatter_share.",
        "configs": {},
    }
    for name, wl in workloads.WORKLOADS.items():
        xs, ss = workloads.generate(wl)
        out = oracle.reduce_scatter_share(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
        result["configs"][name] = {
            "inputs_sha256": input_digest(xs, ss),
            "output_sha256": output_digest(out),
            "out_dtype": wl.out_dtype,
            "shape": [wl.rows, wl.h],
        }
        print(name, result["configs"][name]["output_sha256"], flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "digests.json"), "w") as f:
        json.dump(result, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
