"""Write the stored expected values under tests/golden/.

Only the seeded generator and the oracle are called here; no value comes from
the HIP path. Run from the repository root:  python tests/golden/make_golden.py

* inputs_sha256.json  SHA-256 of each workload's first 2^20 elements (pins the
                      generator against accidental change).
* counts_sha256.json  SHA-256 of the oracle's uint32 counts for each workload
                      at 2^20 elements, and the full-size first workload.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from partitioned_chip_accumulation_amd import inputs  # noqa: E402

N_SMALL = 1 << 20


def main():
    ins, cnt = {}, {}
    for cfg, w in inputs.WORKLOADS.items():
        x = inputs.generate(cfg, n=N_SMALL)
        ins[str(cfg)] = {"n": N_SMALL, "sha256": hashlib.sha256(x.tobytes()).hexdigest()}
        counts, dropped = oracle.hist(x, w.num_bins)
        cnt[str(cfg)] = {"n": N_SMALL, "num_bins": w.num_bins, "dropped": dropped,
                         "sha256": hashlib.sha256(counts.tobytes()).hexdigest()}
    note = "written by tests/golden/make_golden.py from the generator and the oracle only"
    with open(os.path.join(HERE, "inputs_sha256.json"), "w") as f:
        json.dump({"note": note, "inputs": ins}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "counts_sha256.json"), "w") as f:
        json.dump({"note": note, "counts": cnt}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
