"""Writes tests/golden/input_sha256.txt: the SHA-256 of the q, k and v bytes
that seeded_inputs.make_workload gives for each named workload.  It calls
only seeded_inputs (no attention arithmetic, no GPU code); the file pins the
input recipe, so a change of generator, draw order, dtype cast or seed shows
up as a hash mismatch in tests/test_seeded_inputs.py.

    python tests/golden/make_input_sha256.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import seeded_inputs as si  # noqa: E402

NAMES = [w.name for w in si.WORKLOADS] + [w.name for w in si.FP8_WORKLOADS]


def main():
    lines = ["# SHA-256 of the q, k, v bytes of each workload (seeded_inputs.make_workload);",
             "# written by tests/golden/make_input_sha256.py.  Columns: workload q k v"]
    for name in NAMES:
        q, k, v = si.make_workload(si.BY_NAME[name])
        lines.append(" ".join([name, si.sha256(q), si.sha256(k), si.sha256(v)]))
        print(lines[-1], flush=True)
    with open(os.path.join(HERE, "input_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
