"""Writes the stored oracle outputs under tests/golden/ (calls only oracle/ and
the seeded generator). Run from the repository root:

    python tests/golden/make_golden.py

The pages print no worked example values, so these files are regression pins
of the oracle itself: a later change to its arithmetic must either reproduce
them or come with a regenerated file and the passage that justifies it.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as wl  # noqa: E402
from oracle import runs  # noqa: E402


def write_hex(path, header, arrays):
    with open(path, "w") as f:
        for line in header:
            f.write("# " + line + "\n")
        for name, a in arrays:
            a = np.asarray(a, dtype=np.float16).ravel()
            f.write(f"{name} {a.size} " + " ".join(f"{int(v):04x}" for v in a.view(np.uint16)) + "\n")


def main():
    w = wl.layer_mini()
    x = w.x_in().astype(np.float64)
    out, kp, vp = runs.layer_batch(w, 0, x)
    pos = int(w.positions[0])
    page, slot = int(w.page_tables[0][pos // 16]), pos % 16
    write_hex(os.path.join(HERE, "layer_mini_oracle.txt"),
              ["oracle output of one miniature decoder layer (hidden 448, 7 q heads : 1 kv head,",
               "head_dim 64, FFN 1536), batch 1, 64-token context in 4 shuffled pages, seeded",
               "inputs of workloads.layer_mini(); written by tests/golden/make_golden.py.",
               "fields: name count fp16-bits(hex)..."],
              [("x_out", out[0]), ("k_slot", kp[page, :, slot]), ("v_slot", vp[page, :, slot])])


if __name__ == "__main__":
    main()
