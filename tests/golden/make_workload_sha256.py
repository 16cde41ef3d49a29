"""Write workload_sha256.txt: SHA-256 fingerprints of every array the seeded
input generator produces for the five named workloads (little-endian float64
bytes in the field layout [ny, nz, nx]; alpha_h as [ny, nx]).  They pin the
generator: any change to the synthetic inputs shows up as a changed digest.
Calls only matrix_free_pcg_amd.workloads (no solver arithmetic, no GPU).

    python tests/golden/make_workload_sha256.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from matrix_free_pcg_amd import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "workload_sha256.txt")


def digest(a) -> str:
    a = np.ascontiguousarray(np.asarray(a, dtype="<f8"))
    return hashlib.sha256(a.tobytes()).hexdigest()


def fingerprints(cfg: int):
    w = W.make_workload(cfg)
    p = w.problem
    if isinstance(p, W.GeneralProblem):
        rows = [(w.name, name, np.shape(getattr(p, name)), digest(getattr(p, name)))
                for name in ("a", "d", "beta_face", "area", "alpha_x", "alpha_y")]
    else:
        rows = [(w.name, "alpha_z_face", (p.nz + 1,), digest(p.alpha_z_face)),
                (w.name, "alpha_h", (p.ny, p.nx), digest(p.alpha_h_field()))]
    if w.rhs is not None:
        rows.append((w.name, "rhs", w.rhs.shape, digest(w.rhs)))
    if w.x_true is not None:
        rows.append((w.name, "x_true", w.x_true.shape, digest(w.x_true)))
    return rows


def main():
    lines = ["# workload array fingerprints: name, array, shape, sha256 of little-endian float64 bytes",
             "# written by tests/golden/make_workload_sha256.py"]
    for cfg in sorted(W.CONFIG_NAMES):
        for name, arr, shape, h in fingerprints(cfg):
            lines.append(f"{name} {arr} {'x'.join(map(str, shape))} {h}")
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
