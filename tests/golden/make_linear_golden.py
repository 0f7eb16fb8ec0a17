"""Write the FP64 oracle's per-token results for the full-size linear
cross-entropy workloads (M=4096, H=4096, V=131072 with BF16 and with FP32
inputs, and M=16384, H=2304, V=256003) to tests/golden/*.npz.

Calls only the oracle package and the seeded input generators; no value here
comes from the GPU path.  The stored digest of the inputs lets the tests
confirm that they regenerated the same bytes.

    python tests/golden/make_linear_golden.py [linear_4k linear_16k linear_4k_f32]
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import linear  # noqa: E402
from vocabulary_cross_entropy_amd import workloads as wl  # noqa: E402


def digest(case) -> str:
    h = hashlib.sha256()
    for a in (case.X, case.W, case.targets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main(names=None):
    for fn in (wl.linear_4k, wl.linear_16k, wl.linear_4k_f32):
        if names and fn.__name__ not in names:
            continue
        t0 = time.time()
        case = fn()
        loss, stats, lse = linear.forward(case.X, case.W, case.targets, case.label_smoothing,
                                          case.ignore_idx, token_chunk=1024)
        out = os.path.join(HERE, case.name + ".npz")
        np.savez_compressed(out, loss=loss, lse=lse, stats=stats, digest=np.array(digest(case)))
        print(f"{out}: {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
