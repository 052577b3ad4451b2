"""Hash of the HIP library's sources (csrc/*.hip, csrc/*.h, include/*.h).

HBM traffic counted with rocprofv3 belongs to the kernels as they were
built; a recorded traffic figure is only reported while this hash is
unchanged."""
from __future__ import annotations

import glob
import hashlib
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)


def source_sha() -> str:
    files = sorted(glob.glob(os.path.join(_HERE, "csrc", "*.hip")) +
                   glob.glob(os.path.join(_HERE, "csrc", "*.h")) +
                   glob.glob(os.path.join(_ROOT, "include", "*.h")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
