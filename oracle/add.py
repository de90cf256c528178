"""Oracle for the persistent element-wise add.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"Implement persistent kernels" (Helion PR #238), example output, PERSISTENT
BLOCKED KERNEL: each tile loads x and y (masked) and stores x + y.  For fp32
inputs that is one IEEE binary32 add, rounded to nearest even, per element;
the library routine numpy.add in float32 is exactly that.
"""
from __future__ import annotations

import numpy as np


def add_f32(X: np.ndarray, Y: np.ndarray) -> np.ndarray:
    X = np.asarray(X, dtype=np.float32)
    Y = np.asarray(Y, dtype=np.float32)
    if X.shape != Y.shape:
        raise ValueError("shape mismatch")
    return np.add(X, Y, dtype=np.float32)
