"""Runs the unchanged CPU oracle over many independent inputs at once.

The oracle is plain single-threaded C; its functions are called through
ctypes, which releases the GIL for the duration of each call, so host
threads give full-size parity checks the machine's cores without touching
the oracle's arithmetic. Each unit of work is one whole oracle call on one
input (a tensor to encode, or a set of rows of X: row m of X.W depends on
row m of X only).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers():
    """Host threads to use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def gemm_f64_rows(orc, X, W, nthreads=None):
    """orc.gemm_f64(X, W) computed as independent calls on contiguous row
    ranges of X, one per thread; returns (Y, absbound) like orc.gemm_f64."""
    X = np.ascontiguousarray(X)
    M = X.shape[0]
    t = min(nthreads or workers(), M)
    bounds = [M * i // t for i in range(t + 1)]
    with ThreadPoolExecutor(t) as ex:
        parts = list(ex.map(lambda i: orc.gemm_f64(X[bounds[i]:bounds[i + 1]], W), range(t)))
    return np.vstack([p[0] for p in parts]), np.vstack([p[1] for p in parts])
