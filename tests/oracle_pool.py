"""Oracle runs of many requests in parallel, for the GPU parity tests.

Each request of a batched workload is integrated by the oracle alone (batch
1), on a thread of its own with single-threaded BLAS: the oracle's time goes
into NumPy matrix products, which release the interpreter lock, so requests
run side by side on the host's cores.  Test infrastructure only."""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np
from threadpoolctl import threadpool_limits

from oracle import ae_oracle as O


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def per_request(w, W, K, V, m, x0, requests: Sequence[int], steps: Optional[int] = None,
                perturb: Optional[float] = None, seed: int = 11) -> List[Tuple[np.ndarray, Optional[float]]]:
    """For each request b: (oracle actions [1, T, A], floor), where floor is
    the oracle's own max change when the noise is perturbed by a relative
    ``perturb`` (None: not computed).  Masked rows are never read."""
    w1 = dataclasses.replace(w, batch=1)
    E = O.Expert(W, O.Params.like(w1))
    n = w.n_steps if steps is None else steps

    def one(b):
        Kb, Vb, mb, xb = K[:, b:b + 1], V[:, b:b + 1], m[b:b + 1], x0[b:b + 1]
        ref = E.denoise(xb, Kb, Vb, mb, n)
        floor = None
        if perturb is not None:
            rng = np.random.default_rng(seed)
            x1 = (xb * (1.0 + perturb * rng.standard_normal(xb.shape))).astype(np.float32)
            floor = float(np.abs(E.denoise(x1, Kb, Vb, mb, n) - ref).max())
        return ref, floor

    def logged(b):
        r = one(b)
        print(f"[oracle] request {b} integrated", flush=True)  # progress for long batches
        return r

    with threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
            return list(ex.map(logged, requests))
