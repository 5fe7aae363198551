"""Seeded random chunk-step shapes for the GPU parity sweep
(test_gpu_fuzz.py): every supported head dim, page size, GQA group and dtype,
with the edge cases the method has (no prior pages, K = 0, K >= N, a
one-page chunk, spare pool slots, a softmax-scale override) drawn at fixed
rates.  Sizes stay small enough that the fp64 oracle checks every output
element in well under a second per case."""
from __future__ import annotations

import numpy as np

from synth import Problem

N_CASES = 64
SEED = 20261203


def cases(n: int = N_CASES, seed: int = SEED):
    """[(case seed, Problem)] -- deterministic for a given (n, seed)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        d = int(rng.choice([64, 128]))
        ps = int(rng.choice([16, 32, 64, 128]))
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        while hkv * d > 1024:
            hkv //= 2
        g = int(rng.choice([1, 2, 3, 4, 7, 8]))
        hq = hkv * g
        chunk_pages = int(rng.integers(1, 5))
        c = chunk_pages * ps
        u = rng.random()
        if u < 0.1:
            n, k = 0, int(rng.integers(0, 5))             # first chunk: nothing to select from
        else:
            n = int(rng.integers(1, 40))
            v = rng.random()
            k = 0 if v < 0.1 else (n + int(rng.integers(0, 4)) if v < 0.25 else int(rng.integers(1, n + 1)))
        extra = int(rng.integers(0, 6)) if rng.random() < 0.3 else 0
        scale = float(rng.choice([0.05, 0.1])) if rng.random() < 0.15 else 0.0
        p = Problem(hq=hq, hkv=hkv, d=d, ps=ps, c=c, n=n, k=k, dtype=dtype,
                    n_slots=(n + chunk_pages + extra) if extra else 0, scale=scale)
        out.append((1000 + i, p))
    return out
