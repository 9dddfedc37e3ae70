"""Top-k expert selection and gates from router logits (fp64, plain loops).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages keep the model's native top-6 routing and the selected-row order
unchanged ("perf(ds4): extend sparse prefill scheduling to 10K", Summary) but
never state the router's arithmetic.  The reading taken here, which is also
how the synthetic workloads define their routing:

* z[e] = fp32(logits[e] + bias[e]) (bias optional; the addition is one fp32
  rounding, as a router that adds a bias in fp32 would do);
* the k selected experts are the k largest z, in descending order of z; equal
  z go to the lower expert index first (so the result is unique);
* gates are the softmax restricted to the selected experts,
  g_j = exp(z_j - z_max) / sum_i exp(z_i - z_max) over the selected i, where
  z_max is the largest z (the top-1).  The full softmax denominator cancels.
  Evaluated in fp64 and rounded once to fp32.

Logits are finite (NaN has no place in an order); -inf is allowed and gets a
zero gate unless every selected logit is -inf.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


def _f32(v: float) -> float:
    return float(np.float32(v))


def select_topk_row(z: list, k: int) -> list:
    """Indices of the k largest values of z, descending, ties to the lower index.

    Repeated selection of the best remaining index: index a beats index b when
    z[a] > z[b], or z[a] == z[b] and a < b.
    """
    taken = [False] * len(z)
    out = []
    for _ in range(k):
        best = -1
        for e in range(len(z)):
            if taken[e]:
                continue
            if best < 0 or z[e] > z[best]:
                best = e
        taken[best] = True
        out.append(best)
    return out


def route_topk(logits: np.ndarray, bias: Optional[np.ndarray], k: int) -> Tuple[np.ndarray, np.ndarray]:
    """topk_ids int32 [T, k] and topk_w fp32 [T, k] from logits fp32 [T, E]."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    b = None if bias is None else np.asarray(bias, dtype=np.float32).reshape(E)
    ids = np.zeros((T, k), dtype=np.int32)
    gates = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        row = lg[t].tolist()
        z = [_f32(row[e] + float(b[e])) for e in range(E)] if b is not None else row
        sel = select_topk_row(z, k)
        zmax = z[sel[0]]
        p = [math.exp(z[e] - zmax) for e in sel]
        s = 0.0
        for v in p:
            s += v
        for j, e in enumerate(sel):
            ids[t, j] = e
            gates[t, j] = np.float32(p[j] / s)
    return ids, gates
