"""Route table: histogram, prefix and stable scatter (integer, plain loops).

"perf(ds4): batch heterogeneous MoE prefill by expert", Summary: the prefill
groups routed tokens by expert with a route histogram, a prefix over it and a
scatter into expert-major order, for up to 256 experts.  The order inside one
expert's segment is the route order (r = t*k + j), which keeps the
selected-row order ("perf(ds4): extend sparse prefill scheduling to 10K",
Summary of the earlier description).

Readings (the pages give no formulas):
* key[r] = topk_ids[r] if route r is active, else E.  Masked routes fill a
  trailing bin E and are never computed, so counts sum to T*k.
* An active route whose id lies outside [0, E) is treated as masked.
* offsets has E+2 entries: offsets[0] = 0, offsets[b+1] = offsets[b] + counts[b].
* sorted_routes[offsets[key[r]] + #{r' < r : key[r'] = key[r]}] = r, and
  route_rows is its inverse permutation.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

import numpy as np


class RouteTable(NamedTuple):
    counts: np.ndarray  # int32 [E+1]
    offsets: np.ndarray  # int32 [E+2]
    sorted_routes: np.ndarray  # int32 [T*k]
    route_rows: np.ndarray  # int32 [T*k]


def route_keys(topk_ids: np.ndarray, route_mask: Optional[np.ndarray], E: int) -> list:
    ids = np.asarray(topk_ids).reshape(-1).tolist()
    if route_mask is None:
        act = [True] * len(ids)
    else:
        act = (np.asarray(route_mask).reshape(-1) != 0).tolist()
    keys = []
    for r, e in enumerate(ids):
        keys.append(e if (act[r] and 0 <= e < E) else E)
    return keys


def route_table(topk_ids: np.ndarray, route_mask: Optional[np.ndarray], E: int) -> RouteTable:
    keys = route_keys(topk_ids, route_mask, E)
    R = len(keys)
    counts = [0] * (E + 1)
    for b in keys:
        counts[b] += 1
    offsets = [0] * (E + 2)
    for b in range(E + 1):
        offsets[b + 1] = offsets[b] + counts[b]
    fill = offsets[: E + 1]
    fill = list(fill)
    sorted_routes = [0] * R
    for r, b in enumerate(keys):
        sorted_routes[fill[b]] = r
        fill[b] += 1
    route_rows = [0] * R
    for i, r in enumerate(sorted_routes):
        route_rows[r] = i
    return RouteTable(
        counts=np.asarray(counts, dtype=np.int32),
        offsets=np.asarray(offsets, dtype=np.int32),
        sorted_routes=np.asarray(sorted_routes, dtype=np.int32),
        route_rows=np.asarray(route_rows, dtype=np.int32),
    )
