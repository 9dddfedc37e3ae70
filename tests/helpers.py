"""Small shared helpers for the tests (no arithmetic of the path lives here)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_pairs(name):
    """Rows of a golden fixture: list of whitespace-split token lists, comments dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def rel_frob(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def small_problem(seed, T, E, k, d, f, fp8=False, mask_p=0.2, x_std=1.0, w_std=0.05):
    """Random small inputs with the generator's formats, independent of any workload."""
    import torch

    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] if k <= E else rng.integers(0, E, k) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    mask = (rng.random((T, k)) >= mask_p).astype(np.uint8)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32) * np.float32(x_std))
    xb = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    weights = {}
    shapes = {"wg": (E, f, d), "wu": (E, f, d), "wd": (E, d, f)}
    for n, shp in shapes.items():
        z = rng.standard_normal(shp).astype(np.float32)
        if fp8:
            z = np.clip(z * 112.0, -448, 448).astype(np.float32)
            weights[n] = torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            weights[n] = torch.from_numpy(z * np.float32(w_std)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if fp8:
        for n, src in (("sg", "wg"), ("su", "wu"), ("sd", "wd")):
            E_, r, c = shapes[src]
            weights[n] = (rng.uniform(0.5, 2.0, (E_, r // 128, c // 128)) * (w_std / 112.0)).astype(np.float32)
    return ids, w, mask, xb, weights
