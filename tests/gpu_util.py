"""Helpers for the GPU tests: device placement and controlled routings."""
import numpy as np


def torch_dev():
    import torch

    return torch.device("cuda:0")


def bf16_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch_dev())


def np_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def routing_with_counts(counts, k, seed, masked_extra=0, invalid_extra=0):
    """ids [T,k], mask [T,k] such that expert e receives exactly counts[e] active
    routes (duplicates inside a token are allowed); masked_extra masked routes
    and invalid_extra active routes with out-of-range ids fill the rest."""
    rng = np.random.default_rng(seed)
    E = len(counts)
    act = np.repeat(np.arange(E, dtype=np.int32), counts)
    n = act.size + masked_extra + invalid_extra
    T = max(1, -(-n // k))
    pad = T * k - n
    masked_extra += pad
    ids = np.concatenate([act, rng.integers(0, E, masked_extra).astype(np.int32),
                          np.full(invalid_extra, E + 3, np.int32)])
    mask = np.concatenate([np.ones(act.size, np.uint8), np.zeros(masked_extra, np.uint8),
                           np.ones(invalid_extra, np.uint8)])
    perm = rng.permutation(ids.size)
    return ids[perm].reshape(T, k), mask[perm].reshape(T, k)


def rel_frob(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
