"""Seeded synthetic inputs for routed-MoE prefill.

This module only draws inputs.  It holds none of the path's arithmetic (no
histogram, scan, scatter, GEMM, SwiGLU, quantisation of activations or
combine): the oracle and the HIP path both consume what it returns.

Workloads follow the routed-expert setting of the pages: a DeepSeek-V4 style
MoE layer with top-6 routing over up to 256 experts ("perf(ds4): batch
heterogeneous MoE prefill by expert", Summary), at the prompt lengths the pages
measure (401 and 2048 tokens, same page, requalification table) and an
8192-token prefill chunk ("perf(ds4): unify gfx1151 sparse-prefill stack",
Qualification switches).

The router that produces ``topk_ids`` / ``topk_w`` is part of input
generation: softmax over fp32 logits, the top-k experts by descending logit
(ties go to the lower expert index), gates renormalised over the selected k
and rounded to fp32.  Masks are i.i.d. Bernoulli per (token, route) drawn after
routing; a masked route keeps its id and gate but must contribute exactly zero.

Draw order, all from ``numpy.random.Generator(PCG64)``:
  main stream ``SeedSequence(seed)``: logits [T,E] N(0,1) fp32; the per-expert
  bias (bias workloads only); the mask uniforms [T,k]; x [T,d] N(0,1) fp32.
  Expert e has its own stream ``SeedSequence(seed, spawn_key=(e,))`` so one
  expert can be regenerated alone: gate [f,d], up [f,d], down [d,f] normals,
  then (fp8 only) the three block-scale grids.

bf16 values are produced by torch's CPU float32 -> bfloat16 conversion
(round-to-nearest-even) and returned as uint16 bit patterns.  fp8 weight codes
are torch's CPU float32 -> float8_e4m3fn conversion of clamp(112 z, +-448)
returned as uint8 codes; block scales are U[0.5, 2) * 0.02 / 448 in fp32, one
per 128 x 128 block.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, Optional

import numpy as np

SCALE_BLOCK = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    x_std: float
    w_std: float
    mask_p: float
    routing: str  # "softmax" (plain N(0,1) logits), "bias", "zipf"
    dtype: str  # "bf16" or "fp8"
    bias_std: float = 0.0
    zipf_s: float = 0.0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads.  Names state what each one is.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_T32_d512_f256_E16", T=32, d=512, f=256, E=16, k=6,
                 x_std=0.02, w_std=0.02, mask_p=0.10, routing="softmax", dtype="bf16"),
        Workload("prefill_T401_uniform_bf16", T=401, d=4096, f=2048, E=256, k=6,
                 x_std=1.0, w_std=0.02, mask_p=0.05, routing="softmax", dtype="bf16"),
        Workload("prefill_T2048_biased_bf16", T=2048, d=4096, f=2048, E=256, k=6,
                 x_std=1.0, w_std=0.02, mask_p=0.05, routing="bias", dtype="bf16",
                 bias_std=0.5),
        Workload("prefill_T8192_zipf_bf16", T=8192, d=4096, f=2048, E=256, k=6,
                 x_std=1.0, w_std=0.02, mask_p=0.05, routing="zipf", dtype="bf16",
                 zipf_s=1.2),
        Workload("prefill_T8192_uniform_fp8", T=8192, d=4096, f=2048, E=256, k=6,
                 x_std=1.0, w_std=0.02, mask_p=0.05, routing="softmax", dtype="fp8"),
    ]
}
DEFAULT_BENCH_WORKLOAD = "prefill_T401_uniform_bf16"


@dataclasses.dataclass
class Routing:
    """Routed tokens: ids/gates/mask are [T,k]; x is bf16 bits [T,d]."""

    topk_ids: np.ndarray  # int32 [T,k]
    topk_w: np.ndarray  # float32 [T,k]
    route_mask: np.ndarray  # uint8 [T,k], 1 = active
    x: np.ndarray  # uint16 [T,d] bf16 bit patterns


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns through torch's CPU conversion (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 (already within +-448) -> OCP E4M3FN codes through torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _main_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))


def _expert_rng(seed: int, e: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(e,))))


def _select_topk(z: np.ndarray, k: int):
    """Top-k by descending fp32 logit, ties to the lower index; gates renormalised."""
    order = np.argsort(-z, axis=1, kind="stable")[:, :k]
    zsel = np.take_along_axis(z, order, axis=1).astype(np.float64)
    zmax = z.max(axis=1, keepdims=True).astype(np.float64)
    p = np.exp(zsel - zmax)  # softmax numerators; the full denominator cancels
    gates = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), gates


def _draw_logits(rng, wl: Workload) -> np.ndarray:
    """Router logits with the workload's expert bias added in fp32 (first draws)."""
    T, E = wl.T, wl.E
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if wl.routing == "bias":
        bias = (rng.standard_normal(E, dtype=np.float32) * np.float32(wl.bias_std)).astype(np.float32)
    elif wl.routing == "zipf":
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-wl.zipf_s)
        bias = np.log(p / p.sum()).astype(np.float32)
    else:
        bias = np.zeros(E, dtype=np.float32)
    return (logits + bias[None, :]).astype(np.float32)


def make_logits(wl: Workload, seed: int = 0) -> np.ndarray:
    """fp32 [T, E]: the biased router logits make_routing selects from."""
    return _draw_logits(_main_rng(seed), wl)


def owner_mask(topk_ids: np.ndarray, route_mask: np.ndarray, E: int, G: int, g: int) -> np.ndarray:
    """Route mask of owner g of G when experts are split into G contiguous
    ranges of E/G: a route stays active only if its expert lies in
    [g*E/G, (g+1)*E/G).  Other owners' routes fall into the masked bin."""
    if E % G or not 0 <= g < G:
        raise ValueError("need G | E and 0 <= g < G")
    lo, hi = g * (E // G), (g + 1) * (E // G)
    own = (topk_ids >= lo) & (topk_ids < hi)
    return (route_mask.astype(bool) & own).astype(np.uint8)


def make_routing(wl: Workload, seed: int = 0) -> Routing:
    rng = _main_rng(seed)
    T, E, k, d = wl.T, wl.E, wl.k, wl.d
    z = _draw_logits(rng, wl)
    ids, gates = _select_topk(z, k)
    u = rng.random((T, k))
    mask = (u >= wl.mask_p).astype(np.uint8)
    x = rng.standard_normal((T, d), dtype=np.float32) * np.float32(wl.x_std)
    return Routing(topk_ids=ids, topk_w=gates, route_mask=mask, x=f32_to_bf16_bits(x))


def expert_weights(wl: Workload, e: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """One expert's weights.

    bf16: {"wg": uint16 [f,d], "wu": uint16 [f,d], "wd": uint16 [d,f]}.
    fp8:  {"wg","wu","wd": uint8 codes, "sg","su": fp32 [f/128,d/128], "sd": fp32 [d/128,f/128]}.
    """
    rng = _expert_rng(seed, e)
    f, d = wl.f, wl.d
    shapes = {"wg": (f, d), "wu": (f, d), "wd": (d, f)}
    out: Dict[str, np.ndarray] = {}
    if wl.dtype == "bf16":
        for name, shp in shapes.items():
            z = rng.standard_normal(shp, dtype=np.float32)
            z *= np.float32(wl.w_std)
            out[name] = f32_to_bf16_bits(z)
        return out
    if wl.dtype != "fp8":
        raise ValueError(wl.dtype)
    for name, shp in shapes.items():
        z = rng.standard_normal(shp, dtype=np.float32)
        z *= np.float32(112.0)
        np.clip(z, -448.0, 448.0, out=z)
        out[name] = f32_to_e4m3_codes(z)
    for name, src in (("sg", "wg"), ("su", "wu"), ("sd", "wd")):
        r, c = shapes[src]
        u = rng.uniform(0.5, 2.0, size=(r // SCALE_BLOCK, c // SCALE_BLOCK))
        out[name] = (u * (wl.w_std / 448.0)).astype(np.float32)
    return out


def all_expert_weights(wl: Workload, seed: int = 0, threads: Optional[int] = None,
                       sink: Optional[Callable[[int, Dict[str, np.ndarray]], None]] = None):
    """Generate every expert (in parallel threads).

    With ``sink`` each expert is handed to ``sink(e, weights)`` as soon as it
    is ready (e.g. to copy it to the device) and nothing is kept; otherwise the
    stacked host arrays are returned.
    """
    import os

    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    stacked: Dict[str, np.ndarray] = {}

    def one(e):
        w = expert_weights(wl, e, seed)
        if sink is not None:
            sink(e, w)
            return None
        return w

    with ThreadPoolExecutor(threads) as ex:
        for e, w in enumerate(ex.map(one, range(wl.E))):
            if w is None:
                continue
            for name, a in w.items():
                if name not in stacked:
                    stacked[name] = np.empty((wl.E,) + a.shape, dtype=a.dtype)
                stacked[name][e] = a
    return None if sink is not None else stacked


def weight_bytes_per_expert(wl: Workload) -> int:
    per = 3 * wl.f * wl.d
    if wl.dtype == "bf16":
        return 2 * per
    return per + 3 * 4 * (wl.f // SCALE_BLOCK) * (wl.d // SCALE_BLOCK)


def approx_host_bytes(wl: Workload) -> int:
    return wl.E * weight_bytes_per_expert(wl) + wl.T * wl.d * 2


__all__ = [
    "Workload", "WORKLOADS", "DEFAULT_BENCH_WORKLOAD", "Routing", "make_routing", "make_logits",
    "owner_mask",
    "expert_weights", "all_expert_weights", "SCALE_BLOCK", "weight_bytes_per_expert",
    "approx_host_bytes", "f32_to_bf16_bits", "f32_to_e4m3_codes",
]


def device_inputs(wl: Workload, seed: int = 0, device="cuda", threads: Optional[int] = None):
    """Generate a workload straight into device tensors (host memory stays O(one expert)).

    Returns (routing [numpy], tensors dict): x bf16 [T,d], topk_ids int32, topk_w fp32,
    route_mask uint8, w_gate/w_up [E,f,d] and w_down [E,d,f] (bf16, or uint8 E4M3 codes
    with s_gate/s_up/s_down fp32 block scales for fp8 workloads).
    """
    import torch

    dev = torch.device(device)
    r = make_routing(wl, seed)
    T, E, d, f = wl.T, wl.E, wl.d, wl.f
    fp8 = wl.dtype == "fp8"
    wdt = torch.uint8 if fp8 else torch.bfloat16
    ten = {
        "x": torch.from_numpy(r.x.view(np.int16)).view(torch.bfloat16).to(dev),
        "topk_ids": torch.from_numpy(r.topk_ids).to(dev),
        "topk_w": torch.from_numpy(r.topk_w).to(dev),
        "route_mask": torch.from_numpy(r.route_mask).to(dev),
        "w_gate": torch.empty((E, f, d), dtype=wdt, device=dev),
        "w_up": torch.empty((E, f, d), dtype=wdt, device=dev),
        "w_down": torch.empty((E, d, f), dtype=wdt, device=dev),
    }
    if fp8:
        ten["s_gate"] = torch.empty((E, f // SCALE_BLOCK, d // SCALE_BLOCK), dtype=torch.float32, device=dev)
        ten["s_up"] = torch.empty((E, f // SCALE_BLOCK, d // SCALE_BLOCK), dtype=torch.float32, device=dev)
        ten["s_down"] = torch.empty((E, d // SCALE_BLOCK, f // SCALE_BLOCK), dtype=torch.float32, device=dev)
    names = {"wg": "w_gate", "wu": "w_up", "wd": "w_down", "sg": "s_gate", "su": "s_up", "sd": "s_down"}

    def sink(e, w):
        for k, a in w.items():
            src = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            if a.dtype == np.uint16:
                src = src.view(torch.bfloat16)
            ten[names[k]][e].copy_(src)

    all_expert_weights(wl, seed, threads=threads, sink=sink)
    torch.cuda.synchronize(dev)
    return r, ten
