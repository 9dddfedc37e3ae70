"""Routed-MoE FFN and combine in fp64 (plain definitions).

Problem statement ("perf(ds4): batch heterogeneous MoE prefill by expert",
Summary): each token is routed to its selected experts; every expert runs a
gate/up projection, SwiGLU and a down projection on its tokens; the outputs
are summed back per token with the route weights, and a masked route adds an
exact zero.  SwiGLU is the DS4 split op between gate/up and down ("perf(ggml):
reuse ROCmFP4 weights across q=4 columns", DS4 SwiGLU split op plumbing), read
here as silu(gate) * up.  The route-weighted sum is the fused combine
("perf(ds4): accelerate ROCm decode and long-context selection", lucebox8
gfx1151 A/B), summed in ascending route order from +0.0.

Shapes: x [T,d] bf16 bits; topk_ids / topk_w / route_mask [T,k];
gate and up weights [E,f,d] (row n holds output feature n, d contiguous);
down weights [E,d,f].  fp8 weights are E4M3 codes with one fp32 scale per
128 x 128 block: scale[n // 128, c // 128] multiplies element [n, c].

Precision contract (a reading; the pages are silent): inputs are exact in
fp64; h is rounded to bf16 before the down projection; in the fp8 workload x
and h are quantised per row to E4M3 with an fp32 scale (``numerics``) and the
down projection consumes the quantised h.
"""
from __future__ import annotations

from typing import Callable, Dict, Iterable, Optional

import numpy as np

from . import numerics as nx
from .route import route_table

BLOCK = 128
ExpertSource = Callable[[int], Dict[str, np.ndarray]]


def _block_dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W[n, c] = decode(code[n, c]) * scale[n // 128, c // 128]."""
    N, K = codes.shape
    lut = nx.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = lut[codes]
    rows = np.arange(N)[:, None] // BLOCK
    cols = np.arange(K)[None, :] // BLOCK
    return vals * scale.astype(np.float64)[rows, cols]


def dequant_expert(raw: Dict[str, np.ndarray], fp8: bool) -> Dict[str, np.ndarray]:
    """Raw weights of one expert -> fp64 matrices wg [f,d], wu [f,d], wd [d,f]."""
    if not fp8:
        return {n: nx.bf16_bits_to_f64(raw[n]) for n in ("wg", "wu", "wd")}
    return {
        "wg": _block_dequant(raw["wg"], raw["sg"]),
        "wu": _block_dequant(raw["wu"], raw["su"]),
        "wd": _block_dequant(raw["wd"], raw["sd"]),
    }


def x_operand(x_bits_row: np.ndarray, fp8: bool) -> np.ndarray:
    """The activation row the gate/up projection consumes (fp64)."""
    x = nx.bf16_bits_to_f64(x_bits_row)
    if not fp8:
        return x
    q, s = nx.quant_row_fp8(x.astype(np.float32))
    return nx.e4m3_decode(q) * np.float64(s)


def h_operand(g: np.ndarray, u: np.ndarray, fp8: bool) -> np.ndarray:
    """SwiGLU then bf16 rounding (and the per-row fp8 quantisation)."""
    h = nx.bf16_round(nx.silu(g) * u)
    if not fp8:
        return h
    q, s = nx.quant_row_fp8(h.astype(np.float32))
    return nx.e4m3_decode(q) * np.float64(s)


def expert_ffn(xop: np.ndarray, W: Dict[str, np.ndarray], fp8: bool) -> np.ndarray:
    """y = Wd . h(Wg . x, Wu . x) for one token row (fp64)."""
    g = W["wg"] @ xop
    u = W["wu"] @ xop
    h = h_operand(g, u, fp8)
    return W["wd"] @ h


def _active(route_mask, t, j, ids, E):
    on = True if route_mask is None else bool(route_mask[t, j])
    return on and 0 <= int(ids[t, j]) < E


def moe_ref_per_token(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                      route_mask: Optional[np.ndarray], experts: ExpertSource, E: int,
                      fp8: bool = False, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """Literal per-token loop over the selected experts (fp64).

    Returns out [len(tokens), d].  Each active route decodes its expert and
    evaluates the FFN on that token alone; masked routes are skipped, so they
    add nothing and the accumulator of a token with no active route stays +0.0.
    """
    T, k = topk_ids.shape
    d = x.shape[1]
    toks = list(range(T)) if tokens is None else list(tokens)
    out = np.zeros((len(toks), d), dtype=np.float64)
    for row, t in enumerate(toks):
        xop = x_operand(x[t], fp8)
        acc = np.zeros(d, dtype=np.float64)
        for j in range(k):
            if not _active(route_mask, t, j, topk_ids, E):
                continue
            W = dequant_expert(experts(int(topk_ids[t, j])), fp8)
            y = expert_ffn(xop, W, fp8)
            acc = acc + np.float64(topk_w[t, j]) * y
        out[row] = acc
    return out


def route_outputs_ref(x: np.ndarray, topk_ids: np.ndarray, experts: ExpertSource,
                      routes: Iterable[int], fp8: bool = False) -> np.ndarray:
    """y for individual routes r = t*k + j (fp64), before the gate weight."""
    k = topk_ids.shape[1]
    rs = list(routes)
    out = np.zeros((len(rs), x.shape[1]), dtype=np.float64)
    for i, r in enumerate(rs):
        t, j = divmod(int(r), k)
        W = dequant_expert(experts(int(topk_ids[t, j])), fp8)
        out[i] = expert_ffn(x_operand(x[t], fp8), W, fp8)
    return out


def moe_ref_dense(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                  route_mask: Optional[np.ndarray], experts: ExpertSource, E: int,
                  fp8: bool = False) -> np.ndarray:
    """Brute force: every expert on every token, times a dense gate matrix.

    gate[t, e] = sum of topk_w[t, j] over active routes j of token t with
    topk_ids[t, j] == e (zero elsewhere); out = sum_e gate[:, e] * FFN_e(x).
    """
    T, k = topk_ids.shape
    d = x.shape[1]
    gate = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if _active(route_mask, t, j, topk_ids, E):
                gate[t, int(topk_ids[t, j])] += np.float64(topk_w[t, j])
    X = np.stack([x_operand(x[t], fp8) for t in range(T)]) if T else np.zeros((0, d))
    out = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        W = dequant_expert(experts(e), fp8)
        G = X @ W["wg"].T
        U = X @ W["wu"].T
        H = np.stack([h_operand(G[t], U[t], fp8) for t in range(T)]) if T else G
        Y = H @ W["wd"].T
        out += gate[:, e:e + 1] * Y
    return out


def combine_ref(y: np.ndarray, route_rows: np.ndarray, topk_w: np.ndarray,
                route_mask: Optional[np.ndarray], T: int, k: int) -> np.ndarray:
    """out[t] = sum over active j ascending of w[t,j] * y[route_rows[t*k+j]] (fp64).

    Masked routes are never read: their rows of y, their gates and their
    route_rows entries may hold anything, NaN included.
    """
    d = y.shape[1]
    out = np.zeros((T, d), dtype=np.float64)
    rr = np.asarray(route_rows).reshape(T, k)
    for t in range(T):
        acc = np.zeros(d, dtype=np.float64)
        for j in range(k):
            if route_mask is not None and not route_mask[t, j]:
                continue
            acc = acc + np.float64(topk_w[t, j]) * y[rr[t, j]].astype(np.float64)
        out[t] = acc
    return out


def combine_shared_ref(y: np.ndarray, route_rows: np.ndarray, topk_w: np.ndarray,
                       route_mask: Optional[np.ndarray], shared: Optional[np.ndarray], T: int,
                       k: int) -> np.ndarray:
    """The combine writing into a shared-expert output (fp64).

    The fused combine's "shared-output" cases ("perf(ds4): extend sparse
    prefill scheduling to 10K", Historical fused-combine discriminator) add
    the routed sum to the output of the layer's shared expert.  Reading: the
    routed sum is formed exactly as in ``combine_ref`` and the shared row is
    added once at the end, out[t] = routed[t] + shared[t]; with no shared
    output it is the routed sum.  A bf16 copy of out, when asked for, is its
    round-to-nearest-even (``numerics.bf16_round``).
    """
    out = combine_ref(y, route_rows, topk_w, route_mask, T, k)
    if shared is not None:
        out = out + np.asarray(shared, dtype=np.float64)
    return out


def moe_ref_blocked(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
                    route_mask: Optional[np.ndarray], experts: ExpertSource, E: int,
                    fp8: bool = False, expert_subset: Optional[Iterable[int]] = None):
    """Expert-major evaluation of the same fp64 mathematics (BLAS dgemm).

    Builds the route table, evaluates each expert once on its segment of
    routed rows, then combines.  With ``expert_subset`` only those experts are
    evaluated (their rows of y are filled, the rest stay zero) -- used to time
    a bounded sample; the returned ``out`` is then partial.
    Returns (out [T,d], y [T*k, d], route table).
    """
    T, k = topk_ids.shape
    d = x.shape[1]
    rt = route_table(topk_ids, route_mask, E)
    R = T * k
    y = np.zeros((R, d), dtype=np.float64)
    todo = range(E) if expert_subset is None else expert_subset
    xop_cache: Dict[int, np.ndarray] = {}
    for e in todo:
        lo, hi = int(rt.offsets[e]), int(rt.offsets[e + 1])
        if hi == lo:
            continue
        toks = rt.sorted_routes[lo:hi] // k
        X = np.empty((hi - lo, d), dtype=np.float64)
        for i, t in enumerate(toks.tolist()):
            if t not in xop_cache:
                xop_cache[t] = x_operand(x[t], fp8)
            X[i] = xop_cache[t]
        W = dequant_expert(experts(e), fp8)
        G = X @ W["wg"].T
        U = X @ W["wu"].T
        if fp8:
            H = np.stack([h_operand(G[i], U[i], fp8) for i in range(hi - lo)])
        else:
            H = nx.bf16_round(nx.silu(G) * U)
        y[lo:hi] = H @ W["wd"].T
    mask = None if route_mask is None else route_mask.copy()
    if mask is not None:
        bad = (topk_ids < 0) | (topk_ids >= E)
        mask[bad] = 0
    elif np.any((topk_ids < 0) | (topk_ids >= E)):
        mask = ((topk_ids >= 0) & (topk_ids < E)).astype(np.uint8)
    out = combine_ref(y, rt.route_rows, topk_w, mask, T, k)
    return out, y, rt


def dict_source(weights: Dict[str, np.ndarray]) -> ExpertSource:
    """Expert source over stacked arrays {"wg": [E,f,d], ...}."""
    def get(e: int) -> Dict[str, np.ndarray]:
        return {n: a[e] for n, a in weights.items()}
    return get
