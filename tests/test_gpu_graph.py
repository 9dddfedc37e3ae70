"""The whole path (route build, FFN, combine) captured once in a HIP graph
and replayed: every replay, with eager work and synchronisations between
the replays, writes the same bits as the eager call.  The library issues no
memset and allocates nothing inside a call, and its persistent kernels leave
their work-queue heads at zero, so a replayed graph needs nothing reset.

Cases: a decode-sized chunk (at most 32 routed rows: fixed item
assignment), a prefill chunk whose experts fill every tile class (work
queues, several 256-row tiles for one expert), and the fp8 path."""
import numpy as np
import pytest

from gpu_util import bf16_dev, np_dev, routing_with_counts
from test_gpu_ffn import _dev_weights, _weights, _x

pytestmark = pytest.mark.gpu


def _inputs(counts, k, d, f, fp8, seed):
    ids, mask = routing_with_counts(counts, k, seed=seed, masked_extra=5)
    T = ids.shape[0]
    w = np.random.default_rng(seed + 1).random((T, k)).astype(np.float32)
    W = _weights(len(counts), d, f, fp8, seed + 2)
    return ids, mask, w, _x(T, d, seed + 3), W


@pytest.mark.parametrize("name,counts,fp8", [
    ("decode", [1, 0, 2, 0, 0, 3, 1, 0] * 2, False),
    ("prefill", [0, 31, 64, 65, 130, 200, 256, 300, 700, 5, 0, 1], False),
    ("prefill_fp8", [0, 31, 64, 65, 130, 200, 256, 300, 5, 1], True),
])
def test_graph_replays_match_eager(name, counts, fp8):
    import torch

    import routed_expert_prefill_amd as rep

    k, d, f = 6, 512, 256
    ids, mask, w, x, W = _inputs(counts, k, d, f, fp8, seed=len(counts) * 7 + fp8)
    T = ids.shape[0]
    E = len(counts)
    Wd = _dev_weights(W, fp8)
    args = (bf16_dev(x), np_dev(ids), np_dev(w), np_dev(mask), Wd["wg"], Wd["wu"], Wd["wd"],
            Wd.get("sg"), Wd.get("su"), Wd.get("sd"))
    run = rep.MoEPrefill(T, k, E, d, f, fp8=fp8)
    eager = run(*args).clone()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*args)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run(*args)
    torch.cuda.synchronize()

    other = torch.randn(1 << 20, device="cuda:0")
    for i in range(4):
        run.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out.view(torch.int32), eager.view(torch.int32)), (name, i)
        # eager work of the program between the replays: another pass of the
        # path and unrelated torch kernels
        (other * 2).sum().item()
        again = run(*args)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), eager.view(torch.int32)), (name, i)
