"""The calls under HIP graph capture: a captured sequence (decode qmatmul at
one, four and eight activation rows, prefill qmatmul, both MoE forms with and without the routing launch) replayed
several times, with eager work and synchronisations between the replays,
gives bit-identical outputs to the eager calls every time. The library
allocates nothing and records no memset, so its launches can be captured
as they are."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from qhelpers import BF16, activations, dev, log, to_device
from oracle import qref
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


def quantized(n, k, seed):
    w = synth.normal_f32((n, k), 0.02, seed)
    return tuple(to_device(t, BF16) for t in qref.quantize(w, 4, 64, BF16))


def test_graph_replays_match_eager():
    log("graph capture: decode (1, 4, 8 rows), prefill, MoE")
    N, K = 1024, 512
    wq, s, b = quantized(N, K, 501)
    _, x1 = activations((1, K), BF16, 502)
    _, x64 = activations((96, K), BF16, 503)
    _, x4 = activations((4, K), BF16, 509)
    _, x8 = activations((8, K), BF16, 510)
    E, R, C = 8, 128, 256
    g = tuple(t.reshape(E, R, -1) for t in quantized(E * R, C, 504))
    u = tuple(t.reshape(E, R, -1) for t in quantized(E * R, C, 505))
    ids1 = torch.from_numpy(np.array([3, 5], dtype=np.int32)).to(dev())     # 2 pairs: no routing
    idsT = torch.from_numpy(synth.moe_ids(64, 2, E, seed=506).ravel()).to(dev())
    _, a1 = activations((1, C), BF16, 507)
    _, aT = activations((64, C), BF16, 508)
    ws = torch.empty(qp.qgemv_moe_workspace_bytes(128, E), dtype=torch.uint8, device=dev())
    outs = {
        "y1": torch.empty((1, N), dtype=torch.bfloat16, device=dev()),
        "y64": torch.empty((96, N), dtype=torch.bfloat16, device=dev()),
        "y4": torch.empty((4, N), dtype=torch.bfloat16, device=dev()),
        "y8": torch.empty((8, N), dtype=torch.bfloat16, device=dev()),
        "h1": torch.empty((2, R), dtype=torch.bfloat16, device=dev()),
        "hT": torch.empty((128, R), dtype=torch.bfloat16, device=dev()),
        "pT": torch.empty((128, R), dtype=torch.bfloat16, device=dev()),
    }

    def run():
        qp.qmatmul(x1, wq, s, b, 4, 64, out=outs["y1"])
        qp.qmatmul(x64, wq, s, b, 4, 64, out=outs["y64"])
        qp.qmatmul(x4, wq, s, b, 4, 64, out=outs["y4"])
        qp.qmatmul(x8, wq, s, b, 4, 64, out=outs["y8"])
        qp.qgemv_moe_id_gate_up_silu(a1, ids1, 1, 2, 0, 0, g, u, 4, 64, out=outs["h1"],
                                     workspace=ws)
        qp.qgemv_moe_id_gate_up_silu(aT, idsT, 64, 2, C, 0, g, u, 4, 64, out=outs["hT"],
                                     workspace=ws)
        qp.qgemv_moe_id(aT, idsT, 64, 2, C, 0, *g, 4, 64, out=outs["pT"], workspace=ws)

    run()   # eager; also sets every kernel's attributes before capture
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for v in outs.values():
            v.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs"
        run()   # eager work between replays
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"eager after replay {rep}: {k} differs"
