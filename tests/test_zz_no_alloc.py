"""The allocation-free MoE call (qgemv_moe_id_noalloc) against the call with a
caller workspace (qgemv_moe_id), through the C ABI: the same kernels run on the
same inputs, so the outputs must agree bit for bit. Two calls in a row, the
second with fewer pairs, so that the second reads routing tables written over
the first's in the library's scratch; and a call whose pairs each get a tile of
their own (routing skipped), between routed ones."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, TORCH_DT, dev, log, to_device
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


def stack(E, R, C, bits, gs, dt, seed):
    w = synth.normal_f32((E * R, C), 0.02, seed)
    q, s, b = qref.quantize(w, bits, gs, dt)
    return (to_device(q, dt).reshape(E, R, -1), to_device(s, dt).reshape(E, R, -1),
            to_device(b, dt).reshape(E, R, -1))


def both(a, ids, T, top_k, wq, s, b, bits, gs):
    R = wq.shape[1]
    ref = torch.full((T * top_k, R), 7.0, dtype=a.dtype, device=dev())
    got = torch.full((T * top_k, R), -7.0, dtype=a.dtype, device=dev())
    qp.qgemv_moe_id(a, ids, T, top_k, a.shape[1], 0, wq, s, b, bits, gs, out=ref)
    qp.qgemv_moe_id_noalloc(a, ids, T, top_k, a.shape[1], 0, wq, s, b, bits, gs, got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dt", [BF16, F16])
def test_noalloc_matches_workspace_call_twice(dt):
    E, R, C, bits, gs, top_k = 32, 256, 512, 4, 64, 4
    log(f"noalloc dt={dt}")
    wq, s, b = stack(E, R, C, bits, gs, dt, seed=61)
    for T, seed in ((96, 62), (20, 63), (4, 64), (40, 65)):   # routed, routed smaller, 1-pair tiles, routed
        a = torch.from_numpy(synth.normal_f32((T, C), 1.0, seed)).to(TORCH_DT[dt]).to(dev())
        ids = torch.from_numpy(synth.moe_ids(T, top_k, E, seed + 100).ravel()).to(dev())
        ref, got = both(a, ids, T, top_k, wq, s, b, bits, gs)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), f"T={T}"


def test_noalloc_rejects_tables_above_the_scratch():
    E, R, C = 128, 8, 64
    wq = torch.zeros((E, R, C * 4 // 32), dtype=torch.int32, device=dev())
    sb = torch.zeros((E, R, 1), dtype=torch.bfloat16, device=dev())
    T, top_k = 1 << 16, 4
    a = torch.zeros((T, C), dtype=torch.bfloat16, device=dev())
    ids = torch.zeros((T * top_k,), dtype=torch.int32, device=dev())
    out = torch.empty((T * top_k, R), dtype=torch.bfloat16, device=dev())
    with pytest.raises(qp.QpackError, match="WORKSPACE"):
        qp.qgemv_moe_id_noalloc(a, ids, T, top_k, C, 0, wq, sb, sb, 4, 64, out)
