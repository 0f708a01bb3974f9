"""GPU parity of the per-tensor dynamic-range int8 scheme against the oracle,
through the C ABI: quantize (codes and range) and dequantize bit-exact, the
product within tau*S + half an output ulp, and bit-exact where it is exact."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, F32, TORCH_DT, activations, assert_within, dev, log, to_device, to_numpy
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def quantize_both(w):
    rq, rr = qref.quantize_int8_tensor(w)
    gq, gr = qp.qpack_quantize_int8_tensor(torch.from_numpy(w).to(dev()))
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), rq), "codes differ"
    assert np.array_equal(gr.cpu().numpy().view(np.uint32), rr.view(np.uint32)), "range differs"
    return rq, rr, gq, gr


def test_int8_tensor_printed_example_on_device():
    vals = {}
    with open(os.path.join(GOLDEN, "int8_tensor_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = (t.strip() for t in line.split("|"))
                vals[k] = [float(x) for x in v.split()]
    w = np.array(vals["input"], dtype=np.float32)
    _, _, gq, gr = quantize_both(w)
    assert gq.cpu().tolist() == [int(v) for v in vals["codes"]]
    assert gr.cpu().tolist() == vals["range"]


@pytest.mark.parametrize("shape", [(1,), (3, 5), (257, 129), (14336, 4096)])
def test_int8_tensor_quantize_bit_exact(shape):
    log(f"int8 quantize {shape}")
    w = synth.normal_f32(shape, 0.05, 5000 + len(shape))
    if w.size > 1:
        w.reshape(-1)[w.size // 3] = 0.61      # a far value sets the range
    quantize_both(w)


def test_int8_tensor_constant_tensor():
    rq, rr, gq, gr = quantize_both(np.full((40, 7), -1.25, dtype=np.float32))
    assert (gq == -128).all()


@pytest.mark.parametrize("out_dt", [F32, F16, BF16])
def test_int8_tensor_dequantize_bit_exact(out_dt):
    w = synth.normal_f32((129, 300), 0.05, 5100)
    rq, rr, gq, gr = quantize_both(w)
    out = qp.qpack_dequantize_int8_tensor(gq, gr, out_dtype=TORCH_DT[out_dt])
    torch.cuda.synchronize()
    ref = qref.dequantize_int8_tensor(rq, rr)
    if out_dt == F32:
        assert np.array_equal(to_numpy(out).view(np.uint32), ref.view(np.uint32))
    else:
        expect = torch.from_numpy(ref).to(TORCH_DT[out_dt]).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(to_numpy(out), expect)


def run_product(m, n, k, dt, seed, what, x_offset=0):
    w = synth.normal_f32((n, k), 0.05, seed)
    rq, rr, gq, gr = quantize_both(w)
    x_st, _ = activations((m, k), dt, seed + 1)
    xt = to_device(x_st, dt)
    if x_offset:
        buf = torch.empty(m * k + x_offset, dtype=TORCH_DT[dt], device=dev())
        buf[x_offset:] = xt.reshape(-1)
        xt = buf[x_offset:].view(m, k)
    log(f"{what}: m={m} n={n} k={k} dt={dt}")
    y = qp.qmatmul_int8_tensor(xt, gq, gr)
    torch.cuda.synchronize()
    yr, S = qref.qmatmul_int8_tensor(x_st, dt, rq, rr)
    assert_within(y, yr, S, dt, what)


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("m", [1, 2, 5])
@pytest.mark.parametrize("k", [1024, 4096, 14336])
def test_int8_tensor_product_stream(dt, m, k):
    run_product(m, 300, k, dt, 5200 + m + k, "stream")


def test_int8_tensor_product_generic():
    run_product(3, 70, 256, F32, 5300, "generic fp32")
    run_product(2, 33, 48, BF16, 5310, "k=48")
    run_product(2, 40, 512, F16, 5320, "unaligned x", x_offset=1)


def test_int8_tensor_product_full_size_decode():
    run_product(1, 14336, 4096, BF16, 5400, "full size")


def test_int8_tensor_product_exact_case():
    """Range [-8, 7.9375] (step 1/16) and integer activations: every product
    and sum is exact in fp32, so y is the oracle's result rounded once."""
    q = synth.random_ints((96, 1024), -128, 127, 5500).astype(np.int8)
    rng_ = np.array([-8.0, 7.9375], dtype=np.float32)
    x = synth.random_ints((2, 1024), -4, 4, 5501).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(dev())
    y = qp.qmatmul_int8_tensor(xt, torch.from_numpy(q).to(dev()), torch.from_numpy(rng_).to(dev()))
    torch.cuda.synchronize()
    yr, _ = qref.qmatmul_int8_tensor(x, F32, q, rng_)
    assert torch.equal(y.cpu(), torch.from_numpy(yr.astype(np.float32)).to(torch.bfloat16))
