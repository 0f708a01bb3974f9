"""GPU parity of qpack_dequantize against the oracle, through the C ABI.

Both output forms are bit-exact: fp32 output against the oracle's fp32 dense
weight (multiply, then add), 16-bit output against its dense weight in the
scales' own type (product and sum each rounded to that type). Inputs are the
oracle's quantization of seeded weights, or seeded random codes with
full-mantissa scales and biases, never anything the device produced.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, F32, TORCH_DT, dev, log, to_device, to_numpy
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu
ALL_BITS = [2, 3, 4, 6, 8]


def random_case(n, k, bits, gs, dt, seed):
    """Seeded random codes, packed by the oracle, with scales and biases of full
    mantissa in dt (so the products and sums really round)."""
    codes = synth.random_codes((n, k), bits, seed).astype(np.uint8)
    wq = qref.pack(codes, bits)
    s = np.abs(synth.normal_f32((n, k // gs), 0.02, seed + 1)) + 1e-3
    b = synth.normal_f32((n, k // gs), 0.3, seed + 2)
    if dt != F32:
        s = torch.from_numpy(s).to(TORCH_DT[dt]).view(torch.int16).numpy().view(np.uint16)
        b = torch.from_numpy(b).to(TORCH_DT[dt]).view(torch.int16).numpy().view(np.uint16)
    return wq, s, b


def expected(wq, s, b, dt, k, bits, gs, out_dt):
    if out_dt == F32:
        return qref.dequantize(wq, s, b, dt, k, bits, gs)
    return qref.dequantize_typed(wq, s, b, dt, k, bits, gs)


def check(wq, s, b, dt, k, bits, gs, out_dt, what, out=None):
    log(f"{what}: n={wq.shape[0]} k={k} bits={bits} gs={gs} scales={dt} out={out_dt}")
    got = qp.qpack_dequantize(to_device(wq, dt), to_device(s, dt), to_device(b, dt), bits, gs,
                              out_dtype=TORCH_DT[out_dt], out=out)
    torch.cuda.synchronize()
    ref = expected(wq, s, b, dt, k, bits, gs, out_dt)
    g = to_numpy(got)
    if not np.array_equal(g.view(np.uint32 if out_dt == F32 else np.uint16),
                          ref.view(np.uint32 if out_dt == F32 else np.uint16)):
        bad = np.argwhere(g != ref)
        raise AssertionError(f"{what}: {len(bad)} of {ref.size} elements differ; first at "
                             f"{tuple(bad[0])}: gpu={g[tuple(bad[0])]!r} ref={ref[tuple(bad[0])]!r}")


FORMS = [(F32, F32), (F16, F32), (BF16, F32), (F16, F16), (BF16, BF16)]


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt,out_dt", FORMS, ids=[f"s{a}_o{b}" for a, b in FORMS])
def test_dequantize_random_codes_bit_exact(bits, gs, dt, out_dt):
    # 37 rows of 384: 1776 runs of 8 codes, two blocks of 1024 runs with a ragged tail.
    wq, s, b = random_case(37, 384, bits, gs, dt, 1100 + 10 * bits + gs)
    check(wq, s, b, dt, 384, bits, gs, out_dt, "random codes")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_dequantize_quantized_weights_bit_exact(bits, dt):
    w = synth.normal_f32((96, 1024), 0.02, seed=1200 + bits)
    wq, s, b = qref.quantize(w, bits, 64, dt)
    check(wq, s, b, dt, 1024, bits, 64, dt, "quantized weights")
    if dt != F32:
        check(wq, s, b, dt, 1024, bits, 64, F32, "quantized weights, fp32 out")


@pytest.mark.parametrize("dt,out_dt", [(BF16, BF16), (F16, F32)])
def test_dequantize_output_not_16_byte_aligned(dt, out_dt):
    """An output that starts one element into its buffer takes the element-store
    form; nothing outside [out, out + n*k) is written."""
    wq, s, b = random_case(5, 256, 3, 32, dt, 1300)
    buf = torch.full((5 * 256 + 2,), 7.0, dtype=TORCH_DT[out_dt], device=dev())
    out = buf[1:1 + 5 * 256].view(5, 256)
    check(wq, s, b, dt, 256, 3, 32, out_dt, "unaligned output", out=out)
    assert buf[0].item() == 7.0 and buf[-1].item() == 7.0


@pytest.mark.parametrize("bits", ALL_BITS)
def test_dequantize_single_group_rows(bits):
    """k = 32: four runs per row, one group; every row its own scale and bias."""
    wq, s, b = random_case(3, 32, bits, 32, BF16, 1400 + bits)
    check(wq, s, b, BF16, 32, bits, 32, BF16, "k=32")


def test_dequantize_full_size_decode_weight():
    """The 14336 x 4096 4-bit, group-64 bf16 weight of the decode benchmark,
    compared in full."""
    w = synth.normal_f32((14336, 4096), 0.02, seed=1500)
    wq, s, b = qref.quantize(w, 4, 64, BF16)
    check(wq, s, b, BF16, 4096, 4, 64, BF16, "full size")


def test_dequantize_empty_and_rejected_calls():
    wq = torch.zeros((0, 16), dtype=torch.int32, device=dev())
    s = torch.zeros((0, 4), dtype=torch.bfloat16, device=dev())
    out = qp.qpack_dequantize(wq, s, s, 4, 32)
    assert out.shape == (0, 128)
    wq = torch.zeros((2, 16), dtype=torch.int32, device=dev())
    s = torch.ones((2, 4), dtype=torch.bfloat16, device=dev())
    with pytest.raises(qp.QpackError) as e:
        qp.qpack_dequantize(wq, s, s, 4, 32, out_dtype=torch.float16)
    assert e.value.status == 3          # QP_ERR_DTYPE_MISMATCH: fp16 out of bf16 scales
    with pytest.raises(qp.QpackError) as e:
        qp.qpack_dequantize(wq, s, s, 5, 32)
    assert e.value.status == 2          # QP_ERR_UNSUPPORTED: bits = 5
