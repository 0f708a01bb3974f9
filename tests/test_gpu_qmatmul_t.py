"""GPU parity of qmatmul_t (transpose = false: W stored [k, n], grouped along n)
against the oracle, through the C ABI: within tau*S + half an output ulp, and
bit-exact where every product and sum is exact. Weights are the oracle's
quantization of seeded W^T stored row-major [k, n]."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, F32, TORCH_DT, activations, assert_within, dev, log, to_device
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu
ALL_BITS = [2, 3, 4, 6, 8]


def run(m, k, n, bits, gs, dt, seed, what):
    w = synth.normal_f32((k, n), 0.02, seed)          # W [k, n], groups along n
    wq, s, b = qref.quantize(w, bits, gs, dt)
    x_st, _ = activations((m, k), dt, seed + 1)
    log(f"{what}: m={m} k={k} n={n} bits={bits} gs={gs} dt={dt}")
    y = qp.qmatmul_t(to_device(x_st, dt), to_device(wq, dt), to_device(s, dt), to_device(b, dt),
                     bits, gs)
    torch.cuda.synchronize()
    yr, S = qref.qmatmul_t(x_st, dt, wq, s, b, dt, n, bits, gs)
    assert_within(y, yr, S, dt, what)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("m", [1, 3, 6])
def test_qmatmul_t_small(bits, dt, m):
    # n = 640: 80 / 40 / 20 / 160 / 20 lane chunks, a ragged 64-lane tile;
    # k = 200: splits of whole and ragged row ranges.
    run(m, 200, 640, bits, 64, dt, 6000 + 10 * bits + m, "small")


@pytest.mark.parametrize("gs", [32, 128])
def test_qmatmul_t_group_sizes(gs):
    run(2, 384, 1024, 4, gs, BF16, 6100 + gs, f"gs={gs}")


@pytest.mark.parametrize("bits", [4, 8])
def test_qmatmul_t_full_size_decode(bits):
    """W [4096, 14336] stored transposed (the decode shape's weight), x bf16 [1, 4096]."""
    run(1, 4096, 14336, bits, 64, BF16, 6200 + bits, "full size")


def test_qmatmul_t_exact_case():
    """Dyadic codes, scales and biases with integer activations: exact in fp32
    in any order, so y is the oracle's result rounded once."""
    k, n, gs, bits = 256, 512, 32, 4
    codes = synth.random_codes((k, n), bits, 6300).astype(np.uint8)
    wq = qref.pack(codes, bits)
    s = (synth.random_ints((k, n // gs), 1, 16, 6301) / 16.0).astype(np.float32)
    b = (synth.random_ints((k, n // gs), -16, 16, 6302) / 16.0).astype(np.float32)
    x = synth.random_ints((3, k), -4, 4, 6303).astype(np.float32)
    s16 = torch.from_numpy(s).to(torch.bfloat16)
    b16 = torch.from_numpy(b).to(torch.bfloat16)
    y = qp.qmatmul_t(torch.from_numpy(x).to(torch.bfloat16).to(dev()),
                     torch.from_numpy(wq.view(np.int32)).to(dev()), s16.to(dev()), b16.to(dev()),
                     bits, gs)
    torch.cuda.synchronize()
    yr, _ = qref.qmatmul_t(x, F32, wq, s, b, F32, n, bits, gs)
    assert torch.equal(y.cpu(), torch.from_numpy(yr.astype(np.float32)).to(torch.bfloat16))


def test_qmatmul_t_codes_not_16_byte_aligned():
    """Codes one word into their buffer take the word-load form."""
    k, n, bits, gs = 64, 256, 4, 64
    w = synth.normal_f32((k, n), 0.02, 6400)
    wq, s, b = qref.quantize(w, bits, gs, BF16)
    buf = torch.zeros(wq.size + 1, dtype=torch.int32, device=dev())
    buf[1:] = to_device(wq, BF16).reshape(-1)
    wq_d = buf[1:].view(k, -1)
    x_st, _ = activations((2, k), BF16, 6401)
    y = qp.qmatmul_t(to_device(x_st, BF16), wq_d, to_device(s, BF16), to_device(b, BF16), bits, gs)
    torch.cuda.synchronize()
    yr, S = qref.qmatmul_t(x_st, BF16, wq, s, b, BF16, n, bits, gs)
    assert_within(y, yr, S, BF16, "unaligned codes")


def test_qmatmul_t_k0_and_workspace_check():
    x = torch.zeros((2, 0), dtype=torch.bfloat16, device=dev())
    wq = torch.zeros((0, 64), dtype=torch.int32, device=dev())
    s = torch.zeros((0, 4), dtype=torch.bfloat16, device=dev())
    y = qp.qmatmul_t(x, wq, s, s, 4, 128)
    torch.cuda.synchronize()
    assert y.shape == (2, 512) and (y == 0).all()
    x = torch.ones((1, 64), dtype=torch.bfloat16, device=dev())
    wq = torch.zeros((64, 64), dtype=torch.int32, device=dev())
    s = torch.ones((64, 4), dtype=torch.bfloat16, device=dev())
    with pytest.raises(qp.QpackError) as e:
        qp.qmatmul_t(x, wq, s, s, 4, 128, workspace=torch.empty(4, dtype=torch.uint8, device=dev()))
    assert e.value.status == 6
