"""Parity on the inputs where a folded affine product is weakest, on every
product path (emily lib/emily/quantization.ex, `quantized_matmul/2` and
`dequantize_defn/1`: w = q * scale + bias per group).

The kernels sum q * x and x per group and apply the scale and bias once per
group; the oracle forms each weight first. The two agree to the bound
tau * S only if the folded sums carry no error that is large against S.
These weights make S small or zero where the folded sums are not:

- all-zero rows and constant-zero groups: S = 0, so the bound is exactly 0
  and the output must be exactly 0;
- groups of one spike and exact zeros, of either sign (the negative spike
  puts the bias at -spike and every zero at the top code);
- one spike in a whole row, one-sided negative groups, and groups of zeros
  with a spike of each sign.

Activations are same-sign with magnitudes spread over e^-8 .. e^2, and also
N(0, 1). Each case runs at the largest K its kernel takes.

The tile GEMM (17 and more activation rows, 16-bit activations) rounds every
dequantized weight to the activation type before the matrix instruction, as
the prefill design prescribes (weight tiles dequantized to bf16 in LDS). That
rounding alone reaches half a bf16 ulp, 2^-8 of |x w'|, per product, so for
bf16 those cases are held to tau = 2^-8 + 2^-12 (the weight rounding plus the
fp32 accumulation); fp16's rounding, 2^-11, fits inside 2e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, F32, TORCH_DT, assert_within, dev, log, to_device, to_numpy, values
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


TAU_TILE_BF16 = 2.0 ** -8 + 2.0 ** -12


def tile_tau(m, dt):
    return TAU_TILE_BF16 if (m > 16 and dt == BF16) else None


def edge_case(n, k, m, bits, gs, dt, seed, act):
    w = synth.edge_weights(n, k, gs, seed)
    rq, rs, rb = qref.quantize(w, bits, gs, dt)
    if act == "normal":
        x = synth.normal_f32((m, k), 1.0, seed + 1)
    else:
        x = synth.wide_activations((m, k), seed + 1, 1.0 if act == "pos" else -1.0)
    xt = torch.from_numpy(x).to(TORCH_DT[dt])
    xs = to_numpy(xt)
    y = qp.qmatmul(xt.to(dev()), to_device(rq, dt), to_device(rs, dt), to_device(rb, dt), bits, gs)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, dt, rq, rs, rb, dt, k, bits, gs)
    yv = values(y).reshape(y_ref.shape)
    zero = S == 0
    assert zero.any()
    assert np.all(yv[zero] == 0), (
        f"S = 0 but output nonzero at {int((yv[zero] != 0).sum())} places, "
        f"max |y| {np.abs(yv[zero]).max():.3e}")
    assert_within(y, y_ref, S, dt, f"edge b{bits} dt{dt} k{k} m{m} gs{gs} {act}",
                  tau=tile_tau(m, dt))


ACTS = ["pos", "neg", "normal"]

# (m, k, gs): the row kernel at one and two rows (1 to 8 units per lane, 32-lane
# slots at K <= 1024), the four-row matrix-instruction kernel, the skinny
# matrix-core kernel (its row-contiguous form at gs 32, 64 and 128), the tile
# GEMM.
DENSE_16 = [(1, 16384, 128), (1, 4096, 64), (1, 1024, 32), (2, 8192, 64), (2, 16384, 128),
            (3, 4096, 64), (4, 4096, 128), (8, 4096, 64), (12, 2048, 32), (16, 14336, 64),
            (40, 4096, 64)]


def with_dtypes(cases):
    """(m, k, gs) x {bf16, fp16}."""
    return [(m, k, gs, dt) for (m, k, gs) in cases for dt in (BF16, F16)]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("m,k,gs,dt", with_dtypes(DENSE_16))
def test_edge_integral_widths(m, k, gs, bits, dt, act):
    log(f"edge bits={bits} dt={dt} m={m} k={k} gs={gs} act={act}")
    edge_case(64, k, m, bits, gs, dt, seed=9000 + m + k + gs + bits, act=act)


# 3- and 6-bit codes: the row kernel at one and two rows (32-lane slots at K
# <= 1024, seven units per lane at K = 14336) and at three and four rows
# (their slices in registers), the skinny kernel, the tile GEMM.
DENSE_CROSS = [(1, 4096, 32), (1, 4096, 128), (2, 4096, 64), (1, 14336, 64), (1, 1024, 32),
               (3, 4096, 64), (4, 1024, 128), (8, 4096, 64), (12, 2048, 32), (40, 4096, 128)]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("m,k,gs,dt", with_dtypes(DENSE_CROSS))
def test_edge_cross_word_widths(m, k, gs, bits, dt, act):
    log(f"edge cross bits={bits} dt={dt} m={m} k={k} gs={gs} act={act}")
    edge_case(64, k, m, bits, gs, dt, seed=9500 + m + k + gs + bits, act=act)


@pytest.mark.parametrize("act", ["pos", "normal"])
@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("m,k", [(1, 4096), (8, 2048)])
def test_edge_fp32(m, k, bits, act):
    log(f"edge fp32 bits={bits} m={m} k={k} act={act}")
    edge_case(64, k, m, bits, 64, F32, seed=9800 + m + k + bits, act=act)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("gs,dt", [(64, BF16), (128, F16)])
def test_edge_six_bit_row_contiguous(gs, dt, act):
    """6-bit codes take the row-contiguous skinny form from 2^25 codes:
    2368 x 14336 rows of the edge pattern, eight activation rows."""
    log(f"edge six-bit row-contiguous gs={gs} dt={dt} act={act}")
    edge_case(2368, 14336, 8, 6, gs, dt, seed=9700 + gs, act=act)
