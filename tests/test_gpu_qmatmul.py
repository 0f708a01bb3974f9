"""GPU parity of qpack_quantize and qmatmul against the oracle, through the C ABI.

Quantize: bit-exact codes, scales and biases. qmatmul: element by element
within tau*S + half an output ulp (see qhelpers), and bit-exact on inputs
whose arithmetic is exact in fp32. Weights fed to the library's products are
always the oracle's quantization of the seeded fp32 W (never the device's).
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import (BF16, F16, F32, TORCH_DT, activations, assert_within, bits_of, dev, log,
                      rne_to_bits, to_device, to_numpy, values)
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu
ALL_BITS = [2, 3, 4, 6, 8]


def quantize_both(w: np.ndarray, bits: int, gs: int, dt: int):
    """Oracle and device quantization of w; asserts they agree bit for bit and
    returns the oracle's (wq, s, b) as numpy plus device copies of them."""
    rq, rs, rb = qref.quantize(w, bits, gs, dt)
    gq, gs_, gb = qp.qpack_quantize(torch.from_numpy(w).to(dev()), bits, gs, TORCH_DT[dt])
    torch.cuda.synchronize()
    bits_view = np.uint32 if dt == F32 else np.uint16
    assert np.array_equal(to_numpy(gq), rq), "codes differ"
    assert np.array_equal(to_numpy(gs_).view(bits_view), rs.view(bits_view)), "scales differ"
    assert np.array_equal(to_numpy(gb).view(bits_view), rb.view(bits_view)), "biases differ"
    return (rq, rs, rb), (to_device(rq, dt), to_device(rs, dt), to_device(rb, dt))


# ------------------------------------------------------------------ quantize

@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_quantize_bit_exact_small(bits, gs, dt):
    log(f"quantize bits={bits} gs={gs} dt={dt} [97, 384]")
    w = synth.normal_f32((97, 384), 0.02, seed=100 + bits + gs + dt)
    w[3, :gs] = 0.5            # constant group
    w[5, gs:2 * gs] *= 400.0   # large range
    w[7] += 3.0                # far from zero (bias rounding matters)
    quantize_both(w, bits, gs, dt)


def test_quantize_iota_example():
    w = synth.iota_f32((4, 128))
    (rq, rs, rb), _ = quantize_both(w, 4, 64, F32)
    assert np.all(rs == np.float32(63) / np.float32(15))


@pytest.mark.parametrize("shape,bits,gs,dt,seed", [
    ((256, 1024), 4, 64, F32, 11),
    ((14336, 4096), 4, 64, BF16, 21),
    ((14336, 4096), 8, 64, BF16, 21),
    ((14336, 4096), 2, 64, BF16, 21),
    ((4096, 4096), 3, 32, F16, 31), ((4096, 4096), 3, 64, F16, 31), ((4096, 4096), 3, 128, F16, 31),
    ((4096, 4096), 6, 32, F16, 31), ((4096, 4096), 6, 64, F16, 31), ((4096, 4096), 6, 128, F16, 31),
])
def test_quantize_bit_exact_full_configs(shape, bits, gs, dt, seed):
    log(f"quantize full {shape} bits={bits} gs={gs} dt={dt}")
    quantize_both(synth.normal_f32(shape, 0.02, seed), bits, gs, dt)


def test_quantize_empty_is_noop():
    w = torch.empty((0, 64), dtype=torch.float32, device=dev())
    wq, s, b = qp.qpack_quantize(w, 4, 64)
    assert wq.shape == (0, 8)


# ------------------------------------------------------------------ qmatmul

def run_case(n, k, m, bits, gs, dt, seed):
    w = synth.normal_f32((n, k), 0.02, seed)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, bits, gs, dt)
    xs, xt = activations((m, k), dt, seed + 1)
    y = qp.qmatmul(xt, gq, gs_, gb, bits, gs)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, dt, rq, rs, rb, dt, k, bits, gs)
    return y, y_ref, S


SMALL = list(itertools.product(ALL_BITS, [F32, F16, BF16]))


@pytest.mark.parametrize("bits,dt", SMALL)
@pytest.mark.parametrize("k,m", [(32, 1), (96, 3), (768, 2), (1024, 5), (2048, 8), (4096, 16),
                                 (4096, 1), (1024, 13)])
def test_qmatmul_parity_small(bits, dt, k, m):
    gs = {32: 32, 96: 32, 768: 64, 1024: 128, 2048: 64, 4096: 64}[k]
    n = 301  # not a multiple of any block's row count
    log(f"qmatmul bits={bits} dt={dt} n={n} k={k} m={m} gs={gs}")
    y, y_ref, S = run_case(n, k, m, bits, gs, dt, seed=1000 + 7 * bits + k + m + dt)
    assert_within(y, y_ref, S, dt, f"qmatmul b{bits} dt{dt} k{k} m{m}")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("k,m,gs", [(14336, 1, 64), (11008, 1, 128), (8192, 2, 32), (6144, 2, 64),
                                    (2080, 1, 32), (16384, 2, 64), (12288, 1, 32), (2176, 2, 64),
                                    (2176, 1, 32), (2112, 2, 64), (128, 2, 64), (96, 1, 32),
                                    (4096, 4, 64), (2176, 3, 64), (2112, 4, 64), (96, 3, 32),
                                    (1024, 4, 128), (9600, 1, 64), (5120, 2, 32)])
def test_qmatmul_row_stream_units_per_lane(bits, dt, k, m, gs):
    """Decode on the row-per-wave kernel at every code width (3- and 6-bit
    units are 12 and 24 bytes, the fields spread to bytes first): 1 to 8
    units of 32 codes per lane, ragged unit counts (11008 = 344 units, 2176
    = 68, 2080 = 65, 96 = 3), two rows per pass up to K = 8192 and one
    beyond, three and four rows up to K = 4096 (2/4/8-bit: activation
    slices read from LDS, on the 4x4x4 matrix instruction; 3/6-bit: the four
    rows' slices in registers, dot products); rows with an
    even number of groups (scales read as whole rows) and with an odd one
    (2080 / 32 = 65, 2112 / 64 = 33, 96 / 32 = 3); units per lane as the row
    needs them (9600 = 300 units: 5 per lane; 5120 = 160: 3; 11008: 6;
    14336 = 448: 7)."""
    n = 300
    log(f"row stream bits={bits} dt={dt} n={n} k={k} m={m} gs={gs}")
    y, y_ref, S = run_case(n, k, m, bits, gs, dt, seed=7000 + k + m + gs + bits)
    assert_within(y, y_ref, S, dt, f"row stream b{bits} k{k} m{m}")


@pytest.mark.parametrize("bits", [4, 3, 8, 2, 6])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("n,k,m,gs", [(301, 14336, 16, 128), (50, 14336, 7, 64),
                                      (130, 160, 11, 32), (1000, 4096, 2, 64),
                                      (200, 768, 6, 32), (137, 1280, 16, 32)])
def test_qmatmul_skinny_tiles(bits, dt, n, k, m, gs):
    """2..16 activation rows: ragged row counts, K not a multiple of the
    K-split quads, and K long enough that the activation rows go to LDS in
    several chunks (K = 14336); 2-, 3- and 4-bit codes take the row-contiguous
    form where the scales allow it (K = 14336 at gs 64 and 128, and K = 768
    and 1280 at gs 32, whose last K-slice of 16 units is half empty), 6-bit
    codes only on larger matrices."""
    log(f"skinny bits={bits} dt={dt} n={n} k={k} m={m} gs={gs}")
    y, y_ref, S = run_case(n, k, m, bits, gs, dt, seed=5000 + n + k + m + bits)
    assert_within(y, y_ref, S, dt, f"skinny b{bits} n{n} k{k} m{m}")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("m", [1, 2, 4, 16, 64, 300])
def test_qmatmul_exact_arithmetic_is_bit_exact(bits, dt, m):
    """s' = 1/16, b' = -2^(bits-1)/16, integer x in [-8, 8]: every partial sum
    is exact in fp32, so y must be the output rounding of the exact result."""
    n, k, gs = 203, 4096, 64
    log(f"exact bits={bits} dt={dt} m={m}")
    codes = synth.random_codes((n, k), bits, seed=2000 + bits)
    rq = qref.pack(codes, bits)
    sv = np.full((n, k // gs), 1 / 16, dtype=np.float32)
    bv = np.full((n, k // gs), -(2 ** (bits - 1)) / 16, dtype=np.float32)
    rs = sv if dt == F32 else (qref.f32_to_bf16(sv) if dt == BF16 else qref.f32_to_f16(sv))
    rb = bv if dt == F32 else (qref.f32_to_bf16(bv) if dt == BF16 else qref.f32_to_f16(bv))
    x = synth.random_ints((m, k), -8, 8, seed=2100 + bits).astype(np.float32)
    xs = x if dt == F32 else (qref.f32_to_bf16(x) if dt == BF16 else qref.f32_to_f16(x))
    y = qp.qmatmul(to_device(xs, dt), to_device(rq, dt), to_device(rs, dt), to_device(rb, dt),
                   bits, gs)
    torch.cuda.synchronize()
    y_ref, _ = qref.qmatmul(xs, dt, rq, rs, rb, dt, k, bits, gs)
    assert np.array_equal(bits_of(y, dt), rne_to_bits(y_ref, dt))


def test_qmatmul_iota_example_shape_and_values():
    w = synth.iota_f32((4, 128))
    x = synth.iota_f32((3, 128))
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, 4, 64, F32)
    y = qp.qmatmul(torch.from_numpy(x).to(dev()), gq, gs_, gb, 4, 64)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (3, 4)
    y_ref, S = qref.qmatmul(x, F32, rq, rs, rb, F32, 128, 4, 64)
    assert_within(y, y_ref, S, F32, "iota")


@pytest.mark.parametrize("m", [1, 8])
def test_qmatmul_tiny_config_full(m):
    """W fp32 [256, 1024] N(0, 0.02) (seed 11), 4-bit gs64, fp32 scales; x fp32 N(0, 1)."""
    log(f"tiny config m={m}")
    w = synth.normal_f32((256, 1024), 0.02, 11)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, 4, 64, F32)
    xs, xt = activations((m, 1024), F32, 12 if m == 1 else 13)
    y = qp.qmatmul(xt, gq, gs_, gb, 4, 64)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, F32, rq, rs, rb, F32, 1024, 4, 64)
    assert_within(y, y_ref, S, F32, "tiny")


def sampled_check(y, xs, dt, rq, rs, rb, k, bits, gs, n_samples=3000, seed=0, tau=None, blocks=()):
    """Random outputs, the four corners, and every output of each 256 x 256
    block (m0, n0) in `blocks` (whole tiles of the matrix-core GEMM, so every
    lane, register and wave position of a tile is checked)."""
    m, n = y.shape
    g = synth.rng(seed)
    mi = g.integers(0, m, n_samples)
    ni = g.integers(0, n, n_samples)
    # Always include the corners and the last row (ragged tails).
    mi = np.concatenate([mi, [0, m - 1, 0, m - 1]])
    ni = np.concatenate([ni, [0, 0, n - 1, n - 1]])
    for (m0, n0) in blocks:
        bm, bn = np.meshgrid(np.arange(m0, min(m0 + 256, m)), np.arange(n0, min(n0 + 256, n)),
                             indexing="ij")
        mi = np.concatenate([mi, bm.ravel()])
        ni = np.concatenate([ni, bn.ravel()])
    y_ref, S = qref.qmatmul_sampled(xs, dt, rq, rs, rb, dt, k, bits, gs, mi, ni)
    yv = values(y)[mi, ni]
    assert_within(torch.from_numpy(yv), y_ref, S, dt, "sampled", tau=tau)


@pytest.mark.parametrize("bits", [4, 8, 2, 3, 6])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_qmatmul_decode_config_full(bits, m):
    """W [14336, 4096] N(0, 0.02) (seed 21), gs64, bf16 scales; x bf16 [m, 4096]
    (seed 22). Every output against the oracle (at most 16 x 14336 of them).
    At 16 rows (at 4 too for 3- and 6-bit codes) 2-, 3-, 4- and 6-bit codes
    take the row-contiguous skinny form; 6-bit codes take it from 2^25 codes,
    which this matrix has."""
    log(f"decode config bits={bits} m={m}")
    w = synth.normal_f32((14336, 4096), 0.02, 21)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, bits, 64, BF16)
    xs, xt = activations((m, 4096), BF16, 22)
    y = qp.qmatmul(xt, gq, gs_, gb, bits, 64)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, BF16, rq, rs, rb, BF16, 4096, bits, 64)
    assert_within(y, y_ref, S, BF16, f"decode config b{bits} m{m}")


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("m", [5, 16])
def test_qmatmul_six_bit_row_contiguous(dt, gs, m):
    """6-bit codes on the row-contiguous skinny form, which they take from
    2^25 codes: 2403 x 14336 (34.4 M codes; the last block's row groups are
    ragged), every output against the oracle."""
    n, k = 2403, 14336
    log(f"six-bit row-contiguous dt={dt} gs={gs} m={m}")
    y, y_ref, S = run_case(n, k, m, 6, gs, dt, seed=5600 + gs + m)
    assert_within(y, y_ref, S, dt, f"six-bit row-contiguous gs{gs} m{m}")


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("m", [1, 8])
def test_qmatmul_cross_word_config_full(bits, gs, m):
    """W [4096, 4096] N(0, 0.02) (seed 31), fp16 scales; x fp16 [m, 4096]
    (seed 32). Every output against the oracle."""
    log(f"cross-word config bits={bits} gs={gs} m={m}")
    w = synth.normal_f32((4096, 4096), 0.02, 31)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, bits, gs, F16)
    xs, xt = activations((m, 4096), F16, 32)
    y = qp.qmatmul(xt, gq, gs_, gb, bits, gs)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, F16, rq, rs, rb, F16, 4096, bits, gs)
    assert_within(y, y_ref, S, F16, f"cross-word config b{bits} gs{gs} m{m}")


@pytest.mark.parametrize("m", [17, 64, 100, 257])
@pytest.mark.parametrize("bits,dt,gs", [(4, BF16, 64), (2, BF16, 32), (3, F16, 128), (6, F16, 64),
                                        (8, BF16, 64)])
def test_qmatmul_prefill_sizes_small(m, bits, dt, gs):
    log(f"prefill small m={m} bits={bits} dt={dt}")
    y, y_ref, S = run_case(300, 512, m, bits, gs, dt, seed=3000 + m + bits)
    assert_within(y, y_ref, S, dt, f"prefill m{m} b{bits}")


@pytest.mark.parametrize("k", [96, 160, 544])
@pytest.mark.parametrize("bits,dt", [(4, BF16), (3, F16), (8, BF16)])
def test_qmatmul_many_rows_k_not_multiple_of_64(k, bits, dt):
    """More than 16 activation rows with K an odd multiple of 32: every code
    of the last half k-step must count."""
    log(f"many rows k={k} bits={bits} dt={dt}")
    y, y_ref, S = run_case(150, k, 40, bits, 32, dt, seed=3500 + k + bits)
    assert_within(y, y_ref, S, dt, f"k{k} b{bits}")


@pytest.mark.parametrize("shape_x,shape_w,xseed,wseed", [
    ((2048, 4096), (14336, 4096), 43, 41),
    ((2048, 14336), (4096, 14336), 44, 42),
])
def test_qmatmul_prefill_config_sampled(shape_x, shape_w, xseed, wseed):
    """3,000 random outputs and four whole 256 x 256 blocks (the first, the
    last, and two interior ones at different XCD positions of the tile grid)."""
    log(f"prefill config x={shape_x} w={shape_w}")
    w = synth.normal_f32(shape_w, 0.02, wseed)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, 4, 64, BF16)
    xs, xt = activations(shape_x, BF16, xseed)
    y = qp.qmatmul(xt, gq, gs_, gb, 4, 64)
    torch.cuda.synchronize()
    m, n = shape_x[0], shape_w[0]
    blocks = [(0, 0), (m - 256, n - 256), (768, 1280), (1536, n // 2 + 256)]
    sampled_check(y, xs, BF16, rq, rs, rb, shape_w[1], 4, 64, seed=xseed, blocks=blocks)


def test_qmatmul_k_zero_writes_zeros():
    x = torch.ones((3, 0), dtype=torch.bfloat16, device=dev())
    wq = torch.empty((5, 0), dtype=torch.int32, device=dev())
    s = torch.empty((5, 0), dtype=torch.bfloat16, device=dev())
    y = torch.full((3, 5), 7.0, dtype=torch.bfloat16, device=dev())
    qp.qmatmul(x, wq, s, s, 4, 64, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_qmatmul_empty_m_or_n():
    w = synth.normal_f32((8, 64), 0.02, 5)
    _, (gq, gs_, gb) = quantize_both(w, 4, 64, BF16)
    y = qp.qmatmul(torch.empty((0, 64), dtype=torch.bfloat16, device=dev()), gq, gs_, gb, 4, 64)
    assert y.shape == (0, 8)


def test_qmatmul_dtype_mismatch_raises():
    w = synth.normal_f32((8, 64), 0.02, 5)
    _, (gq, gs_, gb) = quantize_both(w, 4, 64, BF16)
    with pytest.raises(qp.QpackError, match="DTYPE_MISMATCH"):
        qp.qmatmul(torch.zeros((1, 64), dtype=torch.float16, device=dev()), gq, gs_, gb, 4, 64)


def shifted_copy(t: torch.Tensor) -> torch.Tensor:
    """A contiguous copy of t placed one element into a fresh buffer (for
    16-bit elements: an address that is 2 mod 4)."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("m", [40, 300])
def test_qmatmul_prefill_scales_not_dword_aligned(m):
    """Scales and biases at an address that is 2 mod 4: the tile GEMM reads
    them as aligned dwords, so such a call takes the 16-row skinny launches;
    both must match the oracle."""
    n, k, bits, gs, dt = 150, 256, 4, 64, BF16
    log(f"prefill unaligned scales m={m}")
    w = synth.normal_f32((n, k), 0.02, 3700 + m)
    (rq, rs, rb), (gq, gs_, gb) = quantize_both(w, bits, gs, dt)
    s2, b2 = shifted_copy(gs_), shifted_copy(gb)
    assert s2.data_ptr() % 4 == 2 and b2.data_ptr() % 4 == 2
    xs, xt = activations((m, k), dt, 3800 + m)
    y_shift = qp.qmatmul(xt, gq, s2, b2, bits, gs)
    y_al = qp.qmatmul(xt, gq, gs_, gb, bits, gs)
    torch.cuda.synchronize()
    y_ref, S = qref.qmatmul(xs, dt, rq, rs, rb, dt, k, bits, gs)
    assert_within(y_shift, y_ref, S, dt, "scales 2 mod 4")
    assert_within(y_al, y_ref, S, dt, "scales aligned")
