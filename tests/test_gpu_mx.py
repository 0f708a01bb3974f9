"""GPU parity of the microscaled modes (mxfp4, mxfp8, nvfp4) against the oracle,
through the C ABI: qpack_dequantize_mx bit-exact, qmatmul_mx within
tau*S + half an output ulp, and bit-exact where every product and sum is exact.

Codes and scale bytes are seeded random bytes (every FP8 code, including the
0x7F / 0xFF that decode to +-480, and for nvfp4 every E4M3 scale byte), never
anything the device produced.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import (BF16, F16, F32, TORCH_DT, activations, assert_within, dev, log, to_device,
                      to_numpy)
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu
MODES = [qref.MXFP4, qref.MXFP8, qref.NVFP4]
MODE_IDS = ["mxfp4", "mxfp8", "nvfp4"]


def mx_weights(n, k, mode, seed, e8m0_lo=118, e8m0_hi=133, small=False):
    """Packed random codes and scale bytes: E8M0 bytes in [lo, hi] (scales
    2^-9 .. 2^6); nvfp4 E4M3 scale bytes of every value. `small` keeps the
    products inside fp16's range (|y| < 65504): E8M0 bytes in [112, 123],
    nvfp4 scale magnitudes below 16."""
    bits, gs = qref.mx_params(mode)
    codes = synth.random_codes((n, k), bits, seed).astype(np.uint8)
    wq = qref.pack(codes, bits)
    if mode == qref.NVFP4:
        if small:
            mag = synth.random_ints((n, k // gs), 0, 0x57, seed + 1)
            sb = mag | (synth.random_ints((n, k // gs), 0, 1, seed + 2) << 7)
        else:
            sb = synth.random_ints((n, k // gs), 0, 255, seed + 1)
    else:
        lo, hi = (112, 123) if small else (e8m0_lo, e8m0_hi)
        sb = synth.random_ints((n, k // gs), lo, hi, seed + 1)
    return wq, sb.astype(np.uint8)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def check_dequant(wq, sb, mode, k, out_dt, what):
    log(f"{what}: mode={mode} n={wq.shape[0]} k={k} out={out_dt}")
    got = qp.qpack_dequantize_mx(to_device(wq, F32), dev_u8(sb), mode,
                                 out_dtype=TORCH_DT[out_dt])
    torch.cuda.synchronize()
    ref = qref.mx_dequantize(wq, sb, mode, k, out_dt)
    view = np.uint32 if out_dt == F32 else np.uint16
    g = to_numpy(got).view(view)
    r = ref.view(view)
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {r.size} differ; first at {i}: "
                             f"gpu=0x{int(g[i]):x} ref=0x{int(r[i]):x}")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("out_dt", [F32, F16, BF16])
def test_mx_dequantize_bit_exact(mode, out_dt):
    # 29 rows of 320: 1160 runs of 8 lanes, two blocks of 1024 runs, ragged tail.
    wq, sb = mx_weights(29, 320, mode, 2000 + mode)
    check_dequant(wq, sb, mode, 320, out_dt, "random")


@pytest.mark.parametrize("mode", [qref.MXFP4, qref.MXFP8], ids=["mxfp4", "mxfp8"])
def test_mx_dequantize_every_e8m0_byte(mode):
    """All 256 scale bytes, including 0 (2^-127, subnormal results) and 255
    (2^128: infinite for nonzero lanes, zero for zero lanes)."""
    wq, _ = mx_weights(256, 64, mode, 2100 + mode)
    sb = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)
    for out_dt in (F32, BF16, F16):
        check_dequant(wq, sb, mode, 64, out_dt, "every e8m0 byte")


def test_mx_dequantize_unaligned_output():
    wq, sb = mx_weights(3, 64, qref.MXFP4, 2200)
    buf = torch.zeros(3 * 64 + 1, dtype=torch.bfloat16, device=dev())
    out = buf[1:].view(3, 64)
    qp.qpack_dequantize_mx(to_device(wq, F32), dev_u8(sb), qref.MXFP4, out=out)
    torch.cuda.synchronize()
    ref = qref.mx_dequantize(wq, sb, qref.MXFP4, 64, BF16)
    assert np.array_equal(to_numpy(out).view(np.uint16), ref)
    assert buf[0].item() == 0.0


def run_mx(m, n, k, mode, dt, seed, what, x_offset=0):
    wq, sb = mx_weights(n, k, mode, seed, small=dt == F16)
    x_st, _ = activations((m, k), dt, seed + 7)
    log(f"{what}: mode={mode} m={m} n={n} k={k} dt={dt}")
    xt = to_device(x_st, dt)
    if x_offset:
        buf = torch.empty(m * k + x_offset, dtype=TORCH_DT[dt], device=dev())
        buf[x_offset:] = xt.reshape(-1)
        xt = buf[x_offset:].view(m, k)
    y = qp.qmatmul_mx(xt, to_device(wq, F32), dev_u8(sb), mode)
    torch.cuda.synchronize()
    yr, S = qref.mx_qmatmul(x_st, dt, wq, sb, mode, k)
    assert_within(y, yr, S, dt, what)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("m", [1, 2, 5])
def test_mx_qmatmul_stream(mode, dt, m):
    # K = 1024: 32 units per row, half the lanes of a wave idle; 300 rows is
    # not a multiple of the rows a block takes.
    run_mx(m, 300, 1024, mode, dt, 2300 + 10 * mode + m, "stream")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("k", [2048, 4096, 14336])
def test_mx_qmatmul_stream_units_per_lane(mode, k):
    """One, two and seven (rounded to eight) units per lane."""
    run_mx(1, 96, k, mode, BF16, 2400 + mode + k, "units per lane")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_mx_qmatmul_generic_fp32(mode):
    run_mx(3, 70, 256, mode, F32, 2500 + mode, "generic fp32")


def test_mx_qmatmul_generic_shapes():
    # nvfp4 with K = 48 (not a multiple of 32); K above the stream kernel's
    # 16384; an activation pointer that is not 16-byte aligned.
    run_mx(2, 33, 48, qref.NVFP4, BF16, 2600, "nvfp4 k=48")
    run_mx(1, 17, 16384 + 32, qref.MXFP4, BF16, 2610, "k above 16384")
    run_mx(2, 40, 512, qref.MXFP8, F16, 2620, "unaligned x", x_offset=1)


def test_mx_qmatmul_fp8_nan_codes_take_the_exact_decode():
    """Rows made only of 0x7F / 0xFF codes (+-480 on the pages, NaN to the
    conversion instructions) must give finite, exact sums."""
    n, k = 8, 256
    codes = np.full((n, k), 0x7F, dtype=np.uint8)
    codes[::2, ::3] = 0xFF
    wq = qref.pack(codes, 8)
    sb = np.full((n, k // 32), 120, dtype=np.uint8)
    x = synth.random_ints((1, k), -4, 4, 2700).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(dev())
    y = qp.qmatmul_mx(xt, to_device(wq, F32), dev_u8(sb), qref.MXFP8)
    torch.cuda.synchronize()
    yr, _ = qref.mx_qmatmul(to_numpy(xt.cpu()), BF16, wq, sb, qref.MXFP8, k)
    assert torch.isfinite(y).all()
    expect = torch.from_numpy(yr.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(y.cpu(), expect)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_mx_qmatmul_exact_integer_case_bit_exact(mode):
    """Integer activations in [-8, 8], scales 2^-2 .. 2^2 (nvfp4: E4M3 bytes
    0x30..0x47, 0.5 .. 3.75) and, for mxfp8, lanes of magnitude 0.5 .. 7.5:
    every product and partial sum is exact in fp32, so y must be the oracle's
    exact result rounded once."""
    n, k = 64, 1024
    wq, sb = mx_weights(n, k, mode, 2800 + mode, 125, 129)
    if mode == qref.NVFP4:
        sb = synth.random_ints(sb.shape, 0x30, 0x47, 2810).astype(np.uint8)
    if mode == qref.MXFP8:
        # E4M3 lanes of exponent field 6..9 (magnitudes 0.5 .. 7.5), both signs.
        e = synth.random_ints((n, k), 6, 9, 2811)
        mant = synth.random_ints((n, k), 0, 7, 2812)
        sign = synth.random_ints((n, k), 0, 1, 2813)
        wq = qref.pack((sign << 7 | e << 3 | mant).astype(np.uint8), 8)
    x = synth.random_ints((2, k), -8, 8, 2820 + mode).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(dev())
    y = qp.qmatmul_mx(xt, to_device(wq, F32), dev_u8(sb), mode)
    torch.cuda.synchronize()
    yr, _ = qref.mx_qmatmul(x, F32, wq, sb, mode, k)
    expect = torch.from_numpy(yr.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(y.cpu(), expect)


def test_mx_qmatmul_full_size_decode():
    """mxfp4 W[14336, 4096], x bf16 [1, 4096], every output against the oracle."""
    run_mx(1, 14336, 4096, qref.MXFP4, BF16, 2900, "full size mxfp4")


def test_mx_qmatmul_k0_and_rejections():
    x = torch.ones((2, 0), dtype=torch.bfloat16, device=dev())
    wq = torch.zeros((3, 0), dtype=torch.int32, device=dev())
    sb = torch.zeros((3, 0), dtype=torch.uint8, device=dev())
    y = qp.qmatmul_mx(x, wq, sb, qref.MXFP4)
    torch.cuda.synchronize()
    assert y.shape == (2, 3) and (y == 0).all()
    x = torch.ones((1, 48), dtype=torch.bfloat16, device=dev())
    wq = torch.zeros((3, 6), dtype=torch.int32, device=dev())
    sb = torch.zeros((3, 1), dtype=torch.uint8, device=dev())
    with pytest.raises(qp.QpackError) as e:
        qp.qmatmul_mx(x, wq, sb, qref.MXFP4)     # K = 48 is not a multiple of 32
    assert e.value.status == 4
    with pytest.raises(qp.QpackError) as e:
        qp.qmatmul_mx(x, wq, sb, 7)
    assert e.value.status == 2


# ------------------------------------------------------------------ prefill tiles (M > 16)

@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dt", [BF16, F16])
def test_mx_qmatmul_prefill_tiles(mode, dt):
    # 300 activation rows (two 256-row tiles, the second ragged), 520 weight
    # rows (ragged 128- or 256-wide tiles), K = 1024: 16 k steps.
    run_mx(300, 520, 1024, mode, dt, 3000 + 10 * mode + dt, "prefill tiles")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_mx_qmatmul_prefill_exact_integer_case(mode):
    """The exact case of the stream kernel on the matrix-core tiles: y must be
    the oracle's exact result rounded once."""
    n, k, m = 96, 512, 40
    wq, sb = mx_weights(n, k, mode, 3100 + mode, 125, 129)
    if mode == qref.NVFP4:
        sb = synth.random_ints(sb.shape, 0x30, 0x47, 3110).astype(np.uint8)
    if mode == qref.MXFP8:
        e = synth.random_ints((n, k), 6, 9, 3111)
        mant = synth.random_ints((n, k), 0, 7, 3112)
        sign = synth.random_ints((n, k), 0, 1, 3113)
        codes = (sign << 7 | e << 3 | mant).astype(np.uint8)
        codes[::7, ::5] = 0x7F      # +480 * scale: the patched conversion
        codes[3::7, 1::5] = 0xFF
        wq = qref.pack(codes, 8)
    x = synth.random_ints((m, k), -2, 2, 3120 + mode).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16).to(dev())
    y = qp.qmatmul_mx(xt, to_device(wq, F32), dev_u8(sb), mode)
    torch.cuda.synchronize()
    yr, _ = qref.mx_qmatmul(x, F32, wq, sb, mode, k)
    expect = torch.from_numpy(yr.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(y.cpu(), expect)


def test_mx_qmatmul_prefill_k_not_multiple_of_64():
    """nvfp4 K = 96: not whole 64-wide tile steps, so the stream kernel runs
    two activation rows at a time."""
    run_mx(20, 70, 96, qref.NVFP4, BF16, 3200, "prefill k=96")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_mx_qmatmul_prefill_full_size_sampled(mode):
    """x bf16 [2048, 4096] times W [14336, 4096] in the launch configuration of
    the benchmark; a 16 x 64 block of outputs (rows and columns spread over
    the tiles) against the oracle."""
    M, N, K = 2048, 14336, 4096
    wq, sb = mx_weights(N, K, mode, 3300 + mode)
    x_st, _ = activations((M, K), BF16, 3310 + mode)
    log(f"full-size prefill: mode={mode}")
    y = qp.qmatmul_mx(to_device(x_st, BF16), to_device(wq, F32), dev_u8(sb), mode)
    torch.cuda.synchronize()
    mi = np.linspace(0, M - 1, 16).astype(np.int64)
    ni = np.linspace(0, N - 1, 64).astype(np.int64)
    yr, S = qref.mx_qmatmul(x_st[mi], BF16, wq[ni], sb[ni], mode, K)
    block = y.cpu()[torch.from_numpy(mi)][:, torch.from_numpy(ni)]
    assert_within(block, yr, S, BF16, "full-size prefill")
