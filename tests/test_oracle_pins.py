"""Pins of the oracle (CPU only) against what the pages and mathematics fix.

Each check compares the oracle with something other than itself: the bit
layout printed as a rule in emily's `dequantize_defn/1` docs (hand-derived
word vectors and a big-integer formulation), library routines (torch / numpy
float conversions, numpy fp64 matmul), closed forms (the iota example of
emily's `quantized_matmul/2` docs, constant groups, exact dyadic arithmetic),
invariants (the quantization round-trip bound, MoE per-pair reduction,
permutation invariance) and brute force on tiny inputs.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import qref
from weight_only_quantized_qgemv_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32, F16, BF16 = qref.F32, qref.F16, qref.BF16
ALL_BITS = [2, 3, 4, 6, 8]


# ---------------------------------------------------------------- helpers

def load_pack_vectors():
    out = []
    with open(os.path.join(GOLDEN, "pack_vectors.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            b, codes, words = (t.strip() for t in line.split("|"))
            out.append((int(b), [int(c) for c in codes.split(",")],
                        [int(w, 16) for w in words.split()]))
    return out


def load_iota_golden():
    d = {}
    with open(os.path.join(GOLDEN, "iota_qmatmul.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split("|"))
            d[key] = val.split()
    return d


def bigint_pack(codes, bits):
    """Independent formulation of the layout: the row is one integer whose
    bits [i*bits, (i+1)*bits) hold lane i; words are its 32-bit limbs."""
    v = 0
    for i, c in enumerate(codes):
        v |= int(c) << (i * bits)
    nw = len(codes) * bits // 32
    return [(v >> (32 * j)) & 0xFFFFFFFF for j in range(nw)]


def to_bits16(a_f32: np.ndarray, dtype_code: int) -> np.ndarray:
    """Round fp32 values to fp16/bf16 with torch (RNE) and return the bits."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    tt = torch.float16 if dtype_code == F16 else torch.bfloat16
    return t.to(tt).view(torch.int16).numpy().view(np.uint16).copy()


def values(a, dtype_code):
    """fp32 values of a stored array, decoded with torch / numpy (not the oracle)."""
    if dtype_code == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype_code == F16:
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)
    t = torch.from_numpy(np.asarray(a, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def store(vals_f32, dtype_code):
    return np.asarray(vals_f32, np.float32) if dtype_code == F32 else to_bits16(vals_f32, dtype_code)


def round_half_away(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    return fl + 1 if v - fl >= Fraction(1, 2) else fl


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("bits,codes,words", load_pack_vectors())
def test_pack_matches_hand_derived_words(bits, codes, words):
    wq = qref.pack(np.array([codes], dtype=np.uint8), bits)
    assert wq[0].tolist() == words
    assert qref.unpack(wq, len(codes), bits)[0].tolist() == codes
    assert bigint_pack(codes, bits) == words


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("k", [32, 96, 160, 1024])
def test_pack_equals_bigint_layout_and_round_trips(bits, k):
    codes = synth.random_codes((5, k), bits, seed=1000 + 10 * bits + k)
    wq = qref.pack(codes, bits)
    for r in range(codes.shape[0]):
        assert wq[r].tolist() == bigint_pack(codes[r], bits)
    assert np.array_equal(qref.unpack(wq, k, bits), codes)


def test_pack_8bit_is_a_byte_copy():
    codes = synth.random_codes((3, 64), 8, seed=7)
    assert np.array_equal(qref.pack(codes, 8), codes.view("<u4"))


def test_pack_4bit_is_nibble_pairs():
    codes = synth.random_codes((3, 64), 4, seed=8)
    bytes_ = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(qref.pack(codes, 4), np.ascontiguousarray(bytes_).view("<u4"))


def test_pack_rejects_ragged_bit_length():
    # emily's build_word_indices: k*bits must be a multiple of 32.
    with pytest.raises(ValueError):
        qref.pack(np.zeros((1, 16), np.uint8), 3)
    with pytest.raises(ValueError):
        qref.quantize(np.zeros((1, 48), np.float32), 4, 32, F32)  # k % gs != 0


# ---------------------------------------------------------------- float formats

def _bf16_probe_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lo = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0x8002, 0xBFFF,
                   0xC000, 0xFFFE, 0xFFFF], dtype=np.uint32)
    lo = np.concatenate([lo, synth.rng(5).integers(0, 1 << 16, 52, dtype=np.uint32)])
    return (hi[:, None] | lo[None, :]).ravel()


def test_bf16_rne_matches_torch():
    """Every bf16 high half crossed with every rounding-relevant low half
    (ties, just below / above ties, extremes) plus random low halves."""
    u = _bf16_probe_patterns()
    f = u.view(np.float32)
    ours = qref.f32_to_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    ours_nan = ours[nan]
    assert np.all((ours_nan & 0x7F80) == 0x7F80) and np.all((ours_nan & 0x7F) != 0)


def test_f16_rne_matches_numpy():
    """Exhaustive over all 2^23 mantissas at the exponents where fp16's
    behaviour changes (below the smallest subnormal, the subnormal range, the
    normal boundary, 1.0, the overflow edge), both signs; every other exponent
    from 2^-27 to 2^17 with all 2^10 kept-mantissa values crossed with the
    rounding-relevant low 13 bits; and a strided sweep of all of fp32."""
    m = np.arange(1 << 23, dtype=np.uint32)
    full = [np.uint32(e << 23) | m for e in (101, 102, 103, 110, 112, 113, 127, 142, 143)]
    keep = np.arange(1 << 10, dtype=np.uint32) << 13
    low = np.array([0, 1, 0x7FF, 0xFFE, 0xFFF, 0x1000, 0x1001, 0x17FF, 0x1FFE, 0x1FFF],
                   dtype=np.uint32)
    mix = (keep[:, None] | low[None, :]).ravel()
    part = [np.uint32(e << 23) | mix for e in range(100, 145)]
    u = np.concatenate(full + part)
    u = np.concatenate([u, u | np.uint32(0x80000000),
                        np.arange(0, 1 << 32, 65537, dtype=np.uint64).astype(np.uint32)])
    f = u.view(np.float32)
    ours = qref.f32_to_f16(f)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x3FF) != 0)


def test_16bit_decoders_match_library():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours_bf = qref.to_f32(h, BF16)
    ref_bf = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    ours_h = qref.to_f32(h, F16)
    ref_h = h.view(np.float16).astype(np.float32)
    for a, b in ((ours_bf, ref_bf), (ours_h, ref_h)):
        nan = np.isnan(b)
        assert np.array_equal(np.isnan(a), nan)
        assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))


# ---------------------------------------------------------------- quantize

def test_quantize_iota_closed_form():
    g = load_iota_golden()
    w = synth.iota_f32((4, 128))
    wq, s, b = qref.quantize(w, 4, 64, F32)
    s_exact = Fraction(g["scale"][0])
    assert np.all(s == np.float32(float(s_exact)))
    assert Fraction(float(np.float32(63) / np.float32(15))) == s_exact
    assert np.array_equal(b, np.array([[128 * n + 64 * gg for gg in range(2)] for n in range(4)],
                                      dtype=np.float32))
    codes = qref.unpack(wq, 128, 4)
    expect = [round_half_away(Fraction(j) / s_exact) for j in range(64)]
    for n in range(4):
        for gg in range(2):
            assert codes[n, 64 * gg:64 * gg + 64].tolist() == expect
    counts = np.bincount(np.array(expect), minlength=16).tolist()
    assert counts == [int(c) for c in g["code_counts"]]
    # No quotient lies near a .5 tie, so fp32 evaluation cannot flip a code.
    assert min(abs(Fraction(j) / s_exact - math.floor(Fraction(j) / s_exact) - Fraction(1, 2))
               for j in range(64)) > Fraction(2, 100)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_quantize_round_trip_bound(bits, gs, dt):
    """|w - w'| <= s'/2 (+ the storage rounding of s and b, + fp32 slack).
    With fp32 storage this is the plain half-step bound."""
    w = synth.normal_f32((12, 512), 0.02, seed=200 + bits * 7 + gs + dt)
    w[0, :gs] = 0.0125  # a constant group
    wq, s, b = qref.quantize(w, bits, gs, dt)
    wd = qref.dequantize(wq, s, b, dt, 512, bits, gs).astype(np.float64)
    sv = np.repeat(values(s, dt).astype(np.float64), gs, axis=1)
    bv = np.repeat(values(b, dt).astype(np.float64), gs, axis=1)
    wg = w.astype(np.float64).reshape(12, -1, gs)
    mn = np.repeat(wg.min(axis=2), gs, axis=1)
    s_true = np.repeat((wg.max(axis=2) - wg.min(axis=2)) / (2 ** bits - 1), gs, axis=1)
    w64 = w.astype(np.float64)
    qmax = 2 ** bits - 1
    slack = 2.0 ** -22 * (np.abs(w64) + np.abs(bv) + qmax * sv + np.abs(wd))
    storage = qmax * np.abs(s_true - sv) * (s_true > 0) + np.abs(mn - bv)
    bound = sv / 2 + storage + slack
    err = np.abs(w64 - wd)
    assert np.all(err <= bound)
    if dt == F32:
        assert np.all(err <= sv / 2 + slack + qmax * np.abs(s_true - sv) * (s_true > 0))
    # The bound is tight: quantization really uses the whole half step.
    assert err.max() > 0.3 * sv.max() / 2


@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_quantize_constant_group_is_exact(dt):
    w = np.full((2, 64), 0.37, dtype=np.float32)
    w[1, 32:] = -3.0
    wq, s, b = qref.quantize(w, 4, 32, dt)
    eps = np.float32(np.finfo(np.float32).eps)
    wd = qref.dequantize(wq, s, b, dt, 64, 4, 32)
    if dt == F32:
        # The scale is floored at FLT_EPSILON, every code is 0, w' = w exactly.
        assert np.all(s == eps)
        assert np.all(qref.unpack(wq, 64, 4) == 0)
        assert np.array_equal(wd, w)
    else:
        # Stored bias b' = RNE(w) != w: the floored scale pushes the residual
        # w - b' to code 0 or 15, so w' stays within the bias rounding of w.
        bv = np.repeat(values(b, dt), 32, axis=1).astype(np.float64)
        codes = qref.unpack(wq, 64, 4)
        assert np.all((codes == 0) | (codes == 15))
        assert np.all(np.abs(wd - w) <= np.abs(w - bv) + 16 * float(eps))


def test_quantize_zero_bias_is_positive_zero():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 1] = -0.0
    w[0, 5] = 1.5
    for dt in (F32, F16, BF16):
        _, _, b = qref.quantize(w[:, ::-1].copy(), 4, 64, dt)
        bits_ = b.view(np.uint32) if dt == F32 else b
        assert int(bits_[0, 0]) == 0


def test_quantize_rounds_half_away_from_zero():
    # 4-bit group spanning [0, 15]: scale 1, bias 0, so the code is round(w).
    w = np.array([[0, 15, 2.5, 0.5, 14.5, 7.5, 7.4999995, 1.0000001] + [0] * 24],
                 dtype=np.float32)
    wq, s, b = qref.quantize(w, 4, 32, F32)
    assert s[0, 0] == 1.0 and b[0, 0] == 0.0
    assert qref.unpack(wq, 32, 4)[0, :8].tolist() == [0, 15, 3, 1, 15, 8, 7, 1]
    # 2-bit group spanning [0, 3]: 1.5 -> 2, 0.5 -> 1, 2.5 -> 3
    w2 = np.array([[0, 3, 1.5, 0.5, 2.5] + [0] * 27], dtype=np.float32)
    wq2, _, _ = qref.quantize(w2, 2, 32, F32)
    assert qref.unpack(wq2, 32, 2)[0, :5].tolist() == [0, 3, 2, 1, 3]


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_quantize_picks_nearest_stored_grid_point(bits, dt):
    """Each code is the grid point q*s' + b' (stored scale and bias) nearest
    to w, over all 2^bits codes; only fp32 rounding may break near-ties."""
    w = synth.normal_f32((6, 256), 0.02, seed=250 + bits + dt)
    w[3] += 3.7   # groups far from zero: bias rounding is large against the step
    w[4] *= 50.0
    wq, s, b = qref.quantize(w, bits, 32, dt)
    codes = qref.unpack(wq, 256, bits).astype(np.float64)
    sv = np.repeat(values(s, dt).astype(np.float64), 32, axis=1)
    bv = np.repeat(values(b, dt).astype(np.float64), 32, axis=1)
    w64 = w.astype(np.float64)
    grid = np.arange(2 ** bits, dtype=np.float64)
    dist_all = np.abs(w64[..., None] - (grid * sv[..., None] + bv[..., None]))
    best = dist_all.min(axis=-1)
    chosen = np.abs(w64 - (codes * sv + bv))
    assert np.all(chosen <= best + 2.0 ** -21 * (np.abs(w64) + np.abs(bv)) + 1e-3 * sv)


def test_quantize_clamps_codes_to_range():
    # bf16 storage, group far from zero. Bias 100.2 is stored as 100.0 (bf16
    # spacing 0.5 there), so (101.2 - b')/s' ~ 306 and the top code clamps to
    # 255; bias 100.3 is stored as 100.5, so (100.3 - b')/s' < 0 clamps to 0.
    for lo, idx, clamped, stored_bias in ((100.2, 1, 255, 100.0), (100.3, 0, 0, 100.5)):
        w = np.full((1, 32), lo + 0.5, dtype=np.float32)
        w[0, 0] = lo
        w[0, 1] = lo + 1.0
        wq, s, b = qref.quantize(w, 8, 32, BF16)
        bv, sv = values(b, BF16)[0, 0], values(s, BF16)[0, 0]
        assert bv == stored_bias
        quotient = (float(w[0, idx]) - float(bv)) / float(sv)
        assert quotient > 255.5 or quotient < -0.5
        assert qref.unpack(wq, 32, 8)[0, idx] == clamped


# ---------------------------------------------------------------- dense weight in the scales' type

def _typed_case(n, k, bits, gs, dt, seed):
    """Random codes with scales and biases of full mantissa in type dt."""
    codes = synth.random_codes((n, k), bits, seed)
    wq = np.array([bigint_pack(codes[r], bits) for r in range(n)], dtype=np.uint32)
    s = store(np.abs(synth.normal_f32((n, k // gs), 0.02, seed + 1)) + 1e-3, dt)
    b = store(synth.normal_f32((n, k // gs), 0.3, seed + 2), dt)
    return codes, wq, s, b


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 128])
def test_dequantize_typed_f16_matches_numpy_half_arithmetic(bits, gs):
    """numpy's float16 multiply and add each round to nearest-even fp16."""
    codes, wq, s, b = _typed_case(24, 512, bits, gs, F16, 900 + bits)
    s16 = np.repeat(s.view(np.float16), gs, axis=1)
    b16 = np.repeat(b.view(np.float16), gs, axis=1)
    expect = (codes.astype(np.float16) * s16 + b16).view(np.uint16)
    got = qref.dequantize_typed(wq, s, b, F16, 512, bits, gs)
    assert got.dtype == np.uint16
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 128])
def test_dequantize_typed_bf16_matches_torch_bf16_arithmetic(bits, gs):
    """torch's CPU bfloat16 multiply and add each round to nearest-even bf16."""
    codes, wq, s, b = _typed_case(24, 512, bits, gs, BF16, 950 + bits)
    st = torch.from_numpy(s.view(np.int16).copy()).view(torch.bfloat16).repeat_interleave(gs, 1)
    bt = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).repeat_interleave(gs, 1)
    prod = torch.from_numpy(codes.astype(np.int32)).to(torch.bfloat16) * st
    expect = (prod + bt).view(torch.int16).numpy().view(np.uint16)
    got = qref.dequantize_typed(wq, s, b, BF16, 512, bits, gs)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("bits", ALL_BITS)
def test_dequantize_typed_f32_is_the_fp32_form(bits):
    codes, wq, s, b = _typed_case(8, 256, bits, 64, F32, 990 + bits)
    expect = (codes.astype(np.float32) * np.repeat(s, 64, axis=1)) + np.repeat(b, 64, axis=1)
    assert np.array_equal(qref.dequantize_typed(wq, s, b, F32, 256, bits, 64), expect)
    assert np.array_equal(qref.dequantize(wq, s, b, F32, 256, bits, 64), expect)


def test_dequantize_typed_rounds_product_then_sum():
    """Worked by hand in bf16 (8 significant bits; spacing 2^-6 on [2, 4)):
    q = 3, s = 1 + 2^-7, b = -2^-7. The product 3 + 3*2^-7 lies halfway
    between 3 + 2^-6 and 3 + 2^-5 and rounds to the even one, 3 + 2^-5; adding
    b gives 3 + 3*2^-7, again a tie, which rounds to 3 + 2^-5. Rounding only
    once would give 3 + 2^-6 (q*s + b = 3 + 2^-6 exactly)."""
    codes = np.zeros((1, 32), dtype=np.int64)
    codes[0, 0] = 3
    wq = np.array([bigint_pack(codes[0], 4)], dtype=np.uint32)
    s = store(np.array([[1.0 + 2.0 ** -7]], np.float32), BF16)
    b = store(np.array([[-(2.0 ** -7)]], np.float32), BF16)
    got = values(qref.dequantize_typed(wq, s, b, BF16, 32, 4, 32), BF16)
    assert got[0, 0] == 3.0 + 2.0 ** -5
    assert got[0, 1] == -(2.0 ** -7)     # code 0: the bias itself
    assert qref.dequantize(wq, s, b, BF16, 32, 4, 32)[0, 0] == 3.0 + 2.0 ** -6


# ---------------------------------------------------------------- transpose = false

@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dt", [F32, BF16])
def test_qmatmul_t_brute_force_dyadic(bits, dt):
    """W [k, n] built from dyadic codes, scales and biases along n: x @ W is
    exact in fp64 in any order, so the oracle equals numpy's product of the
    dequantized weight (and of its transpose, read with transpose = true)."""
    k, n, gs = 96, 128, 32
    wq, s, b, dense = _dyadic_weights(k, n, bits, gs, dt, 2100 + bits)   # dense: [k, n]
    xs, xv = _activation(5, k, dt, 2110 + bits, sigma=1.0)
    if dt == F32:
        xs = np.round(xs * 8).astype(np.float32) / 8
        xv = xs.astype(np.float64)
    y, S = qref.qmatmul_t(xs, dt, wq, s, b, dt, n, bits, gs)
    assert np.array_equal(y, xv @ dense) or np.allclose(y, xv @ dense, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, np.abs(xv) @ np.abs(dense), rtol=1e-12)
    assert np.array_equal(dense, qref.dequantize(wq, s, b, dt, n, bits, gs).astype(np.float64))


# ---------------------------------------------------------------- per-tensor int8

def load_int8_example():
    d = {}
    with open(os.path.join(GOLDEN, "int8_tensor_example.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split("|"))
            d[key] = [float(v) for v in val.split()]
    return d


def test_int8_tensor_printed_round_trip():
    g = load_int8_example()
    w = np.array(g["input"], dtype=np.float32)
    q, rng_ = qref.quantize_int8_tensor(w)
    assert rng_.tolist() == g["range"]
    assert q.tolist() == [int(v) for v in g["codes"]]
    back = qref.dequantize_int8_tensor(q, rng_)
    tol = (rng_[1] - rng_[0]) / 255.0 + 1e-4        # the page's own check
    assert np.all(np.abs(back - w) <= tol)


def test_int8_tensor_dequantize_matches_numpy_fp32_steps():
    q = synth.random_ints((300,), -128, 127, 2050).astype(np.int8)
    rng_ = np.array([-0.37, 0.91], dtype=np.float32)
    step = np.float32((rng_[1] - rng_[0]) / np.float32(255.0))
    expect = (q.astype(np.float32) + np.float32(128.0)) * step + rng_[0]
    assert np.array_equal(qref.dequantize_int8_tensor(q, rng_), expect)


def test_int8_tensor_round_trip_bound_and_constant_tensor():
    w = synth.normal_f32((64, 96), 0.05, 2060)
    q, rng_ = qref.quantize_int8_tensor(w)
    back = qref.dequantize_int8_tensor(q, rng_)
    step = (float(rng_[1]) - float(rng_[0])) / 255.0
    slack = 2.0 ** -21 * (np.abs(w) + abs(float(rng_[0])) + 255 * step)
    assert np.all(np.abs(back.astype(np.float64) - w) <= step / 2 + slack)
    assert q.min() == -128 and q.max() == 127
    c = np.full((5, 7), 0.25, dtype=np.float32)
    qc, rc = qref.quantize_int8_tensor(c)
    assert (qc == -128).all() and rc.tolist() == [0.25, 0.25]
    assert (qref.dequantize_int8_tensor(qc, rc) == 0.25).all()


def test_int8_tensor_qmatmul_exact_case():
    """Range [-8, 7.9375]: step 1/16, every weight (q + 128)/16 - 8 and every
    product with an integer activation exact, so the oracle equals numpy's."""
    q = synth.random_ints((9, 128), -128, 127, 2070).astype(np.int8)
    rng_ = np.array([-8.0, 7.9375], dtype=np.float32)
    x = synth.random_ints((4, 128), -9, 9, 2071).astype(np.float32)
    y, S = qref.qmatmul_int8_tensor(x, F32, q, rng_)
    w = (q.astype(np.float64) + 128.0) / 16.0 - 8.0
    assert np.array_equal(y, x.astype(np.float64) @ w.T)
    assert np.array_equal(S, np.abs(x.astype(np.float64)) @ np.abs(w).T)


# ---------------------------------------------------------------- MoE FFN block

def _ffn_case(T=5, top_k=3, E=6, D=64, F=96, bits=4, gs=32, dt=BF16, seed=1900):
    def stack(rows, cols, s):
        w = synth.normal_f32((E * rows, cols), 0.05, s)
        wq, sc, bi = qref.quantize(w, bits, gs, dt)
        return wq.reshape(E, rows, -1), sc.reshape(E, rows, -1), bi.reshape(E, rows, -1)
    gate, up, down = stack(F, D, seed), stack(F, D, seed + 1), stack(D, F, seed + 2)
    a = store(synth.normal_f32((T, D), 1.0, seed + 3), dt)
    ids = np.stack([synth.rng(seed + 4 + t).permutation(E)[:top_k] for t in range(T)]).ravel()
    rw = synth.normal_f32((T * top_k,), 0.5, seed + 5)
    return dict(a=a, ids=ids.astype(np.int32), rw=rw, T=T, top_k=top_k, E=E, D=D, F=F,
                bits=bits, gs=gs, dt=dt, gate=gate, up=up, down=down)


def _ffn(c, ids=None, rw=None):
    return qref.moe_ffn(c["a"], c["dt"], c["ids"] if ids is None else ids,
                        c["rw"] if rw is None else rw, c["T"], c["top_k"], c["gate"], c["up"],
                        c["down"], c["dt"], c["E"], c["D"], c["F"], c["bits"], c["gs"])


def test_moe_ffn_composes_the_pinned_moe_products():
    """Gate+up+SiLU, rounded to bf16 by torch, then down, rounded by torch, then
    the slot sum in numpy: the block's definition rebuilt from the pinned MoE
    products and library roundings."""
    c = _ffn_case()
    out, h, o = _ffn(c)
    r = qref.moe_gate_up_silu(c["a"], c["dt"], c["ids"], c["T"], c["top_k"], c["D"], 0,
                              c["gate"], c["up"], c["dt"], c["E"], c["F"], c["D"], c["bits"], c["gs"])
    h_ref = to_bits16(r["silu_out"].astype(np.float32), BF16)
    assert np.array_equal(h, h_ref)
    y, _ = qref.moe(h_ref, BF16, c["ids"], c["T"], c["top_k"], c["top_k"] * c["F"], c["F"],
                    *c["down"], c["dt"], c["E"], c["D"], c["F"], c["bits"], c["gs"])
    o_ref = to_bits16(y.astype(np.float32), BF16)
    assert np.array_equal(o, o_ref)
    ov = values(o_ref, BF16).astype(np.float64).reshape(c["T"], c["top_k"], c["D"])
    expect = (c["rw"].astype(np.float64).reshape(c["T"], c["top_k"], 1) * ov).sum(axis=1)
    assert np.allclose(out, expect, rtol=1e-12, atol=1e-12)


def test_moe_ffn_slot_order_and_linearity():
    c = _ffn_case(seed=1950)
    out, _, _ = _ffn(c)
    perm = np.concatenate([t * c["top_k"] + synth.rng(1960 + t).permutation(c["top_k"])
                           for t in range(c["T"])])
    out_p, _, _ = _ffn(c, ids=c["ids"][perm], rw=c["rw"][perm])
    assert np.allclose(out_p, out, rtol=1e-12, atol=1e-12)
    rw2 = synth.normal_f32(c["rw"].shape, 0.5, 1970)
    out2, _, _ = _ffn(c, rw=rw2)
    out12, _, _ = _ffn(c, rw=(c["rw"].astype(np.float64) + rw2).astype(np.float32))
    assert np.allclose(out12, out + out2, rtol=1e-6, atol=1e-6)
    zero, _, _ = _ffn(c, rw=np.zeros_like(c["rw"]))
    assert not zero.any()


# ---------------------------------------------------------------- microscaled modes

def load_mx_luts():
    d = {}
    with open(os.path.join(GOLDEN, "mx_luts.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split("|"))
            d[key] = val.split()
    return d


def test_fp4_e2m1_matches_the_printed_table():
    lut = [float(v) for v in load_mx_luts()["fp4"]]
    got = [qref.fp4_e2m1(c) for c in range(16)]
    assert got == lut
    assert [math.copysign(1.0, g) for g in got] == [math.copysign(1.0, v) for v in lut]


def test_fp8_e4m3_matches_torch_and_the_printed_quirk():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    quirk = dict((int(a, 16), float(b)) for a, b in
                 (t.split(":") for t in load_mx_luts()["e4m3_quirk"]))
    for byte in range(256):
        got = qref.fp8_e4m3(byte)
        if byte in quirk:
            assert got == quirk[byte]
        else:
            assert got == ref[byte] and math.copysign(1, got) == math.copysign(1, ref[byte]), byte


def test_e8m0_matches_torch_and_the_printed_formula():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    ref = ref.to(torch.float64).numpy()
    for s in range(255):
        assert qref.e8m0(s) == ref[s] == 2.0 ** (s - 127)
    assert qref.e8m0(255) == 2.0 ** 128      # torch: NaN; the page's formula: 2^128
    for t in load_mx_luts()["e8m0"]:
        a, b = t.split(":")
        assert qref.e8m0(int(a)) == float(b)


def test_mx_params_follow_the_pages():
    assert qref.mx_params(qref.MXFP4) == (4, 32)
    assert qref.mx_params(qref.MXFP8) == (8, 32)
    assert qref.mx_params(qref.NVFP4) == (4, 16)


def _lut_dense(codes, sbytes, mode):
    """Dense weight from the printed tables (fp4) and torch's decoders (fp8 /
    e8m0, with the printed 0x7F / 0xFF quirk), independent of the oracle."""
    luts = load_mx_luts()
    fp4 = np.array([float(v) for v in luts["fp4"]])
    e4m3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    e4m3 = e4m3.to(torch.float64).numpy().copy()
    e4m3[0x7F], e4m3[0xFF] = 480.0, -480.0
    e8m0 = np.array([2.0 ** (s - 127) for s in range(256)])
    lanes = e4m3[codes] if mode == qref.MXFP8 else fp4[codes]
    scales = e4m3[sbytes] if mode == qref.NVFP4 else e8m0[sbytes]
    gs = qref.mx_params(mode)[1]
    return lanes * np.repeat(scales, gs, axis=1)


def _mx_case(n, k, mode, seed, lo=110, hi=139):
    bits, gs = qref.mx_params(mode)
    codes = synth.random_codes((n, k), bits, seed)
    wq = np.array([bigint_pack(codes[r], bits) for r in range(n)], dtype=np.uint32)
    if mode == qref.NVFP4:   # E4M3 scale bytes of both signs, all exponents
        sbytes = synth.random_ints((n, k // gs), 0, 255, seed + 1)
    else:
        sbytes = synth.random_ints((n, k // gs), lo, hi, seed + 1)
    return codes, wq, sbytes.astype(np.uint8)


@pytest.mark.parametrize("mode", [1, 2, 3], ids=["mxfp4", "mxfp8", "nvfp4"])
def test_mx_dequantize_matches_table_decode(mode):
    codes, wq, sb = _mx_case(16, 256, mode, 1600 + mode)
    dense = _lut_dense(codes, sb, mode)
    assert np.array_equal(qref.mx_dequantize(wq, sb, mode, 256, F32), dense.astype(np.float32))
    assert np.array_equal(qref.mx_dequantize(wq, sb, mode, 256, BF16),
                          to_bits16(dense.astype(np.float32), BF16))


def test_mx_dequantize_extreme_scales_round_to_the_output_type():
    """E8M0 255 is 2^128: lanes +-1 overflow to +-inf in fp32 and bf16, lane
    0.5 gives 2^127. E8M0 0 with lane 0.5 is 2^-128, an fp32 subnormal."""
    codes = np.zeros((1, 32), dtype=np.int64)
    codes[0, 0], codes[0, 1], codes[0, 2] = 2, 10, 1     # +1.0, -1.0, +0.5
    wq = np.array([bigint_pack(codes[0], 4)], dtype=np.uint32)
    big = qref.mx_dequantize(wq, np.array([[255]], np.uint8), qref.MXFP4, 32, F32)
    assert big[0, 0] == np.inf and big[0, 1] == -np.inf
    assert big[0, 2] == np.float32(2.0 ** 127) and big[0, 3] == 0.0
    big16 = values(qref.mx_dequantize(wq, np.array([[255]], np.uint8), qref.MXFP4, 32, BF16), BF16)
    assert big16[0, 0] == np.inf and big16[0, 2] == 2.0 ** 127
    tiny = qref.mx_dequantize(wq, np.array([[0]], np.uint8), qref.MXFP4, 32, F32)
    assert tiny[0, 2] == np.float32(2.0 ** -128) and tiny[0, 0] == np.float32(2.0 ** -127)


@pytest.mark.parametrize("mode", [1, 2, 3], ids=["mxfp4", "mxfp8", "nvfp4"])
def test_mx_qmatmul_exact_integer_case(mode):
    """Integer activations and scales 2^(s-127) with s in [124, 130]: every
    product and partial sum is a short dyadic number, exact in fp64 in any
    order, so the oracle must equal numpy's matmul of the table-decoded weight."""
    codes, wq, sb = _mx_case(12, 128, mode, 1700 + mode, 124, 130)
    if mode == qref.NVFP4:
        sb = synth.random_ints(sb.shape, 0x30, 0x47, 1710).astype(np.uint8)   # 0.5 .. 3.75
    x = synth.random_ints((5, 128), -8, 8, 1720 + mode).astype(np.float32)
    y, S = qref.mx_qmatmul(x, F32, wq, sb, mode, 128)
    dense = _lut_dense(codes, sb, mode)
    assert np.array_equal(y, x.astype(np.float64) @ dense.T)
    assert np.array_equal(S, np.abs(x.astype(np.float64)) @ np.abs(dense).T)


# ---------------------------------------------------------------- products

def test_qmatmul_iota_example():
    g = load_iota_golden()
    w = synth.iota_f32((4, 128))
    x = synth.iota_f32((3, 128))
    wq, s, b = qref.quantize(w, 4, 64, F32)
    y, S = qref.qmatmul(x, F32, wq, s, b, F32, 128, 4, 64)
    assert y.shape == tuple(int(v) for v in g["shape"])
    expect = np.array([[float(v) for v in g[f"y{m}"]] for m in range(3)])
    # Dequantized weights are fp32-rounded (|q*s| < 64, |w'| < 512): each
    # differs from the exact value by at most 2^-24 * (64 + 512).
    tol = np.abs(x).sum(axis=1, keepdims=True) * 2.0 ** -24 * (64 + 512) + 1e-6
    assert np.all(np.abs(y - expect) <= tol)
    # Bias steps by 128 per output row: y[m,n+1] - y[m,n] = 128 * sum_k x[m,k].
    d = np.diff(y, axis=1) - 128.0 * x.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(d) <= 2 * tol)
    dense = x.astype(np.float64) @ w.astype(np.float64).T
    assert dense[0].tolist() == [float(v) for v in g["dense_y0"]]
    assert not np.allclose(dense, y, rtol=0, atol=100)


def _dyadic_weights(n, k, bits, gs, dt, seed):
    """Codes, scales a/64 and biases c/64 chosen directly; every dequantized
    weight q*s+b is then exact in fp32, and s, b exact in fp16/bf16."""
    codes = synth.random_codes((n, k), bits, seed)
    s_vals = (synth.random_ints((n, k // gs), 1, 64, seed + 1) / 64.0).astype(np.float32)
    b_vals = (synth.random_ints((n, k // gs), -128, 128, seed + 2) / 64.0).astype(np.float32)
    wq = np.array([bigint_pack(codes[r], bits) for r in range(n)], dtype=np.uint32)
    dense = (codes.astype(np.float64) * np.repeat(s_vals, gs, axis=1).astype(np.float64)
             + np.repeat(b_vals, gs, axis=1).astype(np.float64))
    return wq, store(s_vals, dt), store(b_vals, dt), dense


def _activation(m, k, dt, seed, sigma=1.0):
    x = synth.normal_f32((m, k), sigma, seed)
    xs = store(x, dt)
    return xs, values(xs, dt).astype(np.float64)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [F32, F16, BF16])
def test_qmatmul_brute_force_dyadic(bits, gs, dt):
    n, k, m = 9, 256, 3
    wq, s, b, dense = _dyadic_weights(n, k, bits, gs, dt, seed=300 + bits + gs + 10 * dt)
    xs, xv = _activation(m, k, dt, seed=400 + bits)
    y, S = qref.qmatmul(xs, dt, wq, s, b, dt, k, bits, gs)
    y_np = xv @ dense.T
    S_np = np.abs(xv) @ np.abs(dense).T
    assert np.all(np.abs(y - y_np) <= 1e-13 * S_np)
    assert np.allclose(S, S_np, rtol=1e-13, atol=0)
    assert np.allclose(qref.dequantize(wq, s, b, dt, k, bits, gs), dense, rtol=0, atol=0)
    mi = np.array([0, 2, 1, 2])
    ni = np.array([8, 0, 4, 8])
    ys, Ss = qref.qmatmul_sampled(xs, dt, wq, s, b, dt, k, bits, gs, mi, ni)
    assert np.array_equal(ys, y[mi, ni]) and np.array_equal(Ss, S[mi, ni])


@pytest.mark.parametrize("bits", ALL_BITS)
def test_qmatmul_exact_integer_case(bits):
    """s = 1/16, b = -2^(bits-1)/16, integer x: every product and partial sum
    is a small dyadic, so the result is exact and equals integer arithmetic."""
    n, k, m, gs = 7, 4096, 2, 64
    codes = synth.random_codes((n, k), bits, seed=500 + bits)
    wq = qref.pack(codes, bits)
    s = np.full((n, k // gs), 1 / 16, dtype=np.float32)
    b = np.full((n, k // gs), -(2 ** (bits - 1)) / 16, dtype=np.float32)
    x = synth.random_ints((m, k), -8, 8, seed=600 + bits).astype(np.float32)
    y, _ = qref.qmatmul(x, F32, wq, s, b, F32, k, bits, gs)
    exact = x.astype(np.int64) @ (codes.astype(np.int64) - 2 ** (bits - 1)).T
    assert np.array_equal(y * 16, exact.astype(np.float64))


# ---------------------------------------------------------------- MoE

def _moe_case(E=6, n_rows=10, n_cols=128, bits=4, gs=32, dt=BF16, seed=700):
    ws = [_dyadic_weights(n_rows, n_cols, bits, gs, dt, seed + 10 * e) for e in range(E)]
    wq = np.stack([t[0] for t in ws])
    s = np.stack([t[1] for t in ws])
    b = np.stack([t[2] for t in ws])
    dense = np.stack([t[3] for t in ws])
    return wq, s, b, dense


@pytest.mark.parametrize("layout", ["shared_row", "per_slot_row", "single_token"])
def test_moe_matches_gathered_dense_product(layout):
    E, n_rows, n_cols, bits, gs, dt = 6, 10, 128, 4, 32, BF16
    wq, s, b, dense = _moe_case(E, n_rows, n_cols, bits, gs, dt)
    T, top_k = 5, 3
    ids = synth.moe_ids(T, top_k, E, seed=710).ravel()
    if layout == "shared_row":      # gate/up: every slot of a token reads the token's row
        a_f, outer, inner, rows = (T, n_cols), n_cols, 0, T
    elif layout == "per_slot_row":  # down: each pair has its own row
        a_f, outer, inner, rows = (T * top_k, n_cols), top_k * n_cols, n_cols, T * top_k
    else:                           # one token, n_selected slots, src1_stride apart
        T, top_k = 1, 4
        ids = synth.moe_ids(1, 4, E, seed=711).ravel()
        a_f, outer, inner, rows = (4, n_cols), 0, n_cols, 4
    a_s, a_v = _activation(rows, n_cols, dt, seed=720)
    out, S = qref.moe(a_s, dt, ids, T, top_k, outer, inner, wq, s, b, dt, E, n_rows, n_cols,
                      bits, gs)
    a_flat = a_v.ravel()
    for p in range(T * top_k):
        off = (p // top_k) * outer + (p % top_k) * inner
        row = a_flat[off:off + n_cols]
        ref = dense[ids[p]] @ row
        refS = np.abs(dense[ids[p]]) @ np.abs(row)
        assert np.all(np.abs(out[p] - ref) <= 1e-13 * refS)
        assert np.allclose(S[p], refS, rtol=1e-13, atol=0)


def test_moe_pair_permutation_invariance_and_per_pair_reduction():
    E, n_rows, n_cols, bits, gs, dt = 5, 8, 96, 6, 32, F16
    wq, s, b, _ = _moe_case(E, n_rows, n_cols, bits, gs, dt, seed=800)
    P = 9
    ids = synth.random_ints((P,), 0, E - 1, seed=801).astype(np.int32)
    a_s, _ = _activation(P, n_cols, dt, seed=802)
    out, _ = qref.moe(a_s, dt, ids, P, 1, n_cols, 0, wq, s, b, dt, E, n_rows, n_cols, bits, gs)
    perm = synth.rng(803).permutation(P)
    out_p, _ = qref.moe(np.ascontiguousarray(a_s[perm]), dt, ids[perm], P, 1, n_cols, 0, wq, s,
                        b, dt, E, n_rows, n_cols, bits, gs)
    assert np.array_equal(out_p, out[perm])
    for p in range(P):
        e = ids[p]
        y, _ = qref.qmatmul(a_s[p:p + 1], dt, wq[e], s[e], b[e], dt, n_cols, bits, gs)
        assert np.array_equal(y[0], out[p])


def test_moe_rejects_out_of_range_ids():
    wq, s, b, _ = _moe_case(3, 4, 64, 4, 32, F32, seed=900)
    a = np.zeros((1, 64), np.float32)
    with pytest.raises(ValueError):
        qref.moe(a, F32, np.array([3], np.int32), 1, 1, 64, 0, wq, s, b, F32, 3, 4, 64, 4, 32)


def test_gate_up_silu_closed_form():
    """Weights built so that g and u take chosen exact values; SiLU(z) =
    z / (1 + e^-z) is then checked against its textbook values."""
    n_rows, n_cols, bits, gs = 3, 32, 4, 32
    x = np.zeros((1, n_cols), np.float32)
    x[0, 0] = 1.0
    # w[r, 0] = q * (1/4) - 2: codes 12, 8, 4 give 1, 0, -1 for the gate; 16ths for up.
    def mk(first_codes):
        codes = np.zeros((n_rows, n_cols), np.uint8)
        codes[:, 0] = first_codes
        return (qref.pack(codes, bits)[None], np.full((1, n_rows, 1), 0.25, np.float32),
                np.full((1, n_rows, 1), -2.0, np.float32))
    gate = mk([12, 8, 4])
    up = mk([15, 15, 0])          # 1.75, 1.75, -2
    res = qref.moe_gate_up_silu(x, F32, np.array([0], np.int32), 1, 1, 0, 0, gate, up, F32, 1,
                                n_rows, n_cols, bits, gs)
    assert res["g"][0].tolist() == [1.0, 0.0, -1.0]
    assert res["u"][0].tolist() == [1.75, 1.75, -2.0]
    sig1 = 1.0 / (1.0 + math.exp(-1.0))   # logistic(1) = 0.7310585786300049
    assert abs(sig1 - 0.7310585786300049) < 1e-16
    expect = [1.0 * sig1 * 1.75, 0.0, -1.0 * (1.0 - sig1) * -2.0]
    assert np.allclose(res["silu_out"][0], expect, rtol=1e-15, atol=0)


def test_gate_up_silu_composes_two_moe_products():
    E, n_rows, n_cols, bits, gs, dt = 4, 6, 64, 3, 32, BF16
    gate = _moe_case(E, n_rows, n_cols, bits, gs, dt, seed=1100)[:3]
    up = _moe_case(E, n_rows, n_cols, bits, gs, dt, seed=1200)[:3]
    ids = synth.moe_ids(2, 2, E, seed=1300).ravel()
    a_s, _ = _activation(2, n_cols, dt, seed=1301, sigma=0.5)
    res = qref.moe_gate_up_silu(a_s, dt, ids, 2, 2, n_cols, 0, gate, up, dt, E, n_rows, n_cols,
                                bits, gs)
    g, _ = qref.moe(a_s, dt, ids, 2, 2, n_cols, 0, *gate, dt, E, n_rows, n_cols, bits, gs)
    u, _ = qref.moe(a_s, dt, ids, 2, 2, n_cols, 0, *up, dt, E, n_rows, n_cols, bits, gs)
    assert np.array_equal(res["g"], g) and np.array_equal(res["u"], u)
    sig = 1.0 / (1.0 + np.exp(-g))
    assert np.allclose(res["silu_out"], g * sig * u, rtol=1e-14, atol=1e-300)
