"""GPU parity of qgemv_moe_ffn (one MoE feed-forward block: gate+up+SiLU, down,
weighted slot sum) against the oracle, through the C ABI.

Bound, propagated through the block (every term from the oracle):
  h:   B_h = tau*(1.1*|u|*S_g + |SiLU(g)|*S_u) + ulp(h)   (device and oracle may
       round the fused value to neighbouring 16-bit numbers: one full ulp)
  o:   B_o = tau*S_o + sum_f |Wd[d, f]| * B_h[f] + ulp(o)
  out: B_out = sum_j |rw_j| * B_o[j] + half an ulp of out
with ulp(v) <= |v| * 2^-7 for bf16 (2^-10 for fp16). S_o and the weighted sum
of B_h are oracle products over the same expert stack (its S term with the
bounds as activations).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import BF16, F16, F32, TAU, half_ulp_out, TORCH_DT, activations, dev, log, to_device, values
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


def stack(E, R, C, bits, gs, dt, seed):
    w = synth.normal_f32((E * R, C), 0.02, seed)
    wq, s, b = qref.quantize(w, bits, gs, dt)
    host = (wq.reshape(E, R, -1), s.reshape(E, R, -1), b.reshape(E, R, -1))
    return host, tuple(to_device(t, dt) for t in host)


def ffn_case(T, top_k, E, D, F, bits, gs, dt, seed):
    gate = stack(E, F, D, bits, gs, dt, seed)
    up = stack(E, F, D, bits, gs, dt, seed + 1)
    down = stack(E, D, F, bits, gs, dt, seed + 2)
    ids = synth.moe_ids(T, top_k, E, seed=seed + 3).ravel().astype(np.int32)
    rw = synth.normal_f32((T * top_k,), 0.4, seed + 4)
    a_s, a_d = activations((T, D), dt, seed + 5)
    return dict(T=T, top_k=top_k, E=E, D=D, F=F, bits=bits, gs=gs, dt=dt, gate=gate, up=up,
                down=down, ids=ids, rw=rw, a_s=a_s, a_d=a_d)


def run_device(c, ids=None):
    ids = c["ids"] if ids is None else ids
    return qp.qgemv_moe_ffn(c["a_d"], torch.from_numpy(ids).to(dev()),
                            torch.from_numpy(c["rw"]).to(dev()), c["top_k"], c["gate"][1],
                            c["up"][1], c["down"][1], c["bits"], c["gs"])


def reference_and_bound(c, ids=None, rw=None, tokens=None):
    """Oracle output and bound, for all tokens or the listed ones."""
    ids = c["ids"] if ids is None else ids
    rw = c["rw"] if rw is None else rw
    T, top_k, dt, D, F = c["T"], c["top_k"], c["dt"], c["D"], c["F"]
    a_s = c["a_s"]
    if tokens is not None:
        a_s = a_s[tokens]
        sel = (np.asarray(tokens)[:, None] * top_k + np.arange(top_k)).ravel()
        ids, rw, T = ids[sel], rw[sel], len(tokens)
    args = (c["gate"][0], c["up"][0], c["down"][0], dt, c["E"], D, F, c["bits"], c["gs"])
    out, h, o = qref.moe_ffn(a_s, dt, ids, rw, T, top_k, *args)
    r = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, D, 0, c["gate"][0], c["up"][0], dt,
                              c["E"], F, D, c["bits"], c["gs"])
    ulp = 2.0 ** -7 if dt == BF16 else 2.0 ** -10
    sig = 1.0 / (1.0 + np.exp(-r["g"]))
    b_h = (TAU[dt] * (1.1 * np.abs(r["u"]) * r["Sg"] + np.abs(r["g"] * sig) * r["Su"])
           + np.abs(r["silu_out"]) * ulp + 1e-30)
    _, s_o = qref.moe(h, dt, ids, T, top_k, top_k * F, F, *c["down"][0], dt, c["E"], D, F,
                      c["bits"], c["gs"])
    _, s_bh = qref.moe(b_h.astype(np.float32), F32, ids, T, top_k, top_k * F, F, *c["down"][0],
                       dt, c["E"], D, F, c["bits"], c["gs"])
    o_vals = values_of(o, dt)
    b_o = TAU[dt] * s_o + s_bh + np.abs(o_vals) * ulp
    b_out = (np.abs(rw.astype(np.float64)).reshape(T, top_k, 1) * b_o.reshape(T, top_k, D)).sum(1)
    b_out += half_ulp_out(out, dt)
    return out, b_out


def values_of(storage, dt):
    if dt == F32:
        return storage.astype(np.float64)
    t = torch.from_numpy(storage.view(np.int16).copy()).view(TORCH_DT[dt])
    return t.double().numpy()


def check(y, out, bound, what):
    err = np.abs(values(y) - out)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside; worst excess "
                           f"{(err - bound).max():.3e}")


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("T,top_k,E", [(1, 4, 8), (6, 3, 8), (48, 8, 16)])
def test_moe_ffn_small(dt, T, top_k, E):
    c = ffn_case(T, top_k, E, 256, 192, 4, 64, dt, 4000 + T)
    log(f"ffn: T={T} top_k={top_k} E={E} dt={dt}")
    y = run_device(c)
    torch.cuda.synchronize()
    out, bound = reference_and_bound(c)
    check(y, out, bound, "ffn small")


@pytest.mark.parametrize("bits", [3, 8])
def test_moe_ffn_other_widths(bits):
    c = ffn_case(16, 4, 8, 256, 128, bits, 32, BF16, 4100 + bits)
    y = run_device(c)
    torch.cuda.synchronize()
    out, bound = reference_and_bound(c)
    check(y, out, bound, f"ffn {bits}-bit")


@pytest.mark.parametrize("T", [1, 64])
def test_moe_ffn_block_shape_sampled_tokens(T):
    """128 experts, top-8, d_model 2048, d_ff 768, 4-bit gs64 bf16: every output
    of up to 8 sampled tokens."""
    c = ffn_case(T, 8, 128, 2048, 768, 4, 64, BF16, 4200 + T)
    y = run_device(c)
    torch.cuda.synchronize()
    tokens = sorted(set(np.linspace(0, T - 1, 8).astype(int).tolist()))
    out, bound = reference_and_bound(c, tokens=tokens)
    check(y[tokens], out, bound, "ffn block shape")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("T,top_k,E,F", [(1, 8, 16, 192), (3, 5, 16, 768), (2, 3, 8, 2048), (1, 4, 8, 4096)])
def test_moe_ffn_fused_down_and_combine(bits, dt, T, top_k, E, F):
    """At most one pair per expert on average: the down projection and the slot
    combine run as one launch (rows of 6, 24, 64 and 128 units: 32- and 64-lane
    slots, one and two units per lane)."""
    c = ffn_case(T, top_k, E, 256, F, bits, 64, dt, 4500 + T + bits + F)
    log(f"ffn fused down+combine: T={T} top_k={top_k} E={E} F={F} bits={bits} dt={dt}")
    y = run_device(c)
    torch.cuda.synchronize()
    out, bound = reference_and_bound(c)
    check(y, out, bound, "ffn fused down+combine")


def test_moe_ffn_fused_invalid_ids_add_nothing():
    """Invalid ids in the one-launch down + combine regime (8 pairs, 16 experts)."""
    c = ffn_case(2, 4, 16, 256, 128, 4, 64, BF16, 4600)
    ids = c["ids"].copy()
    ids[[1, 6]] = [16, -3]                   # outside [0, 16)
    y = run_device(c, ids=ids)
    torch.cuda.synchronize()
    ok_ids = ids.copy()
    rw = c["rw"].copy()
    bad = (ok_ids < 0) | (ok_ids >= 16)
    ok_ids[bad], rw[bad] = 0, 0.0
    out, bound = reference_and_bound(c, ids=ok_ids, rw=rw)
    check(y, out, bound, "ffn fused invalid ids")


def test_moe_ffn_invalid_ids_add_nothing():
    c = ffn_case(6, 4, 8, 256, 128, 4, 64, BF16, 4300)
    ids = c["ids"].copy()
    ids[[1, 6, 15]] = [8, -1, 1000]          # outside [0, 8)
    y = run_device(c, ids=ids)
    torch.cuda.synchronize()
    ok_ids = ids.copy()
    rw = c["rw"].copy()
    bad = (ok_ids < 0) | (ok_ids >= 8)
    ok_ids[bad], rw[bad] = 0, 0.0           # same sum with the slot's weight at zero
    out, bound = reference_and_bound(c, ids=ok_ids, rw=rw)
    check(y, out, bound, "ffn invalid ids")


def test_moe_ffn_zero_slots_and_empty():
    c = ffn_case(3, 2, 4, 64, 64, 4, 32, BF16, 4400)
    out = torch.full((3, 64), 5.0, dtype=torch.bfloat16, device=dev())
    qp.qgemv_moe_ffn(c["a_d"], torch.zeros(0, dtype=torch.int32, device=dev()),
                     torch.zeros(0, dtype=torch.float32, device=dev()), 0, c["gate"][1],
                     c["up"][1], c["down"][1], 4, 32, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()
