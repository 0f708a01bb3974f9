"""GPU parity of the MoE calls (qgemv_moe_id, qgemv_moe_id_gate_up_silu)
against the oracle's per-pair products, through the C ABI.

Bounds: the plain product uses tau*S + half an output ulp. The fused form uses
the first-order propagation of that bound through SiLU(g)*u:
  |d| <= tau * (1.1 |u| S_g + |SiLU(g)| S_u) + half_ulp(out),
where 1.1 >= max |SiLU'(z)| (about 1.0998 near z = 2.4). The down projection is
checked on identical inputs: the oracle's SiLU output rounded to bf16 is fed
to both sides.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from oracle import qref
from qhelpers import (BF16, F16, F32, TAU, half_ulp_out, TORCH_DT, activations, assert_within, dev,
                      log, to_device, to_numpy, values)
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


def stack(E, R, C, bits, gs, dt, seed):
    """Oracle-quantized expert stack (numpy) and its device copy."""
    w = synth.normal_f32((E * R, C), 0.02, seed)
    wq, s, b = qref.quantize(w, bits, gs, dt)
    host = (wq.reshape(E, R, -1), s.reshape(E, R, -1), b.reshape(E, R, -1))
    return host, tuple(to_device(t, dt) for t in host)


def fused_bound(ref, dt):
    sig = 1.0 / (1.0 + np.exp(-ref["g"]))
    return (TAU[dt] * (1.1 * np.abs(ref["u"]) * ref["Sg"] + np.abs(ref["g"] * sig) * ref["Su"])
            + half_ulp_out(ref["silu_out"], dt))


def check_fused(out, ref, dt, what, rows=None):
    y = values(out)
    if rows is not None:
        y = y[rows]
    err = np.abs(y - ref["silu_out"])
    bound = fused_bound(ref, dt)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {int(bad.sum())} outside; worst excess {(err - bound).max():.3e}"


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("dt", [F32, F16, BF16])
@pytest.mark.parametrize("T,top_k,E", [(1, 4, 6), (5, 3, 6), (40, 4, 8)])
def test_moe_gate_up_and_down_small(bits, dt, T, top_k, E):
    R, C, gs = 64, 256, 64        # gate/up: [E, R, C]; down: [E, C, R]
    log(f"moe small bits={bits} dt={dt} T={T} top_k={top_k} E={E}")
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 51 + bits)
    up_h, up_d = stack(E, R, C, bits, gs, dt, 52 + bits)
    down_h, down_d = stack(E, C, R, bits, 32, dt, 53 + bits)
    ids = synth.moe_ids(T, top_k, E, seed=55).ravel()
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 54)
    # gate/up: every slot of a token reads the token's row (outer = C, inner = 0)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    torch.cuda.synchronize()
    ref = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, R, C, bits, gs)
    check_fused(out, ref, dt, "gate_up")
    # plain product with the gate stack
    g = qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *gate_d, bits, gs)
    torch.cuda.synchronize()
    assert_within(g, ref["g"], ref["Sg"], dt, "moe plain")
    # down: pair p reads its own row of the oracle's SiLU output, rounded to dt
    h_f32 = ref["silu_out"].astype(np.float32)
    h_s = h_f32 if dt == F32 else (qref.f32_to_bf16(h_f32) if dt == BF16 else qref.f32_to_f16(h_f32))
    h_d = to_device(np.ascontiguousarray(h_s), dt)
    out_d = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * R, R, *down_d, bits, 32)
    torch.cuda.synchronize()
    ref_d, S_d = qref.moe(h_s, dt, ids, T, top_k, top_k * R, R, *down_h, dt, E, C, R, bits, 32)
    assert_within(out_d, ref_d, S_d, dt, "moe down")


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,top_k,E,R,C,gs", [
    (32, 2, 16, 200, 352, 32),    # 4 pairs per expert: 16-pair tiles
    (64, 4, 8, 96, 256, 64),      # 32 per expert: 32-pair tiles
    (200, 2, 4, 130, 256, 128),   # 100 per expert: 64-pair tiles, several per expert
    (32, 2, 16, 301, 96, 32),     # 16-pair tiles; 1806-byte scale rows per expert (not 16-aligned)
])
def test_moe_matrix_core_tiles(bits, dt, T, top_k, E, R, C, gs):
    """Enough pairs per expert for the matrix-core tiles, with row counts that
    are not multiples of a row group, K not a multiple of 128, and experts
    whose scale and bias rows start off a 16-byte boundary."""
    log(f"moe tiles bits={bits} dt={dt} T={T} top_k={top_k} E={E} R={R} C={C}")
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 61 + bits)
    up_h, up_d = stack(E, R, C, bits, gs, dt, 62 + bits)
    Rd = 96 if R % 32 else R      # the down projection's K (a multiple of its group size)
    down_h, down_d = stack(E, C, Rd, bits, 32, dt, 63 + bits)
    ids = synth.moe_ids(T, top_k, E, seed=65).ravel()
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 64)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    g = qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *gate_d, bits, gs)
    torch.cuda.synchronize()
    ref = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, R, C, bits, gs)
    check_fused(out, ref, dt, "tiles gate_up")
    assert_within(g, ref["g"], ref["Sg"], dt, "tiles plain")
    # Down projection over the pairs' own rows (inner stride = row length).
    h_s, h_d = activations((T * top_k, Rd), dt, 66)
    out_d = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * Rd, Rd, *down_d, bits, 32)
    torch.cuda.synchronize()
    ref_d, S_d = qref.moe(h_s, dt, ids, T, top_k, top_k * Rd, Rd, *down_h, dt, E, C, Rd, bits, 32)
    assert_within(out_d, ref_d, S_d, dt, "tiles down")


def moe_config(T, seed_ids=55):
    E, top_k = 128, 8
    gate_h, gate_d = stack(E, 768, 2048, 4, 64, BF16, 51)
    up_h, up_d = stack(E, 768, 2048, 4, 64, BF16, 52)
    down_h, down_d = stack(E, 2048, 768, 4, 64, BF16, 53)
    ids = synth.moe_ids(T, top_k, E, seed=seed_ids).ravel()
    a_s, a_d = activations((T, 2048), BF16, 54)
    return E, top_k, ids, a_s, a_d, (gate_h, gate_d), (up_h, up_d), (down_h, down_d)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,top_k,E,R,C,gs,skew", [
    (24, 4, 32, 130, 2048, 64, False),   # 3 pairs per expert, K = 2048, ragged rows
    (12, 8, 24, 72, 96, 32, False),      # 4 per expert, 3 units per row, odd group count
    (10, 4, 16, 64, 512, 128, True),     # expert 0 in every token: 10 pairs, two tiles
])
def test_moe_fused_few_pairs_per_expert(bits, dt, T, top_k, E, R, C, gs, skew):
    """The fused form at two to four pairs per expert, where tiles of up to 8
    pairs go to the four-row matrix-instruction kernel: ragged row counts,
    partial unit rounds, and an expert whose pairs span two tiles."""
    log(f"moe few pairs bits={bits} dt={dt} T={T} top_k={top_k} E={E} R={R} C={C} skew={skew}")
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 71 + bits)
    up_h, up_d = stack(E, R, C, bits, gs, dt, 72 + bits)
    if skew:
        ids = np.array([[0] + [1 + (t + j) % (E - 1) for j in range(top_k - 1)] for t in range(T)],
                       dtype=np.int32).ravel()
    else:
        ids = synth.moe_ids(T, top_k, E, seed=75).ravel()
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 74)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    torch.cuda.synchronize()
    ref = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, R, C, bits, gs)
    check_fused(out, ref, dt, "few pairs gate_up")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,top_k,E,R,C,gs", [
    (1, 8, 128, 130, 2048, 64),   # one token over 128 experts, ragged rows
    (2, 3, 96, 64, 96, 32),       # 3 units per row, odd group count
    (1, 4, 64, 72, 4096, 128),    # two units per lane
])
def test_moe_one_pair_tiles(bits, dt, T, top_k, E, R, C, gs):
    """Few pairs over many experts: every pair is its own tile, on the
    dot-product row kernel for the fused form (and for the plain form at this
    density); the plain product also reads through a non-zero inner stride."""
    log(f"moe one-pair bits={bits} dt={dt} T={T} top_k={top_k} E={E} R={R} C={C}")
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 81 + bits)
    up_h, up_d = stack(E, R, C, bits, gs, dt, 82 + bits)
    ids = synth.moe_ids(T, top_k, E, seed=85).ravel()
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 84)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    torch.cuda.synchronize()
    ref = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, R, C, bits, gs)
    check_fused(out, ref, dt, "one-pair gate_up")
    # Plain product over the pairs' own rows (inner stride = row length).
    h_s, h_d = activations((T * top_k, C), dt, 86)
    out_p = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * C, C, *gate_d, bits, gs)
    torch.cuda.synchronize()
    ref_p, S_p = qref.moe(h_s, dt, ids, T, top_k, top_k * C, C, *gate_h, dt, E, R, C, bits, gs)
    assert_within(out_p, ref_p, S_p, dt, "one-pair plain")


@pytest.mark.parametrize("T", [1, 64, 512])
def test_moe_config_sampled(T):
    """128 experts, top-8, gate/up [128, 768, 2048], down [128, 2048, 768], 4-bit
    gs64 bf16; tokens x bf16 [T, 2048]; fused SiLU(gate)*up then down. Every
    output at T = 1 and 64; all pairs of 32 tokens at T = 512."""
    log(f"moe config T={T}")
    E, top_k, ids, a_s, a_d, gate, up, down = moe_config(T)
    P = T * top_k
    ids_d = torch.from_numpy(ids).to(dev())
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, 2048, 0, gate[1], up[1], 4, 64)
    torch.cuda.synchronize()
    # Oracle on every pair up to 64 tokens; at 512, on all pairs of 32 sampled
    # tokens (the first and last among them).
    if T <= 64:
        toks = np.arange(T)
    else:
        g = synth.rng(T)
        toks = np.unique(np.concatenate([g.choice(T, 30, replace=False), [0, T - 1]]))
    sel = np.concatenate([np.arange(t * top_k, (t + 1) * top_k) for t in toks])
    a_sub = np.ascontiguousarray(a_s[toks])
    ref = qref.moe_gate_up_silu(a_sub, BF16, ids[sel], len(toks), top_k, 2048, 0, gate[0], up[0],
                                BF16, E, 768, 2048, 4, 64)
    check_fused(out, ref, BF16, "config gate_up", rows=sel)
    # Down on identical inputs: the oracle's SiLU output for the checked pairs'
    # rows (at T = 512 the other rows are kept from the GPU).
    h = to_numpy(out).copy()
    h[sel] = qref.f32_to_bf16(ref["silu_out"].astype(np.float32))
    h_d = to_device(h, BF16)
    out_d = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * 768, 768, *down[1], 4, 64)
    torch.cuda.synchronize()
    h_sub = np.ascontiguousarray(h[sel])
    ref_d, S_d = qref.moe(h_sub, BF16, ids[sel], len(sel), 1, 768, 0, *down[0], BF16, E, 2048,
                          768, 4, 64)
    assert_within(out_d[torch.from_numpy(sel).to(dev())], ref_d, S_d, BF16, "config down")


def test_moe_single_token_and_offset_forms():
    """Single-token form (n_tokens=1, top_k=n_selected, outer=0, inner=src1_stride)
    and the offset form (pointer arithmetic on a and ids) equal the batched form."""
    E, R, C, bits, gs = 8, 32, 128, 4, 32
    h, d = stack(E, R, C, bits, gs, BF16, 71)
    rows_s, rows_d = activations((6, C), BF16, 72)
    ids = np.array([3, 1, 7, 0, 5, 2], dtype=np.int32)
    ids_d = torch.from_numpy(ids).to(dev())
    full = qp.qgemv_moe_id(rows_d, ids_d, 6, 1, C, 0, *d, bits, gs)
    single = qp.qgemv_moe_id(rows_d, ids_d, 1, 6, 0, C, *d, bits, gs)
    off = qp.qgemv_moe_id(rows_d[2:], ids_d[2:], 1, 4, 0, C, *d, bits, gs)
    torch.cuda.synchronize()
    assert torch.equal(full, single)
    assert torch.equal(full[2:], off)
    ref, S = qref.moe(rows_s, BF16, ids, 1, 6, 0, C, *h, BF16, E, R, C, bits, gs)
    assert_within(single, ref, S, BF16, "single-token")


def test_moe_permutation_of_pairs_permutes_outputs():
    E, R, C, bits, gs = 16, 64, 256, 4, 64
    h, d = stack(E, R, C, bits, gs, BF16, 81)
    P = 64
    ids = synth.random_ints((P,), 0, E - 1, 82).astype(np.int32)
    a_s, a_d = activations((P, C), BF16, 83)
    out = qp.qgemv_moe_id(a_d, torch.from_numpy(ids).to(dev()), P, 1, C, 0, *d, bits, gs)
    perm = synth.rng(84).permutation(P)
    out_p = qp.qgemv_moe_id(a_d[torch.from_numpy(perm).to(dev())].contiguous(),
                            torch.from_numpy(ids[perm]).to(dev()), P, 1, C, 0, *d, bits, gs)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out[torch.from_numpy(perm).to(dev())])


def test_moe_invalid_ids_are_skipped():
    E, R, C, bits, gs = 4, 16, 64, 4, 64
    h, d = stack(E, R, C, bits, gs, BF16, 91)
    ids = np.array([1, -1, 4, 2], dtype=np.int32)
    a_s, a_d = activations((4, C), BF16, 92)
    out = torch.full((4, R), 123.0, dtype=torch.bfloat16, device=dev())
    qp.qgemv_moe_id(a_d, torch.from_numpy(ids).to(dev()), 4, 1, C, 0, *d, bits, gs, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[1] == 123.0) and torch.all(out[2] == 123.0)
    ref, S = qref.moe(np.ascontiguousarray(a_s[[0, 3]]), BF16, ids[[0, 3]], 2, 1, C, 0, *h, BF16,
                      E, R, C, bits, gs)
    assert_within(out[[0, 3]], ref, S, BF16, "valid rows")


def test_moe_expert_with_many_pairs_spans_tiles():
    """All pairs on one expert: several tiles of the same expert."""
    E, R, C, bits, gs = 4, 48, 512, 4, 64
    h, d = stack(E, R, C, bits, gs, BF16, 95)
    P = 37
    ids = np.full(P, 2, dtype=np.int32)
    a_s, a_d = activations((P, C), BF16, 96)
    out = qp.qgemv_moe_id(a_d, torch.from_numpy(ids).to(dev()), P, 1, C, 0, *d, bits, gs)
    torch.cuda.synchronize()
    ref, S = qref.moe(a_s, BF16, ids, P, 1, C, 0, *h, BF16, E, R, C, bits, gs)
    assert_within(out, ref, S, BF16, "one expert")


def skewed_ids(T):
    """Token t picks expert 5 and expert 1 + t % 4 of six: expert 5 serves every
    token (several 64-pair tiles), expert 0 none."""
    return np.stack([np.full(T, 5), 1 + np.arange(T) % 4], axis=1).astype(np.int32).ravel()


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("T,top_k,E,R,C,gs,Rd", [
    (96, 4, 8, 200, 320, 64, 192),    # 48 pairs per expert, ragged row blocks
    (300, 2, 4, 96, 128, 32, 128),    # 150 per expert: three tiles each
    (160, 2, 6, 72, 256, 128, 64),    # skewed: one expert on every token, one on none
])
def test_moe_routed_gemm_tiles(bits, dt, T, top_k, E, R, C, gs, Rd):
    """Dozens of pairs per expert and K a multiple of 64 on both projections:
    the routed matrix-core GEMM (tiles of up to 64 pairs of one expert)."""
    log(f"moe routed gemm bits={bits} dt={dt} T={T} top_k={top_k} E={E} R={R} C={C} gs={gs}")
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 161 + bits)
    up_h, up_d = stack(E, R, C, bits, gs, dt, 162 + bits)
    down_h, down_d = stack(E, C, Rd, bits, 32, dt, 163 + bits)
    ids = skewed_ids(T) if E == 6 else synth.moe_ids(T, top_k, E, seed=165).ravel()
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 164)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    g = qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *gate_d, bits, gs)
    torch.cuda.synchronize()
    ref = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, R, C, bits, gs)
    check_fused(out, ref, dt, "routed gate_up")
    assert_within(g, ref["g"], ref["Sg"], dt, "routed plain")
    # Down projection over the pairs' own rows (inner stride = row length).
    h_s, h_d = activations((T * top_k, Rd), dt, 166)
    out_d = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * Rd, Rd, *down_d, bits, 32)
    torch.cuda.synchronize()
    ref_d, S_d = qref.moe(h_s, dt, ids, T, top_k, top_k * Rd, Rd, *down_h, dt, E, C, Rd, bits, 32)
    assert_within(out_d, ref_d, S_d, dt, "routed down")


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_moe_routed_gemm_32_pair_tiles(bits, dt):
    """Fewer than 16 pairs per expert on average (12 here), K a multiple of 64
    and at most 1024: the plain form takes the routed GEMM in 32-pair tiles.
    Expert 15 serves every token (48 pairs: a full tile and a partial one);
    the other three picks of each token are uniform over experts 0..14."""
    T, E, R, C, gs, Rd = 48, 16, 136, 512, 64, 192
    log(f"moe routed gemm 32-pair tiles bits={bits} dt={dt}")
    ids = np.concatenate([np.full((T, 1), E - 1), synth.moe_ids(T, 3, E - 1, seed=181)],
                         axis=1).astype(np.int32).ravel()
    top_k = 4
    ids_d = torch.from_numpy(ids).to(dev())
    gate_h, gate_d = stack(E, R, C, bits, gs, dt, 182 + bits)
    a_s, a_d = activations((T, C), dt, 183)
    g = qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *gate_d, bits, gs)
    torch.cuda.synchronize()
    ref, S = qref.moe(a_s, dt, ids, T, top_k, C, 0, *gate_h, dt, E, R, C, bits, gs)
    assert_within(g, ref, S, dt, "routed plain, 32-pair tiles")
    down_h, down_d = stack(E, C, Rd, bits, 32, dt, 184 + bits)
    h_s, h_d = activations((T * top_k, Rd), dt, 185)
    out_d = qp.qgemv_moe_id(h_d, ids_d, T, top_k, top_k * Rd, Rd, *down_d, bits, 32)
    torch.cuda.synchronize()
    ref_d, S_d = qref.moe(h_s, dt, ids, T, top_k, top_k * Rd, Rd, *down_h, dt, E, C, Rd, bits, 32)
    assert_within(out_d, ref_d, S_d, dt, "routed down, 32-pair tiles")


def test_moe_routed_gemm_pair_order_does_not_change_values():
    """A pair's output does not depend on which tile slot it lands in: permuting
    the pairs permutes the outputs bit for bit."""
    E, R, C, bits, gs = 4, 136, 256, 4, 64
    h, d = stack(E, R, C, bits, gs, BF16, 171)
    P = 256
    ids = synth.random_ints((P,), 0, E - 1, 172).astype(np.int32)
    a_s, a_d = activations((P, C), BF16, 173)
    out = qp.qgemv_moe_id(a_d, torch.from_numpy(ids).to(dev()), P, 1, C, 0, *d, bits, gs)
    perm = synth.rng(174).permutation(P)
    out_p = qp.qgemv_moe_id(a_d[torch.from_numpy(perm).to(dev())].contiguous(),
                            torch.from_numpy(ids[perm]).to(dev()), P, 1, C, 0, *d, bits, gs)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out[torch.from_numpy(perm).to(dev())])
    ref, S = qref.moe(a_s, BF16, ids, P, 1, C, 0, *h, BF16, E, R, C, bits, gs)
    assert_within(out, ref, S, BF16, "routed")


def test_moe_routed_scales_not_dword_aligned():
    """64 pairs per expert (the routed GEMM's range) with the stack's scales and
    biases at an address that is 2 mod 4: the call takes the matrix-core GEMV
    tiles instead, with the same results."""
    E, R, C, bits, gs = 4, 136, 256, 4, 64
    h, d = stack(E, R, C, bits, gs, BF16, 181)
    wq, s, b = d
    buf_s = torch.empty(s.numel() + 1, dtype=s.dtype, device=s.device)
    buf_b = torch.empty(b.numel() + 1, dtype=b.dtype, device=b.device)
    s2 = buf_s[1:].view(s.shape)
    b2 = buf_b[1:].view(b.shape)
    s2.copy_(s)
    b2.copy_(b)
    assert s2.data_ptr() % 4 == 2
    P = 256
    ids = synth.random_ints((P,), 0, E - 1, 182).astype(np.int32)
    a_s, a_d = activations((P, C), BF16, 183)
    ids_d = torch.from_numpy(ids).to(dev())
    out = qp.qgemv_moe_id(a_d, ids_d, P, 1, C, 0, wq, s2, b2, bits, gs)
    out_al = qp.qgemv_moe_id(a_d, ids_d, P, 1, C, 0, wq, s, b, bits, gs)
    torch.cuda.synchronize()
    ref, S = qref.moe(a_s, BF16, ids, P, 1, C, 0, *h, BF16, E, R, C, bits, gs)
    assert_within(out, ref, S, BF16, "scales 2 mod 4")
    assert_within(out_al, ref, S, BF16, "scales aligned")


@pytest.mark.parametrize("dt", [F16, BF16])
def test_moe_routed_gemm_persistent_blocks_walk_several_items(dt):
    """More (tile, row block) items than the GPU holds routed-GEMM blocks at
    once (two per CU at 4-bit, about 512), so every persistent block walks two
    or three items of its XCD's stretch of the work list: 64 experts with 32
    pairs each (one 64-pair tile per expert) times 23 row blocks is 1472
    items, 184 per XCD, which the 64 blocks of an XCD do not divide."""
    T, top_k, E, C, bits, gs = 256, 8, 64, 128, 4, 64
    log(f"moe routed gemm persistent dt={dt}")
    ids = synth.moe_ids(T, top_k, E, seed=191).ravel()
    assert np.bincount(ids, minlength=E).min() >= 16
    ids_d = torch.from_numpy(ids).to(dev())
    a_s, a_d = activations((T, C), dt, 192)
    R = 23 * 256                      # plain form: 256 rows per item
    w_h, w_d = stack(E, R, C, bits, gs, dt, 193)
    g = qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *w_d, bits, gs)
    torch.cuda.synchronize()
    ref, S = qref.moe(a_s, dt, ids, T, top_k, C, 0, *w_h, dt, E, R, C, bits, gs)
    assert_within(g, ref, S, dt, "routed plain, persistent blocks")
    del w_d
    Rf = 23 * 128                     # fused form: 128 gate + 128 up rows per item
    gate_h, gate_d = stack(E, Rf, C, bits, gs, dt, 194)
    up_h, up_d = stack(E, Rf, C, bits, gs, dt, 195)
    out = qp.qgemv_moe_id_gate_up_silu(a_d, ids_d, T, top_k, C, 0, gate_d, up_d, bits, gs)
    torch.cuda.synchronize()
    ref_f = qref.moe_gate_up_silu(a_s, dt, ids, T, top_k, C, 0, gate_h, up_h, dt, E, Rf, C, bits, gs)
    check_fused(out, ref_f, dt, "routed gate_up, persistent blocks")
