"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/qpack.h declares, and every argument error is reported
with its status before any HIP call is made."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys

import pytest

import weight_only_quantized_qgemv_amd as qp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qpack.h")

OK, INVALID, UNSUPPORTED, MISMATCH, SHAPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5, 6
F32, F16, BF16 = qp.QP_F32, qp.QP_F16, qp.QP_BF16
P = ctypes.c_void_p
A = P(0x10000)      # a well-aligned stand-in address (never dereferenced)
ODD = P(0x10001)    # misaligned for every element size


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
                  - {"if", "defined", "QP_ENUM"})


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(qp.EXPORTS)
    L = qp.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_version_string():
    assert "gfx950" in qp.version()


def qmatmul(x=A, xdt=BF16, m=1, k=64, wq=A, s=A, b=A, sdt=BF16, n=4, bits=4, gs=64, y=A):
    return qp.lib().qmatmul(x, xdt, m, k, wq, s, b, sdt, n, bits, gs, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), UNSUPPORTED), (dict(bits=1), UNSUPPORTED), (dict(bits=16), UNSUPPORTED),
    (dict(gs=16), UNSUPPORTED), (dict(gs=256), UNSUPPORTED), (dict(gs=0), UNSUPPORTED),
    (dict(k=96, gs=64), SHAPE), (dict(k=100, gs=32), SHAPE),
    (dict(xdt=F16, sdt=BF16), MISMATCH), (dict(xdt=F32, sdt=F16), MISMATCH),
    (dict(m=-1), INVALID), (dict(k=-64), INVALID), (dict(n=-2), INVALID),
    (dict(xdt=9), INVALID), (dict(sdt=-1, xdt=-1), INVALID),
    (dict(x=None), INVALID), (dict(wq=None), INVALID), (dict(y=None), INVALID),
    (dict(y=ODD), ALIGN), (dict(x=ODD), ALIGN), (dict(s=ODD), ALIGN), (dict(wq=P(0x10002)), ALIGN),
    (dict(m=1 << 62, n=1 << 62), INVALID),
])
def test_qmatmul_argument_errors(kw, status):
    assert qmatmul(**kw) == status
    assert qp.last_error() != ""


def test_qmatmul_empty_is_a_noop_without_touching_the_device():
    assert qmatmul(m=0) == OK and qp.last_error() == ""
    assert qmatmul(n=0, y=None, x=None) == OK


def test_qmatmul_dtype_rule_follows_scales_dtype():
    # fp32 activations with fp32 scales are fine to validate; a mismatch is not.
    assert qmatmul(xdt=F32, sdt=BF16) == MISMATCH
    assert "match" in qp.last_error()


def quantize(w=A, n=4, k=64, bits=4, gs=64, dt=BF16, wq=A, s=A, b=A):
    return qp.lib().qpack_quantize(w, n, k, bits, gs, dt, wq, s, b, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=7), UNSUPPORTED), (dict(gs=48), UNSUPPORTED), (dict(k=96), SHAPE),
    (dict(n=-1), INVALID), (dict(dt=3), INVALID), (dict(w=None), INVALID),
    (dict(biases=None) if False else dict(b=None), INVALID), (dict(w=P(0x10002)), ALIGN),
    (dict(s=ODD), ALIGN), (dict(dt=F32, s=P(0x10002)), ALIGN),
])
def test_quantize_argument_errors(kw, status):
    assert quantize(**kw) == status


def test_quantize_empty_is_a_noop():
    assert quantize(n=0, w=None) == OK
    assert quantize(k=0, w=None) == OK


def dequantize(wq=A, s=A, b=A, sdt=BF16, n=4, k=64, bits=4, gs=64, odt=BF16, out=A):
    return qp.lib().qpack_dequantize(wq, s, b, sdt, n, k, bits, gs, odt, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=7), UNSUPPORTED), (dict(gs=48), UNSUPPORTED), (dict(k=96), SHAPE),
    (dict(n=-1), INVALID), (dict(sdt=3), INVALID), (dict(odt=3), INVALID),
    (dict(odt=F16), MISMATCH), (dict(sdt=F32, odt=BF16), MISMATCH), (dict(wq=None), INVALID),
    (dict(out=None), INVALID), (dict(wq=P(0x10002)), ALIGN), (dict(s=ODD), ALIGN),
    (dict(odt=F32, out=P(0x10002)), ALIGN), (dict(k=(1 << 33) + 64), UNSUPPORTED),
])
def test_dequantize_argument_errors(kw, status):
    assert dequantize(**kw) == status
    assert qp.last_error() != ""


def test_dequantize_empty_is_a_noop():
    assert dequantize(n=0, wq=None, out=None) == OK
    assert dequantize(k=0, wq=None, out=None) == OK
    assert dequantize(sdt=F16, odt=F32, n=0) == OK


def dequantize_mx(wq=A, s=A, mode=1, n=4, k=64, odt=BF16, out=A):
    return qp.lib().qpack_dequantize_mx(wq, s, mode, n, k, odt, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(mode=0), UNSUPPORTED), (dict(mode=4), UNSUPPORTED), (dict(k=48), SHAPE),
    (dict(mode=3, k=40), SHAPE), (dict(n=-1), INVALID), (dict(odt=3), INVALID),
    (dict(wq=None), INVALID), (dict(s=None), INVALID), (dict(out=None), INVALID),
    (dict(wq=P(0x10002)), ALIGN), (dict(odt=F32, out=P(0x10002)), ALIGN),
])
def test_dequantize_mx_argument_errors(kw, status):
    assert dequantize_mx(**kw) == status
    assert qp.last_error() != ""


def test_dequantize_mx_accepts_nvfp4_group_multiples_and_empty():
    assert dequantize_mx(n=0, mode=3, k=48, wq=None, out=None) == OK
    assert dequantize_mx(k=0, wq=None, out=None) == OK


def qmatmul_mx(x=A, xdt=BF16, m=2, k=64, wq=A, s=A, mode=1, n=4, y=A):
    return qp.lib().qmatmul_mx(x, xdt, m, k, wq, s, mode, n, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(mode=5), UNSUPPORTED), (dict(k=80), SHAPE), (dict(mode=2, k=16), SHAPE),
    (dict(m=-1), INVALID), (dict(xdt=3), INVALID), (dict(x=None), INVALID),
    (dict(wq=None), INVALID), (dict(s=None), INVALID), (dict(y=None), INVALID),
    (dict(y=ODD), ALIGN), (dict(x=ODD), ALIGN), (dict(wq=P(0x10002)), ALIGN),
    (dict(k=1 << 31), INVALID),
])
def test_qmatmul_mx_argument_errors(kw, status):
    assert qmatmul_mx(**kw) == status


def test_qmatmul_mx_empty_is_a_noop():
    assert qmatmul_mx(m=0, x=None, y=None) == OK
    assert qmatmul_mx(n=0, x=None, y=None) == OK


def ffn(a=A, dt=BF16, ids=A, rw=A, T=2, top_k=2, sdt=BF16, E=4, D=64, F=64, bits=4, gs=64,
        out=A, ws=A, ws_bytes=None):
    L = qp.lib()
    if ws_bytes is None:
        ws_bytes = L.qgemv_moe_ffn_workspace_bytes(T, top_k, E, D, F, dt)
    return L.qgemv_moe_ffn(a, dt, ids, rw, T, top_k, *([A] * 9), sdt, E, D, F, bits, gs, out, ws,
                           ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), UNSUPPORTED), (dict(F=96), SHAPE), (dict(D=96), SHAPE), (dict(dt=F16), MISMATCH),
    (dict(T=-1), INVALID), (dict(out=None), INVALID), (dict(ws=None), INVALID),
    (dict(rw=None), INVALID), (dict(ids=None), INVALID), (dict(ws_bytes=64), WORKSPACE),
    (dict(out=ODD), ALIGN), (dict(rw=P(0x10002)), ALIGN), (dict(E=5000), UNSUPPORTED),
])
def test_moe_ffn_argument_errors(kw, status):
    assert ffn(**kw) == status


def test_moe_ffn_empty_and_workspace_size():
    assert ffn(T=0, a=None, out=None, ws=None) == OK
    assert ffn(D=0, a=None, out=None, ws=None) == OK
    L = qp.lib()
    small = L.qgemv_moe_ffn_workspace_bytes(4, 8, 128, 2048, 768, BF16)
    big = L.qgemv_moe_ffn_workspace_bytes(64, 8, 128, 2048, 768, BF16)
    assert small >= 4 * 8 * (2048 + 768) * 2 and big > small
    assert L.qgemv_moe_ffn_workspace_bytes(-1, 8, 128, 2048, 768, BF16) == 0


def test_int8_tensor_argument_errors():
    L = qp.lib()
    assert L.qpack_quantize_int8_tensor(A, -1, A, A, None) == INVALID
    assert L.qpack_quantize_int8_tensor(None, 8, A, A, None) == INVALID
    assert L.qpack_quantize_int8_tensor(P(0x10002), 8, A, A, None) == ALIGN
    assert L.qpack_quantize_int8_tensor(None, 0, None, None, None) == OK
    assert L.qpack_dequantize_int8_tensor(A, 8, A, 3, A, None) == INVALID
    assert L.qpack_dequantize_int8_tensor(A, 8, None, BF16, A, None) == INVALID
    assert L.qpack_dequantize_int8_tensor(A, 8, A, F32, P(0x10002), None) == ALIGN
    assert L.qmatmul_int8_tensor(A, BF16, -1, 64, A, A, 4, A, None) == INVALID
    assert L.qmatmul_int8_tensor(A, 3, 2, 64, A, A, 4, A, None) == INVALID
    assert L.qmatmul_int8_tensor(A, BF16, 2, 64, None, A, 4, A, None) == INVALID
    assert L.qmatmul_int8_tensor(A, BF16, 2, 64, A, None, 4, A, None) == INVALID
    assert L.qmatmul_int8_tensor(ODD, BF16, 2, 64, A, A, 4, A, None) == ALIGN
    assert L.qmatmul_int8_tensor(None, BF16, 0, 64, None, None, 4, None, None) == OK


def qmatmul_t(x=A, xdt=BF16, m=2, k=64, wq=A, s=A, b=A, sdt=BF16, n=128, bits=4, gs=64, y=A,
              ws=A, ws_bytes=1 << 20):
    return qp.lib().qmatmul_t(x, xdt, m, k, wq, s, b, sdt, n, bits, gs, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=7), UNSUPPORTED), (dict(gs=48), UNSUPPORTED), (dict(n=96), SHAPE),
    (dict(xdt=F16), MISMATCH), (dict(m=-1), INVALID), (dict(y=None), INVALID),
    (dict(x=None), INVALID), (dict(ws=None), INVALID), (dict(ws_bytes=8), WORKSPACE),
    (dict(y=ODD), ALIGN), (dict(wq=P(0x10002)), ALIGN), (dict(ws=P(0x10002)), ALIGN),
])
def test_qmatmul_t_argument_errors(kw, status):
    assert qmatmul_t(**kw) == status


def test_qmatmul_t_empty_and_workspace_size():
    assert qmatmul_t(m=0, x=None, y=None, ws=None) == OK
    L = qp.lib()
    assert L.qmatmul_t_workspace_bytes(1, 4096, 14336, 4) >= 14336 * 4
    assert L.qmatmul_t_workspace_bytes(16, 4096, 14336, 4) > L.qmatmul_t_workspace_bytes(1, 4096, 14336, 4)
    assert L.qmatmul_t_workspace_bytes(0, 4096, 14336, 4) == 0


def moe(fused=False, a=A, dt=BF16, ids=A, T=2, top_k=2, outer=64, inner=0, sdt=BF16, E=4, R=8,
        C=64, bits=4, gs=64, out=A, ws=A, ws_bytes=None):
    L = qp.lib()
    if ws_bytes is None:
        ws_bytes = L.qgemv_moe_workspace_bytes(T * top_k, E)
    if fused:
        return L.qgemv_moe_id_gate_up_silu(a, dt, ids, T, top_k, outer, inner, A, A, A, A, A, A,
                                           sdt, E, R, C, bits, gs, out, ws, ws_bytes, None)
    return L.qgemv_moe_id(a, dt, ids, T, top_k, outer, inner, A, A, A, sdt, E, R, C, bits, gs,
                          out, ws, ws_bytes, None)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), UNSUPPORTED), (dict(C=96), SHAPE), (dict(dt=F16), MISMATCH),
    (dict(T=-1), INVALID), (dict(outer=-64), INVALID), (dict(ids=None), INVALID),
    (dict(out=None), INVALID), (dict(ws=None), INVALID), (dict(a=None), INVALID),
    (dict(ws_bytes=16), WORKSPACE), (dict(E=5000), UNSUPPORTED), (dict(E=0), INVALID),
    (dict(out=ODD), ALIGN), (dict(ids=P(0x10002)), ALIGN), (dict(ws=P(0x10008)), ALIGN),
])
def test_moe_argument_errors(fused, kw, status):
    assert moe(fused=fused, **kw) == status


@pytest.mark.parametrize("fused", [False, True])
def test_moe_empty_is_a_noop(fused):
    assert moe(fused=fused, T=0, ids=None, out=None, ws=None) == OK
    assert moe(fused=fused, R=0, ids=None, out=None, ws=None) == OK


def moe_noalloc(a=A, dt=BF16, ids=A, T=2, top_k=2, outer=64, inner=0, sdt=BF16, E=4, R=8, C=64,
                bits=4, gs=64, out=A):
    return qp.lib().qgemv_moe_id_noalloc(a, dt, ids, T, top_k, outer, inner, A, A, A, sdt, E, R,
                                         C, bits, gs, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), UNSUPPORTED), (dict(C=96), SHAPE), (dict(dt=F16), MISMATCH),
    (dict(T=-1), INVALID), (dict(outer=-64), INVALID), (dict(ids=None), INVALID),
    (dict(out=None), INVALID), (dict(a=None), INVALID), (dict(E=5000), UNSUPPORTED),
    (dict(E=0), INVALID), (dict(out=ODD), ALIGN), (dict(ids=P(0x10002)), ALIGN),
    # Routing tables above the scratch maximum: 2^18 pairs need about 4 MB.
    (dict(T=1 << 16, top_k=4, E=128), WORKSPACE),
])
def test_moe_noalloc_argument_errors(kw, status):
    """Every check of the allocation-free call runs before any HIP call."""
    assert moe_noalloc(**kw) == status


def test_moe_noalloc_empty_is_a_noop():
    assert moe_noalloc(T=0, ids=None, out=None) == OK
    assert moe_noalloc(R=0, ids=None, out=None) == OK


def test_moe_noalloc_limit_covers_the_moe_workloads():
    """The largest routed MoE workload here (512 tokens x top-8 over 128
    experts) fits the scratch with room to spare."""
    L = qp.lib()
    assert L.qgemv_moe_workspace_bytes(512 * 8, 128) * 8 < 2 << 20


def test_workspace_bytes_grow_with_pairs_and_experts():
    L = qp.lib()
    a = L.qgemv_moe_workspace_bytes(8, 128)
    b = L.qgemv_moe_workspace_bytes(4096, 128)
    c = L.qgemv_moe_workspace_bytes(4096, 1024)
    assert 0 < a < b < c
    assert b >= 4096 * 4 + (4096 + 128) * 12
    assert L.qgemv_moe_workspace_bytes(-1, 4) == 0


def test_product_path_never_loads_the_oracle():
    """Importing and using the package must not touch oracle/ (no fallback)."""
    code = ("import sys, weight_only_quantized_qgemv_amd as q; q.lib(); "
            "assert not any(m.startswith('oracle') for m in sys.modules), sys.modules.keys()")
    subprocess.check_call([sys.executable, "-c", code], cwd=ROOT)
    pkg = os.path.join(ROOT, "weight_only_quantized_qgemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "qref" not in text and "import oracle" not in text, f


def test_calls_fail_loudly_when_library_is_missing(tmp_path, monkeypatch):
    monkeypatch.setattr(qp, "_lib", None)
    monkeypatch.setattr(qp, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        qp.lib()
