"""ctypes binding of the oracle (``oracle/qref.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never does. Arrays are
numpy arrays on the host; 16-bit floating arrays are carried as ``uint16``
bit patterns together with an element-type code (0 fp32, 1 fp16, 2 bf16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qref.c")
LIB = os.environ.get("QREF_LIB_OVERRIDE") or os.path.join(HERE, "libqref.so")

F32, F16, BF16 = 0, 1, 2

# -ffp-contract=off: a*b+c stays a multiply then an add, as the oracle states.
BUILD_CMD = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", SRC, "-o", LIB, "-lm"]


def build(force: bool = False) -> str:
    if os.environ.get("QREF_LIB_OVERRIDE"):  # a prebuilt variant (mutation tests)
        return LIB
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.check_call(BUILD_CMD)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.qref_f32_to_bf16.restype = ctypes.c_uint16
        L.qref_f32_to_bf16.argtypes = [ctypes.c_float]
        L.qref_f32_to_f16.restype = ctypes.c_uint16
        L.qref_f32_to_f16.argtypes = [ctypes.c_float]
        L.qref_bf16_to_f32.restype = ctypes.c_float
        L.qref_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.qref_f16_to_f32.restype = ctypes.c_float
        L.qref_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.qref_f32_to_bf16_n.argtypes = [P, P, I64]
        L.qref_f32_to_f16_n.argtypes = [P, P, I64]
        L.qref_bf16_to_f32_n.argtypes = [P, P, I64]
        L.qref_f16_to_f32_n.argtypes = [P, P, I64]
        L.qref_pack.argtypes = [P, I64, I64, I, P]
        L.qref_unpack.argtypes = [P, I64, I64, I, P]
        L.qref_quantize.argtypes = [P, I64, I64, I, I, I, P, P, P]
        L.qref_dequantize.argtypes = [P, P, P, I, I64, I64, I, I, P]
        L.qref_dequantize_typed.argtypes = [P, P, P, I, I64, I64, I, I, P]
        L.qref_qmatmul.argtypes = [P, I, I64, I64, P, P, P, I, I64, I, I, P, P]
        L.qref_qmatmul_sampled.argtypes = [P, I, I64, I64, P, P, P, I, I64, I, I, P, P, I64,
                                           P, P]
        L.qref_moe.argtypes = [P, I, P, I64, I64, I64, I64, P, P, P, I, I64, I64, I64, I, I,
                               P, P]
        L.qref_moe_gate_up_silu.argtypes = [P, I, P, I64, I64, I64, I64, P, P, P, P, P, P, I,
                                            I64, I64, I64, I, I, P, P, P, P, P]
        L.qref_mx_params.argtypes = [I, P, P]
        L.qref_qmatmul_t.argtypes = [P, I, I64, I64, P, P, P, I, I64, I, I, P, P]
        L.qref_quantize_int8_tensor.argtypes = [P, I64, P, P]
        L.qref_dequantize_int8_tensor.argtypes = [P, I64, P, P]
        L.qref_qmatmul_int8_tensor.argtypes = [P, I, I64, I64, P, P, I64, P, P]
        L.qref_moe_ffn.argtypes = [P, I, P, P, I64, I64] + [P] * 9 + [I, I64, I64, I64, I, I, P, P, P]
        for f in ("qref_fp4_e2m1", "qref_fp8_e4m3", "qref_e8m0"):
            getattr(L, f).restype = ctypes.c_double
            getattr(L, f).argtypes = [ctypes.c_uint32]
        L.qref_mx_dequantize.argtypes = [P, P, I, I64, I64, I, P]
        L.qref_mx_qmatmul.argtypes = [P, I, I64, I64, P, P, I, I64, P, P]
        L.qref_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _sb_empty(shape, dtype_code):
    return np.empty(shape, dtype=np.float32 if dtype_code == F32 else np.uint16)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return int(lib().qref_num_threads())


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().qref_f32_to_bf16_n(_p(a), _p(out), a.size)
    return out


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().qref_f32_to_f16_n(_p(a), _p(out), a.size)
    return out


def to_f32(bits16: np.ndarray, dtype_code: int) -> np.ndarray:
    """Exact fp32 values of an fp32 / fp16 / bf16 array (as stored)."""
    if dtype_code == F32:
        return np.asarray(bits16, dtype=np.float32)
    L = lib()
    f = L.qref_f16_to_f32_n if dtype_code == F16 else L.qref_bf16_to_f32_n
    a = np.ascontiguousarray(bits16, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    f(_p(a), _p(out), a.size)
    return out


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    wq = np.empty((n, k * bits // 32), dtype=np.uint32)
    _check(lib().qref_pack(_p(codes), n, k, bits, _p(wq)), "pack")
    return wq


def unpack(wq: np.ndarray, k: int, bits: int) -> np.ndarray:
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    n = wq.shape[0]
    codes = np.empty((n, k), dtype=np.uint8)
    _check(lib().qref_unpack(_p(wq), n, k, bits, _p(codes)), "unpack")
    return codes


def quantize(w: np.ndarray, bits: int, group_size: int, sb_dtype: int):
    """Returns (wq [n, k*bits/32] u32, scales [n, k/gs], biases [n, k/gs]);
    scales/biases are fp32 arrays or uint16 bit patterns (fp16/bf16)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    wq = np.empty((n, k * bits // 32), dtype=np.uint32)
    s = _sb_empty((n, k // group_size), sb_dtype)
    b = _sb_empty((n, k // group_size), sb_dtype)
    _check(lib().qref_quantize(_p(w), n, k, bits, group_size, sb_dtype, _p(wq), _p(s), _p(b)),
           "quantize")
    return wq, s, b


def dequantize(wq, s, b, sb_dtype, k, bits, group_size):
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    n = wq.shape[0]
    out = np.empty((n, k), dtype=np.float32)
    _check(lib().qref_dequantize(_p(wq), _p(np.ascontiguousarray(s)), _p(np.ascontiguousarray(b)),
                                 sb_dtype, n, k, bits, group_size, _p(out)), "dequantize")
    return out


def dequantize_typed(wq, s, b, sb_dtype, k, bits, group_size):
    """Dense weight in the scales' type: fp32 array, or uint16 bit patterns for
    fp16 / bf16 scales."""
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    n = wq.shape[0]
    out = _sb_empty((n, k), sb_dtype)
    _check(lib().qref_dequantize_typed(_p(wq), _p(np.ascontiguousarray(s)),
                                       _p(np.ascontiguousarray(b)), sb_dtype, n, k, bits,
                                       group_size, _p(out)), "dequantize_typed")
    return out


def qmatmul(x, x_dtype, wq, s, b, sb_dtype, k, bits, group_size):
    """x: [m,k] fp32 array or uint16 bit patterns. Returns (y, S) fp64 [m, n]."""
    x = np.ascontiguousarray(x)
    m = x.shape[0]
    n = wq.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    S = np.empty((m, n), dtype=np.float64)
    _check(lib().qref_qmatmul(_p(x), x_dtype, m, k, _p(np.ascontiguousarray(wq)),
                              _p(np.ascontiguousarray(s)), _p(np.ascontiguousarray(b)),
                              sb_dtype, n, bits, group_size, _p(y), _p(S)), "qmatmul")
    return y, S


def qmatmul_sampled(x, x_dtype, wq, s, b, sb_dtype, k, bits, group_size, mi, ni):
    x = np.ascontiguousarray(x)
    m = x.shape[0]
    n = wq.shape[0]
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    y = np.empty(mi.shape[0], dtype=np.float64)
    S = np.empty(mi.shape[0], dtype=np.float64)
    _check(lib().qref_qmatmul_sampled(_p(x), x_dtype, m, k, _p(np.ascontiguousarray(wq)),
                                      _p(np.ascontiguousarray(s)), _p(np.ascontiguousarray(b)),
                                      sb_dtype, n, bits, group_size, _p(mi), _p(ni),
                                      mi.shape[0], _p(y), _p(S)), "qmatmul_sampled")
    return y, S


def moe(a, a_dtype, ids, n_tokens, top_k, a_outer, a_inner, wq, s, b, sb_dtype,
        num_experts, n_rows, n_cols, bits, group_size):
    a = np.ascontiguousarray(a)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    P = n_tokens * top_k
    out = np.empty((P, n_rows), dtype=np.float64)
    S = np.empty((P, n_rows), dtype=np.float64)
    _check(lib().qref_moe(_p(a), a_dtype, _p(ids), n_tokens, top_k, a_outer, a_inner,
                          _p(np.ascontiguousarray(wq)), _p(np.ascontiguousarray(s)),
                          _p(np.ascontiguousarray(b)), sb_dtype, num_experts, n_rows, n_cols,
                          bits, group_size, _p(out), _p(S)), "moe")
    return out, S


def moe_gate_up_silu(a, a_dtype, ids, n_tokens, top_k, a_outer, a_inner, gate, up, sb_dtype,
                     num_experts, n_rows, n_cols, bits, group_size):
    """gate, up: (wq, s, b) tuples. Returns dict of fp64 arrays [P, n_rows]:
    silu_out, g, u, Sg, Su."""
    a = np.ascontiguousarray(a)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    P = n_tokens * top_k
    res = {k: np.empty((P, n_rows), dtype=np.float64) for k in ("silu_out", "g", "u", "Sg", "Su")}
    gw, gs_, gb = (np.ascontiguousarray(t) for t in gate)
    uw, us, ub = (np.ascontiguousarray(t) for t in up)
    _check(lib().qref_moe_gate_up_silu(
        _p(a), a_dtype, _p(ids), n_tokens, top_k, a_outer, a_inner, _p(gw), _p(gs_), _p(gb),
        _p(uw), _p(us), _p(ub), sb_dtype, num_experts, n_rows, n_cols, bits, group_size,
        _p(res["silu_out"]), _p(res["g"]), _p(res["u"]), _p(res["Sg"]), _p(res["Su"])),
        "moe_gate_up_silu")
    return res


def moe_ffn(a, a_dtype, ids, rw, n_tokens, top_k, gate, up, down, sb_dtype, num_experts,
            d_model, d_ff, bits, group_size):
    """gate, up, down: (wq, s, b). Returns (out fp64 [T, d_model], h, o) with h
    [P, d_ff] and o [P, d_model] the intermediates in a_dtype storage."""
    a = np.ascontiguousarray(a)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rw = np.ascontiguousarray(rw, dtype=np.float32)
    P = n_tokens * top_k
    out = np.empty((n_tokens, d_model), dtype=np.float64)
    h = _sb_empty((P, d_ff), a_dtype)
    o = _sb_empty((P, d_model), a_dtype)
    ws = [np.ascontiguousarray(x) for trio in (gate, up, down) for x in trio]
    _check(lib().qref_moe_ffn(_p(a), a_dtype, _p(ids), _p(rw), n_tokens, top_k,
                              *[_p(x) for x in ws], sb_dtype, num_experts, d_model, d_ff, bits,
                              group_size, _p(out), _p(h), _p(o)), "moe_ffn")
    return out, h, o


MXFP4, MXFP8, NVFP4 = 1, 2, 3


def mx_params(mode):
    """(bits, group_size) of a microscaled mode."""
    bits, gs = ctypes.c_int(), ctypes.c_int()
    _check(lib().qref_mx_params(mode, ctypes.byref(bits), ctypes.byref(gs)), "mx_params")
    return bits.value, gs.value


def fp4_e2m1(code):
    return lib().qref_fp4_e2m1(code)


def fp8_e4m3(byte):
    return lib().qref_fp8_e4m3(byte)


def e8m0(byte):
    return lib().qref_e8m0(byte)


def mx_dequantize(wq, scales, mode, k, out_dtype=F32):
    """Dense weight [n, k]: fp32 values, or uint16 bit patterns for fp16/bf16."""
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = wq.shape[0]
    out = _sb_empty((n, k), out_dtype)
    _check(lib().qref_mx_dequantize(_p(wq), _p(scales), mode, n, k, out_dtype, _p(out)),
           "mx_dequantize")
    return out


def mx_qmatmul(x, x_dtype, wq, scales, mode, k):
    """x: [m,k] fp32 values or uint16 bit patterns. Returns (y, S) fp64 [m, n]."""
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    m, n = x.shape[0], wq.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    S = np.empty((m, n), dtype=np.float64)
    _check(lib().qref_mx_qmatmul(_p(x), x_dtype, m, k, _p(wq), _p(scales), mode, n, _p(y), _p(S)),
           "mx_qmatmul")
    return y, S


def quantize_int8_tensor(w):
    """fp32 array -> (int8 codes of the same shape, float32 range [lo, hi])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    q = np.empty(w.shape, dtype=np.int8)
    rng_ = np.empty(2, dtype=np.float32)
    _check(lib().qref_quantize_int8_tensor(_p(w), w.size, _p(q), _p(rng_)), "quantize_int8_tensor")
    return q, rng_


def dequantize_int8_tensor(q, rng_):
    q = np.ascontiguousarray(q, dtype=np.int8)
    rng_ = np.ascontiguousarray(rng_, dtype=np.float32)
    w = np.empty(q.shape, dtype=np.float32)
    _check(lib().qref_dequantize_int8_tensor(_p(q), q.size, _p(rng_), _p(w)), "dequantize_int8_tensor")
    return w


def qmatmul_int8_tensor(x, x_dtype, q, rng_):
    """x: [m, k] fp32 values or uint16 bits; q: int8 [n, k]. Returns (y, S) fp64."""
    x = np.ascontiguousarray(x)
    q = np.ascontiguousarray(q, dtype=np.int8)
    rng_ = np.ascontiguousarray(rng_, dtype=np.float32)
    m, k = x.shape
    n = q.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    S = np.empty((m, n), dtype=np.float64)
    _check(lib().qref_qmatmul_int8_tensor(_p(x), x_dtype, m, k, _p(q), _p(rng_), n, _p(y), _p(S)),
           "qmatmul_int8_tensor")
    return y, S


def qmatmul_t(x, x_dtype, wq, s, b, sb_dtype, n, bits, group_size):
    """transpose = false: wq packs W [k, n] along n. Returns (y, S) fp64 [m, n]."""
    x = np.ascontiguousarray(x)
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    m, k = x.shape
    y = np.empty((m, n), dtype=np.float64)
    S = np.empty((m, n), dtype=np.float64)
    _check(lib().qref_qmatmul_t(_p(x), x_dtype, m, k, _p(wq), _p(np.ascontiguousarray(s)),
                                _p(np.ascontiguousarray(b)), sb_dtype, n, bits, group_size,
                                _p(y), _p(S)), "qmatmul_t")
    return y, S
