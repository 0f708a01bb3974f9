"""Weight-only quantized linear layers on MI355X (gfx950).

Thin ctypes binding of ``libqpack.so`` (C ABI in ``include/qpack.h``). This
module only marshals arguments: tensors are passed as device pointers with the
caller's current HIP stream, and every step of the computation runs in the
library's HIP kernels. PyTorch provides device memory and streams. There is no
CPU fallback: without the built library every call raises.

Calls (same names as the C ABI):
    qpack_quantize(w, bits, group_size, sb_dtype)  -> (wq, scales, biases)
    qmatmul(x, wq, scales, biases, bits, group_size) -> y = x @ dequant(W)^T
    qgemv_moe_id(a, ids, ..., wq, scales, biases, ...) -> out
    qgemv_moe_id_gate_up_silu(a, ids, ..., gate, up, ...) -> SiLU(gate) * up
    qgemv_moe_workspace_bytes(n_pairs, num_experts)
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libqpack.so")

QP_F32, QP_F16, QP_BF16 = 0, 1, 2
STATUS = {0: "QP_OK", 1: "QP_ERR_INVALID_ARG", 2: "QP_ERR_UNSUPPORTED",
          3: "QP_ERR_DTYPE_MISMATCH", 4: "QP_ERR_SHAPE", 5: "QP_ERR_ALIGN",
          6: "QP_ERR_WORKSPACE", 7: "QP_ERR_HIP"}

# Every symbol include/qpack.h declares.
EXPORTS = ("qpack_quantize", "qpack_dequantize", "qpack_dequantize_mx", "qmatmul", "qmatmul_mx",
           "qgemv_moe_workspace_bytes", "qgemv_moe_id", "qgemv_moe_id_noalloc",
           "qgemv_moe_id_gate_up_silu",
           "qgemv_moe_ffn_workspace_bytes", "qgemv_moe_ffn", "qpack_quantize_int8_tensor",
           "qpack_dequantize_int8_tensor", "qmatmul_int8_tensor", "qmatmul_t_workspace_bytes",
           "qmatmul_t", "qpack_last_error",
           "qpack_version")


class QpackError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.qpack_quantize.argtypes = [P, I64, I64, I32, I32, ctypes.c_int, P, P, P, P]
        L.qpack_quantize.restype = ctypes.c_int
        L.qpack_dequantize.argtypes = [P, P, P, ctypes.c_int, I64, I64, I32, I32, ctypes.c_int,
                                       P, P]
        L.qpack_dequantize.restype = ctypes.c_int
        L.qpack_dequantize_mx.argtypes = [P, P, ctypes.c_int, I64, I64, ctypes.c_int, P, P]
        L.qpack_dequantize_mx.restype = ctypes.c_int
        L.qmatmul_mx.argtypes = [P, ctypes.c_int, I64, I64, P, P, ctypes.c_int, I64, P, P]
        L.qmatmul_mx.restype = ctypes.c_int
        L.qmatmul.argtypes = [P, ctypes.c_int, I64, I64, P, P, P, ctypes.c_int, I64, I32, I32, P,
                              P]
        L.qmatmul.restype = ctypes.c_int
        L.qgemv_moe_workspace_bytes.argtypes = [I64, I64]
        L.qgemv_moe_workspace_bytes.restype = SZ
        L.qgemv_moe_id.argtypes = [P, ctypes.c_int, P, I64, I64, I64, I64, P, P, P, ctypes.c_int,
                                   I64, I64, I64, I32, I32, P, P, SZ, P]
        L.qgemv_moe_id.restype = ctypes.c_int
        L.qgemv_moe_id_noalloc.argtypes = [P, ctypes.c_int, P, I64, I64, I64, I64, P, P, P,
                                           ctypes.c_int, I64, I64, I64, I32, I32, P, P]
        L.qgemv_moe_id_noalloc.restype = ctypes.c_int
        L.qgemv_moe_id_gate_up_silu.argtypes = [P, ctypes.c_int, P, I64, I64, I64, I64, P, P, P,
                                                P, P, P, ctypes.c_int, I64, I64, I64, I32, I32,
                                                P, P, SZ, P]
        L.qgemv_moe_id_gate_up_silu.restype = ctypes.c_int
        L.qgemv_moe_ffn_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, ctypes.c_int]
        L.qgemv_moe_ffn_workspace_bytes.restype = SZ
        L.qgemv_moe_ffn.argtypes = ([P, ctypes.c_int, P, P, I64, I64] + [P] * 9 +
                                    [ctypes.c_int, I64, I64, I64, I32, I32, P, P, SZ, P])
        L.qgemv_moe_ffn.restype = ctypes.c_int
        L.qpack_quantize_int8_tensor.argtypes = [P, I64, P, P, P]
        L.qpack_quantize_int8_tensor.restype = ctypes.c_int
        L.qpack_dequantize_int8_tensor.argtypes = [P, I64, P, ctypes.c_int, P, P]
        L.qpack_dequantize_int8_tensor.restype = ctypes.c_int
        L.qmatmul_int8_tensor.argtypes = [P, ctypes.c_int, I64, I64, P, P, I64, P, P]
        L.qmatmul_int8_tensor.restype = ctypes.c_int
        L.qmatmul_t_workspace_bytes.argtypes = [I64, I64, I64, I32]
        L.qmatmul_t_workspace_bytes.restype = SZ
        L.qmatmul_t.argtypes = [P, ctypes.c_int, I64, I64, P, P, P, ctypes.c_int, I64, I32, I32, P,
                                P, SZ, P]
        L.qmatmul_t.restype = ctypes.c_int
        L.qpack_last_error.restype = ctypes.c_char_p
        L.qpack_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().qpack_last_error().decode()


def check(status: int) -> None:
    if status != 0:
        raise QpackError(status, last_error())


def version() -> str:
    return lib().qpack_version().decode()


# ------------------------------------------------------------------ tensors

_DTYPE_CODES = None


def dtype_code(dt) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: QP_F32, torch.float16: QP_F16, torch.bfloat16: QP_BF16}
    code = _DTYPE_CODES.get(dt)
    if code is None:
        raise TypeError(f"unsupported dtype {dt}")
    return code


_RAW_STREAM = None


def _stream(t) -> int:
    """The handle of the current stream on t's device. torch's raw-handle query
    costs about 0.06 us per call against about 1.8 us for building the Stream
    object, which matters for calls of a few microseconds issued one by one."""
    global _RAW_STREAM
    if _RAW_STREAM is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _RAW_STREAM = ((lambda dev: raw(dev.index)) if raw is not None
                       else (lambda dev: torch.cuda.current_stream(dev).cuda_stream))
    return _RAW_STREAM(t.device)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _ptr(t) -> int:
    return t.data_ptr()


def qpack_quantize(w, bits: int, group_size: int, sb_dtype=None, wq=None, scales=None,
                   biases=None):
    """Quantize fp32 w [n, k] on the device. Returns (wq u32-as-int32 [n, k*bits/32],
    scales [n, k/gs], biases [n, k/gs]) with scales/biases of `sb_dtype` (default bf16)."""
    import torch
    _dev(w, "w")
    if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous fp32 [n, k] tensor")
    sb_dtype = sb_dtype or torch.bfloat16
    n, k = w.shape
    if wq is None:
        wq = torch.empty((n, k * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // group_size if group_size else 0), dtype=sb_dtype,
                             device=w.device)
    if biases is None:
        biases = torch.empty_like(scales)
    check(lib().qpack_quantize(_ptr(w), n, k, bits, group_size, dtype_code(sb_dtype), _ptr(wq),
                               _ptr(scales), _ptr(biases), _stream(w)))
    return wq, scales, biases


def qpack_dequantize(wq, scales, biases, bits: int, group_size: int, out_dtype=None,
                     out=None):
    """Dense weight [n, k] from packed codes: fp32, or (the default) the scales' own
    dtype, with the product and sum rounded to that dtype."""
    import torch
    for t, nm in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    n = wq.shape[0]
    k = wq.shape[1] * 32 // bits if bits else 0
    out_dtype = out_dtype or scales.dtype
    if out is None:
        out = torch.empty((n, k), dtype=out_dtype, device=wq.device)
    check(lib().qpack_dequantize(_ptr(wq), _ptr(scales), _ptr(biases), dtype_code(scales.dtype),
                                 n, k, bits, group_size, dtype_code(out.dtype), _ptr(out),
                                 _stream(wq)))
    return out


MXFP4, MXFP8, NVFP4 = 1, 2, 3
MX_LAYOUT = {MXFP4: (4, 32), MXFP8: (8, 32), NVFP4: (4, 16)}   # mode -> (bits, group size)


def qpack_dequantize_mx(wq, scales, mode: int, out_dtype=None, out=None):
    """Dense weight [n, k] of a microscaled mode (scales: uint8 [n, k/gs]); bf16 by
    default, as the pages return it."""
    import torch
    for t, nm in ((wq, "wq"), (scales, "scales")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if mode not in MX_LAYOUT:
        raise ValueError(f"unknown microscaled mode {mode}")
    n, k = wq.shape[0], wq.shape[1] * 32 // MX_LAYOUT[mode][0]
    if out is None:
        out = torch.empty((n, k), dtype=out_dtype or torch.bfloat16, device=wq.device)
    check(lib().qpack_dequantize_mx(_ptr(wq), _ptr(scales), mode, n, k, dtype_code(out.dtype),
                                    _ptr(out), _stream(wq)))
    return out


def qmatmul_mx(x, wq, scales, mode: int, out=None):
    """y = x @ dequant(W)^T for a microscaled W; x [m, k] fp32/fp16/bf16, y in x's dtype."""
    import torch
    _dev(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [m, k] tensor")
    for t, nm in ((wq, "wq"), (scales, "scales")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    m, k = x.shape
    n = wq.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    check(lib().qmatmul_mx(_ptr(x), dtype_code(x.dtype), m, k, _ptr(wq), _ptr(scales), mode, n,
                           _ptr(out), _stream(x)))
    return out


def qmatmul(x, wq, scales, biases, bits: int, group_size: int, out=None):
    """y = x @ dequant(W)^T for x [m, k] (fp32/fp16/bf16, same dtype as scales)."""
    import torch
    _dev(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [m, k] tensor")
    m, k = x.shape
    n = wq.shape[0]
    for t, nm in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    check(lib().qmatmul(_ptr(x), dtype_code(x.dtype), m, k, _ptr(wq), _ptr(scales), _ptr(biases),
                        dtype_code(scales.dtype), n, bits, group_size, _ptr(out), _stream(x)))
    return out


def qgemv_moe_workspace_bytes(n_pairs: int, num_experts: int) -> int:
    return int(lib().qgemv_moe_workspace_bytes(n_pairs, num_experts))


def _moe_workspace(a, n_pairs, num_experts, workspace):
    import torch
    need = qgemv_moe_workspace_bytes(n_pairs, num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    return workspace


def qgemv_moe_id(a, ids, n_tokens: int, top_k: int, a_outer: int, a_inner: int, wq, scales,
                 biases, bits: int, group_size: int, out=None, workspace=None):
    """out[p] = a_row(p) @ dequant(W[ids[p]])^T for p < n_tokens*top_k, with
    a_row(p) = a.flat[(p//top_k)*a_outer + (p%top_k)*a_inner : +n_cols].
    wq [E, n_rows, n_cols*bits/32], scales/biases [E, n_rows, n_cols/gs]."""
    import torch
    E, n_rows = wq.shape[0], wq.shape[1]
    n_cols = wq.shape[2] * 32 // bits
    P = n_tokens * top_k
    if out is None:
        out = torch.empty((P, n_rows), dtype=a.dtype, device=a.device)
    workspace = _moe_workspace(a, P, E, workspace)
    check(lib().qgemv_moe_id(_ptr(a), dtype_code(a.dtype), _ptr(ids), n_tokens, top_k, a_outer,
                             a_inner, _ptr(wq), _ptr(scales), _ptr(biases),
                             dtype_code(scales.dtype), E, n_rows, n_cols, bits, group_size,
                             _ptr(out), _ptr(workspace), workspace.numel(), _stream(a)))
    return out


def qgemv_moe_id_noalloc(a, ids, n_tokens: int, top_k: int, a_outer: int, a_inner: int, wq,
                         scales, biases, bits: int, group_size: int, out):
    """qgemv_moe_id with the routing tables in the library's own device
    scratch (no workspace; `out` is the caller's)."""
    E, n_rows = wq.shape[0], wq.shape[1]
    n_cols = wq.shape[2] * 32 // bits
    check(lib().qgemv_moe_id_noalloc(_ptr(a), dtype_code(a.dtype), _ptr(ids), n_tokens, top_k,
                                     a_outer, a_inner, _ptr(wq), _ptr(scales), _ptr(biases),
                                     dtype_code(scales.dtype), E, n_rows, n_cols, bits,
                                     group_size, _ptr(out), _stream(a)))
    return out


def qgemv_moe_id_gate_up_silu(a, ids, n_tokens: int, top_k: int, a_outer: int, a_inner: int,
                              gate, up, bits: int, group_size: int, out=None, workspace=None):
    """silu_out[p] = SiLU(a_row(p) @ dequant(Wg[ids[p]])^T) * (a_row(p) @ dequant(Wu[ids[p]])^T).
    gate, up: (wq, scales, biases) stacks of identical shape."""
    import torch
    gwq, gs_, gb = gate
    uwq, us, ub = up
    if tuple(gwq.shape) != tuple(uwq.shape) or tuple(gs_.shape) != tuple(us.shape):
        raise ValueError("gate and up stacks must match in shape")
    E, n_rows = gwq.shape[0], gwq.shape[1]
    n_cols = gwq.shape[2] * 32 // bits
    P = n_tokens * top_k
    if out is None:
        out = torch.empty((P, n_rows), dtype=a.dtype, device=a.device)
    workspace = _moe_workspace(a, P, E, workspace)
    check(lib().qgemv_moe_id_gate_up_silu(
        _ptr(a), dtype_code(a.dtype), _ptr(ids), n_tokens, top_k, a_outer, a_inner, _ptr(gwq),
        _ptr(gs_), _ptr(gb), _ptr(uwq), _ptr(us), _ptr(ub), dtype_code(gs_.dtype), E, n_rows,
        n_cols, bits, group_size, _ptr(out), _ptr(workspace), workspace.numel(), _stream(a)))
    return out


def qgemv_moe_ffn_workspace_bytes(n_tokens: int, top_k: int, num_experts: int, d_model: int,
                                  d_ff: int, dtype) -> int:
    return int(lib().qgemv_moe_ffn_workspace_bytes(n_tokens, top_k, num_experts, d_model, d_ff,
                                                   dtype_code(dtype)))


def qgemv_moe_ffn(a, ids, route_weights, top_k: int, gate, up, down, bits: int, group_size: int,
                  out=None, workspace=None):
    """One MoE FFN block: a [T, d_model], ids int32 [T*top_k], route_weights fp32
    [T*top_k]; gate / up / down = (wq, scales, biases) expert stacks. Returns
    out [T, d_model] in a's dtype."""
    import torch
    for t, nm in ((a, "a"), (ids, "ids"), (route_weights, "route_weights")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    T, D = a.shape
    E, F = gate[0].shape[0], gate[0].shape[1]
    if workspace is None:
        nbytes = qgemv_moe_ffn_workspace_bytes(T, top_k, E, D, F, a.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=a.device)
    if out is None:
        out = torch.empty((T, D), dtype=a.dtype, device=a.device)
    ptrs = [_ptr(x) for trio in (gate, up, down) for x in trio]
    check(lib().qgemv_moe_ffn(_ptr(a), dtype_code(a.dtype), _ptr(ids), _ptr(route_weights), T,
                              top_k, *ptrs, dtype_code(gate[1].dtype), E, D, F, bits, group_size,
                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(a)))
    return out


def qpack_quantize_int8_tensor(w, q=None, rng=None):
    """Per-tensor dynamic-range int8 of fp32 w: (int8 codes shaped like w, fp32 range [lo, hi])."""
    import torch
    _dev(w, "w")
    if w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError("w must be a contiguous fp32 tensor")
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device) if q is None else q
    rng = torch.empty(2, dtype=torch.float32, device=w.device) if rng is None else rng
    check(lib().qpack_quantize_int8_tensor(_ptr(w), w.numel(), _ptr(q), _ptr(rng), _stream(w)))
    return q, rng


def qpack_dequantize_int8_tensor(q, rng, out_dtype=None, out=None):
    import torch
    _dev(q, "q")
    _dev(rng, "range")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    check(lib().qpack_dequantize_int8_tensor(_ptr(q), q.numel(), _ptr(rng), dtype_code(out.dtype),
                                             _ptr(out), _stream(q)))
    return out


def qmatmul_int8_tensor(x, q, rng, out=None):
    """y = x @ W^T for a per-tensor int8 weight q [n, k] with device range [lo, hi]."""
    import torch
    for t, nm in ((x, "x"), (q, "q"), (rng, "range")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    m, k = x.shape
    n = q.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    check(lib().qmatmul_int8_tensor(_ptr(x), dtype_code(x.dtype), m, k, _ptr(q), _ptr(rng), n,
                                    _ptr(out), _stream(x)))
    return out


def qmatmul_t_workspace_bytes(m: int, k: int, n: int, bits: int) -> int:
    return int(lib().qmatmul_t_workspace_bytes(m, k, n, bits))


def qmatmul_t(x, wq, scales, biases, bits: int, group_size: int, out=None, workspace=None):
    """transpose = false: y = x @ dequant(W) with W stored [k, n] (wq [k, n*bits/32],
    scales / biases [k, n/gs], groups along n)."""
    import torch
    _dev(x, "x")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [m, k] tensor")
    for t, nm in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    m, k = x.shape
    n = wq.shape[1] * 32 // bits
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    if workspace is None:
        nbytes = qmatmul_t_workspace_bytes(m, k, n, bits)
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=x.device)
    check(lib().qmatmul_t(_ptr(x), dtype_code(x.dtype), m, k, _ptr(wq), _ptr(scales), _ptr(biases),
                          dtype_code(scales.dtype), n, bits, group_size, _ptr(out), _ptr(workspace),
                          workspace.numel(), _stream(x)))
    return out
