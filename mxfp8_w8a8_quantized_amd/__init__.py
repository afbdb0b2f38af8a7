"""MXFP8 W8A8 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI in ``include/mx.h`` (same names). It only
marshals arguments: torch tensors in, device pointers and the current HIP
stream out; every step of the computation runs in the library's HIP kernels.
If the built library ``libmxfp8.so`` is missing, every call raises.
"""

import ctypes
import os
from typing import NamedTuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxfp8.so")

MX_OK = 0
MX_ERR_INVALID_ARGUMENT = 1
MX_ERR_UNSUPPORTED = 2
MX_ERR_HIP = 3
MX_EPI_NONE = 0
MX_EPI_GELU_TANH = 1
MX_DT_BF16 = 0
MX_DT_F32 = 1
MX_PLAN_SLAB = 0
MX_PLAN_SPLITK = 1
MX_PLAN_SMALL = 2
MX_PLAN_BALANCED = 3
MX_PLAN_SLAB_M128 = 4
PLAN_NAMES = {MX_PLAN_SLAB: "slab", MX_PLAN_SPLITK: "splitk", MX_PLAN_SMALL: "small", MX_PLAN_BALANCED: "balanced",
              MX_PLAN_SLAB_M128: "slab_m128"}
PLAN_KINDS = {v: k for k, v in PLAN_NAMES.items()}

# Every symbol include/mx.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_PI = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "mx_abi_version": ([], _INT),
    "mx_status_string": ([_INT], ctypes.c_char_p),
    "mx_last_hip_error": ([], _INT),
    "mx_last_error_message": ([], ctypes.c_char_p),
    "mx_quantize_act": ([_P, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_quantize_weight": ([_P, _INT, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_linear_fused": ([_P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
    "mx_linear_q": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
    "mx_slab_rows": ([_I64], _I64),
    "mx_quantize_act_slab": ([_P, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_quantize_weight_slab": ([_P, _INT, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_slab_pack": ([_P, _P, _I64, _I64, _P, _P, _P], _INT),
    "mx_linear_slab": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
    "mx_linear_slab_m128": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
    "mx_linear_slab_requant": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _P], _INT),
    "mx_linear_splitk_ws_bytes": ([_I64, _I64, _INT], _I64),
    "mx_linear_splitk_choose": ([_I64, _I64, _I64], _INT),
    "mx_linear_slab_splitk": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _INT, _P, _I64, _P], _INT),
    "mx_linear_small_ws_bytes": ([_I64, _I64, _INT], _I64),
    "mx_linear_small_choose": ([_I64, _I64, _I64], _INT),
    "mx_linear_slab_small": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _INT, _P, _I64, _P], _INT),
    "mx_linear_balanced_ws_bytes": ([_I64, _I64, _I64], _I64),
    "mx_linear_slab_balanced": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _P], _INT),
    "mx_linear_plan_default": ([_I64, _I64, _I64, _PI, _PI], _INT),
    "mx_linear_plan_ws_bytes": ([_INT, _INT, _I64, _I64, _I64], _I64),
    "mx_linear_slab_plan": ([_INT, _INT, _P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _P], _INT),
    "mx_linear_tune_ws_bytes": ([_I64, _I64, _I64], _I64),
    "mx_linear_tune": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _INT, _P, _PI, _PI], _INT),
    "mx_linear_plan_lookup": ([_I64, _I64, _I64, _INT, _PI, _PI], _INT),
    "mx_linear_slab_auto": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _P], _INT),
    "mx_linear_plan_clear": ([], None),
    "mx_linear_ws_bytes": ([_I64, _I64, _I64], _I64),
    "mx_linear": ([_P, _I64, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P, _I64, _P], _INT),
    "mx_linear_noalloc": ([_P, _I64, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
    "mx_probe_mfma": ([_P, _P, _I64, _INT, _INT, _P, _P], _INT),
    "mx_pc_quantize_act_slab": ([_P, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_pc_quantize_weight_slab": ([_P, _INT, _I64, _I64, _I64, _P, _P, _P], _INT),
    "mx_pc_linear_slab": ([_P, _P, _I64, _I64, _P, _P, _I64, _P, _INT, _P, _P], _INT),
}


class MXError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(message)


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MXError(-1, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(status):
    if status != MX_OK:
        L = lib()
        msg = L.mx_last_error_message().decode()
        name = L.mx_status_string(status).decode()
        raise MXError(status, f"{name}: {msg}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mx_abi_version():
    return lib().mx_abi_version()


def mx_status_string(status):
    return lib().mx_status_string(status).decode()


def mx_last_hip_error():
    return lib().mx_last_hip_error()


def mx_last_error_message():
    return lib().mx_last_error_message().decode()


def mx_quantize_act(x, q=None, s=None):
    """bf16 [M, K] (rows may be strided) -> (codes uint8 [M, K], scales uint8 [M, K/32])."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    dev = x.device
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=dev) if s is None else s
    _need(q, "q", torch.uint8, dev)
    _need(s, "s", torch.uint8, dev)
    ld = x.stride(0) if M > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_quantize_act(_ptr(x), M, K, ld, _ptr(q), _ptr(s), _stream(dev)))
    return q, s


def mx_quantize_weight(w, q=None, s=None):
    """fp32 or bf16 [N, K] -> (codes uint8 [N, K], scales uint8 [N, K/32])."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be 2-D with unit column stride")
    dt = {torch.float32: MX_DT_F32, torch.bfloat16: MX_DT_BF16}.get(w.dtype)
    if dt is None:
        raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
    N, K = w.shape
    dev = w.device
    q = torch.empty((N, K), dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty((N, K // 32), dtype=torch.uint8, device=dev) if s is None else s
    _need(q, "q", torch.uint8, dev)
    _need(s, "s", torch.uint8, dev)
    ld = w.stride(0) if N > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_quantize_weight(_ptr(w), dt, N, K, ld, _ptr(q), _ptr(s), _stream(dev)))
    return q, s


def _linear_common(M, K, wq, ws, bias, y, dev):
    N = wq.shape[0]
    _need(wq, "wq", torch.uint8, dev)
    _need(ws, "ws", torch.uint8, dev)
    if wq.shape != (N, K) or ws.shape != (N, K // 32):
        raise ValueError(f"weights must be [N, {K}] codes and [N, {K // 32}] scales")
    if bias is not None:
        _need(bias, "bias", torch.float16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be f16 [N]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    return N, y


def mx_linear_fused(x, wq, ws, bias=None, gelu=False, y=None):
    """y = bf16(epi(quant_mx(x) @ dequant(wq, ws)^T + bias)) on row-major
    weights, activation quantization fused into the GEMM's prologue (slow:
    see mx.h). x: bf16 [M, K]."""
    dev = x.device
    _need(x, "x", torch.bfloat16, dev)
    M, K = x.shape
    N, y = _linear_common(M, K, wq, ws, bias, y, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(lib().mx_linear_fused(_ptr(x), M, K, _ptr(wq), _ptr(ws), N, _ptr(bias), epi, _ptr(y), _stream(dev)))
    return y


def mx_linear_q(xq, xs, wq, ws, bias=None, gelu=False, y=None):
    """The same linear on pre-quantized activations xq uint8 [M, K], xs uint8 [M, K/32]."""
    dev = xq.device
    _need(xq, "xq", torch.uint8, dev)
    _need(xs, "xs", torch.uint8, dev)
    M, K = xq.shape
    if xs.shape != (M, K // 32):
        raise ValueError("xs must be [M, K/32]")
    N, y = _linear_common(M, K, wq, ws, bias, y, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear_q(_ptr(xq), _ptr(xs), M, K, _ptr(wq), _ptr(ws), N, _ptr(bias), epi, _ptr(y), _stream(dev))
        )
    return y


class Slab(NamedTuple):
    """An operand in the slab layout: codes q uint8 [K/64, R, 64], scales s
    uint8 [K/64, R, 2], R = mx_slab_rows(rows); rows past `rows` are zero."""

    q: torch.Tensor
    s: torch.Tensor
    rows: int

    @property
    def K(self):
        return self.q.shape[0] * 64


def mx_slab_rows(rows):
    return lib().mx_slab_rows(rows)


def _slab_out(rows, K, dev, out):
    R = mx_slab_rows(rows)
    if out is None:
        return Slab(
            torch.empty((K // 64, R, 64), dtype=torch.uint8, device=dev),
            torch.empty((K // 64, R, 2), dtype=torch.uint8, device=dev),
            rows,
        )
    _need(out.q, "out.q", torch.uint8, dev)
    _need(out.s, "out.s", torch.uint8, dev)
    if out.q.shape != (K // 64, R, 64) or out.s.shape != (K // 64, R, 2) or out.rows != rows:
        raise ValueError(f"out must hold [{K // 64}, {R}, 64] codes and [{K // 64}, {R}, 2] scales for {rows} rows")
    return out


def mx_quantize_act_slab(x, out=None):
    """bf16 [M, K] (rows may be strided, K % 64 == 0) -> Slab of its MX codes and scales."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    if K % 64 != 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    dev = x.device
    out = _slab_out(M, K, dev, out)
    ld = x.stride(0) if M > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_quantize_act_slab(_ptr(x), M, K, ld, _ptr(out.q), _ptr(out.s), _stream(dev)))
    return out


def mx_quantize_weight_slab(w, out=None):
    """fp32 or bf16 [N, K] (K % 64 == 0) -> Slab of its MX codes and scales."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be 2-D with unit column stride")
    dt = {torch.float32: MX_DT_F32, torch.bfloat16: MX_DT_BF16}.get(w.dtype)
    if dt is None:
        raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
    N, K = w.shape
    if K % 64 != 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    dev = w.device
    out = _slab_out(N, K, dev, out)
    ld = w.stride(0) if N > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_quantize_weight_slab(_ptr(w), dt, N, K, ld, _ptr(out.q), _ptr(out.s), _stream(dev)))
    return out


def mx_slab_pack(q, s, out=None):
    """Row-major codes uint8 [rows, K] and scales uint8 [rows, K/32] -> Slab."""
    dev = q.device
    _need(q, "q", torch.uint8, dev)
    _need(s, "s", torch.uint8, dev)
    rows, K = q.shape
    if s.shape != (rows, K // 32):
        raise ValueError("s must be [rows, K/32]")
    if K % 64 != 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    out = _slab_out(rows, K, dev, out)
    with torch.cuda.device(dev):
        _check(lib().mx_slab_pack(_ptr(q), _ptr(s), rows, K, _ptr(out.q), _ptr(out.s), _stream(dev)))
    return out


def _slab_linear_args(x, w, bias):
    dev = x.q.device
    for name, t in (("x.q", x.q), ("x.s", x.s), ("w.q", w.q), ("w.s", w.s)):
        _need(t, name, torch.uint8, dev)
    M, N, K = x.rows, w.rows, x.K
    if w.K != K:
        raise ValueError(f"x has K = {K}, w has K = {w.K}")
    for name, sl in (("x", x), ("w", w)):
        R = mx_slab_rows(sl.rows)
        if sl.q.shape != (K // 64, R, 64) or sl.s.shape != (K // 64, R, 2):
            raise ValueError(f"{name} is not a slab of {sl.rows} rows and K = {K}")
    if bias is not None:
        _need(bias, "bias", torch.float16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be f16 [N]")
    return dev, M, N, K


def mx_linear_slab(x, w, bias=None, gelu=False, y=None):
    """y = bf16(epi(xhat @ what^T + bias)) on slab operands x (tokens) and w (weights)."""
    return _slab_call(lib().mx_linear_slab, x, w, bias, gelu, y)


def mx_linear_slab_m128(x, w, bias=None, gelu=False, y=None):
    """mx_linear_slab on 256 (weight rows) x 128 (tokens) tiles: the same y,
    bit for bit, with twice the tiles (for a few hundred tokens)."""
    return _slab_call(lib().mx_linear_slab_m128, x, w, bias, gelu, y)


def _slab_call(fn, x, w, bias, gelu, y):
    dev, M, N, K = _slab_linear_args(x, w, bias)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(fn(_ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), _stream(dev)))
    return y


def mx_linear_slab_requant(x, w, bias=None, gelu=False, out=None):
    """The same linear returning, instead of bf16 y, the Slab of y's MX
    quantization (rows M, K = N): the next linear's activation operand."""
    dev, M, N, K = _slab_linear_args(x, w, bias)
    if N % 64 != 0:
        raise ValueError("the requantized output needs N % 64 == 0")
    out = _slab_out(M, N, dev, out)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear_slab_requant(
                _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(out.q), _ptr(out.s),
                _stream(dev),
            )
        )
    return out


def mx_linear_splitk_ws_bytes(M, N, splits):
    return lib().mx_linear_splitk_ws_bytes(M, N, splits)


def mx_linear_splitk_choose(M, K, N):
    return lib().mx_linear_splitk_choose(M, K, N)


def mx_linear_slab_splitk(x, w, bias=None, gelu=False, y=None, splits=None, workspace=None):
    """mx_linear_slab with split-K over `splits` K ranges (default
    mx_linear_splitk_choose); workspace: uint8 of at least
    mx_linear_splitk_ws_bytes(M, N, splits) bytes (allocated here when None)."""
    dev, M, N, K = _slab_linear_args(x, w, bias)
    splits = mx_linear_splitk_choose(M, K, N) if splits is None else int(splits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    if workspace is None:
        need = mx_linear_splitk_ws_bytes(M, N, splits)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear_slab_splitk(
                _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), splits,
                _ptr(workspace), workspace.numel(), _stream(dev),
            )
        )
    return y


def mx_linear_small_ws_bytes(M, N, splits):
    return lib().mx_linear_small_ws_bytes(M, N, splits)


def mx_linear_small_choose(M, K, N):
    return lib().mx_linear_small_choose(M, K, N)


def mx_linear_slab_small(x, w, bias=None, gelu=False, y=None, splits=None, workspace=None):
    """mx_linear_slab through the few-token kernel (128 x 64 tiles) with
    `splits` K ranges (default mx_linear_small_choose); workspace: uint8 of
    at least mx_linear_small_ws_bytes(M, N, splits) bytes (allocated here
    when None and needed)."""
    dev, M, N, K = _slab_linear_args(x, w, bias)
    splits = mx_linear_small_choose(M, K, N) if splits is None else int(splits)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    need = mx_linear_small_ws_bytes(M, N, splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear_slab_small(
                _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), splits,
                _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev),
            )
        )
    return y


def _plan_out(fn, *args):
    kind, splits = ctypes.c_int(0), ctypes.c_int(0)
    _check(fn(*args, ctypes.byref(kind), ctypes.byref(splits)))
    return PLAN_NAMES[kind.value], splits.value


def plan_linear(M, K, N):
    """The default kernel plan of an M x K x N slab linear
    (mx_linear_plan_default): ("small", splits), ("splitk", splits) or
    ("slab", 1)."""
    return _plan_out(lib().mx_linear_plan_default, M, K, N)


def plan_lookup(M, K, N, gelu=False):
    """The tuned plan of this shape if mx_linear_tune cached one, else the
    default plan (mx_linear_plan_lookup)."""
    return _plan_out(lib().mx_linear_plan_lookup, M, K, N, MX_EPI_GELU_TANH if gelu else MX_EPI_NONE)


def plan_ws_bytes(plan, M, N, K=64):
    """Workspace bytes of a plan (mx_linear_plan_ws_bytes; K matters only to
    "balanced")."""
    kind, sp = plan
    return lib().mx_linear_plan_ws_bytes(PLAN_KINDS[kind], sp, M, K, N)


def mx_linear_tune_ws_bytes(M, K, N):
    return lib().mx_linear_tune_ws_bytes(M, K, N)


def mx_linear_plan_clear():
    lib().mx_linear_plan_clear()


def _plan_call(x, w, bias, y):
    dev, M, N, K = _slab_linear_args(x, w, bias)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    return dev, M, N, K, y


def _ws_args(workspace, dev):
    if workspace is None:
        return None, 0
    _need(workspace, "workspace", torch.uint8, dev)
    return workspace, workspace.numel()


def mx_linear_slab_planned(plan, x, w, bias=None, gelu=False, y=None, workspace=None):
    """mx_linear_slab through the kernel a plan names (mx_linear_slab_plan);
    workspace: uint8 of at least plan_ws_bytes(plan, M, N, K) bytes
    (allocated here when None and needed)."""
    dev, M, N, K, y = _plan_call(x, w, bias, y)
    kind, sp = plan
    need = lib().mx_linear_plan_ws_bytes(PLAN_KINDS[kind], sp, M, K, N)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    workspace, nb = _ws_args(workspace, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(lib().mx_linear_slab_plan(PLAN_KINDS[kind], sp, _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N,
                                         _ptr(bias), epi, _ptr(y), _ptr(workspace), nb, _stream(dev)))
    return y


def mx_linear_tune(x, w, bias=None, gelu=False, y=None, workspace=None, reps=10):
    """Times the candidate plans of this shape on these operands, caches the
    fastest (mx_linear_tune) and returns it as (kind, splits). workspace:
    uint8 of at least mx_linear_tune_ws_bytes(M, K, N) bytes (allocated here
    when None). Synchronizes the current stream."""
    dev, M, N, K, y = _plan_call(x, w, bias, y)
    if workspace is None:
        workspace = torch.empty((max(mx_linear_tune_ws_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)
    workspace, nb = _ws_args(workspace, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        return _plan_out(lib().mx_linear_tune, _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi,
                         _ptr(y), _ptr(workspace), nb, int(reps), _stream(dev))


def mx_linear_slab_auto(x, w, bias=None, gelu=False, y=None, workspace=None):
    """mx_linear_slab through the cached (tuned) or default plan of this shape
    (mx_linear_slab_auto); workspace: uint8 of at least the plan's workspace
    (mx_linear_tune_ws_bytes always suffices; allocated here when None and
    needed)."""
    dev, M, N, K, y = _plan_call(x, w, bias, y)
    if workspace is None:
        with torch.cuda.device(dev):
            kind, sp = plan_lookup(M, K, N, gelu)
        need = lib().mx_linear_plan_ws_bytes(PLAN_KINDS[kind], sp, M, K, N)
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    workspace, nb = _ws_args(workspace, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(lib().mx_linear_slab_auto(_ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi,
                                         _ptr(y), _ptr(workspace), nb, _stream(dev)))
    return y


def mx_probe_mfma(a, b, iters, blocks, sink):
    """Launches the MFMA throughput probe (mx_probe_mfma) on uint8 code
    tensors a, b (same byte count, a multiple of 4) with a float32 sink of at
    least blocks * 256 elements; returns the FLOP it performs. Time it with
    events on the current stream."""
    dev = a.device
    _need(a, "a", torch.uint8, dev)
    _need(b, "b", torch.uint8, dev)
    _need(sink, "sink", torch.float32, dev)
    if a.numel() != b.numel() or sink.numel() < blocks * 256:
        raise ValueError("a and b must have equal sizes and sink at least blocks * 256 floats")
    with torch.cuda.device(dev):
        _check(lib().mx_probe_mfma(_ptr(a), _ptr(b), a.numel(), int(iters), int(blocks), _ptr(sink), _stream(dev)))
    return float(blocks) * 4 * 16 * iters * 2 * 32 * 32 * 64


def mx_linear_balanced_ws_bytes(M, K, N):
    return lib().mx_linear_balanced_ws_bytes(M, K, N)


def mx_linear_slab_balanced(x, w, bias=None, gelu=False, y=None, workspace=None):
    """mx_linear_slab with the last, partial round of tiles split over K;
    workspace: uint8 of at least mx_linear_balanced_ws_bytes(M, K, N) bytes
    (allocated here when None and needed)."""
    dev, M, N, K = _slab_linear_args(x, w, bias)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    need = mx_linear_balanced_ws_bytes(M, K, N)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear_slab_balanced(
                _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), _ptr(workspace),
                0 if workspace is None else workspace.numel(), _stream(dev),
            )
        )
    return y


class PCSlab(NamedTuple):
    """A per-channel FP8 operand: codes q uint8 [K/64, R, 64] (slab layout)
    and one f32 scale per row s [R], R = mx_slab_rows(rows); pad rows zero."""

    q: torch.Tensor
    s: torch.Tensor
    rows: int

    @property
    def K(self):
        return self.q.shape[0] * 64


def _pc_out(rows, K, dev, out):
    R = mx_slab_rows(rows)
    if out is None:
        return PCSlab(
            torch.empty((K // 64, R, 64), dtype=torch.uint8, device=dev),
            torch.empty((R,), dtype=torch.float32, device=dev),
            rows,
        )
    _need(out.q, "out.q", torch.uint8, dev)
    _need(out.s, "out.s", torch.float32, dev)
    if out.q.shape != (K // 64, R, 64) or out.s.shape != (R,) or out.rows != rows:
        raise ValueError(f"out must hold [{K // 64}, {R}, 64] codes and [{R}] scales for {rows} rows")
    return out


def mx_pc_quantize_act_slab(x, out=None):
    """bf16 [M, K] (rows may be strided, K % 64 == 0) -> PCSlab: per-token
    FP8 codes and f32 row scales (max |x| / 448)."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    if K % 64 != 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    dev = x.device
    out = _pc_out(M, K, dev, out)
    ld = x.stride(0) if M > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_pc_quantize_act_slab(_ptr(x), M, K, ld, _ptr(out.q), _ptr(out.s), _stream(dev)))
    return out


def mx_pc_quantize_weight_slab(w, out=None):
    """fp32 or bf16 [N, K] -> PCSlab: per-output-channel FP8 codes and f32 scales."""
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be 2-D with unit column stride")
    dt = {torch.float32: MX_DT_F32, torch.bfloat16: MX_DT_BF16}.get(w.dtype)
    if dt is None:
        raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
    N, K = w.shape
    if K % 64 != 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    dev = w.device
    out = _pc_out(N, K, dev, out)
    ld = w.stride(0) if N > 1 else K
    with torch.cuda.device(dev):
        _check(lib().mx_pc_quantize_weight_slab(_ptr(w), dt, N, K, ld, _ptr(out.q), _ptr(out.s), _stream(dev)))
    return out


def mx_pc_linear_slab(x, w, bias=None, gelu=False, y=None):
    """y = bf16(epi(xs[m] ws[n] (dec(xq) @ dec(wq)^T) + bias)) on PCSlab operands."""
    dev = x.q.device
    for name, t, dt in (("x.q", x.q, torch.uint8), ("x.s", x.s, torch.float32), ("w.q", w.q, torch.uint8),
                        ("w.s", w.s, torch.float32)):
        _need(t, name, dt, dev)
    M, N, K = x.rows, w.rows, x.K
    if w.K != K:
        raise ValueError(f"x has K = {K}, w has K = {w.K}")
    for name, sl in (("x", x), ("w", w)):
        R = mx_slab_rows(sl.rows)
        if sl.q.shape != (K // 64, R, 64) or sl.s.shape != (R,):
            raise ValueError(f"{name} is not a per-channel slab of {sl.rows} rows and K = {K}")
    if bias is not None:
        _need(bias, "bias", torch.float16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be f16 [N]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_pc_linear_slab(
                _ptr(x.q), _ptr(x.s), M, K, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), _stream(dev)
            )
        )
    return y


def mx_linear_ws_bytes(M, K, N):
    return lib().mx_linear_ws_bytes(M, K, N)


def mx_linear(x, w, bias=None, gelu=False, y=None, workspace=None):
    """The linear in one call (mx.h mx_linear): bf16 x [M, K] (rows may be
    strided) is quantized into `workspace` and multiplied by the slab weights
    w through the shape's plan (tuned or default). workspace: uint8 of at
    least mx_linear_ws_bytes(M, K, N) bytes, allocated here when None."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    dev = x.device
    M, K = x.shape
    _need(w.q, "w.q", torch.uint8, dev)
    _need(w.s, "w.s", torch.uint8, dev)
    if w.K != K:
        raise ValueError(f"x has K = {K}, w has K = {w.K}")
    N = w.rows
    if bias is not None:
        _need(bias, "bias", torch.float16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be f16 [N]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    need = mx_linear_ws_bytes(M, K, N)
    if need < 0:
        raise ValueError("the slab layout needs K % 64 == 0")
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    ld = x.stride(0) if M > 1 else K
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(
            lib().mx_linear(
                _ptr(x), M, K, ld, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y), _ptr(workspace),
                workspace.numel(), _stream(dev),
            )
        )
    return y


def mx_linear_noalloc(x, w, bias=None, gelu=False, y=None):
    """mx_linear with the library's own scratch array as its workspace (mx.h
    mx_linear_noalloc: no workspace argument, nothing allocated by the
    library; calls overlapping on one GPU race). y is allocated here when
    None."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    dev = x.device
    M, K = x.shape
    _need(w.q, "w.q", torch.uint8, dev)
    _need(w.s, "w.s", torch.uint8, dev)
    if w.K != K:
        raise ValueError(f"x has K = {K}, w has K = {w.K}")
    N = w.rows
    if bias is not None:
        _need(bias, "bias", torch.float16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be f16 [N]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    _need(y, "y", torch.bfloat16, dev)
    if y.shape != (M, N):
        raise ValueError("y must be bf16 [M, N]")
    ld = x.stride(0) if M > 1 else K
    epi = MX_EPI_GELU_TANH if gelu else MX_EPI_NONE
    with torch.cuda.device(dev):
        _check(lib().mx_linear_noalloc(_ptr(x), M, K, ld, _ptr(w.q), _ptr(w.s), N, _ptr(bias), epi, _ptr(y),
                                       _stream(dev)))
    return y
