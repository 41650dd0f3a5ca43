"""ctypes binding of the gfx950 QLoRA library (``libqlora_gfx950.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qlora.h``.  PyTorch supplies
device memory (``data_ptr()``) and the stream (``cuda_stream``).  There is no
fallback: if the library is missing, every call raises.
"""

import ctypes
import os
import threading
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlora_gfx950.so")

QLORA_F32, QLORA_BF16 = 0, 1
QLORA_NF4_FP32_CONSTANTS = 1
STATUS_NAMES = {0: "QLORA_OK", 1: "QLORA_ERR_NULL", 2: "QLORA_ERR_SHAPE", 3: "QLORA_ERR_ALIGN",
                4: "QLORA_ERR_WORKSPACE", 5: "QLORA_ERR_DTYPE", 6: "QLORA_ERR_HIP",
                7: "QLORA_ERR_NONFINITE", 8: "QLORA_ERR_VALUE", 9: "QLORA_ERR_MEMORY", 10: "QLORA_ERR_SCRATCH"}


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class NF4WeightStruct(ctypes.Structure):
    _fields_ = [("n_out", ctypes.c_int64), ("n_in", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("absmax_fp8", ctypes.c_void_p), ("absmax_scale", ctypes.c_void_p),
                ("absmax_mean", ctypes.c_void_p), ("flags", ctypes.c_uint32)]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "qlora_nf4_sizes": (ctypes.c_int, [_I64, _I64, _P, _P, _P]),
    "qlora_nf4_bytes": (_SZ, [_I64, _I64]),
    "qlora_nf4_bytes_flags": (_SZ, [_I64, _I64, ctypes.c_uint32]),
    "qlora_quantize_workspace_bytes": (_SZ, [_I64, _I64]),
    "qlora_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64, ctypes.c_int]),
    "qlora_nf4_codebook": (None, [_P]),
    "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qlora_version": (ctypes.c_char_p, []),
    "qlora_quantize": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, _SZ, _P]),
    "qlora_dequantize": (ctypes.c_int, [_P, _P, _P]),
    "qlora_dequantize_many": (ctypes.c_int, [_P, ctypes.c_int, _P, _P]),
    "qlora_linear_fwd": (ctypes.c_int, [_P, _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "qlora_linear_bwd": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _P, _P,
                                        _P, _SZ, _P]),
    "qlora_linear_fwd_noalloc_max_bytes": (_SZ, []),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_P, _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _P]),
    "qlora_linear_set_workspace_bytes": (_SZ, [_I64, ctypes.c_int, _P, _I64, ctypes.c_int]),
    "qlora_linear_set_fwd": (ctypes.c_int, [_P, _I64, ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P,
                                            _P, _SZ, _P]),
    "qlora_linear_set_bwd": (ctypes.c_int, [_P, _P, _I64, ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_float,
                                            _P, _P, _P, _P, _P, _SZ, _P]),
    "qlora_linear_dropout_workspace_bytes": (_SZ, [_I64, _I64, _I64, ctypes.c_int]),
    "qlora_linear_fwd_dropout": (ctypes.c_int, [_P, _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                                ctypes.c_uint64, _P, _P, _P, _SZ, _P]),
    "qlora_linear_bwd_dropout": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P, ctypes.c_int, ctypes.c_float,
                                                ctypes.c_double, ctypes.c_uint64, _P, _P, _P, _P, _P, _SZ, _P]),
    "qlora_dropout_mask": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_double, ctypes.c_uint64, _P, _P, _P]),
    "qlora_adamw_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_double, _P]),
    "qlora_status_read": (ctypes.c_int, [_P, _P]),
    "qlora_kernel_timing_enable": (None, [ctypes.c_int]),
    "qlora_kernel_timing_read": (ctypes.c_int, [_P, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_finetuning_quant_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QloraError(status, where)


# ---------------------------------------------------------------- host helpers
def status_string(status: int) -> str:
    return lib().qlora_status_string(int(status)).decode()


def version() -> str:
    return lib().qlora_version().decode()


def nf4_sizes(n_out: int, n_in: int):
    cb, nb, ng = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().qlora_nf4_sizes(n_out, n_in, ctypes.byref(cb), ctypes.byref(nb), ctypes.byref(ng)), "nf4_sizes")
    return cb.value, nb.value, ng.value


def nf4_bytes(n_out: int, n_in: int, double_quant: bool = True) -> int:
    if double_quant:
        return int(lib().qlora_nf4_bytes(n_out, n_in))
    return int(lib().qlora_nf4_bytes_flags(n_out, n_in, QLORA_NF4_FP32_CONSTANTS))


def quantize_workspace_bytes(n_out: int, n_in: int) -> int:
    return int(lib().qlora_quantize_workspace_bytes(n_out, n_in))


def linear_workspace_bytes(tokens: int, n_out: int, n_in: int, r: int) -> int:
    return int(lib().qlora_linear_workspace_bytes(tokens, n_out, n_in, r))


TIMED_KINDS = ("qgemm_fwd", "qgemm_dx", "gemv_fwd", "gemv_bwd", "adamw")


def kernel_timing_enable(on: bool) -> None:
    """Bracket every main-kernel launch with HIP events on its stream (diagnostics)."""
    lib().qlora_kernel_timing_enable(1 if on else 0)


def kernel_timing_read():
    """-> {kind: (launches, total ms)} for the launches timed so far (then cleared)."""
    n = (ctypes.c_int64 * len(TIMED_KINDS))()
    ms = (ctypes.c_double * len(TIMED_KINDS))()
    _check(lib().qlora_kernel_timing_read(n, ms), "kernel_timing_read")
    return {k: (n[i], ms[i]) for i, k in enumerate(TIMED_KINDS)}


def nf4_codebook():
    buf = (ctypes.c_float * 16)()
    lib().qlora_nf4_codebook(buf)
    return list(buf)


# ------------------------------------------------------------- device helpers
def _torch():
    import torch

    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


# The C ABI takes plain pointers and cannot check the extent of a buffer, so every tensor is
# checked here before a call: dtype, contiguity, exact shape, and the device of the packed
# weight.  A wrong tensor raises ValueError and nothing is launched.
_DT = {}  # dtype sets of the checks, filled on first use (torch is imported lazily)


def _dtypes():
    if not _DT:
        torch = _torch()
        _DT.update(tensor=torch.Tensor, bf16=(torch.bfloat16, torch.int16), f32=(torch.float32,))
    return _DT


_TRUST = threading.local()


class trusted_calls:
    """Context manager: inside it the calls of this thread skip the per-tensor checks below (about
    1 us of host time per tensor, which is most of a few-token step's launch cost).  For loops that
    repeat calls on tensors already checked once (the same shapes, dtypes and device)."""

    def __enter__(self):
        self.prev = getattr(_TRUST, "on", False)
        _TRUST.on = True
        return self

    def __exit__(self, *exc):
        _TRUST.on = self.prev
        return False


class _NoChecks:
    __slots__ = ()

    def bf16(self, t, name, shape):
        pass

    def f32(self, t, name, shape):
        pass

    def done(self):
        pass


_NO_CHECKS = _NoChecks()


class _Args:
    """Checks of one call's tensors: dtype, exact shape and contiguity as each is named, then
    (done) that every one of them is on the packed weight's CUDA device."""

    __slots__ = ("device", "named")

    def __new__(cls, device):
        if getattr(_TRUST, "on", False):
            return _NO_CHECKS
        return super().__new__(cls)

    def __init__(self, device):
        self.device = device
        self.named = []

    def _check(self, t, name: str, shape, kind: str) -> None:
        dt = _dtypes()
        if not isinstance(t, dt["tensor"]):
            raise ValueError(f"{name} must be a tensor")
        if t.dtype not in dt[kind]:
            raise ValueError(f"{name} must be {' or '.join(str(d) for d in dt[kind])}, not {t.dtype}")
        if t.shape != shape:
            raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.named.append((name, t))

    def bf16(self, t, name: str, shape) -> None:
        self._check(t, name, shape, "bf16")

    def f32(self, t, name: str, shape) -> None:
        self._check(t, name, shape, "f32")

    def done(self) -> None:
        dev = self.device
        for name, t in self.named:
            if t.device != dev or dev.type != "cuda":
                raise ValueError(f"{name} must be on {dev}, not {t.device}")


def _workspace(ws, device, need) -> int:
    """Checks a caller's workspace (a contiguous uint8 CUDA tensor of at least need() bytes)."""
    if getattr(_TRUST, "on", False):
        return ws.numel()
    torch = _torch()
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.device.type != "cuda" or ws.device != device:
        raise ValueError(f"workspace must be on {device}, not {ws.device}")
    need = need()
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")
    return ws.numel()


def _weight_device(q) -> "object":
    """The device of a packed weight (every call's tensors must be on it)."""
    dev = q.codes.device
    if dev.type != "cuda":
        raise ValueError(f"the packed weight must be on a CUDA device, not {dev}")
    return dev


@dataclass
class NF4Weight:
    """Device buffers of a packed weight (allocated by torch, owned by this object).

    double_quant=False: absmax_scale holds the nblocks fp32 block constants and
    absmax_fp8 / absmax_mean are None (QLORA_NF4_FP32_CONSTANTS)."""
    n_out: int
    n_in: int
    codes: "object"
    absmax_fp8: "object"
    absmax_scale: "object"
    absmax_mean: "object"
    double_quant: bool = True

    @classmethod
    def empty(cls, n_out: int, n_in: int, device="cuda", double_quant: bool = True):
        torch = _torch()
        cb, nb, ng = nf4_sizes(n_out, n_in)
        codes = torch.empty(cb, dtype=torch.uint8, device=device)
        if not double_quant:
            return cls(n_out, n_in, codes, None, torch.empty(nb, dtype=torch.float32, device=device), None, False)
        return cls(n_out, n_in, codes, torch.empty(nb, dtype=torch.uint8, device=device),
                   torch.empty(ng, dtype=torch.float32, device=device),
                   torch.empty(1, dtype=torch.float32, device=device))

    def struct(self) -> NF4WeightStruct:
        return NF4WeightStruct(self.n_out, self.n_in, _ptr(self.codes), _ptr(self.absmax_fp8),
                               _ptr(self.absmax_scale), _ptr(self.absmax_mean),
                               0 if self.double_quant else QLORA_NF4_FP32_CONSTANTS)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.codes, self.absmax_fp8, self.absmax_scale, self.absmax_mean) if t is not None)


def _bits(t):
    """bf16 tensor -> the same memory viewed as int16 (no copy)."""
    torch = _torch()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def quantize(w, out: NF4Weight = None, workspace=None, stream=None, double_quant: bool = True) -> NF4Weight:
    """Quantize a [n_out x n_in] fp32 or bf16 CUDA tensor to NF4 + FP8 double quantization
    (double_quant=False: NF4 + fp32 block constants; ignored when `out` is given, whose
    storage form decides)."""
    torch = _torch()
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    dtype = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}.get(w.dtype)
    if dtype is None:
        raise ValueError("w must be float32 or bfloat16")
    n_out, n_in = w.shape
    if w.device.type != "cuda":
        raise ValueError(f"w must be on a CUDA device, not {w.device}")
    q = out if out is not None else NF4Weight.empty(n_out, n_in, w.device, double_quant=double_quant)
    if (q.n_out, q.n_in) != (n_out, n_in) or _weight_device(q) != w.device:
        raise ValueError("out must be a packed weight of w's shape on w's device")
    wsb = quantize_workspace_bytes(n_out, n_in)
    ws = workspace if workspace is not None else torch.empty(wsb, dtype=torch.uint8, device=w.device)
    wsn = _workspace(ws, w.device, lambda: wsb)
    st = q.struct()
    _check(lib().qlora_quantize(_ptr(w), dtype, ctypes.byref(st), _ptr(ws), wsn, _stream(stream)), "qlora_quantize")
    q.last_workspace = ws
    return q


def status_read(workspace, stream=None) -> int:
    """Synchronise and return the status word a call left in `workspace` (0 = ok)."""
    return int(lib().qlora_status_read(_ptr(workspace), _stream(stream)))


def dequantize(q: NF4Weight, out=None, stream=None):
    torch = _torch()
    dev = _weight_device(q)
    y = out if out is not None else torch.empty((q.n_out, q.n_in), dtype=torch.bfloat16, device=dev)
    chk = _Args(dev)
    chk.bf16(y, "out", (q.n_out, q.n_in))
    chk.done()
    st = q.struct()
    _check(lib().qlora_dequantize(ctypes.byref(st), _ptr(y), _stream(stream)), "qlora_dequantize")
    return y


def dequantize_many(qs, outs=None, stream=None):
    """Decode several packed weights (up to 8) in one launch; returns the bf16 tensors."""
    torch = _torch()
    outs = outs if outs is not None else [torch.empty((q.n_out, q.n_in), dtype=torch.bfloat16, device=q.codes.device)
                                          for q in qs]
    _check_list(outs, len(qs), "outs")
    for i, (q, o) in enumerate(zip(qs, outs)):
        chk = _Args(_weight_device(q))
        chk.bf16(o, f"outs[{i}]", (q.n_out, q.n_in))
        chk.done()
    st = (NF4WeightStruct * len(qs))(*[q.struct() for q in qs])
    ptrs = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    _check(lib().qlora_dequantize_many(st, len(qs), ptrs, _stream(stream)), "qlora_dequantize_many")
    return outs


def linear_workspace(tokens: int, n_out: int, n_in: int, r: int, device="cuda"):
    """A workspace for the linear calls (reusable by successive calls on one stream)."""
    torch = _torch()
    return torch.empty(max(linear_workspace_bytes(tokens, n_out, n_in, r), 1), dtype=torch.uint8, device=device)


def linear_fwd(x, q: NF4Weight, A, B, scale: float, y=None, u_out=None, save_u=True, workspace=None,
               stream=None):
    """y = x W_hat^T + scale (x A^T) B^T (bf16); returns (y, u or None)."""
    torch = _torch()
    T, r = _linear_dims(x, A, q)
    dev = _weight_device(q)
    chk = _Args(dev)
    chk.bf16(x, "x", (T, q.n_in))
    chk.bf16(A, "A", (r, q.n_in))
    chk.bf16(B, "B", (q.n_out, r))
    y = y if y is not None else torch.empty((T, q.n_out), dtype=torch.bfloat16, device=dev)
    chk.bf16(y, "y", (T, q.n_out))
    if save_u and u_out is None:
        u_out = torch.empty((T, r), dtype=torch.bfloat16, device=dev)
    if u_out is not None:
        chk.bf16(u_out, "u_out", (T, r))
    chk.done()
    ws = workspace if workspace is not None else linear_workspace(T, q.n_out, q.n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_workspace_bytes(T, q.n_out, q.n_in, r))
    st = q.struct()
    _check(lib().qlora_linear_fwd(_ptr(x), T, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), _ptr(y),
                                  _ptr(u_out), _ptr(ws), wsb, _stream(stream)), "qlora_linear_fwd")
    return y, u_out


def linear_fwd_noalloc(x, q: NF4Weight, A, B, scale: float, y, u_out=None, stream=None):
    """linear_fwd on the library's fixed per-GPU scratch array instead of a workspace (for callers
    that cannot allocate): y (and u_out, if given) are the caller's; nothing is allocated here.
    Calls that may overlap in time on one GPU share the array and must be ordered."""
    T, r = _linear_dims(x, A, q)
    dev = _weight_device(q)
    chk = _Args(dev)
    chk.bf16(x, "x", (T, q.n_in))
    chk.bf16(A, "A", (r, q.n_in))
    chk.bf16(B, "B", (q.n_out, r))
    chk.bf16(y, "y", (T, q.n_out))
    if u_out is not None:
        chk.bf16(u_out, "u_out", (T, r))
    chk.done()
    st = q.struct()
    _check(lib().qlora_linear_fwd_noalloc(_ptr(x), T, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), _ptr(y),
                                          _ptr(u_out), _stream(stream)), "qlora_linear_fwd_noalloc")
    return y, u_out


def linear_fwd_noalloc_max_bytes() -> int:
    return int(lib().qlora_linear_fwd_noalloc_max_bytes())


def _linear_dims(x, A, q):
    """(T, r) of a linear call from x [T x n_in] and A [r x n_in]."""
    if x.dim() != 2 or A.dim() != 2:
        raise ValueError("x and A must be 2-D")
    return int(x.shape[0]), int(A.shape[0])


def _check_bwd(dy, x, q, A, B, u, chk):
    T, r = _linear_dims(x, A, q)
    chk.bf16(dy, "dy", (T, q.n_out))
    chk.bf16(x, "x", (T, q.n_in))
    chk.bf16(A, "A", (r, q.n_in))
    chk.bf16(B, "B", (q.n_out, r))
    if u is not None:
        chk.bf16(u, "u", (T, r))
    return T, r


def _check_grads(grad_x, grad_A, grad_B, T, r, q, chk):
    if grad_x is not None:
        chk.bf16(grad_x, "grad_x", (T, q.n_in))
    chk.f32(grad_A, "grad_A", (r, q.n_in))
    chk.f32(grad_B, "grad_B", (q.n_out, r))
    chk.done()


def linear_bwd(dy, x, q: NF4Weight, A, B, scale: float, u=None, need_grad_x=True, grad_x=None, grad_A=None,
               grad_B=None, workspace=None, stream=None):
    """Returns (grad_x bf16 or None, grad_A fp32, grad_B fp32)."""
    torch = _torch()
    dev = _weight_device(q)
    chk = _Args(dev)
    T, r = _check_bwd(dy, x, q, A, B, u, chk)
    if need_grad_x and grad_x is None:
        grad_x = torch.empty((T, q.n_in), dtype=torch.bfloat16, device=dev)
    if not need_grad_x:
        grad_x = None
    grad_A = grad_A if grad_A is not None else torch.empty((r, q.n_in), dtype=torch.float32, device=dev)
    grad_B = grad_B if grad_B is not None else torch.empty((q.n_out, r), dtype=torch.float32, device=dev)
    _check_grads(grad_x, grad_A, grad_B, T, r, q, chk)
    ws = workspace if workspace is not None else linear_workspace(T, q.n_out, q.n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_workspace_bytes(T, q.n_out, q.n_in, r))
    st = q.struct()
    _check(lib().qlora_linear_bwd(_ptr(dy), _ptr(x), T, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale),
                                  _ptr(u), _ptr(grad_x), _ptr(grad_A), _ptr(grad_B), _ptr(ws), wsb,
                                  _stream(stream)), "qlora_linear_bwd")
    return grad_x, grad_A, grad_B


def adamw_step(param, param_bf16, grad, exp_avg, exp_avg_sq, step: int, lr: float, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0, stream=None) -> None:
    """One AdamW update of a flat fp32 adapter buffer, in place (see qlora_adamw_step).

    param, grad, exp_avg, exp_avg_sq: contiguous float32 tensors of n elements;
    param_bf16: bfloat16 (or int16) tensor of n elements.  The states may be
    pinned host tensors (``pin_memory=True``): the kernel reads them in place.
    """
    torch = _torch()
    n = param.numel()
    for name, t, dt in (("param", param, torch.float32), ("grad", grad, torch.float32),
                        ("exp_avg", exp_avg, torch.float32), ("exp_avg_sq", exp_avg_sq, torch.float32)):
        if t.dtype != dt or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    if param_bf16.dtype not in (torch.bfloat16, torch.int16) or not param_bf16.is_contiguous() \
            or param_bf16.numel() != n:
        raise ValueError(f"param_bf16 must be a contiguous bfloat16 tensor of {n} elements")
    _check(lib().qlora_adamw_step(_ptr(param), _ptr(param_bf16), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n,
                                  int(step), float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                                  _stream(stream)), "qlora_adamw_step")


# ------------------------------------------------------------------ LoRA dropout
def linear_dropout_workspace_bytes(tokens: int, n_out: int, n_in: int, r: int) -> int:
    return int(lib().qlora_linear_dropout_workspace_bytes(tokens, n_out, n_in, r))


def linear_dropout_workspace(tokens: int, n_out: int, n_in: int, r: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(linear_dropout_workspace_bytes(tokens, n_out, n_in, r), 1), dtype=torch.uint8,
                       device=device)


def linear_fwd_dropout(x, q: NF4Weight, A, B, scale: float, p: float, seed: int, y=None, u_out=None, save_u=True,
                       workspace=None, stream=None):
    """linear_fwd with LoRA dropout of probability p on the adapter input (mask from seed)."""
    torch = _torch()
    T, r = _linear_dims(x, A, q)
    dev = _weight_device(q)
    chk = _Args(dev)
    chk.bf16(x, "x", (T, q.n_in))
    chk.bf16(A, "A", (r, q.n_in))
    chk.bf16(B, "B", (q.n_out, r))
    y = y if y is not None else torch.empty((T, q.n_out), dtype=torch.bfloat16, device=dev)
    chk.bf16(y, "y", (T, q.n_out))
    if save_u and u_out is None:
        u_out = torch.empty((T, r), dtype=torch.bfloat16, device=dev)
    if u_out is not None:
        chk.bf16(u_out, "u_out", (T, r))
    chk.done()
    ws = workspace if workspace is not None else linear_dropout_workspace(T, q.n_out, q.n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_dropout_workspace_bytes(T, q.n_out, q.n_in, r))
    st = q.struct()
    _check(lib().qlora_linear_fwd_dropout(_ptr(x), T, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), float(p),
                                          int(seed), _ptr(y), _ptr(u_out), _ptr(ws), wsb, _stream(stream)),
           "qlora_linear_fwd_dropout")
    return y, u_out


def linear_bwd_dropout(dy, x, q: NF4Weight, A, B, scale: float, p: float, seed: int, u=None, need_grad_x=True,
                       grad_x=None, grad_A=None, grad_B=None, workspace=None, stream=None):
    """linear_bwd with the forward's dropout mask (same p and seed)."""
    torch = _torch()
    dev = _weight_device(q)
    chk = _Args(dev)
    T, r = _check_bwd(dy, x, q, A, B, u, chk)
    if need_grad_x and grad_x is None:
        grad_x = torch.empty((T, q.n_in), dtype=torch.bfloat16, device=dev)
    if not need_grad_x:
        grad_x = None
    grad_A = grad_A if grad_A is not None else torch.empty((r, q.n_in), dtype=torch.float32, device=dev)
    grad_B = grad_B if grad_B is not None else torch.empty((q.n_out, r), dtype=torch.float32, device=dev)
    _check_grads(grad_x, grad_A, grad_B, T, r, q, chk)
    ws = workspace if workspace is not None else linear_dropout_workspace(T, q.n_out, q.n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_dropout_workspace_bytes(T, q.n_out, q.n_in, r))
    st = q.struct()
    _check(lib().qlora_linear_bwd_dropout(_ptr(dy), _ptr(x), T, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale),
                                          float(p), int(seed), _ptr(u), _ptr(grad_x), _ptr(grad_A), _ptr(grad_B),
                                          _ptr(ws), wsb, _stream(stream)), "qlora_linear_bwd_dropout")
    return grad_x, grad_A, grad_B


def dropout_mask(x, p: float, seed: int, stream=None):
    """(keep_words [ceil(T/32) x K] int32, x_drop [T x K] bf16) for a [T x K] bf16 tensor."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    T, K = x.shape
    chk = _Args(x.device)
    chk.bf16(x, "x", (T, K))
    chk.done()
    keep = torch.empty(((T + 31) // 32, K), dtype=torch.int32, device=x.device)
    xd = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    _check(lib().qlora_dropout_mask(_ptr(x), T, K, float(p), int(seed), _ptr(keep), _ptr(xd), _stream(stream)),
           "qlora_dropout_mask")
    return keep, xd


# ------------------------------------------------------------ projection sets
def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


def linear_set_workspace_bytes(tokens: int, n_outs, n_in: int, r: int) -> int:
    arr = (ctypes.c_int64 * len(n_outs))(*n_outs)
    return int(lib().qlora_linear_set_workspace_bytes(tokens, len(n_outs), arr, n_in, r))


def linear_set_workspace(tokens: int, n_outs, n_in: int, r: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(linear_set_workspace_bytes(tokens, n_outs, n_in, r), 1), dtype=torch.uint8, device=device)


def linear_set_fwd(x, qs, A_set, Bs, scale: float, ys=None, u_out=None, save_u=True, workspace=None, stream=None):
    """Projection set forward: y_i = x W_hat_i^T + scale (x A_i^T) B_i^T for every member, with
    A_set [count r x n_in] the members' A matrices back to back.  Returns (ys, u_set or None)."""
    torch = _torch()
    T, count, r, dev, chk = _set_dims(x, qs, A_set)
    _check_list(Bs, count, "Bs")
    for i, (q, b) in enumerate(zip(qs, Bs)):
        chk.bf16(b, f"Bs[{i}]", (q.n_out, r))
    ys = ys if ys is not None else [torch.empty((T, q.n_out), dtype=torch.bfloat16, device=dev) for q in qs]
    _check_list(ys, count, "ys")
    for i, (q, y) in enumerate(zip(qs, ys)):
        chk.bf16(y, f"ys[{i}]", (T, q.n_out))
    if save_u and u_out is None:
        u_out = torch.empty((T, count * r), dtype=torch.bfloat16, device=dev)
    if u_out is not None:
        chk.bf16(u_out, "u_out", (T, count * r))
    chk.done()
    n_outs = [q.n_out for q in qs]
    ws = workspace if workspace is not None else linear_set_workspace(T, n_outs, qs[0].n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_set_workspace_bytes(T, n_outs, qs[0].n_in, r))
    st = (NF4WeightStruct * count)(*[q.struct() for q in qs])
    _check(lib().qlora_linear_set_fwd(_ptr(x), T, count, st, _ptr(A_set), _ptrs(Bs), r, float(scale), _ptrs(ys),
                                      _ptr(u_out), _ptr(ws), wsb, _stream(stream)), "qlora_linear_set_fwd")
    return ys, u_out


def _check_list(ts, count: int, name: str) -> None:
    if len(ts) != count:
        raise ValueError(f"{name} must hold {count} tensors, not {len(ts)}")


def _set_dims(x, qs, A_set):
    """(T, count, r, device, checker) of a projection-set call; A_set must hold count whole [r x n_in] blocks."""
    count = len(qs)
    if count < 1:
        raise ValueError("a projection set needs at least one member")
    dev = _weight_device(qs[0])
    for i, q in enumerate(qs):
        if q.n_in != qs[0].n_in:
            raise ValueError(f"member {i} has n_in {q.n_in}, member 0 has {qs[0].n_in}")
        if _weight_device(q) != dev:
            raise ValueError(f"member {i} is on {q.codes.device}, member 0 on {dev}")
    if x.dim() != 2 or A_set.dim() != 2:
        raise ValueError("x and A_set must be 2-D")
    if A_set.shape[0] % count:
        raise ValueError(f"A_set has {A_set.shape[0]} rows, not a multiple of the {count} members")
    T, r = int(x.shape[0]), int(A_set.shape[0]) // count
    chk = _Args(dev)
    chk.bf16(x, "x", (T, qs[0].n_in))
    chk.bf16(A_set, "A_set", (count * r, qs[0].n_in))
    return T, count, r, dev, chk


def linear_set_bwd(dys, x, qs, A_set, Bs, scale: float, u=None, need_grad_x=True, grad_x=None, grad_A_set=None,
                   grad_Bs=None, workspace=None, stream=None):
    """Projection set backward: (grad_x summed over the members or None, grad_A_set, [grad_B_i])."""
    torch = _torch()
    T, count, r, dev, chk = _set_dims(x, qs, A_set)
    _check_list(dys, count, "dys")
    _check_list(Bs, count, "Bs")
    for i, (q, d, b) in enumerate(zip(qs, dys, Bs)):
        chk.bf16(d, f"dys[{i}]", (T, q.n_out))
        chk.bf16(b, f"Bs[{i}]", (q.n_out, r))
    if u is not None:
        chk.bf16(u, "u", (T, count * r))
    if need_grad_x and grad_x is None:
        grad_x = torch.empty((T, qs[0].n_in), dtype=torch.bfloat16, device=dev)
    if not need_grad_x:
        grad_x = None
    if grad_x is not None:
        chk.bf16(grad_x, "grad_x", (T, qs[0].n_in))
    grad_A_set = grad_A_set if grad_A_set is not None else torch.empty((count * r, qs[0].n_in), dtype=torch.float32,
                                                                       device=dev)
    chk.f32(grad_A_set, "grad_A_set", (count * r, qs[0].n_in))
    grad_Bs = grad_Bs if grad_Bs is not None else [torch.empty((q.n_out, r), dtype=torch.float32, device=dev)
                                                   for q in qs]
    _check_list(grad_Bs, count, "grad_Bs")
    for i, (q, g) in enumerate(zip(qs, grad_Bs)):
        chk.f32(g, f"grad_Bs[{i}]", (q.n_out, r))
    chk.done()
    n_outs = [q.n_out for q in qs]
    ws = workspace if workspace is not None else linear_set_workspace(T, n_outs, qs[0].n_in, r, dev)
    wsb = _workspace(ws, dev, lambda: linear_set_workspace_bytes(T, n_outs, qs[0].n_in, r))
    st = (NF4WeightStruct * count)(*[q.struct() for q in qs])
    _check(lib().qlora_linear_set_bwd(_ptrs(dys), _ptr(x), T, count, st, _ptr(A_set), _ptrs(Bs), r, float(scale),
                                      _ptr(u), _ptr(grad_x), _ptr(grad_A_set), _ptrs(grad_Bs), _ptr(ws), wsb,
                                      _stream(stream)), "qlora_linear_set_bwd")
    return grad_x, grad_A_set, grad_Bs
