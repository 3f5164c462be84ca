"""Thin ctypes binding over libqat.so (the HIP kernels + C ABI in include/qat.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current HIP stream. If the library is
not built, importing the functions raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqat.so")

QAT_OK = 0
GROUP = 64

_c_i32, _c_i64, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> argument types (all pointers as void*)
_SIGS = {
    "qat_init_minmax": [_c_vp, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp],
    "qat_quant_codes": [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp],
    "qat_fakequant_linear_fwd": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                 _c_vp, _c_vp, _c_sz, _c_vp],
    "qat_fakequant_linear_bwd": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32,
                                 _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp],
    "qat_pack": [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp],
    "qat_dequant_gemm_fwd": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                             _c_vp, _c_vp, _c_sz, _c_vp],
    "qat_dequant_gemm_bwd_s": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32,
                               _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp],
    "qat_fakequant_linear_bwd_saved": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                       _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp],
    "qat_dequant_gemm_bwd_s_saved": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64,
                                     _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp],
    "qat_deploy_zq_stride": [_c_i64, _c_i32, _c_i32],
    "qat_deploy_qparams": [_c_vp, _c_vp, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp],
    "qat_deploy_gemv": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp],
    "qat_fakequant_ws_bytes": [_c_i64, _c_i64, _c_i32],
    "qat_dequant_ws_bytes": [_c_i64, _c_i64, _c_i32],
    "qat_timing_enable": [_c_i32],
    "qat_timing_count": [],
    "qat_timing_select": [ctypes.c_char_p],
    "qat_timing_get": [_c_i32, ctypes.c_char_p, _c_sz, ctypes.POINTER(ctypes.c_double),
                       ctypes.POINTER(_c_i64)],
    "qat_peak_mfma_flops": [_c_i32, _c_i32],
    "qat_peak_scratch_bytes": [_c_i32],
    "qat_peak_mfma": [_c_i32, _c_i32, _c_vp, _c_vp],
    "qat_peak_read": [_c_vp, _c_sz, _c_i32, _c_vp, _c_vp],
    "qat_peak_write": [_c_vp, _c_sz, _c_i32, _c_vp],
    "qat_fakequant_linear_fwd_noalloc": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32,
                                         _c_vp, _c_vp],
    "qat_noalloc_max_weights": [],
    "qat_status_string": [_c_i32],
    "qat_last_error": [],
}
_RES = {"qat_deploy_zq_stride": _c_i64, "qat_noalloc_max_weights": _c_i64, "qat_fakequant_ws_bytes": _c_sz, "qat_dequant_ws_bytes": _c_sz, "qat_peak_mfma_flops": _c_i64,
        "qat_peak_scratch_bytes": _c_sz,
        "qat_status_string": ctypes.c_char_p, "qat_last_error": ctypes.c_char_p}

# include/qat_block.h
BLOCK_LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
_LIN_FIELDS = ("W", "s", "z", "dW", "ds", "dz", "m_W", "v_W", "m_s", "v_s", "m_z", "v_z")


class BlockShape(ctypes.Structure):
    _fields_ = [("hidden", _c_i64), ("heads", _c_i64), ("inter", _c_i64), ("seq", _c_i64),
                ("batch", _c_i64), ("bits", _c_i32), ("group", _c_i32)]


class BlockLinear(ctypes.Structure):
    _fields_ = [(f, _c_vp) for f in _LIN_FIELDS]


class BlockAdamW(ctypes.Structure):
    _fields_ = [("lr_weight", ctypes.c_double), ("lr_quant", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", _c_i64), ("total_steps", _c_i64)]


_SIGS.update({
    "qat_block_ws_bytes": [ctypes.POINTER(BlockShape)],
    "qat_block_forward": [ctypes.POINTER(BlockShape), ctypes.POINTER(BlockLinear), _c_vp, _c_vp, _c_vp, _c_vp,
                          _c_vp, _c_vp, _c_vp, _c_sz, _c_vp],
    "qat_block_ap_step": [ctypes.POINTER(BlockShape), ctypes.POINTER(BlockLinear), _c_vp, _c_vp, _c_vp, _c_vp,
                          ctypes.POINTER(BlockAdamW), _c_vp, _c_vp, _c_vp, _c_sz, _c_vp],
})
_RES["qat_block_ws_bytes"] = _c_sz

_lib = None


def lib() -> ctypes.CDLL:
    """Load libqat.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m weight_quantization_aware_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = _RES.get(name, _c_i32)
        _lib = h
    return _lib


class QatError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.qat_status_string(status).decode()
        if status == 7:
            msg += ": " + L.qat_last_error().decode()
        super().__init__(f"{fn} -> {status} ({msg})")
        self.status = status


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != QAT_OK:
        raise QatError(name, st)


# ---------------------------------------------------------------------------
# Argument checks. The C ABI sees raw pointers and sizes only, so every
# wrapper checks here, before the call, that each tensor has the dtype and the
# exact shape the sizes imply, is contiguous, and lives on the same GPU as the
# first tensor of the call (dtype and shape are checked first, so the checks
# also run on a host without a GPU).
# ---------------------------------------------------------------------------

F32 = (torch.float32,)
U8 = (torch.uint8,)
BF16 = (torch.bfloat16, torch.int16, torch.uint16)   # bf16, or its 16-bit patterns
F16 = (torch.float16, torch.int16, torch.uint16)     # fp16, or its 16-bit patterns


class _Args:
    """Collects the tensors of one call; every tensor must sit on one CUDA device."""

    def __init__(self, fn: str):
        self.fn = fn
        self.seen = []

    def t(self, name: str, t, dtypes, shape=None, optional: bool = False, min_bytes: Optional[int] = None):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.fn}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError(f"{self.fn}: {name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
            raise ValueError(f"{self.fn}: {name} holds {t.numel() * t.element_size()} bytes, "
                             f"needs at least {min_bytes}")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous")
        self.seen.append((name, t))
        return t.data_ptr()

    def done(self) -> None:
        """After every tensor's dtype and shape: all on one CUDA (HIP) device."""
        dev = None
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{self.fn}: {name} must be a CUDA (HIP) device tensor, got {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.fn}: {name} is on {t.device}, the call's other tensors on {dev}")


def _dims2(fn: str, name: str, t, what: str):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{fn}: {name} must be a 2-D tensor ({what})")
    return int(t.shape[0]), int(t.shape[1])


def _groups(fn: str, inp: int, group: int) -> int:
    if group <= 0 or inp % group != 0:
        raise ValueError(f"{fn}: group {group} must divide in = {inp}")
    return inp // group


def _packed_cols(fn: str, inp: int, bits: int) -> int:
    if bits not in (2, 3, 4):
        raise ValueError(f"{fn}: bits must be 2, 3 or 4, got {bits}")
    return inp * bits // 8


def _ws(a: _Args, ws, need: int):
    """A workspace: any contiguous device tensor of at least `need` bytes."""
    if ws is None:
        return None, 0
    p = a.t("ws", ws, None, min_bytes=need)
    return p, ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# Workspace size queries
# ---------------------------------------------------------------------------

def fakequant_ws_bytes(out: int, inp: int, bits: int) -> int:
    return int(lib().qat_fakequant_ws_bytes(out, inp, bits))


def dequant_ws_bytes(out: int, inp: int, bits: int) -> int:
    return int(lib().qat_dequant_ws_bytes(out, inp, bits))


def workspace(nbytes: int, device=None) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------------------
# The C-ABI calls, same names as in include/qat.h
# ---------------------------------------------------------------------------

def qat_init_minmax(W: torch.Tensor, bits: int, s: torch.Tensor, z: torch.Tensor, group: int = GROUP) -> None:
    fn = "qat_init_minmax"
    out, inp = _dims2(fn, "W", W, "[out, in]")
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("W", W, F32), out, inp, group, bits, a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)))
    a.done()
    _call(fn, *args, _stream())


def qat_quant_codes(W, s, z, bits, codes=None, W_hat=None, group: int = GROUP) -> None:
    fn = "qat_quant_codes"
    out, inp = _dims2(fn, "W", W, "[out, in]")
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("W", W, F32), a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), out, inp, group, bits,
            a.t("codes", codes, U8, (out, inp), optional=True), a.t("W_hat", W_hat, BF16, (out, inp), optional=True))
    a.done()
    _call(fn, *args, _stream())


def qat_fakequant_linear_fwd(X, W, s, z, bits, Y, ws=None, group: int = GROUP) -> None:
    fn = "qat_fakequant_linear_fwd"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "W", W, "[out, in]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("X", X, BF16), a.t("W", W, F32, (out, inp)), a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)),
            M, out, inp, group, bits, a.t("Y", Y, BF16, (M, out)))
    a.done()
    _call(fn, *args, *_ws(a, ws, fakequant_ws_bytes(out, inp, bits)), _stream())


def noalloc_max_weights() -> int:
    return int(lib().qat_noalloc_max_weights())


def qat_fakequant_linear_fwd_noalloc(X, W, s, z, bits, Y, group: int = GROUP) -> None:
    """The staged forward with W_hat in the library's static device scratch
    (allocates nothing; out * in <= noalloc_max_weights())."""
    fn = "qat_fakequant_linear_fwd_noalloc"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "W", W, "[out, in]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("X", X, BF16), a.t("W", W, F32, (out, inp)), a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)),
            M, out, inp, group, bits, a.t("Y", Y, BF16, (M, out)))
    a.done()
    _call(fn, *args, _stream())


def qat_fakequant_linear_bwd(dY, X, W, s, z, bits, dX=None, dW=None, ds=None, dz=None, ws=None,
                             group: int = GROUP) -> None:
    """ws None: W_hat is recomputed from W, s, z inside the dX GEMM (no workspace)."""
    fn = "qat_fakequant_linear_bwd"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "W", W, "[out, in]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("dY", dY, BF16, (M, out)), a.t("X", X, BF16), a.t("W", W, F32, (out, inp)),
            a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), M, out, inp, group, bits,
            a.t("dX", dX, BF16, (M, inp), optional=True), a.t("dW", dW, F32, (out, inp), optional=True),
            a.t("ds", ds, F32, (out, G), optional=True), a.t("dz", dz, F32, (out, G), optional=True))
    a.done()
    _call(fn, *args, *_ws(a, ws, fakequant_ws_bytes(out, inp, bits)), _stream())


def _saved(a: _Args, w_hat, out: int, inp: int, required: bool):
    """w_hat: a forward's workspace (any dtype, >= out * in * 2 bytes) or a bf16
    W_hat [out, in]."""
    if w_hat is not None and w_hat.dtype in BF16 and w_hat.dim() == 2:
        return a.t("w_hat", w_hat, BF16, (out, inp))
    return a.t("w_hat", w_hat, None, optional=not required, min_bytes=out * inp * 2)


def qat_fakequant_linear_bwd_saved(dY, X, W, s, z, w_hat, bits, dX=None, dW=None, ds=None, dz=None,
                                   group: int = GROUP) -> None:
    """Backward on the W_hat [out, in] (bf16) its forward staged: the forward's
    workspace, or qat_quant_codes' W_hat."""
    fn = "qat_fakequant_linear_bwd_saved"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "W", W, "[out, in]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("dY", dY, BF16, (M, out)), a.t("X", X, BF16), a.t("W", W, F32, (out, inp)),
            a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), _saved(a, w_hat, out, inp, dX is not None),
            M, out, inp, group, bits,
            a.t("dX", dX, BF16, (M, inp), optional=True), a.t("dW", dW, F32, (out, inp), optional=True),
            a.t("ds", ds, F32, (out, G), optional=True), a.t("dz", dz, F32, (out, G), optional=True))
    a.done()
    _call(fn, *args, _stream())


def qat_pack(W, s, z, bits, Wq, z_round=None, group: int = GROUP) -> None:
    fn = "qat_pack"
    out, inp = _dims2(fn, "W", W, "[out, in]")
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("W", W, F32), a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), out, inp, group, bits,
            a.t("Wq", Wq, U8, (out, _packed_cols(fn, inp, bits))),
            a.t("z_round", z_round, F32, (out, G), optional=True))
    a.done()
    _call(fn, *args, _stream())


def qat_dequant_gemm_fwd(X, Wq, s, z, bits, Y, ws=None, group: int = GROUP) -> None:
    fn = "qat_dequant_gemm_fwd"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "Wq", Wq, "[out, in * bits / 8]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("X", X, BF16), a.t("Wq", Wq, U8, (out, _packed_cols(fn, inp, bits))),
            a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), M, out, inp, group, bits,
            a.t("Y", Y, BF16, (M, out)))
    a.done()
    _call(fn, *args, *_ws(a, ws, dequant_ws_bytes(out, inp, bits)), _stream())


def qat_dequant_gemm_bwd_s(dY, X, Wq, s, z, bits, ds, dX=None, dz=None, ws=None, group: int = GROUP) -> None:
    """ws None: W_hat is dequantised from the packed codes inside the dX GEMM."""
    fn = "qat_dequant_gemm_bwd_s"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "Wq", Wq, "[out, in * bits / 8]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("dY", dY, BF16, (M, out)), a.t("X", X, BF16), a.t("Wq", Wq, U8, (out, _packed_cols(fn, inp, bits))),
            a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), M, out, inp, group, bits,
            a.t("dX", dX, BF16, (M, inp), optional=True), a.t("ds", ds, F32, (out, G)),
            a.t("dz", dz, F32, (out, G), optional=True))
    a.done()
    _call(fn, *args, *_ws(a, ws, dequant_ws_bytes(out, inp, bits)), _stream())


def qat_dequant_gemm_bwd_s_saved(dY, X, Wq, s, z, w_hat, bits, ds, dX=None, dz=None, group: int = GROUP) -> None:
    """E2E-QP backward on the W_hat [out, in] (bf16) its forward staged."""
    fn = "qat_dequant_gemm_bwd_s_saved"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "Wq", Wq, "[out, in * bits / 8]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("dY", dY, BF16, (M, out)), a.t("X", X, BF16), a.t("Wq", Wq, U8, (out, _packed_cols(fn, inp, bits))),
            a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), _saved(a, w_hat, out, inp, dX is not None),
            M, out, inp, group, bits,
            a.t("dX", dX, BF16, (M, inp), optional=True), a.t("ds", ds, F32, (out, G)),
            a.t("dz", dz, F32, (out, G), optional=True))
    a.done()
    _call(fn, *args, _stream())


def deploy_zq_stride(inp: int, bits: int, group: int = GROUP) -> int:
    return int(lib().qat_deploy_zq_stride(inp, group, bits))


def qat_deploy_qparams(s, z, bits, s16, zq, inp: int, group: int = GROUP) -> None:
    fn = "qat_deploy_qparams"
    out = _dims2(fn, "s", s, "[out, in / group]")[0]
    G = _groups(fn, inp, group)
    stride = deploy_zq_stride(inp, bits, group)
    a = _Args(fn)
    args = (a.t("s", s, F32, (out, G)), a.t("z", z, F32, (out, G)), out, inp, group, bits,
            a.t("s16", s16, F16, (out, G)), a.t("zq", zq, U8, (out, stride)))
    a.done()
    _call(fn, *args, _stream())


def qat_deploy_gemv(X, Wq, s16, zq, bits, Y, group: int = GROUP) -> None:
    fn = "qat_deploy_gemv"
    M, inp = _dims2(fn, "X", X, "[M, in]")
    out = _dims2(fn, "Wq", Wq, "[out, in * bits / 8]")[0]
    G = _groups(fn, inp, group)
    a = _Args(fn)
    args = (a.t("X", X, F16), a.t("Wq", Wq, U8, (out, _packed_cols(fn, inp, bits))), a.t("s16", s16, F16, (out, G)),
            a.t("zq", zq, U8, (out, deploy_zq_stride(inp, bits, group))), M, out, inp, group, bits,
            a.t("Y", Y, F16, (M, out)))
    a.done()
    _call(fn, *args, _stream())


# ---------------------------------------------------------------------------
# Kernel timing (HIP events recorded by the library around each launch)
# ---------------------------------------------------------------------------

def timing_enable(on: bool) -> None:
    lib().qat_timing_enable(1 if on else 0)


def timing_select(label: Optional[str]) -> None:
    """Time only launches of this kernel label (None: every launch)."""
    lib().qat_timing_select(None if label is None else label.encode())


def timing_report() -> dict:
    """{label: (total_ms, launches)} for the kernels launched while enabled."""
    L = lib()
    n = L.qat_timing_count()
    if n < 0:
        raise QatError("qat_timing_count", -n)
    out = {}
    buf = ctypes.create_string_buffer(128)
    for i in range(n):
        ms, cnt = ctypes.c_double(), _c_i64()
        st = L.qat_timing_get(i, buf, 128, ctypes.byref(ms), ctypes.byref(cnt))
        if st != QAT_OK:
            raise QatError("qat_timing_get", st)
        out[buf.value.decode()] = (ms.value, int(cnt.value))
    return out


# ---------------------------------------------------------------------------
# Practical-peak probes (include/qat_peaks.h)
# ---------------------------------------------------------------------------

def peak_mfma(blocks: int, iters: int, scratch: torch.Tensor) -> int:
    """Launch the MFMA loop on the current stream; returns its flop count."""
    _call("qat_peak_mfma", blocks, iters, _p(scratch), _stream())
    return int(lib().qat_peak_mfma_flops(blocks, iters))


def peak_read(buf: torch.Tensor, blocks: int, scratch: torch.Tensor) -> int:
    """Launch the read-stream kernel over buf on the current stream; returns bytes read."""
    nbytes = buf.numel() * buf.element_size()
    _call("qat_peak_read", _p(buf), nbytes, blocks, _p(scratch), _stream())
    return nbytes - nbytes % 16


def peak_write(buf: torch.Tensor, blocks: int) -> int:
    """Launch the write-stream kernel over buf (overwritten) on the current stream; returns bytes written."""
    nbytes = buf.numel() * buf.element_size()
    _call("qat_peak_write", _p(buf), nbytes, blocks, _stream())
    return nbytes - nbytes % 16


# ---------------------------------------------------------------------------
# One Block-AP step on a Llama-2 decoder block (include/qat_block.h)
# ---------------------------------------------------------------------------

def block_shape(hidden, heads, inter, seq, batch, bits, group: int = GROUP) -> BlockShape:
    return BlockShape(hidden, heads, inter, seq, batch, bits, group)


def block_ws_bytes(shape: BlockShape) -> int:
    return int(lib().qat_block_ws_bytes(ctypes.byref(shape)))


def _block_linear_shapes(shape: BlockShape):
    """(out, in) of q, k, v, o, gate, up, down (include/qat_block.h)."""
    H, I = int(shape.hidden), int(shape.inter)
    return [(H, H)] * 4 + [(I, H), (I, H), (H, I)]


def _linears(a: _Args, shape: BlockShape, lins, step: bool):
    """lins: 7 dicts (q, k, v, o, gate, up, down) of fp32 tensors keyed by
    W, s, z, dW, ds, dz, m_W, v_W, m_s, v_s, m_z, v_z (missing keys: NULL).
    Each must have its parameter's shape."""
    if len(lins) != 7:
        raise ValueError("seven linears: q, k, v, o, gate, up, down")
    group = int(shape.group)
    arr = (BlockLinear * 7)()
    for i, (d, (o, inp)) in enumerate(zip(lins, _block_linear_shapes(shape))):
        G = _groups("qat_block", inp, group)
        for f in _LIN_FIELDS:
            shp = (o, inp) if f.endswith("W") else (o, G)
            need = f in ("W", "s", "z") or (step and f != "dW")
            setattr(arr[i], f, a.t(f"{BLOCK_LINEARS[i]}.{f}", d.get(f), F32, shp, optional=not need))
    return arr


def _block_io(a: _Args, shape: BlockShape, g1, g2, x, target, y, loss):
    H, BT = int(shape.hidden), int(shape.batch) * int(shape.seq)
    return (a.t("g1", g1, F32, (H,)), a.t("g2", g2, F32, (H,)), a.t("x", x, BF16, (BT, H)),
            a.t("target", target, BF16, (BT, H)), a.t("y", y, F32, (BT, H), optional=True),
            a.t("loss", loss, F32, (1,)))


def qat_block_forward(shape: BlockShape, lins, g1, g2, x, target, loss, y=None, ws=None) -> None:
    a = _Args("qat_block_forward")
    arr = _linears(a, shape, lins, step=False)
    G1, G2, X, T, Yp, L = _block_io(a, shape, g1, g2, x, target, y, loss)
    wp, wn = _ws(a, ws, block_ws_bytes(shape))
    a.done()
    _call("qat_block_forward", ctypes.byref(shape), arr, G1, G2, X, T, Yp, L, wp, wn, _stream())


def qat_block_ap_step(shape: BlockShape, lins, g1, g2, x, target, opt: dict, loss, y=None, ws=None) -> None:
    """opt: lr_weight, lr_quant, beta1, beta2, eps, weight_decay, step (0-based), total_steps."""
    o = BlockAdamW(opt["lr_weight"], opt["lr_quant"], opt["beta1"], opt["beta2"], opt["eps"],
                   opt["weight_decay"], opt["step"], opt["total_steps"])
    a = _Args("qat_block_ap_step")
    arr = _linears(a, shape, lins, step=True)
    G1, G2, X, T, Yp, L = _block_io(a, shape, g1, g2, x, target, y, loss)
    wp, wn = _ws(a, ws, block_ws_bytes(shape))
    a.done()
    _call("qat_block_ap_step", ctypes.byref(shape), arr, G1, G2, X, T, ctypes.byref(o), Yp, L, wp, wn, _stream())
