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
    "qat_fakequant_ws_bytes": [_c_i64, _c_i64, _c_i64],
    "qat_dequant_ws_bytes": [_c_i64, _c_i64, _c_i64],
    "qat_timing_enable": [_c_i32],
    "qat_timing_count": [],
    "qat_timing_select": [ctypes.c_char_p],
    "qat_timing_get": [_c_i32, ctypes.c_char_p, _c_sz, ctypes.POINTER(ctypes.c_double),
                       ctypes.POINTER(_c_i64)],
    "qat_peak_mfma_flops": [_c_i32, _c_i32],
    "qat_peak_scratch_bytes": [_c_i32],
    "qat_peak_mfma": [_c_i32, _c_i32, _c_vp, _c_vp],
    "qat_peak_read": [_c_vp, _c_sz, _c_i32, _c_vp, _c_vp],
    "qat_status_string": [_c_i32],
    "qat_last_error": [],
}
_RES = {"qat_deploy_zq_stride": _c_i64, "qat_fakequant_ws_bytes": _c_sz, "qat_dequant_ws_bytes": _c_sz, "qat_peak_mfma_flops": _c_i64,
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


def _u16(t: torch.Tensor) -> torch.Tensor:
    """bf16 (or, for the deployment calls, fp16) tensors travel as their 16-bit
    patterns."""
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected a bf16 tensor, got {t.dtype}")


# ---------------------------------------------------------------------------
# Workspace size queries
# ---------------------------------------------------------------------------

def fakequant_ws_bytes(M: int, out: int, inp: int) -> int:
    return int(lib().qat_fakequant_ws_bytes(M, out, inp))


def dequant_ws_bytes(M: int, out: int, inp: int) -> int:
    return int(lib().qat_dequant_ws_bytes(M, out, inp))


def workspace(nbytes: int, device=None) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------------------
# The C-ABI calls, same names as in include/qat.h
# ---------------------------------------------------------------------------

def qat_init_minmax(W: torch.Tensor, bits: int, s: torch.Tensor, z: torch.Tensor, group: int = GROUP) -> None:
    out, inp = W.shape
    _call("qat_init_minmax", _p(W), out, inp, group, bits, _p(s), _p(z), _stream())


def qat_quant_codes(W, s, z, bits, codes=None, W_hat=None, group: int = GROUP) -> None:
    out, inp = W.shape
    _call("qat_quant_codes", _p(W), _p(s), _p(z), out, inp, group, bits, _p(codes),
          _p(None if W_hat is None else _u16(W_hat)), _stream())


def qat_fakequant_linear_fwd(X, W, s, z, bits, Y, ws=None, group: int = GROUP) -> None:
    M, inp = X.shape
    out = W.shape[0]
    _call("qat_fakequant_linear_fwd", _p(_u16(X)), _p(W), _p(s), _p(z), M, out, inp, group, bits,
          _p(_u16(Y)), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())


def qat_fakequant_linear_bwd(dY, X, W, s, z, bits, dX=None, dW=None, ds=None, dz=None, ws=None,
                             group: int = GROUP) -> None:
    M, inp = X.shape
    out = W.shape[0]
    _call("qat_fakequant_linear_bwd", _p(_u16(dY)), _p(_u16(X)), _p(W), _p(s), _p(z), M, out, inp,
          group, bits, _p(None if dX is None else _u16(dX)), _p(dW), _p(ds), _p(dz), _p(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream())


def qat_pack(W, s, z, bits, Wq, z_round=None, group: int = GROUP) -> None:
    out, inp = W.shape
    _call("qat_pack", _p(W), _p(s), _p(z), out, inp, group, bits, _p(Wq), _p(z_round), _stream())


def qat_dequant_gemm_fwd(X, Wq, s, z, bits, Y, ws=None, group: int = GROUP) -> None:
    M, inp = X.shape
    out = Wq.shape[0]
    _call("qat_dequant_gemm_fwd", _p(_u16(X)), _p(Wq), _p(s), _p(z), M, out, inp, group, bits,
          _p(_u16(Y)), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())


def _check_saved(w_hat, out: int, inp: int) -> None:
    """w_hat: a forward's workspace (any dtype) or a bf16 W_hat, at least out * in * 2 bytes."""
    if w_hat is not None and w_hat.numel() * w_hat.element_size() < out * inp * 2:
        raise ValueError("w_hat holds fewer than out * in bf16 values")


def qat_fakequant_linear_bwd_saved(dY, X, W, s, z, w_hat, bits, dX=None, dW=None, ds=None, dz=None,
                                   group: int = GROUP) -> None:
    """Backward on the W_hat [out, in] (bf16) its forward staged: the forward's
    workspace, or qat_quant_codes' W_hat."""
    M, inp = X.shape
    out = W.shape[0]
    _check_saved(w_hat, out, inp)
    _call("qat_fakequant_linear_bwd_saved", _p(_u16(dY)), _p(_u16(X)), _p(W), _p(s), _p(z), _p(w_hat),
          M, out, inp, group, bits,
          _p(None if dX is None else _u16(dX)), _p(dW), _p(ds), _p(dz), _stream())


def qat_dequant_gemm_bwd_s_saved(dY, X, Wq, s, z, w_hat, bits, ds, dX=None, dz=None, group: int = GROUP) -> None:
    """E2E-QP backward on the W_hat [out, in] (bf16) its forward staged."""
    M, inp = X.shape
    out = Wq.shape[0]
    _check_saved(w_hat, out, inp)
    _call("qat_dequant_gemm_bwd_s_saved", _p(_u16(dY)), _p(_u16(X)), _p(Wq), _p(s), _p(z), _p(w_hat),
          M, out, inp, group, bits,
          _p(None if dX is None else _u16(dX)), _p(ds), _p(dz), _stream())


def qat_dequant_gemm_bwd_s(dY, X, Wq, s, z, bits, ds, dX=None, dz=None, ws=None, group: int = GROUP) -> None:
    M, inp = X.shape
    out = Wq.shape[0]
    _call("qat_dequant_gemm_bwd_s", _p(_u16(dY)), _p(_u16(X)), _p(Wq), _p(s), _p(z), M, out, inp,
          group, bits, _p(None if dX is None else _u16(dX)), _p(ds), _p(dz), _p(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream())


def _f16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.float16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected an fp16 tensor, got {t.dtype}")


def deploy_zq_stride(inp: int, bits: int, group: int = GROUP) -> int:
    return int(lib().qat_deploy_zq_stride(inp, group, bits))


def qat_deploy_qparams(s, z, bits, s16, zq, inp: int, group: int = GROUP) -> None:
    out = s.shape[0]
    _call("qat_deploy_qparams", _p(s), _p(z), out, inp, group, bits, _p(_f16(s16)), _p(zq), _stream())


def qat_deploy_gemv(X, Wq, s16, zq, bits, Y, group: int = GROUP) -> None:
    M, inp = X.shape
    out = Wq.shape[0]
    _call("qat_deploy_gemv", _p(_f16(X)), _p(Wq), _p(_f16(s16)), _p(zq), M, out, inp, group, bits,
          _p(_f16(Y)), _stream())


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


# ---------------------------------------------------------------------------
# One Block-AP step on a Llama-2 decoder block (include/qat_block.h)
# ---------------------------------------------------------------------------

def block_shape(hidden, heads, inter, seq, batch, bits, group: int = GROUP) -> BlockShape:
    return BlockShape(hidden, heads, inter, seq, batch, bits, group)


def block_ws_bytes(shape: BlockShape) -> int:
    return int(lib().qat_block_ws_bytes(ctypes.byref(shape)))


def _linears(lins):
    """lins: 7 dicts (q, k, v, o, gate, up, down) of fp32 tensors keyed by
    W, s, z, dW, ds, dz, m_W, v_W, m_s, v_s, m_z, v_z (missing keys: NULL)."""
    if len(lins) != 7:
        raise ValueError("seven linears: q, k, v, o, gate, up, down")
    arr = (BlockLinear * 7)()
    for i, d in enumerate(lins):
        for f in _LIN_FIELDS:
            t = d.get(f)
            if t is not None and t.dtype != torch.float32:
                raise TypeError(f"linear {i} {f}: expected fp32, got {t.dtype}")
            setattr(arr[i], f, _p(t))
    return arr


def qat_block_forward(shape: BlockShape, lins, g1, g2, x, target, loss, y=None, ws=None) -> None:
    arr = _linears(lins)
    _call("qat_block_forward", ctypes.byref(shape), arr, _p(g1), _p(g2), _p(_u16(x)), _p(_u16(target)), _p(y),
          _p(loss), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())


def qat_block_ap_step(shape: BlockShape, lins, g1, g2, x, target, opt: dict, loss, y=None, ws=None) -> None:
    """opt: lr_weight, lr_quant, beta1, beta2, eps, weight_decay, step (0-based), total_steps."""
    o = BlockAdamW(opt["lr_weight"], opt["lr_quant"], opt["beta1"], opt["beta2"], opt["eps"],
                   opt["weight_decay"], opt["step"], opt["total_steps"])
    arr = _linears(lins)
    _call("qat_block_ap_step", ctypes.byref(shape), arr, _p(g1), _p(g2), _p(_u16(x)), _p(_u16(target)),
          ctypes.byref(o), _p(y), _p(loss), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream())
