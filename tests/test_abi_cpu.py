"""CPU checks of the C ABI: the library loads, exports every symbol that
include/qat.h declares, and rejects bad arguments on the host before any HIP
call (these calls return before touching a device)."""
import ctypes
import os
import re

import numpy as np
import pytest

from weight_quantization_aware_amd import _lib as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(qat_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_calls():
    names = declared()
    for n in ["qat_init_minmax", "qat_fakequant_linear_fwd", "qat_fakequant_linear_bwd", "qat_pack",
              "qat_dequant_gemm_fwd", "qat_dequant_gemm_bwd_s", "qat_quant_codes", "qat_block_ap_step",
              "qat_fakequant_linear_bwd_saved", "qat_dequant_gemm_bwd_s_saved",
              "qat_block_forward", "qat_block_ws_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(Q.LIB_PATH)
    for n in declared():
        assert hasattr(h, n), n
    assert set(declared()) <= set(Q._SIGS)


def test_status_strings():
    L = Q.lib()
    for st in range(10):
        assert L.qat_status_string(st) != b"unknown status"
    assert L.qat_status_string(10) == b"unknown status"
    assert L.qat_last_error() == b""


def test_workspace_sizes():
    # one bf16 W_hat [out, in], rounded up to 256 bytes, at every bit width
    assert Q.fakequant_ws_bytes(4096, 4096, 2) == 4096 * 4096 * 2
    assert Q.fakequant_ws_bytes(64, 64, 4) == 64 * 64 * 2
    assert Q.fakequant_ws_bytes(4100, 64, 3) == 4100 * 64 * 2
    assert Q.fakequant_ws_bytes(7, 64, 2) == 1024
    assert Q.fakequant_ws_bytes(0, 64, 2) == 0
    assert Q.fakequant_ws_bytes(64, 64, 5) == 0
    assert Q.dequant_ws_bytes(192, 128, 3) == Q.fakequant_ws_bytes(192, 128, 3)


FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced on the error paths


@pytest.mark.parametrize("args,status", [
    ((FAKE, 64, 128, 64, 5, FAKE, FAKE + 4096, None), 3),        # bits
    ((FAKE, 64, 128, 48, 2, FAKE, FAKE + 4096, None), 4),        # group not 32, 64, 128 or in
    ((FAKE, 64, 128, 96, 2, FAKE, FAKE + 4096, None), 4),        # group not 32, 64, 128 or in
    ((FAKE, 64, 192, 128, 2, FAKE, FAKE + 4096, None), 4),       # group 128 does not divide in
    ((FAKE, 64, 128, 0, 2, FAKE, FAKE + 4096, None), 4),         # group 0
    ((FAKE, 64, 96, 64, 2, FAKE, FAKE + 4096, None), 2),         # in % 64
    ((FAKE, 0, 128, 64, 2, FAKE, FAKE + 4096, None), 2),         # out <= 0
    ((None, 64, 128, 64, 2, FAKE, FAKE + 4096, None), 1),        # null W
    ((FAKE + 4, 64, 128, 64, 2, FAKE, FAKE + 4096, None), 5),    # misaligned
    ((FAKE, 64, 128, 64, 2, FAKE, FAKE, None), 8),               # s aliases z
    ((FAKE, 64, 128, 64, 2, FAKE + 16, FAKE + 1 << 30, None), 8),  # s inside W
])
def test_init_validation(args, status):
    assert Q.lib().qat_init_minmax(*args) == status


def test_fwd_bwd_validation():
    L = Q.lib()
    A, B, C, D, E = (FAKE * k for k in range(1, 6))
    # fwd: workspace given but too small
    assert L.qat_fakequant_linear_fwd(A, B, C, D, 8, 64, 128, 64, 2, E, FAKE * 7, 16, None) == 6
    # fwd: M <= 0
    assert L.qat_fakequant_linear_fwd(A, B, C, D, 0, 64, 128, 64, 2, E, None, 0, None) == 2
    # bwd: a workspace, when given for dX, must hold W_hat (NULL: W_hat is made inside the dX GEMM)
    assert L.qat_fakequant_linear_bwd(A, B, C, D, E, 8, 64, 128, 64, 2, FAKE * 6, None, None, None,
                                      FAKE * 7, 16, None) == 6
    assert L.qat_dequant_gemm_bwd_s(A, B, C, D, E, 8, 64, 128, 64, 2, FAKE * 6, FAKE * 8, None, FAKE * 7,
                                    16, None) == 6
    # the GEMM calls need out % 4 == 0 (8-byte aligned rows of Y and dY)
    for out in (98, 97, 1):
        assert L.qat_fakequant_linear_fwd(A, B, C, D, 8, out, 128, 64, 2, E, None, 0, None) == 2
        assert L.qat_dequant_gemm_fwd(A, B, C, D, 8, out, 128, 64, 2, E, None, 0, None) == 2
    # bwd: ds without dz
    assert L.qat_fakequant_linear_bwd(A, B, C, D, E, 8, 64, 128, 64, 2, None, None, FAKE * 6, None,
                                      FAKE * 7, 1 << 30, None) == 1
    # e2e bwd: ds is required
    assert L.qat_dequant_gemm_bwd_s(A, B, C, D, E, 8, 64, 128, 64, 2, None, None, None, FAKE * 7,
                                    1 << 30, None) == 1
    # e2e fwd: workspace given but too small; M <= 0
    assert L.qat_dequant_gemm_fwd(A, B, C, D, 8, 64, 128, 64, 2, E, FAKE * 7, 16, None) == 6
    assert L.qat_dequant_gemm_fwd(A, B, C, D, 0, 64, 128, 64, 2, E, None, 0, None) == 2
    # pack: 3 bits with a group-aligned row is fine shape-wise, bits 1 is not
    assert L.qat_pack(A, B, C, 64, 128, 64, 1, D, None, None) == 3


def test_saved_backward_validation():
    L = Q.lib()
    A, B, C, D, E, WH, DX = (FAKE * k for k in range(1, 8))
    # dX wanted without the saved W_hat
    assert L.qat_fakequant_linear_bwd_saved(A, B, C, D, E, None, 8, 64, 128, 64, 2, DX, None, None, None,
                                            None) == 1
    assert L.qat_dequant_gemm_bwd_s_saved(A, B, C, D, E, None, 8, 64, 128, 64, 2, DX, FAKE * 9, None,
                                          None) == 1
    # dX writing over the saved W_hat
    assert L.qat_fakequant_linear_bwd_saved(A, B, C, D, E, WH, 8, 64, 128, 64, 2, WH, None, None, None,
                                            None) == 8
    # misaligned W_hat; ds without dz; e2e without ds
    assert L.qat_fakequant_linear_bwd_saved(A, B, C, D, E, WH + 8, 8, 64, 128, 64, 2, DX, None, None, None,
                                            None) == 5
    assert L.qat_fakequant_linear_bwd_saved(A, B, C, D, E, WH, 8, 64, 128, 64, 2, None, None, FAKE * 9, None,
                                            None) == 1
    assert L.qat_dequant_gemm_bwd_s_saved(A, B, C, D, E, WH, 8, 64, 128, 64, 2, DX, None, None, None) == 1
    # shapes as in the staging variants
    assert L.qat_fakequant_linear_bwd_saved(A, B, C, D, E, WH, 0, 64, 128, 64, 2, DX, None, None, None,
                                            None) == 2
    assert L.qat_dequant_gemm_bwd_s_saved(A, B, C, D, E, WH, 8, 64, 128, 64, 5, DX, FAKE * 9, None, None) == 3


def test_noalloc_forward_validation():
    L = Q.lib()
    A, B, C, D, E = ((FAKE << 12) * k for k in range(1, 6))        # 4 GiB apart: no overlaps
    assert L.qat_noalloc_max_weights() == 48 << 20
    # more weights than the static scratch holds: refused before any launch
    assert L.qat_fakequant_linear_fwd_noalloc(A, B, C, D, 1, 8192, 8192, 64, 2, E, None) == 9
    # the checks of the workspace forward
    assert L.qat_fakequant_linear_fwd_noalloc(A, B, C, D, 0, 64, 128, 64, 2, E, None) == 2
    assert L.qat_fakequant_linear_fwd_noalloc(A, None, C, D, 8, 64, 128, 64, 2, E, None) == 1
    assert L.qat_fakequant_linear_fwd_noalloc(A, B, C, D, 8, 64, 128, 64, 2, A, None) == 8


def test_timing_registry_host_side():
    # enabling, selecting and reading the registry records nothing without launches
    Q.timing_select("gemm_fwd")
    Q.timing_enable(True)
    Q.timing_enable(False)
    Q.timing_select(None)
    assert Q.timing_report() == {}


def test_peak_probe_host_validation():
    L = Q.lib()
    assert L.qat_peak_mfma_flops(256, 100) == 256 * 8 * 8 * 100 * 16 * 16 * 32 * 2
    assert L.qat_peak_mfma_flops(0, 100) == -1
    assert L.qat_peak_scratch_bytes(4) == 4 * 512 * 4
    assert L.qat_peak_mfma(0, 10, FAKE, None) == 1
    assert L.qat_peak_read(None, 1 << 20, 16, FAKE, None) == 1
    assert L.qat_peak_read(FAKE + 4, 1 << 20, 16, FAKE, None) == 1
    assert L.qat_peak_write(None, 1 << 20, 16, None) == 1
    assert L.qat_peak_write(FAKE + 4, 1 << 20, 16, None) == 1
    assert L.qat_peak_write(FAKE, 8, 16, None) == 1


def test_deploy_validation():
    L = Q.lib()
    A, B, C, D, E = (FAKE * k for k in range(1, 6))
    # M must be 1..16
    assert L.qat_deploy_gemv(A, B, C, D, 0, 64, 256, 64, 2, E, None) == 2
    assert L.qat_deploy_gemv(A, B, C, D, 17, 64, 256, 64, 2, E, None) == 2
    # bits, group, in % 64
    assert L.qat_deploy_gemv(A, B, C, D, 1, 64, 256, 64, 5, E, None) == 3
    assert L.qat_deploy_gemv(A, B, C, D, 1, 64, 256, 48, 2, E, None) == 4
    assert L.qat_deploy_gemv(A, B, C, D, 1, 64, 96, 32, 2, E, None) == 2
    # null and misaligned pointers, Y overlapping the codes
    assert L.qat_deploy_gemv(A, None, C, D, 1, 64, 256, 64, 2, E, None) == 1
    assert L.qat_deploy_gemv(A, B + 4, C, D, 1, 64, 256, 64, 2, E, None) == 5
    assert L.qat_deploy_gemv(A, B, C, D, 1, 64, 256, 64, 2, B + 16, None) == 8
    # qparams: s16 overlapping s
    assert L.qat_deploy_qparams(A, B, 64, 256, 64, 2, A + 16, C, None) == 8
    assert L.qat_deploy_qparams(A, B, 64, 256, 64, 7, C, D, None) == 3
    # zq row stride: ceil(G N / 8); 0 for invalid arguments
    assert Q.deploy_zq_stride(256, 2) == 1
    assert Q.deploy_zq_stride(192, 3) == 2
    assert Q.deploy_zq_stride(192, 3, group=192) == 1
    assert Q.deploy_zq_stride(4096, 4) == 32
    assert Q.deploy_zq_stride(4096, 4, group=48) == 0


# ---------------------------------------------------------------------------
# The Block-AP step (include/qat_block.h): host-side validation only
# ---------------------------------------------------------------------------

def _block_args(shape, n_lin=7, step=True):
    lins = (Q.BlockLinear * 7)()
    for i in range(n_lin):
        for j, f in enumerate(Q._LIN_FIELDS):
            if step or f in ("W", "s", "z"):
                setattr(lins[i], f, FAKE * (1 + 64 * i + 4 * j))
    return lins


def test_block_ws_bytes():
    sh = Q.block_shape(4096, 32, 11008, 2048, 2, 2)
    n = Q.block_ws_bytes(sh)
    BT, H, I, S = 4096, 4096, 11008, 2 * 32 * 2048 * 2048
    # at least the activations the backward reads and the probabilities in bf16
    # (the forward keeps the scores in registers)
    assert n >= S * 2 + BT * H * 2 * 4 + BT * I * 2 * 3
    assert n % 256 == 0 and n < 2 * 2 ** 30
    for bad in [Q.block_shape(4096, 30, 11008, 2048, 2, 2),    # head size not 128
                Q.block_shape(4096, 32, 11000, 2048, 2, 2),    # inter % 64
                Q.block_shape(4096, 32, 11008, 2000, 2, 2),    # seq % 64
                Q.block_shape(4096, 32, 11008, 8192, 1, 2),    # seq > 4096
                Q.block_shape(16384, 128, 11008, 2048, 2, 2),  # hidden > 8192
                Q.block_shape(4096, 32, 11008, 2048, 2, 5),    # bits
                Q.block_shape(4096, 32, 11008, 2048, 2, 2, 96),
                Q.block_shape(4096, 32, 11072, 2048, 2, 2, 128)]:  # group does not divide inter
        assert Q.block_ws_bytes(bad) == 0


def test_block_validation():
    L = Q.lib()
    sh = Q.block_shape(256, 2, 704, 192, 2, 2)
    need = Q.block_ws_bytes(sh)
    opt = Q.BlockAdamW(2e-5, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0, 4096)
    X, T, G1, G2, Y, LOSS, WS = (FAKE << 12) * np.arange(1, 8)
    X, T, G1, G2, Y, LOSS, WS = (int(v) for v in (X, T, G1, G2, Y, LOSS, WS))
    lins = _block_args(sh)
    step = lambda **kw: L.qat_block_ap_step(kw.get("shape", ctypes.byref(sh)), kw.get("lins", lins), G1, G2, X, T,
                                            kw.get("opt", ctypes.byref(opt)), Y, LOSS, WS, kw.get("ws", need), None)
    assert step(ws=need - 256) == 6                               # workspace too small
    bad = Q.block_shape(256, 2, 704, 100, 2, 2)
    assert step(shape=ctypes.byref(bad)) == 2
    bad = Q.block_shape(256, 2, 704, 192, 2, 2, 48)
    assert step(shape=ctypes.byref(bad)) == 4
    assert step(opt=None) == 1
    o2 = Q.BlockAdamW(2e-5, 1e-4, 1.0, 0.999, 1e-8, 0.0, 0, 4096)    # beta1 outside [0, 1)
    assert step(opt=ctypes.byref(o2)) == 2
    o3 = Q.BlockAdamW(2e-5, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0, 0)       # no schedule length
    assert step(opt=ctypes.byref(o3)) == 2
    assert step(lins=_block_args(sh, step=False)) == 1             # gradients and moments required
    l2 = _block_args(sh)
    l2[3].ds = l2[3].dz                                            # two outputs share memory
    assert step(lins=l2) == 8
    l3 = _block_args(sh)
    l3[6].W = l3[6].W + 4                                          # misaligned
    assert step(lins=l3) == 5
    l4 = _block_args(sh)
    l4[0].m_W = X                                                  # a moment over the input
    assert step(lins=l4) == 8
    l5 = _block_args(sh)
    l5[2].dW = None                                                # dW is optional at every group size
    assert step(lins=l5, ws=need - 256) == 6                       # (validation reaches the workspace check)
    sh32 = Q.block_shape(256, 2, 704, 192, 2, 2, 32)
    l5 = _block_args(sh32)
    l5[2].dW = None
    assert step(shape=ctypes.byref(sh32), lins=l5, ws=need - 256) == 6
    # the forward call needs only W, s, z but checks the same shapes and regions
    fwd = L.qat_block_forward(ctypes.byref(sh), _block_args(sh, step=False), G1, G2, X, T, Y, LOSS, WS, need - 1,
                              None)
    assert fwd == 6
    assert L.qat_block_forward(ctypes.byref(sh), _block_args(sh, step=False), G1, G2, X, T, X, LOSS, WS, need,
                               None) == 8                          # y over x


# ---------------------------------------------------------------------------
# The Python binding checks dtype, shape and device before the C call (the C
# ABI sees raw pointers only). Dtype and shape are checked first, so host
# tensors exercise them here; a host tensor that passes them is refused as
# not on the GPU.
# ---------------------------------------------------------------------------

def _fq_args(M=8, out=64, inp=128, g=64):
    import torch
    return dict(X=torch.zeros(M, inp, dtype=torch.bfloat16), W=torch.zeros(out, inp),
                s=torch.ones(out, inp // g), z=torch.zeros(out, inp // g),
                Y=torch.zeros(M, out, dtype=torch.bfloat16))


def test_binding_rejects_wrong_dtype_shape_device():
    import torch
    a = _fq_args()
    fwd = lambda **kw: Q.qat_fakequant_linear_fwd(kw.get("X", a["X"]), kw.get("W", a["W"]), kw.get("s", a["s"]),
                                                  kw.get("z", a["z"]), 2, kw.get("Y", a["Y"]), group=kw.get("g", 64))
    with pytest.raises(TypeError, match="X must be"):
        fwd(X=a["X"].float())                                          # X not bf16
    with pytest.raises(TypeError, match="W must be"):
        fwd(W=a["W"].double())
    with pytest.raises(ValueError, match="s must have shape"):
        fwd(s=torch.ones(64, 4))                                       # s sized for group 32
    with pytest.raises(ValueError, match="W must have shape"):
        fwd(W=torch.zeros(64, 256))                                    # W's in differs from X's
    with pytest.raises(ValueError, match="Y must have shape"):
        fwd(Y=torch.zeros(8, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="group 48 must divide"):
        fwd(g=48, s=torch.ones(64, 2), z=torch.zeros(64, 2))
    with pytest.raises(ValueError, match="contiguous"):
        fwd(W=torch.zeros(128, 64).t())
    with pytest.raises(ValueError, match="CUDA"):
        fwd()                                                          # right shapes, host memory
    # packed weights at another bit width; bwd outputs of the wrong shape
    Wq = torch.zeros(64, 128 * 3 // 8, dtype=torch.uint8)
    with pytest.raises(ValueError, match="Wq must have shape"):
        Q.qat_dequant_gemm_fwd(a["X"], Wq, a["s"], a["z"], 2, a["Y"])
    with pytest.raises(ValueError, match="bits must be"):
        Q.qat_pack(a["W"], a["s"], a["z"], 5, Wq)
    dY = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dX must have shape"):
        Q.qat_fakequant_linear_bwd(dY, a["X"], a["W"], a["s"], a["z"], 2, dX=torch.zeros(8, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="dW must be"):
        Q.qat_fakequant_linear_bwd(dY, a["X"], a["W"], a["s"], a["z"], 2, dW=torch.zeros(64, 128, dtype=torch.half))
    with pytest.raises(ValueError, match="ds must have shape"):
        Q.qat_dequant_gemm_bwd_s(dY, a["X"], torch.zeros(64, 32, dtype=torch.uint8), a["s"], a["z"], 2,
                                 torch.zeros(64, 4))
    with pytest.raises(ValueError, match="w_hat holds"):
        Q.qat_fakequant_linear_bwd_saved(dY, a["X"], a["W"], a["s"], a["z"], torch.zeros(100, dtype=torch.uint8), 2,
                                         dX=torch.zeros(8, 128, dtype=torch.bfloat16))
    # deployment: fp16 operands
    with pytest.raises(TypeError, match="X must be"):
        Q.qat_deploy_gemv(a["X"], torch.zeros(64, 32, dtype=torch.uint8), torch.zeros(64, 2, dtype=torch.half),
                          torch.zeros(64, 1, dtype=torch.uint8), 2, torch.zeros(8, 64, dtype=torch.half))


def test_binding_block_checks():
    import torch
    sh = Q.block_shape(256, 2, 704, 192, 2, 2)
    lins = []
    for o, i in [(256, 256)] * 4 + [(704, 256), (704, 256), (256, 704)]:
        e = {"W": torch.zeros(o, i), "s": torch.ones(o, i // 64), "z": torch.zeros(o, i // 64)}
        lins.append(e)
    x = torch.zeros(384, 256, dtype=torch.bfloat16)
    g = torch.ones(256)
    loss = torch.zeros(1)
    bad = [dict(d) for d in lins]
    bad[6] = {"W": torch.zeros(704, 256), "s": torch.ones(704, 4), "z": torch.zeros(704, 4)}   # down transposed
    with pytest.raises(ValueError, match="down_proj.W must have shape"):
        Q.qat_block_forward(sh, bad, g, g, x, x, loss)
    with pytest.raises(ValueError, match="x must have shape"):
        Q.qat_block_forward(sh, lins, g, g, x[:100], x, loss)
    with pytest.raises(ValueError, match="q_proj.ds is required"):
        Q.qat_block_ap_step(sh, lins, g, g, x, x, {"lr_weight": 0, "lr_quant": 0, "beta1": 0.9, "beta2": 0.999,
                                                   "eps": 1e-8, "weight_decay": 0, "step": 0, "total_steps": 1}, loss)
    with pytest.raises(ValueError, match="CUDA"):
        Q.qat_block_forward(sh, lins, g, g, x, x, loss)
