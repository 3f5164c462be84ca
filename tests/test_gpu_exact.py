"""Exact-sum parity: the GEMM outputs of every path, bit for bit against the
fp64 oracle.

Inputs come from synth.exact_sum_inputs: integer activations and output
gradients in [-2, 2], power-of-two step sizes (2^-5 .. 2^-7) and integer zero
points in use. Every product of an activation and a dequantised weight is then
a multiple of 2^-7 and one output's products add up to less than 2^17 in
magnitude (asserted per case), so every fp32 partial sum is exact whatever the
order of the additions (tests/test_exact_cpu.py shows it on the CPU). The
oracle's fp64 products, rounded once to bf16 (Y, dX) or fp32 (dW), must
therefore equal the GPU's outputs bit for bit, on every tile, for the staged
path (W_hat in a workspace), the fused paths (W_hat made in LDS from the fp32
master weight or from packed codes, no workspace) and the backwards on the
forward's saved W_hat. A wrong code, a dropped k-chunk or a tile stored twice
breaks that equality where the element-wise bf16 bound of the other parity
tests could still let it pass. dz of the straight-through backward and ds, dz
of E2E-QP are integer sums times a power of two, exact too; ds of the
straight-through backward depends on W / s - rint(W / s) and is held to the
fp32 tolerance (relative Frobenius 1e-5).
Zeros compare as values (+0 and -0 alike).
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import dev_bf16, dev_f32, dev_u8, host_bits, rel_fro, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _bits_of(ref: np.ndarray) -> np.ndarray:
    """bf16 bits of exact fp64 values that are exact in fp32 (one rounding)."""
    b = O.f64_to_bf16_bits(O.bf16_round(O.fl32(ref)))
    return np.where(b == 0x8000, 0, b).astype(np.uint16)


def _same_bits(name: str, got: np.ndarray, ref_bits: np.ndarray) -> None:
    got = np.where(got == 0x8000, 0, got)
    bad = got != ref_bits
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outputs differ; first at {i}: "
                             f"got {O.bf16_bits_to_f64(got[i])!r} ref {O.bf16_bits_to_f64(ref_bits[i])!r}")


def _same_f32(name: str, got: np.ndarray, ref: np.ndarray) -> None:
    bad = got.astype(np.float64) != ref
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outputs differ; first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")


def _premise(a: np.ndarray, w: np.ndarray) -> None:
    """One output's products add up to less than 2^17 in magnitude (a @ w^T)."""
    assert (np.abs(a) @ np.abs(w).T).max() < 2.0 ** 17


# (M, out, in, bits): several tiles with ragged edges in M, out and in; a
# short contraction; a long one that is not a multiple of 64 in out; the
# Llama-2-7B q_proj workload at full size; and q_proj-sized products with
# out = 4100 at 4096 tokens, whose dX contractions end mid-slab on the tile
# shapes that large ragged products take (128x128 fused, 128x256 staged);
# and a Llama-2-7B down projection at 2048 tokens, whose 2048 x 11008 dX
# takes 128x256 tiles because 256x256 ones would leave their second round
# mostly empty.
CASES = [(300, 320, 512, 3), (2085, 4096, 256, 2), (100, 4160, 4160, 3), (257, 4100, 192, 4),
         (2048, 4096, 4096, 2), (4096, 4100, 4096, 2), (2048, 4096, 11008, 3)]


@pytest.mark.parametrize("M,out,inp,bits", CASES)
def test_fakequant_exact(M, out, inp, bits):
    say(f"exact fake-quant M={M} out={out} in={inp} bits={bits}")
    e = synth.exact_sum_inputs(500 + bits, M, out, inp, bits)
    X, dY = O.bf16_bits_to_f64(e.X), O.bf16_bits_to_f64(e.dY)
    t = O.quantize(e.W, e.s, e.z, bits)
    w_hat = O.dequantize_exact(t["q"], t["zr"], t["s"])
    _premise(X, w_hat)
    _premise(dY, w_hat.T)
    y_bits = _bits_of(X @ w_hat.T)
    r = O.fakequant_bwd_values(dY, X, e.W, e.s, e.z, bits)
    dx_bits = _bits_of(r["dX"])
    del w_hat, t

    X_, dY_, W_, s_, z_ = dev_bf16(e.X), dev_bf16(e.dY), dev_f32(e.W), dev_f32(e.s), dev_f32(e.z)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    for name, w in (("staged", ws), ("fused", None)):
        Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
        Q.qat_fakequant_linear_fwd(X_, W_, s_, z_, bits, Y, ws=w)
        torch.cuda.synchronize()
        _same_bits(f"Y {name}", host_bits(Y), y_bits)
    ws_bwd = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    for name in ("staged", "fused", "saved"):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gW = torch.empty(out, inp, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        gz = torch.empty_like(gs)
        if name == "saved":      # ws holds the staged forward's W_hat
            Q.qat_fakequant_linear_bwd_saved(dY_, X_, W_, s_, z_, ws, bits, dX=gX, dW=gW, ds=gs, dz=gz)
        else:
            Q.qat_fakequant_linear_bwd(dY_, X_, W_, s_, z_, bits, dX=gX, dW=gW, ds=gs, dz=gz,
                                       ws=ws_bwd if name == "staged" else None)
        torch.cuda.synchronize()
        _same_bits(f"dX {name}", host_bits(gX), dx_bits)
        _same_f32(f"dW {name}", gW.cpu().numpy(), r["dW"])
        _same_f32(f"dz {name}", gz.cpu().numpy(), r["dz"])
        assert rel_fro(gs.cpu().numpy(), r["ds"]) < TOL_F32, name


# + the E2E-QP MLP's gate/up shape, and the same at 2048 tokens (a 2048 x
# 11008 forward on 128x256 tiles)
E2E_CASES = CASES + [(4096, 11008, 4096, 2), (2048, 11008, 4096, 2)]


@pytest.mark.parametrize("M,out,inp,bits", E2E_CASES)
def test_e2e_exact(M, out, inp, bits):
    say(f"exact e2e M={M} out={out} in={inp} bits={bits}")
    e = synth.exact_sum_inputs(600 + bits, M, out, inp, bits)
    X, dY = O.bf16_bits_to_f64(e.X), O.bf16_bits_to_f64(e.dY)
    w_hat = O.e2e_w_hat(e.Wq, e.s, e.zp, inp, bits)
    _premise(X, w_hat)
    _premise(dY, w_hat.T)
    y_bits = _bits_of(X @ w_hat.T)
    del w_hat
    r = O.dequant_gemm_bwd_s(e.dY, e.X, e.Wq, e.s, e.zp, inp, bits)
    q = O.unpack_codes(e.Wq, inp, bits).astype(np.float64)
    gsum = (np.abs(r["Gw"]) * np.abs(q - np.repeat(e.zp.astype(np.float64), 64, axis=1)))
    assert gsum.reshape(out, inp // 64, 64).sum(-1).max() < 2.0 ** 24      # ds sums exactly
    del q, gsum
    dx_bits = _bits_of(r["dX"])

    X_, dY_, Wq_, s_, zp_ = dev_bf16(e.X), dev_bf16(e.dY), dev_u8(e.Wq), dev_f32(e.s), dev_f32(e.zp)
    ws = Q.workspace(Q.dequant_ws_bytes(out, inp, bits))
    for name, w in (("staged", ws), ("fused", None)):
        Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
        Q.qat_dequant_gemm_fwd(X_, Wq_, s_, zp_, bits, Y, ws=w)
        torch.cuda.synchronize()
        _same_bits(f"Y {name}", host_bits(Y), y_bits)
    ws_bwd = Q.workspace(Q.dequant_ws_bytes(out, inp, bits))
    for name in ("staged", "fused", "saved"):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        gz = torch.empty_like(gs)
        if name == "saved":
            Q.qat_dequant_gemm_bwd_s_saved(dY_, X_, Wq_, s_, zp_, ws, bits, gs, dX=gX, dz=gz)
        else:
            Q.qat_dequant_gemm_bwd_s(dY_, X_, Wq_, s_, zp_, bits, gs, dX=gX, dz=gz,
                                     ws=ws_bwd if name == "staged" else None)
        torch.cuda.synchronize()
        _same_bits(f"dX {name}", host_bits(gX), dx_bits)
        _same_f32(f"ds {name}", gs.cpu().numpy(), r["ds"])
        _same_f32(f"dz {name}", gz.cpu().numpy(), r["dz"])
