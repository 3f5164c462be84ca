"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded inputs.

Codes, W_hat bits, s, z and packed bytes must match bit-exactly. bf16 GEMM
outputs (Y, dX) must lie, element by element, within the bound that bf16
operands, fp32 accumulation and one bf16 rounding allow
(tests/helpers.bf16_gemm_bound: 2^-8 |ref| + ~2^-8 sum |a||w_hat|), and within
relative Frobenius error 2e-2 over the tensor; fp32 dW within an fp32
accumulation bound element by element and 1e-5 relative; ds and dz within
1e-5 relative; dz at min-max init must be exactly zero. Shapes span
several tiles of every tile configuration with ragged M and out tails; the
perturbed-qparams variant (s * 0.75, z moved by one on a quarter of the
groups) makes the clamp, the mask and dz non-trivial.
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import (check_bound, check_gemm_bf16, dev_bf16, dev_f32, dev_u8, e2e_w_hat_exact, f32_gemm_bound,
                           host_bits, rel_fro, say, w_hat_exact)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5

FQ_CASES = [
    # M, out, in, bits
    (128, 256, 256, 2),
    (300, 320, 512, 3),
    (1, 64, 64, 4),
    (2085, 4096, 256, 2),
    (100, 4160, 4160, 3),
    (4196, 4160, 128, 2),
    (2000, 3136, 128, 4),
]
E2E_CASES = [
    (128, 256, 256, 2),
    (300, 320, 512, 3),
    (77, 192, 128, 4),
    (2085, 4096, 256, 3),
    (100, 4160, 4160, 4),
]


def _inputs(M, out, inp, seed):
    W = synth.weight(seed, 0, out, inp, 0.02, True)
    X = synth.activations(seed, 0, M, inp, 4 if inp >= 64 else 0)
    dY = synth.grad_out(seed, 0, M, out)
    return W, X, dY


def _qparams(W, bits, perturb, seed):
    s, z = O.init_minmax(W, bits)
    if perturb:
        s, z = synth.perturb_qparams(seed, s, z, bits)
    return s, z


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


# ---------------------------------------------------------------------------
# a1 init, a2+a3 codes, a8 pack: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out,inp", [(256, 256), (100, 192), (7, 64), (4096, 4096)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_init_minmax_bit_exact(out, inp, bits):
    say(f"init out={out} in={inp} bits={bits}")
    W = synth.weight(7, bits, out, inp, 0.02, True)
    W[0, :64] = 0.25                                   # a constant group (degenerate floor)
    s_ref, z_ref = O.init_minmax(W, bits)
    s = torch.empty(out, inp // 64, device="cuda")
    z = torch.empty_like(s)
    Q.qat_init_minmax(dev_f32(W), bits, s, z)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(z.cpu().numpy(), z_ref)


@pytest.mark.parametrize("out,inp", [(256, 256), (130, 320), (4096, 4096)])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("perturb", [False, True])
def test_quant_codes_bit_exact(out, inp, bits, perturb):
    say(f"codes out={out} in={inp} bits={bits} perturb={perturb}")
    W = synth.weight(11, bits, out, inp, 0.02, True)
    s, z = _qparams(W, bits, perturb, 5)
    if perturb:
        z = (z + np.float32(0.4)).astype(np.float32)   # float z: the forward rounds it
    codes_ref, what_ref = O.quant_codes(W, s, z, bits)
    codes = torch.empty(out, inp, dtype=torch.uint8, device="cuda")
    what = torch.empty(out, inp, dtype=torch.bfloat16, device="cuda")
    Q.qat_quant_codes(dev_f32(W), dev_f32(s), dev_f32(z), bits, codes, what)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(host_bits(what), what_ref)


@pytest.mark.parametrize("out,inp", [(256, 256), (130, 320), (4096, 4096)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_bit_exact(out, inp, bits):
    say(f"pack out={out} in={inp} bits={bits}")
    W = synth.weight(13, bits, out, inp, 0.02, True)
    s, z = _qparams(W, bits, True, 9)
    z = (z + np.float32(0.3)).astype(np.float32)
    wq_ref, zp_ref = O.pack(W, s, z, bits)
    Wq = torch.empty(out, inp * bits // 8, dtype=torch.uint8, device="cuda")
    zp = torch.empty(out, inp // 64, device="cuda")
    Q.qat_pack(dev_f32(W), dev_f32(s), dev_f32(z), bits, Wq, zp)
    torch.cuda.synchronize()
    assert np.array_equal(Wq.cpu().numpy(), wq_ref)
    assert np.array_equal(zp.cpu().numpy(), zp_ref)


# ---------------------------------------------------------------------------
# a2-a7 fake-quant linear forward and STE backward
# ---------------------------------------------------------------------------

def _run_fq(M, out, inp, bits, W, X, dY, s, z, fused=False):
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    dW_, dX_ = dev_f32(W), dev_bf16(X)
    ds_, zs_ = dev_f32(s), dev_f32(z)
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_fakequant_linear_fwd(dX_, dW_, ds_, zs_, bits, Y, ws=None if fused else ws)
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gW = torch.empty(out, inp, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_fakequant_linear_bwd(dev_bf16(dY), dX_, dW_, ds_, zs_, bits, dX=gX, dW=gW, ds=gs, dz=gz, ws=ws)
    torch.cuda.synchronize()
    return host_bits(Y), host_bits(gX), gW.cpu().numpy(), gs.cpu().numpy(), gz.cpu().numpy()


def check_dw(dW, dY, X, m, r):
    """dW element by element: exactly 0 where the oracle's mask clamps, else
    within the fp32 accumulation bound over the M tokens of dY^T X."""
    a, x = O.bf16_bits_to_f64(dY), O.bf16_bits_to_f64(X)
    check_bound("dW", dW, r["dW"], np.where(m, f32_gemm_bound(np.abs(a).T @ np.abs(x), a.shape[0]), 0.0))
    assert np.array_equal(dW == 0, ~m | (r["Gw"] == 0))      # the mask itself


@pytest.mark.parametrize("M,out,inp,bits", FQ_CASES)
@pytest.mark.parametrize("perturb", [False, True])
def test_fakequant_fwd_bwd_parity(M, out, inp, bits, perturb):
    say(f"fakequant M={M} out={out} in={inp} bits={bits} perturb={perturb}")
    W, X, dY = _inputs(M, out, inp, 21 + bits)
    s, z = _qparams(W, bits, perturb, 3)
    Y, dX, dW, ds, dz = _run_fq(M, out, inp, bits, W, X, dY, s, z)
    r = O.fakequant_bwd(dY, X, W, s, z, bits)
    wh = w_hat_exact(W, s, z, bits)
    check_gemm_bf16("Y", Y, X, wh, TOL_BF16)
    check_gemm_bf16("dX", dX, dY, wh.T.copy(), TOL_BF16)
    m = O.quantize(W, s, z, bits)["m"]
    check_dw(dW, dY, X, m, r)
    assert rel_fro(dW, r["dW"]) < TOL_F32
    assert rel_fro(ds, r["ds"]) < TOL_F32
    assert np.array_equal(dW == 0, ~m | (r["Gw"] == 0))      # the mask itself
    if np.all(r["dz"] == 0):
        assert np.max(np.abs(dz)) <= 1e-30
    else:
        assert rel_fro(dz, r["dz"]) < TOL_F32
    if perturb:
        assert (~m).sum() > 0


@pytest.mark.parametrize("M,out,inp,bits", [(300, 320, 512, 3), (2085, 4096, 256, 2), (4196, 4160, 128, 4)])
def test_fused_forward_equals_staged_forward(M, out, inp, bits):
    # The fused kernel quantises fp32 tiles into LDS; the staged path writes a bf16
    # W_hat first. Same codes and same MFMA order -> identical bf16 outputs.
    say(f"fused-vs-staged M={M} out={out} in={inp} bits={bits}")
    W, X, _ = _inputs(M, out, inp, 31)
    s, z = _qparams(W, bits, True, 4)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    args = (dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits)
    Y1 = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty_like(Y1)
    Q.qat_fakequant_linear_fwd(*args, Y1, ws=ws)
    Q.qat_fakequant_linear_fwd(*args, Y2, ws=None)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Y1), host_bits(Y2))


def test_fused_forward_near_tie_fallback():
    # Weights placed exactly on and next to rounding ties exercise the exact
    # division path of the fused loader.
    say("fused near-tie")
    M, out, inp, bits = 64, 128, 256, 2
    g = np.random.default_rng(5)
    s = g.uniform(0.01, 0.02, (out, inp // 64)).astype(np.float32)
    z = np.full((out, inp // 64), 1.0, np.float32)
    half = g.integers(-2, 3, (out, inp)) + 0.5
    se = np.repeat(s, 64, 1)
    W = (half * se).astype(np.float32)
    W[:, ::3] = np.nextafter(W[:, ::3], np.float32(np.inf))
    W[:, 1::3] = np.nextafter(W[:, 1::3], np.float32(-np.inf))
    X = synth.activations(40, 0, M, inp)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    args = (dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits)
    Y1 = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty_like(Y1)
    Q.qat_fakequant_linear_fwd(*args, Y1, ws=ws)
    Q.qat_fakequant_linear_fwd(*args, Y2, ws=None)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Y1), host_bits(Y2))
    check_gemm_bf16("Y", host_bits(Y2), X, w_hat_exact(W, s, z, bits), TOL_BF16)


def test_ste_backward_near_tie_mask_exact():
    # Weights on and one ulp beside rounding ties, with zero points that push
    # codes past both ends, through the backward epilogue: its clamp mask (the
    # zero pattern of dW) must be exactly the oracle's fp32-quotient decision.
    say("bwd near-tie")
    M, out, inp, bits = 96, 128, 256, 2
    g = np.random.default_rng(9)
    s = g.uniform(0.01, 0.02, (out, inp // 64)).astype(np.float32)
    z = g.integers(0, 4, (out, inp // 64)).astype(np.float32)
    half = g.integers(-4, 5, (out, inp)) + 0.5
    W = (half * np.repeat(s, 64, 1)).astype(np.float32)
    W[:, ::3] = np.nextafter(W[:, ::3], np.float32(np.inf))
    W[:, 1::3] = np.nextafter(W[:, 1::3], np.float32(-np.inf))
    X = synth.activations(41, 0, M, inp)
    dY = synth.grad_out(41, 0, M, out)
    gW = torch.empty(out, inp, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_fakequant_linear_bwd(dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits,
                               dW=gW, ds=gs, dz=gz)
    torch.cuda.synchronize()
    m = O.quantize(W, s, z, bits)["m"]
    r = O.fakequant_bwd(dY, X, W, s, z, bits)
    assert 0.05 < m.mean() < 0.95
    assert np.array_equal(gW.cpu().numpy() != 0, m & (r["Gw"] != 0))
    assert rel_fro(gW.cpu().numpy(), r["dW"]) < TOL_F32
    assert rel_fro(gs.cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32


def test_bwd_optional_outputs():
    say("bwd optional outputs")
    M, out, inp, bits = 96, 192, 256, 3
    W, X, dY = _inputs(M, out, inp, 50)
    s, z = _qparams(W, bits, True, 6)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    r = O.fakequant_bwd(dY, X, W, s, z, bits)
    gW = torch.full((out, inp), 7.0, device="cuda")
    Q.qat_fakequant_linear_bwd(dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits,
                               dW=gW, ws=ws)
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    Q.qat_fakequant_linear_bwd(dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits,
                               dX=gX, ws=ws)
    torch.cuda.synchronize()
    assert rel_fro(gW.cpu().numpy(), r["dW"]) < TOL_F32
    check_gemm_bf16("dX", host_bits(gX), dY, w_hat_exact(W, s, z, bits).T.copy(), TOL_BF16)


# ---------------------------------------------------------------------------
# a9/a10 E2E-QP
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,out,inp,bits", E2E_CASES)
def test_e2e_parity(M, out, inp, bits):
    say(f"e2e M={M} out={out} in={inp} bits={bits}")
    Wq = synth.packed_codes(61, bits, out, inp, bits)
    s = synth.e2e_scales(61, bits, out, inp)
    z = synth.e2e_zeros(61, bits, out, inp, bits)
    X = synth.activations(61, bits, M, inp)
    dY = synth.grad_out(61, bits, M, out)
    ws = Q.workspace(Q.dequant_ws_bytes(out, inp, bits))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    dq, ds_, dz_ = dev_u8(Wq), dev_f32(s), dev_f32(z)
    Q.qat_dequant_gemm_fwd(dev_bf16(X), dq, ds_, dz_, bits, Y)
    Y_staged = torch.empty_like(Y)
    Q.qat_dequant_gemm_fwd(dev_bf16(X), dq, ds_, dz_, bits, Y_staged, ws=ws)
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_dequant_gemm_bwd_s(dev_bf16(dY), dev_bf16(X), dq, ds_, dz_, bits, gs, dX=gX, dz=gz, ws=ws)
    torch.cuda.synchronize()
    r = O.dequant_gemm_bwd_s(dY, X, Wq, s, z, inp, bits)
    wh = e2e_w_hat_exact(Wq, s, z, inp, bits)
    check_gemm_bf16("Y", host_bits(Y), X, wh, TOL_BF16)
    # fused (codes dequantised into LDS) and staged (W_hat in the workspace)
    # forwards multiply the same bf16 operand in the same k order
    assert np.array_equal(host_bits(Y), host_bits(Y_staged))
    check_gemm_bf16("dX", host_bits(gX), dY, wh.T.copy(), TOL_BF16)
    assert rel_fro(gs.cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32


@pytest.mark.parametrize("M,out,inp,bits", [(300, 320, 512, 3), (2085, 4096, 256, 2), (100, 4160, 4160, 3),
                                             (4196, 4160, 128, 4), (2048, 4096, 4096, 2)])
def test_saved_backward_equals_staging_backward(M, out, inp, bits):
    # The backward on the forward's saved W_hat (dX reads W_hat [out, in] in
    # place) against the staging backward (W_hat^T staged from W): the same
    # bf16 operand in the same k order, so every output is bit-identical; the
    # E2E pair likewise, on the W_hat its staged forward left in the workspace.
    say(f"saved backward M={M} out={out} in={inp} bits={bits}")
    W, X, dY = _inputs(M, out, inp, 90 + bits)
    s, z = _qparams(W, bits, True, 9)
    dY_, X_, W_, s_, z_ = dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z)
    ws_fwd = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    ws_bwd = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_fakequant_linear_fwd(X_, W_, s_, z_, bits, Y, ws=ws_fwd)
    outs = []
    for saved in (False, True):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gW = torch.empty(out, inp, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        gz = torch.empty_like(gs)
        if saved:
            Q.qat_fakequant_linear_bwd_saved(dY_, X_, W_, s_, z_, ws_fwd, bits, dX=gX, dW=gW, ds=gs, dz=gz)
        else:
            Q.qat_fakequant_linear_bwd(dY_, X_, W_, s_, z_, bits, dX=gX, dW=gW, ds=gs, dz=gz, ws=ws_bwd)
        outs.append((host_bits(gX), gW.cpu().numpy(), gs.cpu().numpy(), gz.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    Wq = synth.packed_codes(62, bits, out, inp, bits)
    es, ez = dev_f32(synth.e2e_scales(62, bits, out, inp)), dev_f32(synth.e2e_zeros(62, bits, out, inp, bits))
    dq = dev_u8(Wq)
    Q.qat_dequant_gemm_fwd(X_, dq, es, ez, bits, Y, ws=ws_fwd)
    outs = []
    for saved in (False, True):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        gz = torch.empty_like(gs)
        if saved:
            Q.qat_dequant_gemm_bwd_s_saved(dY_, X_, dq, es, ez, ws_fwd, bits, gs, dX=gX, dz=gz)
        else:
            Q.qat_dequant_gemm_bwd_s(dY_, X_, dq, es, ez, bits, gs, dX=gX, dz=gz, ws=ws_bwd)
        outs.append((host_bits(gX), gs.cpu().numpy(), gz.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M,out,inp,bits", [(128, 256, 256, 2), (300, 320, 512, 3), (1, 64, 64, 4),
                                             (2085, 4096, 256, 2), (100, 4160, 4160, 3), (4196, 4160, 128, 4)])
def test_backward_without_workspace(M, out, inp, bits):
    # ws = NULL: the dX GEMM makes W_hat in LDS from the fp32 master weight
    # (fake-quant) or the packed codes (E2E-QP), read along the weight's rows.
    # Same bf16 operand, same k order as the staging backward: every output is
    # bit-identical to it, and dX is inside the element-wise bound.
    say(f"no-workspace backward M={M} out={out} in={inp} bits={bits}")
    W, X, dY = _inputs(M, out, inp, 110 + bits)
    s, z = _qparams(W, bits, True, 11)
    dY_, X_, W_, s_, z_ = dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    outs = []
    for w in (ws, None):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gW = torch.empty(out, inp, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        gz = torch.empty_like(gs)
        Q.qat_fakequant_linear_bwd(dY_, X_, W_, s_, z_, bits, dX=gX, dW=gW, ds=gs, dz=gz, ws=w)
        outs.append((gX, gW, gs, gz))
    torch.cuda.synchronize()
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    check_gemm_bf16("dX", host_bits(outs[1][0]), dY, w_hat_exact(W, s, z, bits).T.copy(), TOL_BF16)
    Wq = synth.packed_codes(112, bits, out, inp, bits)
    es, ez = synth.e2e_scales(112, bits, out, inp), synth.e2e_zeros(112, bits, out, inp, bits)
    dq, es_, ez_ = dev_u8(Wq), dev_f32(es), dev_f32(ez)
    outs = []
    for w in (ws, None):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gs = torch.empty(out, inp // 64, device="cuda")
        Q.qat_dequant_gemm_bwd_s(dY_, X_, dq, es_, ez_, bits, gs, dX=gX, ws=w)
        outs.append((gX, gs))
    torch.cuda.synchronize()
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    check_gemm_bf16("dX", host_bits(outs[1][0]), dY, e2e_w_hat_exact(Wq, es, ez, inp, bits).T.copy(), TOL_BF16)


def test_backward_without_workspace_near_tie():
    # weights on and one ulp beside rounding ties through the transposed fp32
    # ring of the no-workspace dX: the exact-division fallback gives the
    # staging backward's W_hat, so dX is bit-identical
    say("no-workspace backward near-tie")
    M, out, inp, bits = 96, 128, 256, 2
    g = np.random.default_rng(12)
    s = g.uniform(0.01, 0.02, (out, inp // 64)).astype(np.float32)
    z = g.integers(0, 4, (out, inp // 64)).astype(np.float32)
    half = g.integers(-4, 5, (out, inp)) + 0.5
    W = (half * np.repeat(s, 64, 1)).astype(np.float32)
    W[:, ::3] = np.nextafter(W[:, ::3], np.float32(np.inf))
    W[:, 1::3] = np.nextafter(W[:, 1::3], np.float32(-np.inf))
    dY = synth.grad_out(42, 0, M, out)
    args = (dev_bf16(dY), dev_bf16(synth.activations(42, 0, M, inp)), dev_f32(W), dev_f32(s), dev_f32(z), bits)
    g1 = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    g2 = torch.empty_like(g1)
    Q.qat_fakequant_linear_bwd(*args, dX=g1, ws=Q.workspace(Q.fakequant_ws_bytes(out, inp, bits)))
    Q.qat_fakequant_linear_bwd(*args, dX=g2)
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    check_gemm_bf16("dX", host_bits(g2), dY, w_hat_exact(W, s, z, bits).T.copy(), TOL_BF16)


RAGGED_OUT = [
    # M, out, in, bits, group: out a multiple of 4 but not of 64
    (300, 4100, 512, 2, 64),
    (77, 11000, 256, 3, 64),
    (130, 100, 256, 4, 32),
    (64, 36, 128, 2, 128),
    (1, 4100, 192, 3, 192),          # channel-wise
]


@pytest.mark.parametrize("M,out,inp,bits,group", RAGGED_OUT)
def test_ragged_out(M, out, inp, bits, group):
    # every GEMM call with out not a multiple of 64 (rows of dY only 8-byte
    # aligned when out % 8 == 4; the dX contraction over out ends mid-slab):
    # forward staged and fused, the three backwards (staging, saved W_hat, no
    # workspace) against the oracle and against each other, and the E2E-QP pair
    say(f"ragged out M={M} out={out} in={inp} bits={bits} group={group}")
    W = synth.weight(120, bits, out, inp, 0.02, True)
    X = synth.activations(120, bits, M, inp, 4)
    dY = synth.grad_out(120, bits, M, out)
    s, z = O.init_minmax(W, bits, group)
    s, z = synth.perturb_qparams(12, s, z, bits)
    G = inp // group
    dY_, X_, W_, s_, z_ = dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Yf = torch.empty_like(Y)
    Q.qat_fakequant_linear_fwd(X_, W_, s_, z_, bits, Y, ws=ws, group=group)
    saved = ws.clone()
    Q.qat_fakequant_linear_fwd(X_, W_, s_, z_, bits, Yf, group=group)
    outs = []
    for variant in ("staging", "saved", "no workspace"):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gW = torch.empty(out, inp, device="cuda")
        gs = torch.empty(out, G, device="cuda")
        gz = torch.empty_like(gs)
        if variant == "saved":
            Q.qat_fakequant_linear_bwd_saved(dY_, X_, W_, s_, z_, saved, bits, dX=gX, dW=gW, ds=gs, dz=gz, group=group)
        else:
            Q.qat_fakequant_linear_bwd(dY_, X_, W_, s_, z_, bits, dX=gX, dW=gW, ds=gs, dz=gz,
                                       ws=ws if variant == "staging" else None, group=group)
        outs.append((gX, gW, gs, gz))
    torch.cuda.synchronize()
    assert torch.equal(Y, Yf)
    for o in outs[1:]:
        assert torch.equal(outs[0][0], o[0]) and torch.equal(outs[0][1], o[1])
        assert rel_fro(o[2].cpu().numpy(), outs[0][2].cpu().numpy()) < 1e-6
    wh = w_hat_exact(W, s, z, bits, group)
    check_gemm_bf16("Y", host_bits(Y), X, wh, TOL_BF16)
    check_gemm_bf16("dX", host_bits(outs[0][0]), dY, wh.T.copy(), TOL_BF16)
    r = O.fakequant_bwd(dY, X, W, s, z, bits, group)
    m = O.quantize(W, s, z, bits, group)["m"]
    gX, gW, gs, gz = outs[0]
    check_dw(gW.cpu().numpy(), dY, X, m, r)
    assert rel_fro(gs.cpu().numpy(), r["ds"]) < TOL_F32
    if np.any(r["dz"] != 0):
        assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32
    # E2E-QP on the packed weight of the same shape
    Wq = synth.packed_codes(121, bits, out, inp, bits)
    g = np.random.default_rng(121)
    es = g.uniform(0.005, 0.05, (out, G)).astype(np.float32)
    ez = g.integers(0, 1 << bits, (out, G)).astype(np.float32)
    dq, es_, ez_ = dev_u8(Wq), dev_f32(es), dev_f32(ez)
    Y1 = torch.empty_like(Y)
    Y2 = torch.empty_like(Y)
    Q.qat_dequant_gemm_fwd(X_, dq, es_, ez_, bits, Y1, ws=ws, group=group)
    Q.qat_dequant_gemm_fwd(X_, dq, es_, ez_, bits, Y2, group=group)
    outs = []
    for w in (ws, None):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gs = torch.empty(out, G, device="cuda")
        gz = torch.empty_like(gs)
        Q.qat_dequant_gemm_bwd_s(dY_, X_, dq, es_, ez_, bits, gs, dX=gX, dz=gz, ws=w, group=group)
        outs.append((gX, gs, gz))
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(outs[0][0], outs[1][0])
    whe = e2e_w_hat_exact(Wq, es, ez, inp, bits, group)
    check_gemm_bf16("Y", host_bits(Y1), X, whe, TOL_BF16)
    check_gemm_bf16("dX", host_bits(outs[0][0]), dY, whe.T.copy(), TOL_BF16)
    r = O.dequant_gemm_bwd_s(dY, X, Wq, es, ez, inp, bits, group)
    assert rel_fro(outs[0][1].cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(outs[0][2].cpu().numpy(), r["dz"]) < TOL_F32


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_then_dequant_gemm_equals_fakequant_forward(bits):
    # Cross-path: with the hard-rounded zero point, dequant(pack(W)) is the same
    # bf16 operand as the fake-quant W_hat, so the two forwards agree bit for bit.
    say(f"cross-path bits={bits}")
    M, out, inp = 300, 320, 512
    W, X, _ = _inputs(M, out, inp, 70 + bits)
    s, z = _qparams(W, bits, True, 8)
    dW_, ds_, dz_ = dev_f32(W), dev_f32(s), dev_f32(z)
    Wq = torch.empty(out, inp * bits // 8, dtype=torch.uint8, device="cuda")
    zp = torch.empty(out, inp // 64, device="cuda")
    Q.qat_pack(dW_, ds_, dz_, bits, Wq, zp)
    Y1 = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty_like(Y1)
    Xd = dev_bf16(X)
    Y3 = torch.empty_like(Y1)
    Q.qat_dequant_gemm_fwd(Xd, Wq, ds_, zp, bits, Y1)
    Q.qat_dequant_gemm_fwd(Xd, Wq, ds_, zp, bits, Y3, ws=Q.workspace(Q.dequant_ws_bytes(out, inp, bits)))
    Q.qat_fakequant_linear_fwd(Xd, dW_, ds_, dz_, bits, Y2, ws=Q.workspace(Q.fakequant_ws_bytes(out, inp, bits)))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Y1), host_bits(Y2))
    assert np.array_equal(host_bits(Y3), host_bits(Y2))


# ---------------------------------------------------------------------------
# ABI contract on the device: errors touch nothing
# ---------------------------------------------------------------------------

def test_errors_leave_outputs_untouched():
    # through the raw C ABI (the binding would refuse these before the call):
    # every refused call leaves its outputs as they were
    say("abi errors")
    L = Q.lib()
    st = torch.cuda.current_stream().cuda_stream
    W = torch.randn(64, 128, device="cuda")
    s = torch.full((64, 2), 3.0, device="cuda")
    z = torch.full((64, 2), 4.0, device="cuda")
    p = lambda t: t.data_ptr()
    assert L.qat_init_minmax(p(W), 64, 128, 64, 5, p(s), p(z), st) == 3           # bits
    assert L.qat_init_minmax(p(W), 64, 96, 64, 2, p(s), p(z), st) == 2            # in % 64 != 0
    X = torch.zeros(8, 128, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((8, 64), 1.5, dtype=torch.bfloat16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    gX = torch.empty(8, 128, dtype=torch.bfloat16, device="cuda")
    assert L.qat_fakequant_linear_fwd(p(X), p(W), p(s), p(z), 8, 64, 128, 64, 2, p(Y), p(small), 16, st) == 6
    assert L.qat_quant_codes(p(W), p(s), p(z), 64, 128, 64, 2, None, p(W), st) == 8   # output over input
    assert L.qat_fakequant_linear_bwd(p(Y), p(X), p(W), p(s), p(z), 8, 64, 128, 64, 2, p(gX), None, p(s), None,
                                      None, 0, st) == 1                                # ds without dz
    torch.cuda.synchronize()
    assert torch.all(s == 3.0) and torch.all(z == 4.0) and torch.all(Y == 1.5)
