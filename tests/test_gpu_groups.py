"""GPU parity at the other group sizes (groups of 32 and 128 along `in`, and
channel-wise: one group per weight row), every C-ABI call against the fp64
oracle. Same bars as at group 64: s, z, codes, W_hat bits, packed bytes and
zp bit-exact; bf16 Y and dX within the element-wise bf16 GEMM bound
(tests/helpers.bf16_gemm_bound) and relative Frobenius 2e-2; fp32 dW, ds, dz
within 1e-5; the fused (no-workspace) forwards bit-identical to the staged
ones. Shapes cover both gradient tile configurations, ragged output tiles and
a channel-wise row length that is not a power of two (192), and each way
the gradient epilogue finishes a group: stored per 64- or 32-column chunk,
summed over the tile's chunks and stored (group 128, or a whole row that fits
one tile), or summed per tile and accumulated (whole rows over several
tiles). The backwards on the forward's saved W_hat, and those without a
workspace (W_hat made in the dX GEMM's LDS), match the staging ones bit
for bit at every group size (ds, dz of whole-row groups to fp32 reassociation:
their per-tile atomic adds meet in no fixed order).
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import (check_gemm_bf16, dev_bf16, dev_f32, dev_u8, e2e_w_hat_exact, host_bits, rel_fro, say,
                           w_hat_exact)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5

CASES = [
    # M, out, in, group (None: the whole row), bits
    (300, 320, 512, 32, 2),
    (300, 320, 512, 128, 3),
    (300, 320, 512, None, 4),
    (77, 192, 192, None, 2),
    (128, 256, 256, 32, 4),
    (100, 4096, 4096, 128, 2),
    (100, 4096, 4096, 32, 3),
    (64, 192, 128, None, 3),          # whole row = one 128-column tile: stored
    (100, 4096, 4096, None, 2),       # whole row over 16 tiles of 256: accumulated
    (16, 65536, 256, None, 4),        # whole row = one 256-column tile: stored
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _gs(group, inp):
    return inp if group is None else group


@pytest.mark.parametrize("M,out,inp,group,bits", CASES)
def test_init_codes_pack_bit_exact(M, out, inp, group, bits):
    gs = _gs(group, inp)
    say(f"groups init/codes/pack out={out} in={inp} group={gs} bits={bits}")
    W = synth.weight(90, bits, out, inp, 0.02, True)
    Wd = dev_f32(W)
    s = torch.empty(out, inp // gs, device="cuda")
    z = torch.empty_like(s)
    Q.qat_init_minmax(Wd, bits, s, z, group=gs)
    codes = torch.empty(out, inp, dtype=torch.uint8, device="cuda")
    W_hat = torch.empty(out, inp, dtype=torch.bfloat16, device="cuda")
    Q.qat_quant_codes(Wd, s, z, bits, codes=codes, W_hat=W_hat, group=gs)
    Wq = torch.empty(out, inp * bits // 8, dtype=torch.uint8, device="cuda")
    zp = torch.empty_like(s)
    Q.qat_pack(Wd, s, z, bits, Wq, zp, group=gs)
    torch.cuda.synchronize()
    s_ref, z_ref = O.init_minmax(W, bits, gs)
    assert np.array_equal(s.cpu().numpy(), s_ref) and np.array_equal(z.cpu().numpy(), z_ref)
    c_ref, wh_ref = O.quant_codes(W, s_ref, z_ref, bits, gs)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_bits(W_hat), wh_ref)
    Wq_ref, zp_ref = O.pack(W, s_ref, z_ref, bits, gs)
    assert np.array_equal(Wq.cpu().numpy(), Wq_ref) and np.array_equal(zp.cpu().numpy(), zp_ref)


def _same_backward(outs, whole_rows, n_exact):
    """The saved-W_hat backward against the staging one: the first n_exact
    outputs (dX, dW) bit-identical; ds and dz too, except for whole-row groups,
    whose sums over rows wider than a gradient tile meet by one atomic add per
    tile in no fixed order, so they agree to fp32 reassociation."""
    for k, (a_, b_) in enumerate(zip(*outs)):
        if k < n_exact or not whole_rows:
            assert torch.equal(a_, b_), k
        else:
            assert rel_fro(a_.cpu().numpy(), b_.cpu().numpy()) < 1e-6, k


@pytest.mark.parametrize("M,out,inp,group,bits", CASES)
def test_fakequant_fwd_bwd(M, out, inp, group, bits):
    gs = _gs(group, inp)
    say(f"groups fakequant M={M} out={out} in={inp} group={gs} bits={bits}")
    W = synth.weight(91, bits, out, inp, 0.02, True)
    X = synth.activations(91, bits, M, inp, 4)
    dY = synth.grad_out(91, bits, M, out)
    s, z = O.init_minmax(W, bits, gs)
    s, z = synth.perturb_qparams(5, s, z, bits)
    Wd, sd, zd, Xd, dYd = dev_f32(W), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, bits))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Yf = torch.empty_like(Y)
    Q.qat_fakequant_linear_fwd(Xd, Wd, sd, zd, bits, Y, ws=ws, group=gs)
    saved = ws.clone()                                          # the forward's W_hat
    Q.qat_fakequant_linear_fwd(Xd, Wd, sd, zd, bits, Yf, ws=None, group=gs)
    outs = []
    for variant in ("staging", "saved", "no workspace"):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gW = torch.empty(out, inp, device="cuda")
        gs_ = torch.full((out, inp // gs), 9.0, device="cuda")  # must be overwritten, not accumulated
        gz = torch.full_like(gs_, 9.0)
        if variant == "saved":
            Q.qat_fakequant_linear_bwd_saved(dYd, Xd, Wd, sd, zd, saved, bits, dX=gX, dW=gW, ds=gs_, dz=gz,
                                             group=gs)
        else:
            Q.qat_fakequant_linear_bwd(dYd, Xd, Wd, sd, zd, bits, dX=gX, dW=gW, ds=gs_, dz=gz,
                                       ws=ws if variant == "staging" else None, group=gs)
        outs.append((gX, gW, gs_, gz))
    torch.cuda.synchronize()
    _same_backward(outs[:2], gs == inp, 2)
    _same_backward(outs[::2], gs == inp, 2)
    gX, gW, gs_, gz = outs[0]
    assert torch.equal(Y, Yf)
    wh = w_hat_exact(W, s, z, bits, gs)
    check_gemm_bf16("Y", host_bits(Y), X, wh, TOL_BF16)
    r = O.fakequant_bwd(dY, X, W, s, z, bits, gs)
    check_gemm_bf16("dX", host_bits(gX), dY, wh.T.copy(), TOL_BF16)
    assert rel_fro(gW.cpu().numpy(), r["dW"]) < TOL_F32
    assert rel_fro(gs_.cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32


@pytest.mark.parametrize("M,out,inp,group,bits", CASES)
def test_e2e_fwd_bwd(M, out, inp, group, bits):
    gs = _gs(group, inp)
    say(f"groups e2e M={M} out={out} in={inp} group={gs} bits={bits}")
    g = np.random.default_rng(92 + bits)
    Wq = synth.packed_codes(92, bits, out, inp, bits)
    s = g.uniform(0.005, 0.05, (out, inp // gs)).astype(np.float32)
    z = g.integers(0, 1 << bits, (out, inp // gs)).astype(np.float32)
    X = synth.activations(92, bits, M, inp)
    dY = synth.grad_out(92, bits, M, out)
    Wqd, sd, zd, Xd, dYd = dev_u8(Wq), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.dequant_ws_bytes(out, inp, bits))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Yf = torch.empty_like(Y)
    Q.qat_dequant_gemm_fwd(Xd, Wqd, sd, zd, bits, Y, ws=ws, group=gs)
    saved = ws.clone()                                          # the forward's W_hat
    Q.qat_dequant_gemm_fwd(Xd, Wqd, sd, zd, bits, Yf, group=gs)
    outs = []
    for variant in ("staging", "saved", "no workspace"):
        gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
        gs_ = torch.full((out, inp // gs), 9.0, device="cuda")
        gz = torch.full_like(gs_, 9.0)
        if variant == "saved":
            Q.qat_dequant_gemm_bwd_s_saved(dYd, Xd, Wqd, sd, zd, saved, bits, gs_, dX=gX, dz=gz, group=gs)
        else:
            Q.qat_dequant_gemm_bwd_s(dYd, Xd, Wqd, sd, zd, bits, gs_, dX=gX, dz=gz,
                                     ws=ws if variant == "staging" else None, group=gs)
        outs.append((gX, gs_, gz))
    torch.cuda.synchronize()
    _same_backward(outs[:2], gs == inp, 1)
    _same_backward(outs[::2], gs == inp, 1)
    gX, gs_, gz = outs[0]
    assert torch.equal(Y, Yf)
    wh = e2e_w_hat_exact(Wq, s, z, inp, bits, gs)
    check_gemm_bf16("Y", host_bits(Y), X, wh, TOL_BF16)
    r = O.dequant_gemm_bwd_s(dY, X, Wq, s, z, inp, bits, gs)
    check_gemm_bf16("dX", host_bits(gX), dY, wh.T.copy(), TOL_BF16)
    assert rel_fro(gs_.cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32
