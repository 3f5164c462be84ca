"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (staged W_hat workspaces), against the fp64 oracle.

The Llama-2-7B q_proj workload (4096 x 4096, 2048 tokens) is compared whole:
every element of Y and dX within the element-wise bf16 GEMM bound
(tests/helpers.bf16_gemm_bound), every element of dW within the fp32
accumulation bound and exactly 0 where the oracle's quantiser clamps, ds and
dz over the whole tensor.

The larger workloads (the 7B MLP, the 70B gate and down at 2, 3 and 4 bits,
the E2E-QP MLP) are compared on samples that cross every output tile: one
token in every band of 128 tokens and one output (or input) column in every
band of 64, each as a whole row or column of Y and dX, against exact
restrictions the oracle computes from its full W_hat; dW, ds and dz on one
weight row in every band of 128 rows (all tokens, all inputs) and dW on one
input column in every band of 64. The backward formulas separate by weight
row and column, and quantisation is elementwise inside a group, so these are
exact restrictions of the full results. Samples include the first and last
token, row and column (the ragged edges of the tile grid).
Tolerances: the element-wise bounds above, and beside them relative
Frobenius 2e-2 for bf16 outputs and 1e-5 for fp32 outputs; codes bit-exact.
The backwards without a workspace (W_hat made inside the dX GEMM) give the
staging backward's dX bit for bit at q_proj and at the E2E-QP workloads.
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import (bf16_gemm_bound, check_bound, check_gemm_bf16, dev_bf16, dev_f32, dev_u8,
                           e2e_w_hat_exact, f32_gemm_bound, host_bits, rel_fro, say, tile_samples, w_hat_exact)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _lin(cfg, name, bits=None):
    for lin in synth.config(cfg, bits):
        if lin.name == name:
            return lin
    raise KeyError(name)


def _rows(t, idx):
    return t[torch.as_tensor(idx, device=t.device)]


def _cols(t, idx):
    return t[:, torch.as_tensor(idx, device=t.device)]


def _check_sampled_gemm(name, got_rows, got_cols, a_bits, w_hat, T, R):
    """Rows T of got = a w_hat^T (all columns) and columns R (all rows) within
    the element-wise bound, from the oracle's exact W_hat."""
    check_gemm_bf16(f"{name}[T,:]", got_rows, a_bits[T], w_hat, TOL_BF16)
    check_gemm_bf16(f"{name}[:,R]", got_cols, a_bits, w_hat[R], TOL_BF16)


def _check_grads_rows(gW, gs, gz, dY, X, W, s, z, b, R):
    """dW, ds, dz on weight rows R against the oracle (all tokens, all inputs)."""
    r = O.fakequant_bwd(dY[:, R], X, W[R], s[R], z[R], b)
    m = O.quantize(W[R], s[R], z[R], b)["m"]
    a, x = O.bf16_bits_to_f64(dY[:, R]), O.bf16_bits_to_f64(X)
    dw = _rows(gW, R).cpu().numpy()
    check_bound("dW[R,:]", dw, r["dW"], np.where(m, f32_gemm_bound(np.abs(a).T @ np.abs(x), a.shape[0]), 0.0))
    assert rel_fro(dw, r["dW"]) < TOL_F32
    assert np.array_equal(dw != 0, m & (r["Gw"] != 0))          # the clamp mask, exactly
    assert rel_fro(_rows(gs, R).cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(_rows(gz, R).cpu().numpy(), r["dz"]) < TOL_F32


def _check_dw_cols(gW, dY, X, W, s, z, b, C):
    """dW on input columns C (all weight rows): Gw[:, C] = dY^T X[:, C] masked by
    the quantiser of those elements (each with its own group's s, z)."""
    a, x = O.bf16_bits_to_f64(dY), O.bf16_bits_to_f64(X[:, C])
    gw = a.T @ x
    m = O.quantize(W[:, C], s[:, C // 64], z[:, C // 64], b, 1)["m"]
    ref = np.where(m, gw, 0.0)
    dw = _cols(gW, C).cpu().numpy()
    check_bound("dW[:,C]", dw, ref, np.where(m, f32_gemm_bound(np.abs(a).T @ np.abs(x), a.shape[0]), 0.0))


def _run_fakequant(lin, W, X, dY, s, z):
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    dW_, s_, z_, X_, dY_ = dev_f32(W), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.fakequant_ws_bytes(out, inp, b))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_fakequant_linear_fwd(X_, dW_, s_, z_, b, Y, ws=ws)
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gW = torch.empty(out, inp, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_fakequant_linear_bwd(dY_, X_, dW_, s_, z_, b, dX=gX, dW=gW, ds=gs, dz=gz, ws=ws)
    torch.cuda.synchronize()
    del dW_, ws
    return Y, gX, gW, gs, gz


def test_fakequant_q_proj_whole():
    lin = _lin(2, "q_proj")
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full fakequant q_proj whole M={M} out={out} in={inp} bits={b}")
    W, X, dY = lin.W(), lin.X(), lin.dY()
    s, z = O.init_minmax(W, b)
    s, z = synth.perturb_qparams(7, s, z, b)          # make clamp, mask and dz non-trivial
    Y, gX, gW, gs, gz = _run_fakequant(lin, W, X, dY, s, z)
    # the backward without a workspace (W_hat made in the dX GEMM's LDS)
    gX2 = torch.empty_like(gX)
    Q.qat_fakequant_linear_bwd(dev_bf16(dY), dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), b, dX=gX2)
    torch.cuda.synchronize()
    assert torch.equal(gX, gX2)
    del gX2
    wh = w_hat_exact(W, s, z, b)
    ry = check_gemm_bf16("Y", host_bits(Y), X, wh, TOL_BF16)
    rx = check_gemm_bf16("dX", host_bits(gX), dY, wh.T.copy(), TOL_BF16)
    r = O.fakequant_bwd(dY, X, W, s, z, b)
    m = O.quantize(W, s, z, b)["m"]
    a, x = O.bf16_bits_to_f64(dY), O.bf16_bits_to_f64(X)
    dw = gW.cpu().numpy()
    rw = check_bound("dW", dw, r["dW"], np.where(m, f32_gemm_bound(np.abs(a).T @ np.abs(x), M), 0.0))
    assert np.array_equal(dw != 0, m & (r["Gw"] != 0))
    assert rel_fro(dw, r["dW"]) < TOL_F32
    assert rel_fro(gs.cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(gz.cpu().numpy(), r["dz"]) < TOL_F32
    say(f"  largest error / bound: Y {ry:.3f} dX {rx:.3f} dW {rw:.3f}")


FQ_FULL = [
    # workload, linear, bits
    (3, "gate_proj", None),
    (3, "down_proj", None),
    (5, "gate_proj", 2),
    (5, "down_proj", 3),
    (5, "gate_proj", 4),
]


@pytest.mark.parametrize("cfg,name,bits", FQ_FULL)
def test_fakequant_full_size_every_tile(cfg, name, bits):
    lin = _lin(cfg, name, bits)
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full fakequant C{cfg} {name} M={M} out={out} in={inp} bits={b}")
    g = np.random.default_rng(1000 + cfg * 10 + b)
    W, X, dY = lin.W(), lin.X(), lin.dY()
    s, z = O.init_minmax(W, b)
    s, z = synth.perturb_qparams(7, s, z, b)
    Y, gX, gW, gs, gz = _run_fakequant(lin, W, X, dY, s, z)
    T, R, C = tile_samples(M, 128, g), tile_samples(out, 64, g), tile_samples(inp, 64, g)
    wh = w_hat_exact(W, s, z, b)
    _check_sampled_gemm("Y", host_bits(_rows(Y, T)), host_bits(_cols(Y, R)), X, wh, T, R)
    wht = wh.T.copy()
    del wh
    _check_sampled_gemm("dX", host_bits(_rows(gX, T)), host_bits(_cols(gX, C)), dY, wht, T, C)
    del wht
    _check_grads_rows(gW, gs, gz, dY, X, W, s, z, b, tile_samples(out, 128, g))
    _check_dw_cols(gW, dY, X, W, s, z, b, C)


def test_fakequant_full_size_fused_forward_bit_identical():
    # The no-workspace forward (fp32 weights quantised into LDS) at the q_proj
    # workload equals the staged forward bit for bit.
    lin = _lin(2, "q_proj")
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full fused forward M={M} out={out} in={inp}")
    W, X = lin.W(), lin.X()
    s, z = O.init_minmax(W, b)
    args = (dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), b)
    Y1 = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty_like(Y1)
    Q.qat_fakequant_linear_fwd(*args, Y1, ws=Q.workspace(Q.fakequant_ws_bytes(out, inp, b)))
    Q.qat_fakequant_linear_fwd(*args, Y2, ws=None)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


E2E_FULL = [
    (4, "gate_proj", None),
    (4, "down_proj", None),
    (5, "gate_proj", 2),
    (5, "down_proj", 4),
]


@pytest.mark.parametrize("cfg,name,bits", E2E_FULL)
def test_e2e_full_size_every_tile(cfg, name, bits):
    lin = _lin(cfg, name, bits)
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full e2e C{cfg} {name} M={M} out={out} in={inp} bits={b}")
    g = np.random.default_rng(2000 + cfg * 10 + b)
    Wq, s, z, X, dY = lin.Wq(), lin.s_e2e(), lin.z_e2e(), lin.X(), lin.dY()

    Wq_, s_, z_, X_, dY_ = dev_u8(Wq), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.dequant_ws_bytes(out, inp, b))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_dequant_gemm_fwd(X_, Wq_, s_, z_, b, Y, ws=ws)
    Yf = torch.empty_like(Y)
    Q.qat_dequant_gemm_fwd(X_, Wq_, s_, z_, b, Yf)               # fused, no workspace
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_dequant_gemm_bwd_s(dY_, X_, Wq_, s_, z_, b, gs, dX=gX, dz=gz, ws=ws)
    gX2 = torch.empty_like(gX)
    gs2 = torch.empty_like(gs)
    Q.qat_dequant_gemm_bwd_s(dY_, X_, Wq_, s_, z_, b, gs2, dX=gX2)            # no workspace
    torch.cuda.synchronize()
    assert torch.equal(Y, Yf)
    assert torch.equal(gX, gX2) and torch.equal(gs, gs2)
    del gX2, gs2

    T, R, C = tile_samples(M, 128, g), tile_samples(out, 64, g), tile_samples(inp, 64, g)
    wh = e2e_w_hat_exact(Wq, s, z, inp, b)
    _check_sampled_gemm("Y", host_bits(_rows(Y, T)), host_bits(_cols(Y, R)), X, wh, T, R)
    wht = wh.T.copy()
    del wh
    _check_sampled_gemm("dX", host_bits(_rows(gX, T)), host_bits(_cols(gX, C)), dY, wht, T, C)
    del wht
    Rg = tile_samples(out, 128, g)
    r = O.dequant_gemm_bwd_s(dY[:, Rg], X, Wq[Rg], s[Rg], z[Rg], inp, b)
    assert rel_fro(_rows(gs, Rg).cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(_rows(gz, Rg).cpu().numpy(), r["dz"]) < TOL_F32


@pytest.mark.parametrize("cfg,name,bits", [(2, "q_proj", None), (5, "down_proj", 3)])
def test_init_pack_full_size_bit_exact(cfg, name, bits):
    # init (s, z) and the codes over the whole weight at q_proj, on one row in
    # every band of 64 at the 70B down_proj; pack (bytes, zp) on those rows
    # (both are row-separable).
    lin = _lin(cfg, name, bits)
    out, inp, b = lin.out, lin.inp, lin.bits
    say(f"full init+pack C{cfg} {name} out={out} in={inp} bits={b}")
    g = np.random.default_rng(3000 + cfg)
    W = lin.W()
    W_ = dev_f32(W)
    s_ = torch.empty(out, inp // 64, device="cuda")
    z_ = torch.empty_like(s_)
    Q.qat_init_minmax(W_, b, s_, z_)
    Wq_ = torch.empty(out, inp * b // 8, dtype=torch.uint8, device="cuda")
    zp_ = torch.empty_like(s_)
    Q.qat_pack(W_, s_, z_, b, Wq_, zp_)
    torch.cuda.synchronize()
    R = np.arange(out) if cfg == 2 else tile_samples(out, 64, g)
    s_ref, z_ref = O.init_minmax(W[R], b)
    assert np.array_equal(_rows(s_, R).cpu().numpy(), s_ref)
    assert np.array_equal(_rows(z_, R).cpu().numpy(), z_ref)
    if cfg == 2:
        codes = torch.empty(out, inp, dtype=torch.uint8, device="cuda")
        Q.qat_quant_codes(W_, s_, z_, b, codes=codes)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), O.quant_codes(W, s_ref, z_ref, b)[0])
        R = tile_samples(out, 64, g)
        s_ref, z_ref = s_ref[R], z_ref[R]
    Wq_ref, zp_ref = O.pack(W[R], s_ref, z_ref, b)
    assert np.array_equal(_rows(Wq_, R).cpu().numpy(), Wq_ref)
    assert np.array_equal(_rows(zp_, R).cpu().numpy(), zp_ref)
