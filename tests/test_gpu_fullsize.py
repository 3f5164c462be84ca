"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (staged W_hat / W_hat^T workspaces), on sampled outputs.

The oracle computes the sampled outputs one by one from its own definitions:
the backward formulas are separable by weight row and quantisation is
elementwise within a group, so
  Y[T, R]      = oracle forward of X[T] against the rows R of W,
  dX[T, cols]  = oracle backward of dY[T] against the column groups J of W,
  dW, ds, dz   = oracle backward of dY[:, R] against the rows R of W,
are exact restrictions of the full results. Samples always include the first
and last token, row and group (the ragged edges of the tile grid).
Tolerances as in the small-shape tests: relative Frobenius error over the
samples, 2e-2 for bf16 outputs, 1e-5 for fp32 outputs; codes bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import dev_bf16, dev_f32, dev_u8, host_bits, rel_fro, say

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
NS = 16          # sampled tokens / rows
NJ = 4           # sampled 64-column groups


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _pick(n, k, rng):
    """k sorted distinct indices in [0, n) including 0 and n - 1."""
    mid = rng.choice(np.arange(1, n - 1), size=min(k, n) - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid]))


def _cols(J):
    return (J[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)


def _packed_cols(Wq, J, bits):
    """Byte columns of the packed rows that hold the code groups J."""
    gb = 64 * bits // 8
    return Wq[:, (J[:, None] * gb + np.arange(gb)[None, :]).reshape(-1)]


def _lin(cfg, name, bits=None):
    for lin in synth.config(cfg, bits):
        if lin.name == name:
            return lin
    raise KeyError(name)


def _rows(t, idx):
    return t[torch.as_tensor(idx, device=t.device)]


FQ_FULL = [
    # workload, linear, bits
    (2, "q_proj", None),
    (3, "gate_proj", None),
    (3, "down_proj", None),
    (5, "gate_proj", 2),
    (5, "down_proj", 3),
    (5, "gate_proj", 4),
]


@pytest.mark.parametrize("cfg,name,bits", FQ_FULL)
def test_fakequant_full_size_sampled(cfg, name, bits):
    lin = _lin(cfg, name, bits)
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full fakequant C{cfg} {name} M={M} out={out} in={inp} bits={b}")
    g = np.random.default_rng(1000 + cfg * 10 + b)
    W, X, dY = lin.W(), lin.X(), lin.dY()
    s, z = O.init_minmax(W, b)
    s, z = synth.perturb_qparams(7, s, z, b)          # make clamp, mask and dz non-trivial

    dW_, s_, z_, X_, dY_ = dev_f32(W), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.fakequant_ws_bytes(M, out, inp))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_fakequant_linear_fwd(X_, dW_, s_, z_, b, Y, ws=ws)
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gW = torch.empty(out, inp, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_fakequant_linear_bwd(dY_, X_, dW_, s_, z_, b, dX=gX, dW=gW, ds=gs, dz=gz, ws=ws)
    torch.cuda.synchronize()

    T, R, J = _pick(M, NS, g), _pick(out, NS, g), _pick(inp // 64, NJ, g)
    C = _cols(J)
    # forward on sampled tokens x rows
    y = O.bf16_bits_to_f64(host_bits(_rows(Y, T)))[:, R]
    y_ref = O.fakequant_fwd(X[T], W[R], s[R], z[R], b)
    assert rel_fro(y, y_ref) < TOL_BF16
    # dX on sampled tokens x column groups
    dx = O.bf16_bits_to_f64(host_bits(_rows(gX, T)))[:, C]
    dx_ref = O.fakequant_bwd(dY[T], X[T][:, C], W[:, C], s[:, J], z[:, J], b)["dX"]
    assert rel_fro(dx, dx_ref) < TOL_BF16
    # dW, ds, dz on sampled weight rows (all tokens, all inputs)
    r = O.fakequant_bwd(dY[:, R], X, W[R], s[R], z[R], b)
    assert rel_fro(_rows(gW, R).cpu().numpy(), r["dW"]) < TOL_F32
    assert rel_fro(_rows(gs, R).cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(_rows(gz, R).cpu().numpy(), r["dz"]) < TOL_F32
    # the clamp mask of the sampled rows is exactly the oracle's
    m = O.quantize(W[R], s[R], z[R], b)["m"]
    assert np.array_equal(_rows(gW, R).cpu().numpy() != 0, m & (r["Gw"] != 0))


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
    Q.qat_fakequant_linear_fwd(*args, Y1, ws=Q.workspace(Q.fakequant_ws_bytes(M, out, inp)))
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
def test_e2e_full_size_sampled(cfg, name, bits):
    lin = _lin(cfg, name, bits)
    M, out, inp, b = lin.m, lin.out, lin.inp, lin.bits
    say(f"full e2e C{cfg} {name} M={M} out={out} in={inp} bits={b}")
    g = np.random.default_rng(2000 + cfg * 10 + b)
    Wq, s, z, X, dY = lin.Wq(), lin.s_e2e(), lin.z_e2e(), lin.X(), lin.dY()

    Wq_, s_, z_, X_, dY_ = dev_u8(Wq), dev_f32(s), dev_f32(z), dev_bf16(X), dev_bf16(dY)
    ws = Q.workspace(Q.dequant_ws_bytes(M, out, inp))
    Y = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
    Q.qat_dequant_gemm_fwd(X_, Wq_, s_, z_, b, Y, ws=ws)
    Yf = torch.empty_like(Y)
    Q.qat_dequant_gemm_fwd(X_, Wq_, s_, z_, b, Yf)               # fused, no workspace
    gX = torch.empty(M, inp, dtype=torch.bfloat16, device="cuda")
    gs = torch.empty(out, inp // 64, device="cuda")
    gz = torch.empty_like(gs)
    Q.qat_dequant_gemm_bwd_s(dY_, X_, Wq_, s_, z_, b, gs, dX=gX, dz=gz, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yf)

    T, R, J = _pick(M, NS, g), _pick(out, NS, g), _pick(inp // 64, NJ, g)
    C = _cols(J)
    y = O.bf16_bits_to_f64(host_bits(_rows(Y, T)))[:, R]
    assert rel_fro(y, O.dequant_gemm_fwd(X[T], Wq[R], s[R], z[R], inp, b)) < TOL_BF16
    dx = O.bf16_bits_to_f64(host_bits(_rows(gX, T)))[:, C]
    dx_ref = O.dequant_gemm_bwd_s(dY[T], X[T][:, C], _packed_cols(Wq, J, b), s[:, J], z[:, J], 64 * len(J), b)["dX"]
    assert rel_fro(dx, dx_ref) < TOL_BF16
    r = O.dequant_gemm_bwd_s(dY[:, R], X, Wq[R], s[R], z[R], inp, b)
    assert rel_fro(_rows(gs, R).cpu().numpy(), r["ds"]) < TOL_F32
    assert rel_fro(_rows(gz, R).cpu().numpy(), r["dz"]) < TOL_F32


@pytest.mark.parametrize("cfg,name,bits", [(2, "q_proj", None), (5, "down_proj", 3)])
def test_init_pack_full_size_bit_exact_rows(cfg, name, bits):
    # init (s, z), pack (bytes, zp) at the full weight shapes, checked on
    # sampled rows (both are row-separable).
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
    R = _pick(out, NS, g)
    s_ref, z_ref = O.init_minmax(W[R], b)
    assert np.array_equal(_rows(s_, R).cpu().numpy(), s_ref)
    assert np.array_equal(_rows(z_, R).cpu().numpy(), z_ref)
    Wq_ref, zp_ref = O.pack(W[R], s_ref, z_ref, b)
    assert np.array_equal(_rows(Wq_, R).cpu().numpy(), Wq_ref)
    assert np.array_equal(_rows(zp_, R).cpu().numpy(), zp_ref)
