"""Pins for the oracle's deployment format and inference linear (paperlayer.ai
summary of EfficientQAT, Appendix D: each group of g weights shares an FP16
step size and an N-bit zero point; Appendix A and section 4: the INT2 model's
linear-layer matrix-vector product against PyTorch's FP16 linear).

Each check is against something other than the oracle: Python's own IEEE
half packing (struct 'e') and torch's half conversion for the fp16 rounding,
hand-derived bytes for the zero-point bitstream, exact rational sums
(fractions.Fraction) for the product, closed forms for one-hot and
group-constant inputs, and the pages' storage accounting.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import qat_oracle as O


def half_struct(x: float) -> float:
    """IEEE binary16 round-to-nearest-even by Python's struct module."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def test_f16_rounding_matches_struct_and_torch():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-7, 4, 2000),
        # exact ties between neighbouring halves: 1 + (2k+1) 2^-11
        1.0 + (2 * np.arange(0, 20) + 1) * 2.0 ** -11,
        # subnormal range and its ties
        np.arange(1, 40) * 2.0 ** -25,
        [0.0, -0.0, 65504.0, 65519.0, 6.103515625e-05, 5.960464477539063e-08],
    ])
    bits = O.f64_to_f16_bits(vals)
    got = O.f16_bits_to_f64(bits)
    for v, g in zip(vals, got):
        assert g == half_struct(float(v)) or (np.isnan(g) and np.isnan(half_struct(float(v))))
    t = torch.from_numpy(vals).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, t)
    # overflow: the nearest-even rounding of anything at or above 65520 is inf
    assert np.isinf(O.f16_bits_to_f64(O.f64_to_f16_bits(np.array([65520.0, 1e6])))).all()


def test_deploy_qparams_hand_derived_bytes():
    z = np.array([[1, 2, 3, 0, 1]], np.float32)
    s = np.full((1, 5), 0.5, np.float32)
    assert O.deploy_qparams(s, z, 2)[1].tolist() == [[0x39, 0x01]]
    # 3 bits: byte 0 = 001 | 010 << 3 | (011 & 3) << 6 ; byte 1 = 0 | 000 << 1 | 001 << 4
    assert O.deploy_qparams(s, z, 3)[1].tolist() == [[0xD1, 0x10]]
    z4 = np.array([[5, 10, 15]], np.float32)
    assert O.deploy_qparams(np.ones((1, 3), np.float32), z4, 4)[1].tolist() == [[0xA5, 0x0F]]
    # rint (half to even) then clamp to [0, K]
    zr = np.array([[-0.6, 1.6, 2.5, 0.5, 3.5, 7.2]], np.float32)
    got = O.unpack_codes(O.deploy_qparams(np.ones((1, 6), np.float32), zr, 2)[1], 6, 2)
    assert got.tolist() == [[0, 2, 2, 0, 3, 3]]
    # s16 is torch's half of the fp32 step size
    s = np.array([[0.1, 1e-5, 0.0123, 70000.0, 3.0517578e-05]], np.float32)
    s16 = O.deploy_qparams(s, np.zeros_like(s), 2)[0]
    assert np.array_equal(s16, torch.from_numpy(s).half().view(torch.int16).numpy().view(np.uint16))


def _rand_deploy(rng, out, inp, bits, group):
    K = (1 << bits) - 1
    G = inp // group
    Wq = rng.integers(0, 256, (out, inp * bits // 8), dtype=np.uint8)
    s = rng.uniform(0.002, 0.05, (out, G)).astype(np.float32)
    z = rng.integers(0, K + 1, (out, G)).astype(np.float32)
    s16, zq = O.deploy_qparams(s, z, bits)
    return Wq, s16, zq


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("group", [32, 64, "row"])
def test_w_hat_brute_force(bits, group):
    rng = np.random.default_rng(10 + bits)
    out, inp = 3, 128
    g = inp if group == "row" else group
    Wq, s16, zq = _rand_deploy(rng, out, inp, bits, g)
    W = O.deploy_w_hat(Wq, s16, zq, inp, bits, g)
    row_bits = [[int(b) for byte in Wq[o] for b in ((byte >> k) & 1 for k in range(8))] for o in range(out)]
    z_bits = [[int(b) for byte in zq[o] for b in ((byte >> k) & 1 for k in range(8))] for o in range(out)]
    for o in range(out):
        for i in range(inp):
            q = sum(row_bits[o][bits * i + b] << b for b in range(bits))
            j = i // g
            zz = sum(z_bits[o][bits * j + b] << b for b in range(bits))
            sv = struct.unpack("<e", struct.pack("<H", int(s16[o, j])))[0]
            assert W[o, i] == half_struct((q - zz) * sv)


@pytest.mark.parametrize("bits", [2, 4])
def test_gemv_exact_rational_sum(bits):
    rng = np.random.default_rng(20 + bits)
    M, out, inp, g = 3, 4, 256, 64
    Wq, s16, zq = _rand_deploy(rng, out, inp, bits, g)
    X = O.f64_to_f16_bits(rng.standard_normal((M, inp)))
    y, ybits = O.deploy_gemv(X, Wq, s16, zq, inp, bits, g)
    W = O.deploy_w_hat(Wq, s16, zq, inp, bits, g)
    Xv = O.f16_bits_to_f64(X)
    for m in range(M):
        for o in range(out):
            exact = sum((Fraction(float(Xv[m, i])) * Fraction(float(W[o, i])) for i in range(inp)), Fraction(0))
            assert abs(y[m, o] - float(exact)) <= 1e-15 * sum(abs(Xv[m] * W[o]))
            assert O.f16_bits_to_f64(ybits[m, o]) == half_struct(float(exact))


def test_gemv_closed_forms():
    rng = np.random.default_rng(30)
    out, inp, bits, g = 5, 128, 2, 64
    Wq, s16, zq = _rand_deploy(rng, out, inp, bits, g)
    W = O.deploy_w_hat(Wq, s16, zq, inp, bits, g)
    # one-hot activations pick a column of W_hat exactly
    X = np.zeros((inp, inp))
    X[np.arange(inp), np.arange(inp)] = 1.0
    _, yb = O.deploy_gemv(O.f64_to_f16_bits(X), Wq, s16, zq, inp, bits, g)
    assert np.array_equal(O.f16_bits_to_f64(yb), W.T)
    # every code of row 0 equal to c: a row of ones gives fp16(sum_j 64 (c - z_j) s_j)
    c = 2
    Wc = np.full((1, inp * bits // 8), sum(c << (2 * k) for k in range(4)), np.uint8)
    z = O.unpack_codes(zq[:1], inp // g, bits)[0]
    sv = O.f16_bits_to_f64(s16[0])
    expect = sum(64 * half_struct((c - z[j]) * sv[j]) for j in range(inp // g))
    _, yb = O.deploy_gemv(O.f64_to_f16_bits(np.ones((1, inp))), Wc, s16[:1], zq[:1], inp, bits, g)
    assert O.f16_bits_to_f64(yb[0, 0]) == half_struct(expect)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_storage_accounting_matches_the_pages(bits):
    # Appendix D: per group of g weights, an FP16 step size and an N-bit zero
    # point -> N + (16 + N) / g bits per weight, with nothing else stored.
    out, inp, g = 64, 4096, 64
    rng = np.random.default_rng(40)
    Wq, s16, zq = _rand_deploy(rng, out, inp, bits, g)
    total_bits = 8 * (Wq.nbytes + s16.nbytes + zq.nbytes)
    assert total_bits / (out * inp) == bits + (16 + bits) / g


def test_deploy_w_hat_is_fp16_of_the_e2e_dequantisation():
    # With an fp16-representable step size and integer zero points, the
    # deployment weight is the fp16 rounding of the E2E-QP dequantisation.
    rng = np.random.default_rng(50)
    out, inp, bits, g = 4, 256, 3, 64
    Wq, s16, zq = _rand_deploy(rng, out, inp, bits, g)
    s = O.f16_bits_to_f64(s16).astype(np.float32)
    z = O.unpack_codes(zq, inp // g, bits).astype(np.float32)
    e2e = O.e2e_w_hat(Wq, s, z, inp, bits, g)
    assert np.array_equal(O.deploy_w_hat(Wq, s16, zq, inp, bits, g), O.f16_bits_to_f64(O.f64_to_f16_bits(e2e)))
