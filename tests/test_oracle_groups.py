"""Pins for the oracle at the other group sizes the EfficientQAT pages ablate
(Summary, Appendix F: group 32 and 128; channel-wise quantisation, one group
per weight row). Every check is against something other than the oracle
itself: per-group brute force in plain Python, closed forms (endpoint codes,
the s/2 bound), finite differences of the straight-through surrogate, the
exact E2E scale gradient, and invariants that hold at any group size.
"""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O

GROUPS = [32, 128, "row"]


def bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _g(group, inp):
    return inp if group == "row" else group


@pytest.mark.parametrize("group", GROUPS)
def test_init_matches_per_group_loops(group):
    # s and z from plain Python min / max over each group, with the fp32
    # operations written out one by one (numpy float32 scalars).
    rng = np.random.default_rng(40)
    out, inp = 6, 256
    gs = _g(group, inp)
    W = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        K = np.float32((1 << bits) - 1)
        s, z = O.init_minmax(W, bits, gs)
        assert s.shape == (out, inp // gs)
        for o in range(out):
            for j in range(inp // gs):
                vals = [W[o, i] for i in range(j * gs, (j + 1) * gs)]
                lo, hi = min(vals), max(vals)
                sv = max(np.float32(np.float32(hi - lo) / K), np.float32(1e-5))
                zv = np.float32(np.rint(np.float32(-lo / sv)))
                assert s[o, j] == sv and z[o, j] == zv


@pytest.mark.parametrize("group", GROUPS)
def test_endpoints_and_half_scale_bound(group):
    rng = np.random.default_rng(41)
    out, inp = 64, 512
    gs = _g(group, inp)
    W = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        K = (1 << bits) - 1
        s, z = O.init_minmax(W, bits, gs)
        t = O.quantize(W, s, z, bits, gs)
        q = t["q"].reshape(out, inp // gs, gs)
        Wg = W.reshape(out, inp // gs, gs)
        qmin = np.take_along_axis(q, Wg.argmin(-1)[..., None], -1)[..., 0]
        qmax = np.take_along_axis(q, Wg.argmax(-1)[..., None], -1)[..., 0]
        assert np.all(qmin == 0)
        a = O.fl32(-Wg.min(-1).astype(np.float64) / s.astype(np.float64)).astype(np.float64)
        near_tie = np.abs(np.abs(a - np.floor(a)) - 0.5) < 1e-5
        assert np.all((qmax == K) | near_tie)
        err = np.abs(O.dequantize_exact(t["q"], t["zr"], t["s"]) - W)
        assert np.all(err <= t["s"] * (0.5 + 1e-5))


@pytest.mark.parametrize("group", GROUPS)
def test_requantising_is_idempotent(group):
    rng = np.random.default_rng(42)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    gs = _g(group, 256)
    for bits in (2, 3, 4):
        s, z = O.init_minmax(W, bits, gs)
        t = O.quantize(W, s, z, bits, gs)
        w32 = O.fl32(O.dequantize_exact(t["q"], t["zr"], t["s"]))
        assert np.array_equal(O.quantize(w32, s, z, bits, gs)["q"], t["q"])


def _off_kink(rng, out, inp, bits, gs):
    K = (1 << bits) - 1
    G = inp // gs
    s = rng.uniform(0.005, 0.03, (out, G)).astype(np.float32)
    z = rng.integers(0, K + 1, (out, G)).astype(np.float32)
    inside = rng.choice(np.arange(1, K), size=(out, inp))
    outside = rng.choice(np.array([-3, -2, -1, K + 1, K + 2, K + 3]), size=(out, inp))
    v = np.where(rng.random((out, inp)) < 0.6, inside, outside)
    f = rng.uniform(-0.4, 0.4, (out, inp))
    se, ze = np.repeat(s, gs, 1).astype(np.float64), np.repeat(z, gs, 1).astype(np.float64)
    return O.fl32((v - ze + f) * se), s, z


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [2, 4])
def test_ste_gradients_by_finite_differences(group, bits):
    # Central differences of <dY, X W_hat^T> with rint frozen at the base point
    # (value kept, slope one), inputs built away from the clamp kinks.
    rng = np.random.default_rng(50 + bits)
    M, out, inp = 3, 4, 128
    gs = _g(group, inp)
    K = (1 << bits) - 1
    W, s, z = _off_kink(rng, out, inp, bits, gs)
    Xb = bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    X, dY = O.bf16_bits_to_f64(Xb), O.bf16_bits_to_f64(dYb)
    r = O.fakequant_bwd(dYb, Xb, W, s, z, bits, gs)
    W64, s64, z64 = W.astype(np.float64), s.astype(np.float64), z.astype(np.float64)
    base_u = W64 / np.repeat(s64, gs, 1)

    def L(W_, s_, z_):
        se, ze = np.repeat(s_, gs, 1), np.repeat(z_, gs, 1)
        zr = ze + np.repeat(np.rint(z64) - z64, gs, 1)
        w_hat = (np.clip(W_ / se + (np.rint(base_u) - base_u) + zr, 0, K) - zr) * se
        return float(np.sum(dY * (X @ w_hat.T)))

    def fd(arr, idx, f, h):
        a1, a2 = arr.copy(), arr.copy()
        a1[idx] += h
        a2[idx] -= h
        return (f(a1) - f(a2)) / (2 * h)

    for (o, i) in [(0, 0), (1, gs - 1), (3, inp - 1), (2, 40)]:
        h = 1e-4 * abs(W64[o, i]) + 1e-9
        assert abs(fd(W64, (o, i), lambda a: L(a, s64, z64), h) - r["dW"][o, i]) <= 1e-6 * np.abs(r["Gw"]).max()
    for o in range(out):
        for j in range(inp // gs):
            num = fd(s64, (o, j), lambda a: L(W64, a, z64), 1e-6 * s64[o, j])
            assert abs(num - r["ds"][o, j]) <= 1e-5 * (abs(num) + np.abs(r["ds"]).max())
            num = fd(z64, (o, j), lambda a: L(W64, s64, a), 1e-3)
            assert abs(num - r["dz"][o, j]) <= 1e-6 * (abs(num) + np.abs(r["dz"]).max())


@pytest.mark.parametrize("group", GROUPS)
def test_euler_identity(group):
    rng = np.random.default_rng(60)
    M, out, inp, bits = 5, 12, 256, 3
    gs = _g(group, inp)
    W = (rng.standard_normal((out, inp)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, bits, gs)
    s = (s * np.float32(0.7)).astype(np.float32)
    Xb = bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    Y = O.fakequant_fwd(Xb, W, s, z, bits, gs)
    r = O.fakequant_bwd(dYb, Xb, W, s, z, bits, gs)
    lhs = np.sum(s * r["ds"]) + np.sum(W * r["dW"])
    rhs = np.sum(O.bf16_bits_to_f64(dYb) * Y)
    assert abs(lhs - rhs) <= 1e-6 * np.sum(np.abs(r["Gw"]) * np.abs(W))


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_e2e_scale_gradient_exact(group, bits):
    # Y is linear in s, so central differences are exact up to rounding.
    rng = np.random.default_rng(70 + bits)
    M, out, inp = 3, 4, 256
    gs = _g(group, inp)
    G = inp // gs
    Wq = rng.integers(0, 256, (out, inp * bits // 8), dtype=np.uint8)
    s = rng.uniform(0.005, 0.05, (out, G)).astype(np.float32)
    z = rng.integers(0, 1 << bits, (out, G)).astype(np.float32)
    Xb = bf16_bits(rng.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(rng.standard_normal((M, out)).astype(np.float32))
    dY, X = O.bf16_bits_to_f64(dYb), O.bf16_bits_to_f64(Xb)
    r = O.dequant_gemm_bwd_s(dYb, Xb, Wq, s, z, inp, bits, gs)
    q = O.unpack_codes(Wq, inp, bits).astype(np.float64)

    def L(s_):
        w_hat = (q - np.repeat(z.astype(np.float64), gs, 1)) * np.repeat(s_, gs, 1)
        return float(np.sum(dY * (X @ w_hat.T)))

    s64 = s.astype(np.float64)
    for o in range(out):
        for j in range(G):
            a, b = s64.copy(), s64.copy()
            h = 1e-3 * s64[o, j]
            a[o, j] += h
            b[o, j] -= h
            La, Lb = L(a), L(b)
            num = (La - Lb) / (2 * h)
            roundoff = 8 * np.finfo(np.float64).eps * (abs(La) + abs(Lb)) / (2 * h)
            assert abs(num - r["ds"][o, j]) <= 1e-10 * abs(num) + roundoff


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_groups_are_byte_aligned(group, bits):
    # Each group of `group` codes is exactly group*N/8 whole bytes of the row's
    # LSB-first bit stream: re-packing one group alone gives those bytes.
    rng = np.random.default_rng(80 + bits)
    W = (rng.standard_normal((5, 256)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, bits, group)
    Wq, zp = O.pack(W, s, z, bits, group)
    q = O.quantize(W, s, zp, bits, group)["q"]
    nb = group * bits // 8
    for j in range(256 // group):
        one = O.pack_codes(q[:, j * group:(j + 1) * group], bits)
        assert np.array_equal(one, Wq[:, j * nb:(j + 1) * nb])
    assert np.array_equal(O.unpack_codes(Wq, 256, bits), q.astype(O.unpack_codes(Wq, 256, bits).dtype))
