"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a closed form the EfficientQAT pages state, a hand-evaluated example,
brute force on tiny inputs, finite differences, an exact invariant, or a
library routine for the rounding helpers. A plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong rounding
mode) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import qat_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def facts():
    with open(os.path.join(GOLD, "page_facts.json")) as f:
        return json.load(f)


def bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------------------
# rounding helpers against library routines
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        g.standard_normal(2000).astype(np.float32) * np.float32(1e-30),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of bit 16
    bits = g.integers(0, 2**31, size=4000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties]).astype(np.float32)
    ref = O.bf16_bits_to_f64(bf16_bits(x))
    assert np.array_equal(O.bf16_round(x), ref)


def test_fl32_division_matches_numpy_fp32():
    g = np.random.default_rng(2)
    a = (g.standard_normal(100000) * 0.05).astype(np.float32)
    b = g.uniform(1e-4, 0.1, 100000).astype(np.float32)
    assert np.array_equal(O.fl32(a.astype(np.float64) / b.astype(np.float64)), a / b)
    assert np.array_equal(O.fl32(a.astype(np.float64) - b.astype(np.float64)), a - b)


def test_bf16_decode_encode_roundtrip():
    g = np.random.default_rng(3)
    b = g.integers(0, 2**16, size=5000, dtype=np.uint16)
    b = b[np.isfinite(O.bf16_bits_to_f64(b))]
    assert np.array_equal(O.f64_to_bf16_bits(O.bf16_bits_to_f64(b)), b)


# ---------------------------------------------------------------------------
# a1 init: closed form, hand examples
# ---------------------------------------------------------------------------

def test_init_hand_example_on_grid():
    # A group lying on the grid (q - 2) * 0.25, q in 0..3:
    # min = -0.5, max = 0.25 -> s = 0.75/3 = 0.25, z = rint(0.5/0.25) = 2.
    q = np.tile(np.array([0, 1, 2, 3], np.float32), 16)
    W = ((q - 2) * np.float32(0.25)).reshape(1, 64).astype(np.float32)
    s, z = O.init_minmax(W, 2)
    assert s[0, 0] == np.float32(0.25) and z[0, 0] == 2.0
    t = O.quantize(W, s, z, 2)
    assert np.array_equal(t["q"][0], q) and t["m"].all()


def test_init_hand_example_4bit():
    # N = 4, K = 15: min = -0.75, max = 3.0 -> s = 3.75/15 = 0.25, z = rint(3) = 3.
    W = np.linspace(-0.75, 3.0, 64, dtype=np.float32).reshape(1, 64)
    W[0, 0], W[0, -1] = -0.75, 3.0
    s, z = O.init_minmax(W, 4)
    assert s[0, 0] == np.float32(0.25) and z[0, 0] == 3.0


def test_init_fp32_order_of_operations():
    # s = fl32(fl32(max - min) / K), z = rint(fl32(-min / s)), evaluated in
    # numpy's own fp32 arithmetic on random groups.
    g = np.random.default_rng(4)
    W = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        s, z = O.init_minmax(W, bits)
        Wg = W.reshape(16, 4, 64)
        d = Wg.max(-1) - Wg.min(-1)                      # fp32 subtraction
        s_ref = np.maximum(d / np.float32((1 << bits) - 1), O.S_MIN)
        z_ref = np.rint(-Wg.min(-1) / s_ref)
        assert np.array_equal(s, s_ref) and np.array_equal(z, z_ref)


def test_init_degenerate_group_floor():
    W = np.full((2, 64), 0.125, np.float32)
    s, z = O.init_minmax(W, 2)
    assert np.all(s == O.S_MIN)
    assert np.all(z == np.rint(np.float32(-0.125) / O.S_MIN))


def test_scale_fraction_matches_page():
    f = facts()["scale_fraction_g64"]
    W = np.zeros((8, 4096), np.float32)
    W[:, ::2] = 1.0
    s, _ = O.init_minmax(W, 2)
    frac = s.size / W.size
    assert frac == 1 / 64
    assert abs(frac - f["value"]) / f["value"] < f["rel_tol"]


# ---------------------------------------------------------------------------
# a2/a3 quantise / dequantise
# ---------------------------------------------------------------------------

def test_grid_structure_2bit():
    f = facts()["grid_levels_2bit"]
    g = np.random.default_rng(5)
    W = (g.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, 2)
    assert np.all((z >= 0) & (z <= 3))
    for o, j in [(0, 0), (3, 7), (63, 15)]:
        lv = (np.arange(4) - z[o, j]) * np.float64(s[o, j])
        assert len(np.unique(lv)) == f["value"]
        assert np.allclose(np.diff(lv), s[o, j])                 # affine
        assert (0.0 in lv) == f["zero_exactly_representable"]


def test_minmax_endpoints_land_on_first_and_last_code():
    g = np.random.default_rng(6)
    W = (g.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    W.reshape(-1)[g.choice(W.size, 262, replace=False)] *= 10
    for bits in (2, 3, 4):
        K = (1 << bits) - 1
        s, z = O.init_minmax(W, bits)
        t = O.quantize(W, s, z, bits)
        q = t["q"].reshape(256, 16, 64)
        Wg = W.reshape(256, 16, 64)
        qmin = np.take_along_axis(q, Wg.argmin(-1)[..., None], -1)[..., 0]
        qmax = np.take_along_axis(q, Wg.argmax(-1)[..., None], -1)[..., 0]
        assert np.all(qmin == 0)
        # the max lands on K unless fl32(-min/s) sits within a few ulp of a half
        a = O.fl32(-Wg.min(-1).astype(np.float64) / s.astype(np.float64)).astype(np.float64)
        near_tie = np.abs(np.abs(a - np.floor(a)) - 0.5) < 1e-5
        assert np.all((qmax == K) | near_tie)
        # dequantised endpoints within s/2 (plus fp32 slack)
        wh = O.dequantize_exact(t["q"], t["zr"], t["s"]).reshape(256, 16, 64)
        err_min = np.abs(np.take_along_axis(wh - Wg, Wg.argmin(-1)[..., None], -1)[..., 0])
        err_max = np.abs(np.take_along_axis(wh - Wg, Wg.argmax(-1)[..., None], -1)[..., 0])
        tol = s * (0.5 + 1e-5)
        assert np.all(err_min <= tol) and np.all(err_max <= tol)


def test_tie_case_hand_example():
    # min = -1.5, max = 1.5, K = 3: s = 1, z = rint(1.5) = 2 (half to even);
    # the max gives rint(1.5) + 2 = 4 -> clamped to 3 and masked; -0.5 -> 2, 0.5 -> 2.
    W = np.zeros((1, 64), np.float32)
    W[0, :4] = [-1.5, -0.5, 0.5, 1.5]
    s, z = O.init_minmax(W, 2)
    assert s[0, 0] == 1.0 and z[0, 0] == 2.0
    t = O.quantize(W, s, z, 2)
    assert list(t["q"][0, :4]) == [0, 2, 2, 3]
    assert list(t["m"][0, :4]) == [True, True, True, False]


def test_codes_are_nearest_grid_point_brute_force():
    g = np.random.default_rng(7)
    for bits in (2, 3, 4):
        K = (1 << bits) - 1
        W = (g.standard_normal((8, 128)) * 0.03).astype(np.float32)
        s = g.uniform(0.004, 0.02, (8, 2)).astype(np.float32)
        z = g.uniform(-1.3, K + 1.3, (8, 2)).astype(np.float32)     # exercises the zero-point clamp
        t = O.quantize(W, s, z, bits)
        for o in range(8):
            for i in range(128):
                sj, zj = float(s[o, i // 64]), float(z[o, i // 64])
                zr = min(max(round(zj), 0), K) if abs(zj - np.floor(zj) - 0.5) > 1e-6 else None
                if zr is None:
                    continue
                u = float(np.float32(W[o, i]) / np.float32(sj))
                d = [abs((c - zr) - u) for c in range(K + 1)]
                best = int(np.argmin(d))
                if abs(u - np.floor(u) - 0.5) < 1e-6:
                    continue                                    # exact tie: rounding rule decides
                assert t["q"][o, i] == best
                inside = -0.5 < u + zr < K + 0.5
                assert t["m"][o, i] == inside


def test_inclusive_mask_boundary():
    # s = 1, z = 1, K = 3: v = rint(W) + 1. W = -1 -> v = 0 (kept), W = 2 -> v = 3
    # (kept), W = -2 -> v = -1 (masked), W = 3 -> v = 4 (masked).
    W = np.zeros((1, 64), np.float32)
    W[0, :4] = [-1.0, 2.0, -2.0, 3.0]
    s = np.ones((1, 1), np.float32)
    z = np.ones((1, 1), np.float32)
    t = O.quantize(W, s, z, 2)
    assert list(t["v"][0, :4]) == [0, 3, -1, 4]
    assert list(t["m"][0, :4]) == [True, True, False, False]
    assert list(t["q"][0, :4]) == [0, 3, 0, 3]


def test_zero_point_round_and_clamp():
    # zr = clamp(rint(z), 0, K): z = 2.5 -> 2 (ties to even), 3.5 -> 4 -> 3, -0.7 -> -1 -> 0.
    W = np.zeros((3, 64), np.float32)
    s = np.ones((3, 1), np.float32)
    z = np.array([[2.5], [3.5], [-0.7]], np.float32)
    t = O.quantize(W, s, z, 2)
    assert list(t["zr"][:, 0]) == [2, 3, 0]


def test_requantising_w_hat_is_idempotent():
    g = np.random.default_rng(8)
    W = (g.standard_normal((64, 512)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        s, z = O.init_minmax(W, bits)
        s2, z2 = s * np.float32(0.8), z
        for ss, zz in ((s, z), (s2, z2)):
            t = O.quantize(W, ss, zz, bits)
            w32 = O.fl32(O.dequantize_exact(t["q"], t["zr"], t["s"]))
            t2 = O.quantize(w32, ss, zz, bits)
            assert np.array_equal(t2["q"], t["q"])
            assert t2["m"].all()


def test_high_bit_limit_error_bound():
    g = np.random.default_rng(9)
    W = (g.standard_normal((32, 256)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, 8)
    t = O.quantize(W, s, z, 8)
    err = np.abs(O.dequantize_exact(t["q"], t["zr"], t["s"]) - W)
    assert np.all(err <= t["s"] * (0.5 + 1e-5))


def test_round_ste_forward_value_is_round():
    g = np.random.default_rng(10)
    W = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, 3)
    t = O.quantize(W, s, z, 3)
    wh = O.dequantize_exact(t["q"], t["zr"], t["s"])
    m = t["m"]
    assert np.array_equal(wh[m], (np.rint(t["u"]) * t["s"])[m])


def test_quant_codes_export_matches_fp32_then_bf16():
    g = np.random.default_rng(11)
    W = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, 2)
    codes, wh = O.quant_codes(W, s, z, 2)
    t = O.quantize(W, s, z, 2)
    assert np.array_equal(codes, t["q"].astype(np.uint8))
    # fp32 product computed by numpy, then torch's bf16 cast
    w32 = ((t["q"] - t["zr"]).astype(np.float32) * t["s"].astype(np.float32)).astype(np.float32)
    assert np.array_equal(wh, bf16_bits(w32))


# ---------------------------------------------------------------------------
# a4-a7 forward and STE backward
# ---------------------------------------------------------------------------

def test_forward_bruteforce_loops():
    g = np.random.default_rng(12)
    M, out, inp, bits = 3, 4, 128, 2
    K = 3
    W = (g.standard_normal((out, inp)) * 0.02).astype(np.float32)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    s, z = O.init_minmax(W, bits)
    Y = O.fakequant_fwd(Xb, W, s, z, bits)
    X = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    for mi in range(M):
        for o in range(out):
            acc = 0.0
            for i in range(inp):
                sj, zj = float(s[o, i // 64]), float(z[o, i // 64])
                u = float(np.float32(W[o, i]) / np.float32(sj))
                code = min(max(int(np.rint(u)) + int(zj), 0), K)
                acc += X[mi, i] * (code - zj) * sj
            assert abs(acc - Y[mi, o]) <= 1e-12 * max(1.0, abs(acc))


def _off_kink_inputs(g, out, inp, bits, group=64):
    """W built from chosen integers v = rint(u) + z away from the clamp kinks
    {0, K}, with fractional offsets in (-0.4, 0.4) so no element sits on a
    rounding tie; roughly a third of the elements are clamped."""
    K = (1 << bits) - 1
    G = inp // group
    s = g.uniform(0.005, 0.03, (out, G)).astype(np.float32)
    z = g.integers(0, K + 1, (out, G)).astype(np.float32)
    inside = g.choice(np.arange(1, K), size=(out, inp))
    outside = g.choice(np.array([-3, -2, -1, K + 1, K + 2, K + 3]), size=(out, inp))
    v = np.where(g.random((out, inp)) < 0.6, inside, outside)
    f = g.uniform(-0.4, 0.4, (out, inp))
    se, ze = np.repeat(s, group, 1).astype(np.float64), np.repeat(z, group, 1).astype(np.float64)
    W = O.fl32((v - ze + f) * se)
    return W, s, z


def _ste_surrogate_loss(W, s, z, X, dY, base_u, base_z, bits, group=64):
    """<dY, X W_hat^T> with rint replaced by its value at the base point plus
    an identity-slope term, for both the scaled weight and the zero point."""
    K = (1 << bits) - 1
    se = np.repeat(s, group, 1)
    ze = np.repeat(z, group, 1)
    zc = np.repeat(np.rint(base_z) - base_z, group, 1)
    u = W / se
    c = np.rint(base_u) - base_u
    zr = ze + zc
    w_hat = (np.clip(u + c + zr, 0, K) - zr) * se
    return float(np.sum(dY * (X @ w_hat.T)))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_ste_gradients_match_finite_differences(bits):
    g = np.random.default_rng(100 + bits)
    M, out, inp = 3, 5, 128
    W, s, z = _off_kink_inputs(g, out, inp, bits)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(g.standard_normal((M, out)).astype(np.float32))
    X, dY = O.bf16_bits_to_f64(Xb), O.bf16_bits_to_f64(dYb)
    r = O.fakequant_bwd(dYb, Xb, W, s, z, bits)
    t = O.quantize(W, s, z, bits)
    assert 0.15 < 1 - t["m"].mean() < 0.7          # both branches exercised

    W64, s64, z64 = W.astype(np.float64), s.astype(np.float64), z.astype(np.float64)
    base_u = W64 / np.repeat(s64, 64, 1)
    L = lambda W_, s_, z_, X_: _ste_surrogate_loss(W_, s_, z_, X_, dY, base_u, z64, bits)

    def fd(arr, idx, f, h):
        a1, a2 = arr.copy(), arr.copy()
        a1[idx] += h
        a2[idx] -= h
        return (f(a1) - f(a2)) / (2 * h)

    for (o, i) in [(0, 0), (1, 63), (2, 64), (4, 127), (3, 17), (0, 100)]:
        h = 1e-4 * abs(W64[o, i]) + 1e-9
        num = fd(W64, (o, i), lambda a: L(a, s64, z64, X), h)
        assert abs(num - r["dW"][o, i]) <= 1e-6 * np.abs(r["Gw"]).max()
    for (o, j) in [(0, 0), (1, 1), (4, 0), (2, 1)]:
        h = 1e-6 * s64[o, j]
        num = fd(s64, (o, j), lambda a: L(W64, a, z64, X), h)
        assert abs(num - r["ds"][o, j]) <= 1e-5 * (abs(num) + np.abs(r["ds"]).max())
        num = fd(z64, (o, j), lambda a: L(W64, s64, a, X), 1e-3)
        assert abs(num - r["dz"][o, j]) <= 1e-6 * (abs(num) + np.abs(r["dz"]).max())
    for (mi, i) in [(0, 0), (2, 127), (1, 64)]:
        num = fd(X, (mi, i), lambda a: L(W64, s64, z64, a), 1e-3)
        assert abs(num - r["dX"][mi, i]) <= 1e-9 * (1 + abs(num))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_euler_identities(bits):
    # Scaling W and s together leaves u and q unchanged and scales Y, so
    # <s, ds> + <W, dW> = <dY, Y>; and <dX, X> = <dY, Y> (Y is linear in X).
    g = np.random.default_rng(200 + bits)
    M, out, inp = 7, 24, 256
    W = (g.standard_normal((out, inp)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, bits)
    s = (s * np.float32(0.7)).astype(np.float32)                       # force clamping
    z = np.clip(z + g.integers(-1, 2, z.shape), 0, (1 << bits) - 1).astype(np.float32)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(g.standard_normal((M, out)).astype(np.float32))
    Y = O.fakequant_fwd(Xb, W, s, z, bits)
    r = O.fakequant_bwd(dYb, Xb, W, s, z, bits)
    dY, X = O.bf16_bits_to_f64(dYb), O.bf16_bits_to_f64(Xb)
    lhs = np.sum(s * r["ds"]) + np.sum(W * r["dW"])
    rhs = np.sum(dY * Y)
    scale = np.sum(np.abs(r["Gw"]) * np.abs(W))
    assert abs(lhs - rhs) <= 1e-6 * scale
    assert abs(np.sum(r["dX"] * X) - rhs) <= 1e-10 * np.sum(np.abs(dY) * np.abs(Y))
    assert (~O.quantize(W, s, z, bits)["m"]).sum() > 0


def test_min_max_init_mask_all_ones_and_dz_zero():
    g = np.random.default_rng(13)
    W = (g.standard_normal((32, 512)) * 0.02).astype(np.float32)
    Xb = bf16_bits(g.standard_normal((9, 512)).astype(np.float32))
    dYb = bf16_bits((g.standard_normal((9, 32)) * 1e-3).astype(np.float32))
    for bits in (2, 3, 4):
        s, z = O.init_minmax(W, bits)
        r = O.fakequant_bwd(dYb, Xb, W, s, z, bits)
        m = O.quantize(W, s, z, bits)["m"]
        if m.all():
            assert np.all(r["dz"] == 0) and np.array_equal(r["dW"], r["Gw"])
        else:                                    # only max elements at rounding ties
            assert (~m).sum() <= 2


def test_backward_transposition_shapes():
    g = np.random.default_rng(14)
    M, out, inp = 5, 3, 192
    W = (g.standard_normal((out, inp)) * 0.02).astype(np.float32)
    s, z = O.init_minmax(W, 2)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(g.standard_normal((M, out)).astype(np.float32))
    r = O.fakequant_bwd(dYb, Xb, W, s, z, 2)
    assert r["dX"].shape == (M, inp) and r["dW"].shape == (out, inp)
    assert r["ds"].shape == (out, 3) and r["dz"].shape == (out, 3)
    # Gw[o, i] = sum_m dY[m, o] X[m, i], by loops
    dY, X = O.bf16_bits_to_f64(dYb), O.bf16_bits_to_f64(Xb)
    for o, i in [(0, 0), (2, 191), (1, 77)]:
        assert abs(sum(dY[mm, o] * X[mm, i] for mm in range(M)) - r["Gw"][o, i]) < 1e-12


# ---------------------------------------------------------------------------
# a8 pack
# ---------------------------------------------------------------------------

def test_pack_layout_hand_examples():
    with open(os.path.join(GOLD, "pack_layout.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array([c["codes"]])
        assert list(O.pack_codes(q, c["bits"])[0]) == c["bytes"]
        assert list(O.unpack_codes(np.array([c["bytes"]], np.uint8), len(c["codes"]), c["bits"])[0]) == c["codes"]


@settings(max_examples=40, deadline=None)
@given(bits=st.sampled_from([2, 3, 4]), out=st.integers(1, 5), ng=st.integers(1, 3), seed=st.integers(0, 2**31))
def test_pack_roundtrip(bits, out, ng, seed):
    g = np.random.default_rng(seed)
    q = g.integers(0, 1 << bits, (out, 64 * ng))
    b = O.pack_codes(q, bits)
    assert b.shape == (out, 64 * ng * bits // 8) and b.dtype == np.uint8
    assert np.array_equal(O.unpack_codes(b, 64 * ng, bits), q)


def test_pack_dequant_equals_fakequant_w_hat():
    g = np.random.default_rng(15)
    W = (g.standard_normal((16, 512)) * 0.02).astype(np.float32)
    for bits in (2, 3, 4):
        s, z = O.init_minmax(W, bits)
        z = (z + np.float32(0.3)).astype(np.float32)             # float z: pack hard-rounds it
        Wq, zp = O.pack(W, s, z, bits)
        assert np.array_equal(zp, np.clip(np.rint(z), 0, (1 << bits) - 1))
        t = O.quantize(W, s, z, bits)
        assert np.array_equal(O.e2e_w_hat(Wq, s, zp, 512, bits), O.dequantize_exact(t["q"], t["zr"], t["s"]))


# ---------------------------------------------------------------------------
# a9/a10 E2E-QP
# ---------------------------------------------------------------------------

def test_e2e_integer_weight_gemm_bruteforce():
    g = np.random.default_rng(16)
    M, out, inp, bits = 2, 3, 64, 3
    q = g.integers(0, 8, (out, inp))
    Wq = O.pack_codes(q, bits)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    s = np.ones((out, 1), np.float32)
    z = np.zeros((out, 1), np.float32)
    Y = O.dequant_gemm_fwd(Xb, Wq, s, z, inp, bits)
    X = O.bf16_bits_to_f64(Xb)
    for mi in range(M):
        for o in range(out):
            assert Y[mi, o] == sum(X[mi, i] * int(q[o, i]) for i in range(inp))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_e2e_scale_gradient_exact_by_finite_differences(bits):
    tol = facts()["e2e_scale_grad_fd_rel"]["value"]
    g = np.random.default_rng(300 + bits)
    M, out, inp = 4, 6, 192
    Wq = g.integers(0, 256, (out, inp * bits // 8), dtype=np.uint8)
    s = g.uniform(0.005, 0.05, (out, 3)).astype(np.float32)
    z = g.integers(0, 1 << bits, (out, 3)).astype(np.float32)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(g.standard_normal((M, out)).astype(np.float32))
    dY = O.bf16_bits_to_f64(dYb)
    r = O.dequant_gemm_bwd_s(dYb, Xb, Wq, s, z, inp, bits)

    q = O.unpack_codes(Wq, inp, bits).astype(np.float64)
    X = O.bf16_bits_to_f64(Xb)

    def L(s_):                      # fp64 throughout: Y = X ((q - z) s)^T
        w_hat = (q - np.repeat(z.astype(np.float64), 64, 1)) * np.repeat(s_, 64, 1)
        return float(np.sum(dY * (X @ w_hat.T)))

    s64 = s.astype(np.float64)
    for o in range(out):
        for j in range(3):
            h = 1e-3 * s64[o, j]
            a, b = s64.copy(), s64.copy()
            a[o, j] += h
            b[o, j] -= h
            num = (L(a) - L(b)) / (2 * h)
            assert abs(num - r["ds"][o, j]) <= tol * max(abs(num), 1e-3)
    # Y is homogeneous of degree one in s: <s, ds> = <dY, Y>.
    Y = O.dequant_gemm_fwd(Xb, Wq, s, z, inp, bits)
    assert abs(np.sum(s64 * r["ds"]) - np.sum(dY * Y)) <= 1e-12 * np.sum(np.abs(dY * Y))
    # dz variant: shifting z by t shifts W_hat by -t*s.
    def Lz(z_):
        return float(np.sum(dY * O.dequant_gemm_fwd(Xb, Wq, s, z_, inp, bits)))
    z64 = z.astype(np.float64)
    a, b = z64.copy(), z64.copy()
    a[1, 2] += 0.5
    b[1, 2] -= 0.5
    assert abs((Lz(a) - Lz(b)) - r["dz"][1, 2]) <= 1e-10 * (abs(r["dz"][1, 2]) + 1e-12)


def test_e2e_dx_transpose_by_loops():
    g = np.random.default_rng(17)
    M, out, inp, bits = 2, 3, 64, 4
    Wq = g.integers(0, 256, (out, inp * bits // 8), dtype=np.uint8)
    s = g.uniform(0.005, 0.05, (out, 1)).astype(np.float32)
    z = g.integers(0, 16, (out, 1)).astype(np.float32)
    Xb = bf16_bits(g.standard_normal((M, inp)).astype(np.float32))
    dYb = bf16_bits(g.standard_normal((M, out)).astype(np.float32))
    r = O.dequant_gemm_bwd_s(dYb, Xb, Wq, s, z, inp, bits)
    q = O.unpack_codes(Wq, inp, bits)
    dY = O.bf16_bits_to_f64(dYb)
    for mi in range(M):
        for i in (0, 31, 63):
            ref = sum(dY[mi, o] * (q[o, i] - z[o, 0]) * float(s[o, 0]) for o in range(out))
            assert abs(ref - r["dX"][mi, i]) < 1e-12
