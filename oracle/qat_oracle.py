"""Plain fp64 CPU oracle for EfficientQAT's group-wise fake-quantised linear.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the entry module and
the CPU-baseline leg of the benchmark may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product.

Every function is a direct, slow, obviously-correct statement of what the
EfficientQAT pages define. Sources (page title -- section / equation):

* [Notes-Eq1]  "EfficientQAT" paper note (zhaoyang97 Paper-Notes, ACL2025) --
               method details, Block-AP: the uniform quantiser
               W_int = clamp(round(W/s) + z, 0, 2^N - 1) (Eq. 1) and the
               dequantiser W_hat = (W_int - z) * s (Eq. 2); E2E-QP gradient
               dW_hat/ds = W_q - z.
* [Note-Init]  "EfficientQAT, low-bit training on a single GPU"
               (modelfoundations.com) -- Phase 1: per-group min-max init
               s = (x_max - x_min)/(2^N - 1), z = round(-x_min/s), both trainable.
* [Note-E2E]   same note -- Phase 2: with frozen integers the forward is only a
               dequantisation, linear in s, so dW_hat/ds = W_int - z is exact.
* [Note-Code]  same note -- "Paper vs. code": zero points are float parameters
               rounded through a straight-through round in every forward and
               hard-rounded at pack time; blocks train in FP32.
* [Summ-A]     paperlayer.ai summary of arXiv 2407.11062v3 -- Appendix A:
               Block-AP uses a straight-through estimator through the rounding,
               with gradients for step size, zero point and weight.
* [Summ-D]     same summary -- Appendix D: each group of g weights shares a
               step size and an N-bit zero point; stored for deployment, the
               step size is FP16.
* [Summ-A-inf] same summary -- Appendix A and section 4: the deployed INT2
               model's linear-layer matrix-vector product, compared against the
               FP16 PyTorch linear.

Readings where the pages are silent (the kernel follows the same readings):

* rounding is round-half-to-even (``np.rint``);
* s, z and u = W/s are IEEE fp32 values, each produced by one correctly
  rounded fp32 operation in the order written below. Here each such operation
  is done in fp64 and rounded once to fp32, which equals the fp32 result
  because 53 >= 2*24 + 2 (double rounding is innocuous);
* groups are g consecutive elements along the input dimension of W [out, in],
  g = 64 by default (32, 128, or the whole row for channel-wise);
* a degenerate group (max == min) gets s = S_MIN = fp32(1e-5);
* the zero point used in the Block-AP forward is zr = clamp(rint(z), 0, K)
  with identity derivative (straight-through round and clamp);
* the clamp mask is m = [0 <= rint(u) + zr <= K], inclusive;
* the STE backward keeps the value of rint and uses derivative 1 for it:
  in range dW_hat/dW = 1, dW_hat/ds = rint(u) - u, dW_hat/dzr = 0;
  clamped  dW_hat/dW = 0, dW_hat/ds = q - zr,     dW_hat/dzr = -s;
* GEMMs take bf16 activations at their exact values and an exact fp64 W_hat;
  the kernel's bf16 rounding of W_hat lies inside the stated tolerance;
* packed weights: each row is an LSB-first bitstream, code i in bits
  [N*i, N*i + N) of the row's bytes, row stride in*N/8 bytes.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py, tests/test_oracle_groups.py and
tests/test_oracle_deploy.py (closed forms, brute force, finite differences,
exact rational sums, invariants, and library routines for the rounding
helpers). The absolute
values the method produces on real weights are not pinned by any page
(the pages print no worked example).
"""
from __future__ import annotations

import numpy as np

GROUP = 64
S_MIN = np.float32(1e-5)


def levels(bits: int) -> int:
    """K = 2^N - 1, the largest code ([Notes-Eq1])."""
    return (1 << bits) - 1


# ---------------------------------------------------------------------------
# Rounding helpers (IEEE definitions)
# ---------------------------------------------------------------------------

def fl32(x) -> np.ndarray:
    """Round an fp64 value to the nearest fp32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to their exact values in fp64."""
    u32 = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (8 significant bits, ties to
    even), returned as exact fp64 values. Written from the definition: scale by
    the bf16 unit in the last place of x, round half-to-even, scale back.
    Finite inputs only."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])                  # |x| = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, -126)             # exponent of the leading bit, normal range floor
    ulp = np.ldexp(1.0, e - 7)              # bf16 keeps 7 fraction bits
    out[nz] = np.rint(x[nz] / ulp) * ulp    # exact in fp64
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127    # largest finite bf16
    out[np.abs(out) > big] = np.inf * np.sign(out[np.abs(out) > big])
    return out


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Encode values that are exactly bf16-representable as bf16 bits."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _groups(a: np.ndarray, group: int = GROUP) -> np.ndarray:
    out, inp = a.shape
    return a.reshape(out, inp // group, group)


def _expand(p: np.ndarray, group: int = GROUP) -> np.ndarray:
    return np.repeat(np.asarray(p), group, axis=1)


# ---------------------------------------------------------------------------
# a1: min-max init  [Note-Init]
# ---------------------------------------------------------------------------

def init_minmax(W: np.ndarray, bits: int, group: int = GROUP):
    """Per (row, group): s = fl32(fl32(max - min) / K), floored at S_MIN, and
    z = rint(fl32(-min / s)). Returns fp32 arrays s, z of shape [out, in/g]."""
    K = levels(bits)
    g = _groups(np.asarray(W, dtype=np.float32).astype(np.float64), group)
    xmin = g.min(axis=-1)
    xmax = g.max(axis=-1)
    d = fl32(xmax - xmin).astype(np.float64)
    s = fl32(d / K)
    s = np.maximum(s, S_MIN).astype(np.float32)
    z = np.rint(fl32(-xmin / s.astype(np.float64)).astype(np.float64)).astype(np.float32)
    return s, z


# ---------------------------------------------------------------------------
# a2/a3: quantise (Eq. 1) and dequantise (Eq. 2)  [Notes-Eq1], [Note-Code]
# ---------------------------------------------------------------------------

def quantize(W: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int, group: int = GROUP) -> dict:
    """Eq. 1 with the straight-through zero point.

    Returns a dict of per-element arrays (all [out, in]):
      zr : clamp(rint(z), 0, K)            the zero point used in the forward
      u  : fl32(W / s)                     the scaled weight (fp32 value)
      v  : rint(u) + zr                    the unclamped integer
      q  : clamp(v, 0, K)                  the code W_int
      m  : 0 <= v <= K                     the clamp mask (inclusive)
      s  : s expanded to elements
    """
    K = levels(bits)
    se = _expand(np.asarray(s, dtype=np.float32), group).astype(np.float64)
    ze = _expand(np.asarray(z, dtype=np.float32), group).astype(np.float64)
    zr = np.clip(np.rint(ze), 0, K)
    u = fl32(np.asarray(W, dtype=np.float32).astype(np.float64) / se).astype(np.float64)
    v = np.rint(u) + zr
    q = np.clip(v, 0, K)
    m = (v >= 0) & (v <= K)
    return {"zr": zr, "u": u, "v": v, "q": q, "m": m, "s": se}


def dequantize_exact(q: np.ndarray, zr: np.ndarray, se: np.ndarray) -> np.ndarray:
    """Eq. 2 in fp64: (q - zr) * s, exact (small integer times an fp32)."""
    return (q - zr) * se


def quant_codes(W, s, z, bits, group: int = GROUP):
    """The code export: u8 codes and W_hat as bf16 bits, where the bf16 value is
    the round-to-nearest-even of the fp32 product fl32((q - zr) * s)."""
    t = quantize(W, s, z, bits, group)
    w32 = fl32(dequantize_exact(t["q"], t["zr"], t["s"]))
    w_hat_bits = f64_to_bf16_bits(bf16_round(w32))
    return t["q"].astype(np.uint8), w_hat_bits


# ---------------------------------------------------------------------------
# a4-a7: fake-quant linear forward and STE backward  [Notes-Eq1], [Summ-A]
# ---------------------------------------------------------------------------

def fakequant_fwd(X_bits: np.ndarray, W, s, z, bits, group: int = GROUP) -> np.ndarray:
    """Y = X W_hat^T with X the exact bf16 values and W_hat exact (fp64)."""
    t = quantize(W, s, z, bits, group)
    w_hat = dequantize_exact(t["q"], t["zr"], t["s"])
    return bf16_bits_to_f64(X_bits) @ w_hat.T


def fakequant_bwd(dY_bits, X_bits, W, s, z, bits, group: int = GROUP) -> dict:
    """Straight-through backward of Y = X W_hat^T.

    dX = dY W_hat;  Gw = dY^T X;  dW = Gw * m;
    ds[o, j] = sum_{i in j} Gw[o, i] * (m_i ? rint(u_i) - u_i : q_i - zr);
    dz[o, j] = sum_{i in j} Gw[o, i] * (m_i ? 0 : -s[o, j]).
    """
    return fakequant_bwd_values(bf16_bits_to_f64(dY_bits), bf16_bits_to_f64(X_bits), W, s, z, bits, group)


def fakequant_bwd_values(dY, X, W, s, z, bits, group: int = GROUP) -> dict:
    """The same straight-through backward for dY and X given as fp64 values."""
    t = quantize(W, s, z, bits, group)
    w_hat = dequantize_exact(t["q"], t["zr"], t["s"])
    dY = np.asarray(dY, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    dX = dY @ w_hat
    Gw = dY.T @ X
    m = t["m"]
    dW = np.where(m, Gw, 0.0)
    dwhat_ds = np.where(m, np.rint(t["u"]) - t["u"], t["q"] - t["zr"])
    dwhat_dz = np.where(m, 0.0, -t["s"])
    ds = _groups(Gw * dwhat_ds, group).sum(axis=-1)
    dz = _groups(Gw * dwhat_dz, group).sum(axis=-1)
    return {"dX": dX, "dW": dW, "ds": ds, "dz": dz, "Gw": Gw}


# ---------------------------------------------------------------------------
# a8: pack  [Note-Code] (hard-rounded zero point), [Summ-D] (N-bit codes)
# ---------------------------------------------------------------------------

def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """LSB-first bitstream per row: code i sits in bits [N*i, N*i+N). A row
    whose bit count is not a multiple of 8 ends in a zero-padded byte."""
    q = np.asarray(q).astype(np.int64)
    out, inp = q.shape
    nbytes = -(-inp * bits // 8)
    res = np.zeros((out, nbytes), dtype=np.int64)
    for b in range(bits):                       # bit b of code i -> stream bit N*i + b
        pos = np.arange(inp) * bits + b
        bit = (q >> b) & 1
        np.add.at(res, (slice(None), pos // 8), bit << (pos % 8))
    return res.astype(np.uint8)


def unpack_codes(Wq: np.ndarray, inp: int, bits: int) -> np.ndarray:
    """Inverse of pack_codes: [out, in] integer codes."""
    Wq = np.asarray(Wq, dtype=np.uint8).astype(np.int64)
    out = Wq.shape[0]
    q = np.zeros((out, inp), dtype=np.int64)
    for b in range(bits):
        pos = np.arange(inp) * bits + b
        bit = (Wq[:, pos // 8] >> (pos % 8)) & 1
        q |= bit << b
    return q


def pack(W, s, z, bits, group: int = GROUP):
    """Hard-round the zero point (zp = clamp(rint(z), 0, K)), quantise with it
    and pack the codes. Returns (packed bytes [out, in*N/8], zp fp32 [out, G])."""
    K = levels(bits)
    zp = np.clip(np.rint(np.asarray(z, dtype=np.float32)), 0, K).astype(np.float32)
    t = quantize(W, s, zp, bits, group)
    return pack_codes(t["q"], bits), zp


# ---------------------------------------------------------------------------
# a9/a10: E2E-QP dequant GEMM and the exact scale gradient  [Note-E2E]
# ---------------------------------------------------------------------------

def e2e_w_hat(Wq, s, z, inp, bits, group: int = GROUP) -> np.ndarray:
    """W_hat = (q - z) * s with z used as stored (frozen, integer valued)."""
    q = unpack_codes(Wq, inp, bits).astype(np.float64)
    return (q - _expand(np.asarray(z, np.float32), group)) * _expand(np.asarray(s, np.float32), group)


def dequant_gemm_fwd(X_bits, Wq, s, z, inp, bits, group: int = GROUP) -> np.ndarray:
    return bf16_bits_to_f64(X_bits) @ e2e_w_hat(Wq, s, z, inp, bits, group).T


def dequant_gemm_bwd_s(dY_bits, X_bits, Wq, s, z, inp, bits, group: int = GROUP) -> dict:
    """dX = dY W_hat;  ds[o, j] = sum_{i in j} Gw[o, i] * (q_i - z[o, j]);
    dz (the train-s-and-z variant) = -s * sum_{i in j} Gw[o, i]."""
    q = unpack_codes(Wq, inp, bits).astype(np.float64)
    ze = _expand(np.asarray(z, np.float32), group).astype(np.float64)
    se = _expand(np.asarray(s, np.float32), group).astype(np.float64)
    dY = bf16_bits_to_f64(dY_bits)
    X = bf16_bits_to_f64(X_bits)
    dX = dY @ ((q - ze) * se)
    Gw = dY.T @ X
    ds = _groups(Gw * (q - ze), group).sum(axis=-1)
    dz = -np.asarray(s, np.float64) * _groups(Gw, group).sum(axis=-1)
    return {"dX": dX, "ds": ds, "dz": dz, "Gw": Gw}


# ---------------------------------------------------------------------------
# Deployment format and the inference linear  [Summ-D], [Summ-A-inf]
#
# Readings: the deployed model is FP16 (activations, outputs and the step
# size); a group's step size is fp16(s), rounded to nearest even; its zero
# point is the N-bit integer clamp(rint(z), 0, K), stored as an LSB-first
# bitstream per row like the codes (row stride ceil(G*N/8) bytes); the
# dequantised weight is fp16((q - z) * s16), one rounding of the exact
# product; the linear sums x * W_hat exactly and rounds once to fp16.
# ---------------------------------------------------------------------------

def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """Round to nearest even fp16 (numpy's double -> half conversion); values
    beyond the fp16 range become infinities."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def deploy_qparams(s, z, bits: int):
    """(s16 bits [out, G] uint16, zq [out, ceil(G*N/8)] uint8) from the fp32
    step sizes and zero points."""
    K = levels(bits)
    s16 = f64_to_f16_bits(np.asarray(s, dtype=np.float32).astype(np.float64))
    zint = np.clip(np.rint(np.asarray(z, dtype=np.float32)), 0, K).astype(np.int64)
    return s16, pack_codes(zint, bits)


def deploy_w_hat(Wq, s16_bits, zq, inp: int, bits: int, group: int = GROUP) -> np.ndarray:
    """W_hat = fp16((q - z) * s16), as fp64 values [out, in]."""
    G = inp // group
    q = unpack_codes(Wq, inp, bits)
    z = unpack_codes(zq, G, bits)
    prod = (q - _expand(z, group)).astype(np.float64) * _expand(f16_bits_to_f64(s16_bits), group)
    return f16_bits_to_f64(f64_to_f16_bits(prod))


def deploy_gemv(X16_bits, Wq, s16_bits, zq, inp: int, bits: int, group: int = GROUP) -> np.ndarray:
    """Y = fp16(X W_hat^T) for fp16 activations X [M, in]; returns the exact
    (unrounded) fp64 product and the rounded fp16 bits."""
    y = f16_bits_to_f64(X16_bits) @ deploy_w_hat(Wq, s16_bits, zq, inp, bits, group).T
    return y, f64_to_f16_bits(y)
