"""Seeded synthetic inputs for the group-wise fake-quant linear.

This module only draws random tensors. It holds none of the method's
arithmetic (no scale, zero point, code, dequantisation or gradient): both the
HIP path and the fp64 oracle take its outputs as plain inputs.

Shapes and distributions follow the workloads of the EfficientQAT pages:
Llama-2-7B / 70B linear shapes, Block-AP on 2048-token samples and E2E-QP on
4096-token samples ("The recipe in numbers" table on the modelfoundations.com
EfficientQAT note). No dataset or pretrained weight is used; the tensors stand
in for RedPajama activations and Llama weights.

Conventions
-----------
* Generator: ``numpy.random.Generator(PCG64(seed))`` with
  ``seed = 1000 * cfg + 10 * layer + tensor_id`` and tensor ids
  W=1, X=2, dY=3, outlier positions=4, s=5, codes/z=6.
* Values are drawn in fp32. bf16 tensors are produced by round-to-nearest-even
  from fp32 through torch's CPU conversion and returned as uint16 bit patterns.
* "0.1% entries x10 outliers": exactly round(0.001*out*in) distinct positions,
  uniform without replacement, multiplied by 10 (sign kept).
* "8 outlier channels x20": 8 distinct input-feature columns of X scaled by 20
  before the bf16 rounding.
* E2E-QP packed weights with uniform codes: every N-bit field uniform on
  0..2^N-1 and independent is the same as every byte uniform on 0..255, so the
  packed tensor is drawn directly as uniform random bytes of shape
  [out, in*N/8]; no packing is done here.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np

GROUP = 64

TID_W, TID_X, TID_DY, TID_OUTL, TID_S, TID_CODES = 1, 2, 3, 4, 5, 6


def rng(cfg: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg + 10 * layer + tensor_id))


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) as uint16 bits, via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 (round to nearest even) as uint16 bits, via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def weight(cfg: int, layer: int, out: int, inp: int, sigma: float, outliers: bool) -> np.ndarray:
    """fp32 master weight [out, in] ~ N(0, sigma), optional 0.1% x10 outliers."""
    w = rng(cfg, layer, TID_W).standard_normal((out, inp), dtype=np.float32)
    w *= np.float32(sigma)
    if outliers:
        n = int(round(0.001 * out * inp))
        pos = rng(cfg, layer, TID_OUTL).choice(out * inp, size=n, replace=False)
        flat = w.reshape(-1)
        flat[pos] *= np.float32(10.0)
    return w


def activations(cfg: int, layer: int, m: int, inp: int, outlier_channels: int = 0) -> np.ndarray:
    """bf16 bits [m, in] ~ N(0, 1), optional outlier columns x20 before rounding."""
    x = rng(cfg, layer, TID_X).standard_normal((m, inp), dtype=np.float32)
    if outlier_channels:
        cols = rng(cfg, layer, TID_OUTL + 100).choice(inp, size=outlier_channels, replace=False)
        x[:, cols] *= np.float32(20.0)
    return to_bf16_bits(x)


def activations_f16(cfg: int, layer: int, m: int, inp: int, outlier_channels: int = 0) -> np.ndarray:
    """fp16 bits [m, in] ~ N(0, 1), optional outlier columns x20 before rounding
    (the inputs of a deployed FP16 model's linear layers)."""
    x = rng(cfg, layer, TID_X).standard_normal((m, inp), dtype=np.float32)
    if outlier_channels:
        cols = rng(cfg, layer, TID_OUTL + 100).choice(inp, size=outlier_channels, replace=False)
        x[:, cols] *= np.float32(20.0)
    return to_f16_bits(x)


def grad_out(cfg: int, layer: int, m: int, out: int, std: float = 1e-3) -> np.ndarray:
    """bf16 bits [m, out] ~ N(0, std)."""
    g = rng(cfg, layer, TID_DY).standard_normal((m, out), dtype=np.float32)
    g *= np.float32(std)
    return to_bf16_bits(g)


def packed_codes(cfg: int, layer: int, out: int, inp: int, bits: int) -> np.ndarray:
    """Uniform random packed bytes [out, in*bits/8] (uniform independent codes)."""
    assert (inp * bits) % 8 == 0
    return rng(cfg, layer, TID_CODES).integers(0, 256, size=(out, inp * bits // 8), dtype=np.uint8)


def e2e_scales(cfg: int, layer: int, out: int, inp: int, lo: float = 0.005, hi: float = 0.05) -> np.ndarray:
    """fp32 step sizes [out, in/64] ~ U(lo, hi)."""
    return rng(cfg, layer, TID_S).uniform(lo, hi, size=(out, inp // GROUP)).astype(np.float32)


def e2e_zeros(cfg: int, layer: int, out: int, inp: int, bits: int) -> np.ndarray:
    """fp32 integer-valued zero points [out, in/64], uniform over {0..2^bits-1}."""
    k = (1 << bits) - 1
    return rng(cfg, layer, TID_CODES + 100).integers(0, k + 1, size=(out, inp // GROUP)).astype(np.float32)


def perturb_qparams(seed: int, s: np.ndarray, z: np.ndarray, bits: int, frac: float = 0.25):
    """Parity-only variant that makes the clamp, the mask and dz non-trivial.

    s <- 0.75*s everywhere; on a seeded `frac` of the groups z moves by +1 or -1
    and is kept inside [0, 2^bits-1]. Returns new (s, z) fp32 arrays.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    k = (1 << bits) - 1
    s2 = (s.astype(np.float32) * np.float32(0.75)).astype(np.float32)
    pick = g.random(z.shape) < frac
    step = np.where(g.random(z.shape) < 0.5, -1.0, 1.0).astype(np.float32)
    z2 = np.where(pick, np.clip(z + step, 0, k), z).astype(np.float32)
    return s2, z2


@dataclasses.dataclass
class ExactSum:
    """Inputs on which every GEMM of the path sums exactly in fp32 (see exact_sum_inputs)."""
    X: np.ndarray        # bf16 bits [m, in], integer values in [-amp, amp]
    dY: np.ndarray       # bf16 bits [m, out], integer values in [-amp, amp]
    W: np.ndarray        # fp32 [out, in] = s * t, t ~ U(-(K + 2), K + 2) per element
    s: np.ndarray        # fp32 [out, G], powers of two 2^-5, 2^-6 or 2^-7
    z: np.ndarray        # fp32 [out, G], an integer in [0, K] plus U(-0.4, 0.4)
    zp: np.ndarray       # fp32 [out, G], integers in [0, K] (a frozen zero point)
    Wq: np.ndarray       # uint8 [out, in*bits/8], uniform random packed bytes


def exact_sum_inputs(seed: int, m: int, out: int, inp: int, bits: int, amp: int = 2,
                     group: int = GROUP) -> ExactSum:
    """Seeded inputs whose GEMMs are exact in fp32 in any summation order.

    Activations and output gradients are small integers, step sizes are powers
    of two 2^-e (e in 5..7) and the zero points used are integers, so any
    dequantised weight (q - z) s is an integer times 2^-e and every product of
    an activation and a weight is a multiple of 2^-7. While the sum of the
    magnitudes of one output's products stays below 2^17 (amp * K * 2^-5 per
    product, at most 2^-2 * K_dim * amp * K), every partial sum is a multiple
    of 2^-7 below 2^24 * 2^-7 and hence exact in fp32, whatever the order of
    the additions. The same holds for dY^T X (integers below 2^24). W = s * t
    is exact in fp32 (a power-of-two scaling), so W / s = t exactly.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    k = (1 << bits) - 1
    G = inp // group
    X = g.integers(-amp, amp + 1, size=(m, inp)).astype(np.float32)
    dY = g.integers(-amp, amp + 1, size=(m, out)).astype(np.float32)
    s = np.ldexp(np.float32(1.0), -g.integers(5, 8, size=(out, G))).astype(np.float32)
    zi = g.integers(0, k + 1, size=(out, G))
    z = (zi + g.uniform(-0.4, 0.4, size=(out, G))).astype(np.float32)
    zp = g.integers(0, k + 1, size=(out, G)).astype(np.float32)
    t = g.uniform(-(k + 2), k + 2, size=(out, inp)).astype(np.float32)
    W = (np.repeat(s, group, axis=1) * t).astype(np.float32)
    assert (inp * bits) % 8 == 0
    Wq = g.integers(0, 256, size=(out, inp * bits // 8), dtype=np.uint8)
    return ExactSum(to_bf16_bits(X), to_bf16_bits(dY), W, s, z, zp, Wq)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Linear:
    name: str
    out: int
    inp: int
    m: int
    bits: int
    sigma: float = 0.02
    outliers: bool = True
    x_outlier_channels: int = 0
    cfg: int = 0
    layer: int = 0

    @property
    def groups(self) -> int:
        return self.inp // GROUP

    def W(self) -> np.ndarray:
        return weight(self.cfg, self.layer, self.out, self.inp, self.sigma, self.outliers)

    def X(self) -> np.ndarray:
        return activations(self.cfg, self.layer, self.m, self.inp, self.x_outlier_channels)

    def dY(self) -> np.ndarray:
        return grad_out(self.cfg, self.layer, self.m, self.out)

    def Wq(self) -> np.ndarray:
        return packed_codes(self.cfg, self.layer, self.out, self.inp, self.bits)

    def s_e2e(self) -> np.ndarray:
        return e2e_scales(self.cfg, self.layer, self.out, self.inp)

    def z_e2e(self) -> np.ndarray:
        return e2e_zeros(self.cfg, self.layer, self.out, self.inp, self.bits)


def config(cfg: int, bits: Optional[int] = None) -> List[Linear]:
    """The linears of workload `cfg` (1..5).

    1: toy 256x256, M=128, w2g64.
    2: Llama-2-7B q_proj 4096x4096, M=2048, w2g64, X with 8 outlier channels.
    3: the seven linears of a Llama-2-7B block, M=2048, w3g64, no outliers.
    4: E2E-QP Llama-2-7B MLP (gate, up 11008x4096; down 4096x11008), M=4096, w2.
    5: Llama-2-70B gate 28672x8192 and down 8192x28672, M=4096, w2/w3/w4.
    """
    if cfg == 1:
        return [Linear("toy", 256, 256, 128, 2, cfg=1)]
    if cfg == 2:
        return [Linear("q_proj", 4096, 4096, 2048, 2, x_outlier_channels=8, cfg=2)]
    if cfg == 3:
        shapes = [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
                  ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                  ("down_proj", 4096, 11008)]
        return [Linear(n, o, i, 2048, 3, outliers=False, cfg=3, layer=li)
                for li, (n, o, i) in enumerate(shapes)]
    if cfg == 4:
        shapes = [("gate_proj", 11008, 4096), ("up_proj", 11008, 4096), ("down_proj", 4096, 11008)]
        return [Linear(n, o, i, 4096, 2, cfg=4, layer=li) for li, (n, o, i) in enumerate(shapes)]
    if cfg == 5:
        b = 2 if bits is None else bits
        shapes = [("gate_proj", 28672, 8192), ("down_proj", 8192, 28672)]
        return [Linear(n, o, i, 4096, b, sigma=0.015, cfg=5, layer=li + 10 * b)
                for li, (n, o, i) in enumerate(shapes)]
    raise ValueError(f"unknown workload {cfg}")


# Linear layers of the deployed Llama-2 models (name, out, in) for the
# inference linear: token-by-token decoding runs one matrix-vector product (or
# a few, M <= 16) per layer.
DEPLOY_SHAPES = {
    "7b": [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096), ("o_proj", 4096, 4096),
           ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096), ("down_proj", 4096, 11008)],
    "70b": [("q_proj", 8192, 8192), ("k_proj", 1024, 8192), ("v_proj", 1024, 8192), ("o_proj", 8192, 8192),
            ("gate_proj", 28672, 8192), ("up_proj", 28672, 8192), ("down_proj", 8192, 28672)],
}


# --------------------------------------------------------------------------
# One Llama-2 decoder block for the Block-AP step
# --------------------------------------------------------------------------

BLOCK_LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
TID_TARGET, TID_NORM1, TID_NORM2 = 7, 8, 9

# (hidden, heads, inter, seq, batch): Llama-2-7B's block on the pages' Block-AP
# samples (2048 tokens, batch 2); head size 128 as in every Llama-2 model.
BLOCK_7B = (4096, 32, 11008, 2048, 2)


def block_linear_shapes(hidden: int, inter: int):
    """(name, out, in) of the seven linears, in the order q, k, v, o, gate, up, down."""
    H, I = hidden, inter
    return [("q_proj", H, H), ("k_proj", H, H), ("v_proj", H, H), ("o_proj", H, H),
            ("gate_proj", I, H), ("up_proj", I, H), ("down_proj", H, I)]


def block_inputs(cfg: int, hidden: int, inter: int, tokens: int, outlier_channels: int = 8,
                 sigma: float = 0.02, target_std: float = 0.1):
    """Seeded inputs of one block step.

    W: per linear fp32 ~ N(0, sigma) with 0.1% x10 outliers (layer index =
    position in BLOCK_LINEARS); x: bf16 bits [tokens, hidden] ~ N(0, 1) with
    `outlier_channels` columns x20; target: bf16 bits of x + N(0, target_std)
    (a stand-in for the full-precision block's output, which sits close to its
    input through the residual); g1, g2: fp32 norm weights ~ 1 + N(0, 0.1).
    """
    W = {n: weight(cfg, li, o, i, sigma, True) for li, (n, o, i) in enumerate(block_linear_shapes(hidden, inter))}
    x32 = rng(cfg, 0, TID_X).standard_normal((tokens, hidden), dtype=np.float32)
    if outlier_channels:
        cols = rng(cfg, 0, TID_OUTL + 100).choice(hidden, size=outlier_channels, replace=False)
        x32[:, cols] *= np.float32(20.0)
    x = to_bf16_bits(x32)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    noise = rng(cfg, 0, TID_TARGET).standard_normal((tokens, hidden), dtype=np.float32)
    target = to_bf16_bits(xv + np.float32(target_std) * noise)
    g1 = (1.0 + 0.1 * rng(cfg, 0, TID_NORM1).standard_normal(hidden)).astype(np.float32)
    g2 = (1.0 + 0.1 * rng(cfg, 0, TID_NORM2).standard_normal(hidden)).astype(np.float32)
    return {"W": W, "x": x, "target": target, "g1": g1, "g2": g2}
