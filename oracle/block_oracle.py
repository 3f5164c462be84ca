"""Plain fp64 CPU oracle of one Block-AP training step on a Llama-2 decoder
block whose seven linears are fake-quantised.

TEST INFRASTRUCTURE, like qat_oracle (which it uses for the quantiser and the
straight-through linear). Only the tests, the smoke check of the entry module
and the CPU-baseline leg of the benchmark may import it; the product path
never does.

Sources (page title -- section):
* [Note-AP]   "EfficientQAT, low-bit training on a single GPU"
              (modelfoundations.com) -- Phase 1 (Block-AP): each transformer
              block is trained alone, all its linear weights together with
              the step sizes and zero points, on a mean-squared error to the
              full-precision block's outputs (the inputs come from the
              quantised stream); the step sizes and weights have separate
              learning rates on separate cosine schedules (quant 1e-4,
              weights 2e-5 at 2 bits) with AdamW; "The recipe in numbers":
              4096 samples of 2048 tokens, batch 2, 2 epochs per block.
* [Summ-A]    paperlayer.ai summary -- Appendix A: gradients through the
              rounding by a straight-through estimator (see qat_oracle).

Readings where the pages are silent (the GPU path follows the same):
* the block is the Llama-2 decoder block: RMSNorm, q/k/v, rotary position
  embedding (base 10000, the two halves of each head rotated), causal
  softmax attention scaled by 1/sqrt(head_dim), o, residual, RMSNorm,
  gate/up, SiLU-gated product, down, residual; RMSNorm epsilon 1e-5;
* trained: W, s and z of the seven linears; the two RMSNorm weights stay
  frozen (they are not quantised and the pages name only those groups);
* loss: mean over all elements of (y - target)^2;
* AdamW as in torch.optim.AdamW (decoupled weight decay, bias-corrected
  moments, eps added after the square root), betas (0.9, 0.999), eps 1e-8,
  weight decay 0 (the pages mention none);
* cosine schedule as torch's CosineAnnealingLR with eta_min 0 over T_max
  steps: optimizer step k (0-based) uses lr0 * (1 + cos(pi k / T_max)) / 2;
* all arithmetic fp64 here; the quantiser's own fp32 operations are those of
  qat_oracle.

block_forward_rows gives the output at a few tokens of one sequence (the
check of the full-size GPU forward on sampled tokens).

Parity status: pinned by tests/test_oracle_block.py (finite differences of
the whole block loss under the straight-through surrogate, torch autograd on
an independent float64 statement of the block, torch's AdamW and
CosineAnnealingLR, and closed forms of the components).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from oracle import qat_oracle as Q

LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
RMS_EPS = 1e-5
ROPE_BASE = 10000.0


@dataclasses.dataclass(frozen=True)
class BlockShape:
    hidden: int
    heads: int
    inter: int
    seq: int
    batch: int
    bits: int
    group: int = 64

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def linear_shapes(self):
        H, I = self.hidden, self.inter
        return {"q_proj": (H, H), "k_proj": (H, H), "v_proj": (H, H), "o_proj": (H, H),
                "gate_proj": (I, H), "up_proj": (I, H), "down_proj": (H, I)}


# ---------------------------------------------------------------------------
# Components
# ---------------------------------------------------------------------------

def rmsnorm(x, g):
    """h = x / sqrt(mean(x^2) + eps) * g, per row; returns (h, r) with r the
    reciprocal root."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)
    return x * r * g, r


def rmsnorm_bwd(dh, x, g, r):
    """Gradient of rmsnorm w.r.t. x: r (g dh) - r^3 x mean(x g dh)."""
    gd = dh * g
    return r * gd - (r ** 3) * x * np.mean(x * gd, axis=-1, keepdims=True)


def rope_angles(seq: int, head_dim: int):
    half = head_dim // 2
    inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)                     # [seq, half]


def rope_at(x, pos, heads: int, head_dim: int, inverse: bool = False):
    """Rotate each head's pair (i, i + head_dim/2) of row r by the angle
    pos[r] * theta_i, theta_i = 10000^(-2 i / head_dim) (the inverse rotation
    for the gradient). x: [rows, heads * head_dim]."""
    half = head_dim // 2
    inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    v = x.reshape(x.shape[0], heads, head_dim)
    a, b = v[..., :half], v[..., half:]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return out.reshape(x.shape[0], heads * head_dim)


def rope(x, shape: BlockShape, inverse: bool = False):
    """rope_at over a [batch * seq, hidden] tensor: row b * seq + t is at
    position t."""
    pos = np.tile(np.arange(shape.seq), shape.batch)
    return rope_at(x, pos, shape.heads, shape.head_dim, inverse)


def attention(q, k, v, shape: BlockShape):
    """Causal softmax attention per (sequence, head); returns (out, P)."""
    B, T, nh, hd = shape.batch, shape.seq, shape.heads, shape.head_dim
    q4 = q.reshape(B, T, nh, hd).transpose(0, 2, 1, 3)
    k4 = k.reshape(B, T, nh, hd).transpose(0, 2, 1, 3)
    v4 = v.reshape(B, T, nh, hd).transpose(0, 2, 1, 3)
    S = q4 @ k4.transpose(0, 1, 3, 2) / math.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    S = np.where(mask, -np.inf, S)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=-1, keepdims=True)
    out = (P @ v4).transpose(0, 2, 1, 3).reshape(B * T, nh * hd)
    return out, P


def attention_bwd(dout, q, k, v, P, shape: BlockShape):
    B, T, nh, hd = shape.batch, shape.seq, shape.heads, shape.head_dim
    tr = lambda a: a.reshape(B, T, nh, hd).transpose(0, 2, 1, 3)
    do4, q4, k4, v4 = tr(dout), tr(q), tr(k), tr(v)
    dv = P.transpose(0, 1, 3, 2) @ do4
    dP = do4 @ v4.transpose(0, 1, 3, 2)
    dS = P * (dP - np.sum(dP * P, axis=-1, keepdims=True))
    dq = dS @ k4 / math.sqrt(hd)
    dk = dS.transpose(0, 1, 3, 2) @ q4 / math.sqrt(hd)
    back = lambda a: a.transpose(0, 2, 1, 3).reshape(B * T, nh * hd)
    return back(dq), back(dk), back(dv)


def silu(x):
    return x / (1.0 + np.exp(-x))


def silu_grad(x):
    sg = 1.0 / (1.0 + np.exp(-x))
    return sg * (1.0 + x * (1.0 - sg))


def fq(x, p, shape: BlockShape):
    t = Q.quantize(p["W"], p["s"], p["z"], shape.bits, shape.group)
    return x @ Q.dequantize_exact(t["q"], t["zr"], t["s"]).T


def fq_bwd(dy, x, p, shape: BlockShape):
    return Q.fakequant_bwd_values(dy, x, p["W"], p["s"], p["z"], shape.bits, shape.group)


# ---------------------------------------------------------------------------
# The block: forward, loss, backward
# ---------------------------------------------------------------------------

def block_forward(x, params, g1, g2, shape: BlockShape):
    """Returns the output and everything the backward needs."""
    c = {"x": x}
    c["h1"], c["r1"] = rmsnorm(x, g1)
    c["q0"] = fq(c["h1"], params["q_proj"], shape)
    c["k0"] = fq(c["h1"], params["k_proj"], shape)
    c["v"] = fq(c["h1"], params["v_proj"], shape)
    c["q"] = rope(c["q0"], shape)
    c["k"] = rope(c["k0"], shape)
    c["attn"], c["P"] = attention(c["q"], c["k"], c["v"], shape)
    c["x2"] = x + fq(c["attn"], params["o_proj"], shape)
    c["h2"], c["r2"] = rmsnorm(c["x2"], g2)
    c["gate"] = fq(c["h2"], params["gate_proj"], shape)
    c["up"] = fq(c["h2"], params["up_proj"], shape)
    c["a"] = silu(c["gate"]) * c["up"]
    c["y"] = c["x2"] + fq(c["a"], params["down_proj"], shape)
    return c


def block_forward_rows(x, params, g1, g2, shape: BlockShape, b: int, rows):
    """The block output y at tokens `rows` (positions within sequence b), from
    that sequence's tokens 0 .. max(rows) only (attention is causal; every
    other step works row by row). Returns [len(rows), hidden]."""
    T, nh, hd = shape.seq, shape.heads, shape.head_dim
    rows = np.asarray(rows)
    tmax = int(rows.max())
    xb = x[b * T: b * T + tmax + 1]
    h1, _ = rmsnorm(xb, g1)
    k = rope_at(fq(h1, params["k_proj"], shape), np.arange(tmax + 1), nh, hd)
    v = fq(h1, params["v_proj"], shape)
    q = rope_at(fq(h1[rows], params["q_proj"], shape), rows, nh, hd)
    attn = np.empty((len(rows), nh * hd))
    for r, t in enumerate(rows):
        for h in range(nh):
            cols = slice(h * hd, (h + 1) * hd)
            sc = k[: t + 1, cols] @ q[r, cols] / math.sqrt(hd)
            p = np.exp(sc - sc.max())
            attn[r, cols] = (p / p.sum()) @ v[: t + 1, cols]
    x2 = xb[rows] + fq(attn, params["o_proj"], shape)
    h2, _ = rmsnorm(x2, g2)
    a = silu(fq(h2, params["gate_proj"], shape)) * fq(h2, params["up_proj"], shape)
    return x2 + fq(a, params["down_proj"], shape)


def mse(y, target):
    """Mean over all elements of (y - target)^2 and its gradient."""
    d = y - target
    return float(np.mean(d * d)), 2.0 * d / d.size


def block_backward(dy, c, params, g1, g2, shape: BlockShape):
    """Gradients of W, s, z of the seven linears (dict of dicts)."""
    grads = {}
    r = fq_bwd(dy, c["a"], params["down_proj"], shape)
    grads["down_proj"] = r
    da = r["dX"]
    dgate = da * c["up"] * silu_grad(c["gate"])
    dup = da * silu(c["gate"])
    rg = fq_bwd(dgate, c["h2"], params["gate_proj"], shape)
    ru = fq_bwd(dup, c["h2"], params["up_proj"], shape)
    grads["gate_proj"], grads["up_proj"] = rg, ru
    dx2 = dy + rmsnorm_bwd(rg["dX"] + ru["dX"], c["x2"], g2, c["r2"])
    ro = fq_bwd(dx2, c["attn"], params["o_proj"], shape)
    grads["o_proj"] = ro
    dq, dk, dv = attention_bwd(ro["dX"], c["q"], c["k"], c["v"], c["P"], shape)
    dq0 = rope(dq, shape, inverse=True)
    dk0 = rope(dk, shape, inverse=True)
    grads["q_proj"] = fq_bwd(dq0, c["h1"], params["q_proj"], shape)
    grads["k_proj"] = fq_bwd(dk0, c["h1"], params["k_proj"], shape)
    grads["v_proj"] = fq_bwd(dv, c["h1"], params["v_proj"], shape)
    return {n: {"W": g["dW"], "s": g["ds"], "z": g["dz"]} for n, g in grads.items()}


# ---------------------------------------------------------------------------
# Optimiser: AdamW with two parameter groups on cosine schedules
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AdamW:
    lr_weight: float = 2e-5
    lr_quant: float = 1e-4
    betas: tuple = (0.9, 0.999)
    eps: float = 1e-8
    weight_decay: float = 0.0
    total_steps: int = 4096


def cosine_lr(lr0: float, k: int, total: int) -> float:
    """Learning rate of optimizer step k (0-based) under a cosine schedule
    from lr0 to 0 over `total` steps."""
    return lr0 * (1.0 + math.cos(math.pi * k / total)) / 2.0


def adamw_update(p, g, m, v, lr: float, t: int, opt: AdamW):
    """One AdamW step (t is 1-based) on fp64 arrays; returns new (p, m, v)."""
    b1, b2 = opt.betas
    p = p * (1.0 - lr * opt.weight_decay)
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mh = m / (1.0 - b1 ** t)
    vh = v / (1.0 - b2 ** t)
    return p - lr * mh / (np.sqrt(vh) + opt.eps), m, v


def block_ap_step(x, target, params, state, g1, g2, shape: BlockShape, k: int, opt: AdamW = AdamW()):
    """One Block-AP optimizer step (k 0-based). params[name] = {W, s, z};
    state[name][key] = (m, v). Returns (loss, new params, new state, grads)."""
    c = block_forward(x, params, g1, g2, shape)
    loss, dy = mse(c["y"], target)
    grads = block_backward(dy, c, params, g1, g2, shape)
    lr_w = cosine_lr(opt.lr_weight, k, opt.total_steps)
    lr_q = cosine_lr(opt.lr_quant, k, opt.total_steps)
    new_p, new_s = {}, {}
    for n in LINEARS:
        new_p[n], new_s[n] = {}, {}
        for key in ("W", "s", "z"):
            m, v = state[n][key]
            lr = lr_w if key == "W" else lr_q
            p, m, v = adamw_update(np.asarray(params[n][key], np.float64), grads[n][key], m, v, lr, k + 1, opt)
            new_p[n][key], new_s[n][key] = Q.fl32(p), (m, v)   # the parameters are stored in fp32
    return loss, new_p, new_s, grads
