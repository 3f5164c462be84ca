"""Pins for the Block-AP step oracle (modelfoundations.com EfficientQAT note,
Phase 1 and "The recipe in numbers"; paperlayer.ai summary, Appendix A).

Checked against things other than the oracle's own code:
* torch autograd on an independent float64 torch statement of the block
  (torch's softmax, SiLU and tensor algebra, a straight-through fake-quant
  autograd function) -- forward output and every W, s, z gradient;
* central finite differences of the whole block loss under the
  straight-through surrogate (rounding frozen at the base point);
* torch.optim.AdamW with two parameter groups and CosineAnnealingLR;
* closed forms of the components (RoPE is a rotation, the identity at
  position 0; RMSNorm output has unit mean square over g; causal softmax rows
  sum to one with zeros above the diagonal; attention over one key returns
  its value; the first AdamW step is lr * g / (|g| + eps)).
"""
import math

import numpy as np
import pytest
import torch

from oracle import block_oracle as B
from oracle import qat_oracle as Q

TINY = B.BlockShape(hidden=32, heads=2, inter=48, seq=6, batch=2, bits=2, group=16)


def _params(shape, rng, perturb=True):
    params = {}
    K = (1 << shape.bits) - 1
    for n, (o, i) in shape.linear_shapes().items():
        W = (rng.standard_normal((o, i)) * 0.2).astype(np.float32)
        s, z = Q.init_minmax(W, shape.bits, shape.group)
        if perturb:
            s = (s * np.float32(0.8)).astype(np.float32)
            z = np.clip(z + rng.integers(-1, 2, z.shape), 0, K).astype(np.float32)
        params[n] = {"W": W, "s": s, "z": z}
    return params


def _inputs(shape, rng):
    M = shape.batch * shape.seq
    x = rng.standard_normal((M, shape.hidden))
    tgt = x + 0.3 * rng.standard_normal((M, shape.hidden))
    g1 = 1.0 + 0.1 * rng.standard_normal(shape.hidden)
    g2 = 1.0 + 0.1 * rng.standard_normal(shape.hidden)
    return x, tgt, g1, g2


# ---------------------------------------------------------------------------
# components
# ---------------------------------------------------------------------------

def test_rope_is_a_rotation():
    rng = np.random.default_rng(1)
    sh = B.BlockShape(hidden=64, heads=4, inter=64, seq=9, batch=2, bits=2)
    x = rng.standard_normal((sh.batch * sh.seq, sh.hidden))
    y = B.rope(x, sh)
    half = sh.head_dim // 2
    xv = x.reshape(sh.batch, sh.seq, sh.heads, sh.head_dim)
    yv = y.reshape(xv.shape)
    # pair norms are kept, position 0 is untouched, the inverse undoes it
    nx = xv[..., :half] ** 2 + xv[..., half:] ** 2
    ny = yv[..., :half] ** 2 + yv[..., half:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)
    assert np.allclose(yv[:, 0], xv[:, 0], rtol=0, atol=0)
    assert np.allclose(B.rope(y, sh, inverse=True), x, rtol=1e-12, atol=1e-12)
    # pair 0 rotates by exactly pos radians (theta_0 = 1)
    t = 5
    c, s = math.cos(t), math.sin(t)
    a, b = xv[0, t, 1, 0], xv[0, t, 1, half]
    assert math.isclose(yv[0, t, 1, 0], a * c - b * s, rel_tol=1e-12)
    assert math.isclose(yv[0, t, 1, half], b * c + a * s, rel_tol=1e-12)


def test_rmsnorm_unit_mean_square():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 64)) * 3.0
    g = 1.0 + rng.random(64)
    h, r = B.rmsnorm(x, g)
    ms = np.mean((h / g) ** 2, axis=-1)
    expect = np.mean(x * x, axis=-1) / (np.mean(x * x, axis=-1) + B.RMS_EPS)
    assert np.allclose(ms, expect, rtol=1e-12)


def test_causal_softmax_and_single_key():
    rng = np.random.default_rng(3)
    sh = B.BlockShape(hidden=32, heads=2, inter=32, seq=7, batch=2, bits=2)
    q, k, v = (rng.standard_normal((sh.batch * sh.seq, sh.hidden)) for _ in range(3))
    out, P = B.attention(q, k, v, sh)
    assert np.allclose(P.sum(-1), 1.0, rtol=1e-12)
    assert np.all(np.triu(P[0, 0], 1) == 0)
    # the first query sees only the first key: its output is that key's value
    vv = v.reshape(sh.batch, sh.seq, sh.heads, sh.head_dim)
    oo = out.reshape(vv.shape)
    assert np.allclose(oo[:, 0], vv[:, 0], rtol=1e-12)


def test_cosine_schedule_and_adamw_match_torch():
    rng = np.random.default_rng(4)
    opt = B.AdamW(lr_weight=2e-5, lr_quant=1e-4, total_steps=5, weight_decay=0.01)
    shapes = {"W": (6, 8), "s": (6, 2), "z": (6, 2)}
    p0 = {k: rng.standard_normal(v) for k, v in shapes.items()}
    grads = [{k: rng.standard_normal(v) * 1e-3 for k, v in shapes.items()} for _ in range(4)]
    # torch: one optimizer with two groups, a cosine schedule on each group
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p0.items()}
    topt = torch.optim.AdamW([{"params": [tp["W"]], "lr": opt.lr_weight},
                              {"params": [tp["s"], tp["z"]], "lr": opt.lr_quant}],
                             betas=opt.betas, eps=opt.eps, weight_decay=opt.weight_decay)
    sched = torch.optim.lr_scheduler.CosineAnnealingLR(topt, T_max=opt.total_steps, eta_min=0.0)
    mine = {k: (v.copy(), np.zeros_like(v), np.zeros_like(v)) for k, v in p0.items()}
    for kstep, g in enumerate(grads):
        for key in tp:
            tp[key].grad = torch.tensor(g[key])
        assert math.isclose(topt.param_groups[0]["lr"], B.cosine_lr(opt.lr_weight, kstep, opt.total_steps),
                            rel_tol=1e-12)
        topt.step()
        sched.step()
        for key in mine:
            p, m, v = mine[key]
            lr = B.cosine_lr(opt.lr_weight if key == "W" else opt.lr_quant, kstep, opt.total_steps)
            mine[key] = B.adamw_update(p, g[key], m, v, lr, kstep + 1, opt)
        for key in mine:
            assert np.allclose(mine[key][0], tp[key].detach().numpy(), rtol=1e-13, atol=1e-16)
    assert B.cosine_lr(1.0, 0, 10) == 1.0 and math.isclose(B.cosine_lr(1.0, 5, 10), 0.5)
    assert abs(B.cosine_lr(1.0, 10, 10)) < 1e-15


def test_first_adamw_step_closed_form():
    rng = np.random.default_rng(5)
    p, g = rng.standard_normal(100), rng.standard_normal(100) * 1e-4
    opt = B.AdamW()
    new, _, _ = B.adamw_update(p, g, np.zeros(100), np.zeros(100), 1e-4, 1, opt)
    assert np.allclose(new, p - 1e-4 * g / (np.abs(g) + opt.eps), rtol=1e-12)


# ---------------------------------------------------------------------------
# the whole block against torch autograd on an independent statement
# ---------------------------------------------------------------------------

class _FakeQuant(torch.autograd.Function):
    """Eq. 1-2 with the straight-through rules (in range: dW 1, ds rint(u) - u;
    clamped: dW 0, ds q - zr, dz -s), written with torch ops."""

    @staticmethod
    def forward(ctx, W, s, z, K, group):
        se = s.repeat_interleave(group, dim=1)
        zr = torch.clamp(torch.round(z), 0, K).repeat_interleave(group, dim=1)
        u = (W.float() / se.float()).double()     # the quotient is one fp32 division
        v = torch.round(u) + zr
        q = torch.clamp(v, 0, K)
        m = (v >= 0) & (v <= K)
        ctx.save_for_backward(u, q, zr, se, m)
        ctx.group = group
        return (q - zr) * se

    @staticmethod
    def backward(ctx, gw):
        u, q, zr, se, m = ctx.saved_tensors
        g = ctx.group
        dW = torch.where(m, gw, torch.zeros_like(gw))
        ds = (gw * torch.where(m, torch.round(u) - u, q - zr)).reshape(gw.shape[0], -1, g).sum(-1)
        dz = (gw * torch.where(m, torch.zeros_like(gw), -se)).reshape(gw.shape[0], -1, g).sum(-1)
        return dW, ds, dz, None, None


def _torch_block(x, tgt, g1, g2, params, sh):
    K = (1 << sh.bits) - 1
    T, nh, hd, Bt = sh.seq, sh.heads, sh.head_dim, sh.batch
    tw = {n: {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in p.items()}
          for n, p in params.items()}

    def lin(h, n):
        w = _FakeQuant.apply(tw[n]["W"], tw[n]["s"], tw[n]["z"], K, sh.group)
        return h @ w.T

    def norm(h, g):
        return h * torch.rsqrt((h * h).mean(-1, keepdim=True) + B.RMS_EPS) * g

    def rot(h):
        half = hd // 2
        inv = 1.0 / (B.ROPE_BASE ** (torch.arange(0, half, dtype=torch.float64) * 2 / hd))
        ang = torch.outer(torch.arange(T, dtype=torch.float64), inv)
        cos = torch.cat([ang.cos(), ang.cos()], -1)[None, :, None, :]
        sin = torch.cat([ang.sin(), ang.sin()], -1)[None, :, None, :]
        h4 = h.reshape(Bt, T, nh, hd)
        rh = torch.cat([-h4[..., half:], h4[..., :half]], -1)
        return (h4 * cos + rh * sin).reshape(Bt * T, nh * hd)

    X = torch.tensor(x)
    h1 = norm(X, torch.tensor(g1))
    q, k, v = rot(lin(h1, "q_proj")), rot(lin(h1, "k_proj")), lin(h1, "v_proj")
    q4, k4, v4 = (t.reshape(Bt, T, nh, hd).transpose(1, 2) for t in (q, k, v))
    S = q4 @ k4.transpose(-1, -2) / math.sqrt(hd)
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    attn = (torch.softmax(S, -1) @ v4).transpose(1, 2).reshape(Bt * T, nh * hd)
    x2 = X + lin(attn, "o_proj")
    h2 = norm(x2, torch.tensor(g2))
    a = torch.nn.functional.silu(lin(h2, "gate_proj")) * lin(h2, "up_proj")
    y = x2 + lin(a, "down_proj")
    loss = ((y - torch.tensor(tgt)) ** 2).mean()
    loss.backward()
    grads = {n: {k: t.grad.numpy() for k, t in p.items()} for n, p in tw.items()}
    return y.detach().numpy(), float(loss.detach()), grads


def test_block_matches_torch_autograd():
    rng = np.random.default_rng(6)
    sh = TINY
    params = _params(sh, rng)
    x, tgt, g1, g2 = _inputs(sh, rng)
    c = B.block_forward(x, params, g1, g2, sh)
    loss, dy = B.mse(c["y"], tgt)
    grads = B.block_backward(dy, c, params, g1, g2, sh)
    ty, tloss, tgrads = _torch_block(x, tgt, g1, g2, params, sh)
    assert np.allclose(c["y"], ty, rtol=1e-12, atol=1e-12)
    assert math.isclose(loss, tloss, rel_tol=1e-12)
    for n in B.LINEARS:
        for key in ("W", "s", "z"):
            a, b = grads[n][key], tgrads[n][key]
            assert np.allclose(a, b, rtol=1e-9, atol=1e-12 * np.abs(b).max()), (n, key)


# ---------------------------------------------------------------------------
# finite differences of the block loss (straight-through surrogate)
# ---------------------------------------------------------------------------

def _surrogate_loss(x, tgt, g1, g2, params, frozen, sh):
    """The block loss with W_hat = (clip(W/s + f + zr, 0, K) - zr) s, where f is
    the rounding residual rint(u) - u frozen at the base point and zr the base
    point's rounded zero point plus the change in z."""
    K = (1 << sh.bits) - 1
    w_hat = {}
    for n, p in params.items():
        se = np.repeat(p["s"], sh.group, 1)
        zr = np.repeat(p["z"] + frozen[n]["dz"], sh.group, 1)
        w_hat[n] = (np.clip(p["W"] / se + frozen[n]["f"] + zr, 0, K) - zr) * se

    def lin(h, n):
        return h @ w_hat[n].T

    h1, _ = B.rmsnorm(x, g1)
    q, k, v = B.rope(lin(h1, "q_proj"), sh), B.rope(lin(h1, "k_proj"), sh), lin(h1, "v_proj")
    attn, _ = B.attention(q, k, v, sh)
    x2 = x + lin(attn, "o_proj")
    h2, _ = B.rmsnorm(x2, g2)
    y = x2 + lin(B.silu(lin(h2, "gate_proj")) * lin(h2, "up_proj"), "down_proj")
    return B.mse(y, tgt)[0]


def test_block_gradients_by_finite_differences():
    rng = np.random.default_rng(7)
    sh = TINY
    params = _params(sh, rng)
    # keep weights away from the clamp kinks and rounding ties
    K = (1 << sh.bits) - 1
    for n, p in params.items():
        se = np.repeat(p["s"], sh.group, 1).astype(np.float64)
        ze = np.repeat(p["z"], sh.group, 1).astype(np.float64)
        inside = rng.choice(np.arange(1, K), size=p["W"].shape)
        outside = rng.choice(np.array([-2, -1, K + 1, K + 2]), size=p["W"].shape)
        vint = np.where(rng.random(p["W"].shape) < 0.7, inside, outside)
        p["W"] = Q.fl32((vint - ze + rng.uniform(-0.35, 0.35, p["W"].shape)) * se)
    x, tgt, g1, g2 = _inputs(sh, rng)
    c = B.block_forward(x, params, g1, g2, sh)
    loss, dy = B.mse(c["y"], tgt)
    grads = B.block_backward(dy, c, params, g1, g2, sh)

    p64 = {n: {k: np.asarray(v, np.float64) for k, v in p.items()} for n, p in params.items()}
    frozen = {}
    for n, p in p64.items():
        t = Q.quantize(params[n]["W"], params[n]["s"], params[n]["z"], sh.bits, sh.group)
        # residual against the exact quotient, so the surrogate equals the oracle at the base point
        quot = p["W"] / np.repeat(p["s"], sh.group, 1)
        frozen[n] = {"f": np.rint(t["u"]) - quot, "dz": np.rint(p["z"]) - p["z"]}
    base = _surrogate_loss(x, tgt, g1, g2, p64, frozen, sh)
    assert math.isclose(base, loss, rel_tol=1e-9)

    def fd(n, key, idx, h):
        a = {m: {k: v.copy() for k, v in p.items()} for m, p in p64.items()}
        b = {m: {k: v.copy() for k, v in p.items()} for m, p in p64.items()}
        a[n][key][idx] += h
        b[n][key][idx] -= h
        return (_surrogate_loss(x, tgt, g1, g2, a, frozen, sh) - _surrogate_loss(x, tgt, g1, g2, b, frozen, sh)) / (2 * h)

    for n in B.LINEARS:
        o, i = p64[n]["W"].shape
        for idx in [(0, 0), (o - 1, i - 1), (o // 2, i // 3)]:
            h = 1e-6 * max(abs(p64[n]["W"][idx]), 1e-3)
            g = grads[n]["W"][idx]
            assert abs(fd(n, "W", idx, h) - g) <= 1e-6 * np.abs(grads[n]["W"]).max() + 1e-7 * abs(g), (n, idx)
        for idx in [(0, 0), (o - 1, p64[n]["s"].shape[1] - 1)]:
            num = fd(n, "s", idx, 1e-7 * p64[n]["s"][idx])
            assert abs(num - grads[n]["s"][idx]) <= 1e-5 * (abs(num) + np.abs(grads[n]["s"]).max()), (n, "s")
            num = fd(n, "z", idx, 1e-4)
            assert abs(num - grads[n]["z"][idx]) <= 1e-5 * (abs(num) + np.abs(grads[n]["z"]).max()), (n, "z")


def test_block_ap_step_moves_every_parameter_group():
    rng = np.random.default_rng(8)
    sh = TINY
    params = _params(sh, rng)
    x, tgt, g1, g2 = _inputs(sh, rng)
    state = {n: {k: (np.zeros_like(v, np.float64), np.zeros_like(v, np.float64)) for k, v in p.items()}
             for n, p in params.items()}
    opt = B.AdamW(total_steps=10)
    loss, newp, news, grads = B.block_ap_step(x, tgt, params, state, g1, g2, sh, 0, opt)
    for n in B.LINEARS:
        for key, lr in (("W", opt.lr_weight), ("s", opt.lr_quant), ("z", opt.lr_quant)):
            g = grads[n][key]
            expect = Q.fl32(np.asarray(params[n][key], np.float64) - lr * g / (np.abs(g) + opt.eps))
            assert np.array_equal(newp[n][key], expect), (n, key)


def test_forward_rows_match_torch_statement():
    # the sampled-token forward against the independent torch statement's output
    rng = np.random.default_rng(9)
    sh = B.BlockShape(hidden=32, heads=2, inter=48, seq=9, batch=2, bits=3, group=16)
    params = _params(sh, rng)
    x, tgt, g1, g2 = _inputs(sh, rng)
    ty, _, _ = _torch_block(x, tgt, g1, g2, params, sh)
    for b, rows in ((0, [0, 4, 8]), (1, [3]), (1, [0, 1, 2, 5, 6])):
        y = B.block_forward_rows(x, params, g1, g2, sh, b, rows)
        assert np.allclose(y, ty[b * sh.seq + np.asarray(rows)], rtol=1e-12, atol=1e-12), (b, rows)


def test_rope_at_positions():
    # rope over a whole tensor equals rope_at with the tokens' positions; a
    # position-p rotation composed with its inverse is the identity
    rng = np.random.default_rng(10)
    sh = B.BlockShape(hidden=64, heads=2, inter=64, seq=5, batch=3, bits=2)
    x = rng.standard_normal((sh.batch * sh.seq, sh.hidden))
    pos = np.tile(np.arange(sh.seq), sh.batch)
    assert np.array_equal(B.rope(x, sh), B.rope_at(x, pos, sh.heads, sh.head_dim))
    p = rng.integers(0, 4096, x.shape[0])
    back = B.rope_at(B.rope_at(x, p, 2, 32), p, 2, 32, inverse=True)
    assert np.allclose(back, x, rtol=1e-12, atol=1e-12)
