"""CPU checks of the element-wise bound that the GPU parity tests apply to the
bf16 GEMM outputs (Y, dX): a correct bf16 GEMM (bf16 operands, any fp32
accumulation order, one bf16 rounding) stays inside it, and a planted defect
in a single output tile -- one 64-deep slab of the contraction dropped, or one
32-deep k-step of a single 16 x 16 fragment dropped -- falls outside it.

The simulated kernel is numpy's fp32 GEMM on the exact bf16 operands (its
blocked fp32 summation is one of the orders the bound allows)."""
import numpy as np
import pytest

from oracle import qat_oracle as O
from weight_quantization_aware_amd import synth
from tests.helpers import bf16_gemm_bound, check_bound, check_gemm_bf16, w_hat_exact


def _case(M, out, inp, bits, seed):
    W = synth.weight(seed, 0, out, inp, 0.02, True)
    X = synth.activations(seed, 0, M, inp, 8)
    s, z = O.init_minmax(W, bits)
    wh = w_hat_exact(W, s, z, bits)
    return X, wh


def _simulated_kernel(a_bits, wh, drop=None):
    """bf16(fp32 sum of bf16 products); drop = (rows, cols, ks): those products
    are left out of the listed outputs (a planted defect)."""
    a = O.bf16_bits_to_f64(a_bits).astype(np.float32)
    b = O.bf16_round(O.fl32(wh)).astype(np.float32)          # the bf16 W_hat operand
    acc = a @ b.T                                            # fp32 accumulation
    if drop is not None:
        r, c, ks = drop
        part = a[r][:, ks] @ b[c][:, ks].T                   # fp32
        acc[np.ix_(r, c)] = acc[np.ix_(r, c)] - part
    got = O.bf16_round(acc)
    return O.f64_to_bf16_bits(got)


@pytest.fixture(scope="module")
def q_proj_like():
    # the q_proj contraction depth (in = 4096) on half its tokens and rows:
    # 64 output tiles of 128 x 256
    return _case(1024, 2048, 4096, 2, 5)


def test_correct_bf16_gemm_is_inside_the_bound(q_proj_like):
    X, wh = q_proj_like
    got = _simulated_kernel(X, wh)
    r = check_gemm_bf16("Y", got, X, wh)
    assert 0.0 < r < 1.0
    ref = O.bf16_bits_to_f64(X) @ wh.T
    assert not np.array_equal(O.bf16_bits_to_f64(got), ref)   # the rounding is really there


@pytest.mark.parametrize("drop", [
    (np.arange(128, 256), np.arange(256, 512), np.arange(640, 704)),   # one 64-slab of one 128x256 tile
    (np.arange(16, 32), np.arange(32, 48), np.arange(96, 128)),        # one k-step of one 16x16 fragment
    (np.arange(0, 128), np.arange(0, 256), np.arange(4032, 4096)),     # the last slab of the first tile
])
def test_planted_tile_defect_is_outside_the_bound(q_proj_like, drop):
    X, wh = q_proj_like
    bad = _simulated_kernel(X, wh, drop)
    with pytest.raises(AssertionError, match="element-wise bound"):
        check_gemm_bf16("Y", bad, X, wh)
    # the whole-tensor relative Frobenius gate alone does not see it (at the
    # q_proj workload's 256 tiles it would be diluted further)
    ref = O.bf16_bits_to_f64(X) @ wh.T
    fro = np.linalg.norm(O.bf16_bits_to_f64(bad) - ref) / np.linalg.norm(ref)
    assert fro < 2e-2


def test_dx_shaped_contraction():
    # dX = dY W_hat contracts over out (here 512): the same bound with k = out
    out, inp, M = 512, 1024, 256
    W = synth.weight(9, 0, out, inp, 0.02, True)
    dY = synth.grad_out(9, 0, M, out)
    s, z = O.init_minmax(W, 3)
    wh_t = w_hat_exact(W, s, z, 3).T.copy()                  # dX = dY (W_hat^T)^T
    check_gemm_bf16("dX", _simulated_kernel(dY, wh_t), dY, wh_t)
    bad = _simulated_kernel(dY, wh_t, (np.arange(128, 256), np.arange(0, 256), np.arange(64, 128)))
    with pytest.raises(AssertionError):
        check_gemm_bf16("dX", bad, dY, wh_t)


def test_bound_rejects_nan_and_counts_violations():
    ref = np.ones((2, 2))
    b = bf16_gemm_bound(ref, np.ones((2, 2)), 64)
    with pytest.raises(AssertionError, match="1 of 4"):
        check_bound("t", np.array([[1.0, np.nan], [1.0, 1.0]]), ref, b)
