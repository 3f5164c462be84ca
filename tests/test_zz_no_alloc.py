"""The forward entry point that allocates nothing (qat_fakequant_linear_fwd_noalloc):
its W_hat lives in the library's static device scratch. Through the C ABI it
must give the workspace forward's Y bit for bit, on two calls in a row (the
second smaller, so the scratch still holds the first call's larger W_hat),
and refuse a problem larger than the scratch without launching anything."""
import numpy as np
import pytest
import torch

from oracle import qat_oracle as O
from weight_quantization_aware_amd import _lib as Q
from weight_quantization_aware_amd import synth
from tests.helpers import check_gemm_bf16, dev_bf16, dev_f32, host_bits, say, w_hat_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _case(M, out, inp, bits, group, seed):
    W = synth.weight(seed, bits, out, inp, 0.02, True)
    X = synth.activations(seed, bits, M, inp, 4)
    s, z = O.init_minmax(W, bits, group)
    s, z = synth.perturb_qparams(seed, s, z, bits)
    return W, X, s, z


def test_noalloc_forward_equals_workspace_forward_twice():
    # a 7B-MLP-sized weight (11008 x 4096 = 43 Mi of the 48 Mi scratch), then a
    # small ragged one
    for M, out, inp, bits, group in [(300, 11008, 4096, 2, 64), (77, 320, 512, 3, 128)]:
        say(f"noalloc forward M={M} out={out} in={inp} bits={bits} group={group}")
        W, X, s, z = _case(M, out, inp, bits, group, 17)
        args = (dev_bf16(X), dev_f32(W), dev_f32(s), dev_f32(z), bits)
        Y_ws = torch.empty(M, out, dtype=torch.bfloat16, device="cuda")
        Y_na = torch.full_like(Y_ws, 3.0)
        Q.qat_fakequant_linear_fwd(*args, Y_ws, ws=Q.workspace(Q.fakequant_ws_bytes(out, inp, bits)), group=group)
        Q.qat_fakequant_linear_fwd_noalloc(*args, Y_na, group=group)
        torch.cuda.synchronize()
        assert torch.equal(Y_ws, Y_na)
        if out * inp <= 1 << 20:
            check_gemm_bf16("Y", host_bits(Y_na), X, w_hat_exact(W, s, z, bits, group))


def test_noalloc_forward_refuses_more_than_the_scratch():
    n = Q.noalloc_max_weights()
    assert n == 48 << 20
    out, inp = 8192, 8192                       # 64 Mi weights
    W = torch.zeros(out, inp, device="cuda")
    s = torch.ones(out, inp // 64, device="cuda")
    z = torch.zeros_like(s)
    X = torch.zeros(1, inp, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((1, out), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Q.QatError) as e:
        Q.qat_fakequant_linear_fwd_noalloc(X, W, s, z, 2, Y)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert torch.all(Y == 5.0)
