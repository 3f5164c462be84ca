"""Shared helpers for the tests (not a test module)."""
import numpy as np
import torch

from oracle import qat_oracle as O

U_BF16 = 2.0 ** -8        # unit roundoff of bf16 (8 significant bits, round to nearest)
U_F32 = 2.0 ** -24        # unit roundoff of fp32


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def gamma(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32: the relative bound of a sum of
    n terms accumulated in fp32 in any order, relative to the sum of |terms|."""
    return n * U_F32 / (1.0 - n * U_F32)


def bf16_gemm_bound(ref: np.ndarray, absprod: np.ndarray, k: int) -> np.ndarray:
    """Largest |got - ref| that a correct bf16 GEMM output element can show.

    got = bf16(acc), acc = the fp32 sum, in any order, of the k products
    a_i * b_i, where a_i is an exact bf16 input (X or dY), b_i = bf16(fl32(w_i))
    the bf16 operand made from the exact dequantised weight w_i, and every
    product of two bf16 values is exact in fp32. ref = sum a_i w_i (fp64) and
    absprod = sum |a_i| |w_i|. The matrix cores' adders are allowed an error of
    up to one fp32 ulp (2u, as if truncating) per addition, hence 2 gamma_k.
    With e_b = 2^-8 + 2^-23 (fp32 then bf16 rounding of w_i):
      |sum a_i b_i - ref| <= e_b absprod
      |acc - sum a_i b_i| <= 2 gamma_k (1 + e_b) absprod
      |got - acc|         <= 2^-8 |acc|
    so |got - ref| <= 2^-8 |ref| + (1 + 2^-8) (e_b + 2 gamma_k (1 + e_b)) absprod.
    A tiny absolute term covers fp32 subnormals flushed by the matrix cores."""
    e_b = U_BF16 + 2.0 * U_F32
    c = (1.0 + U_BF16) * (e_b + 2.0 * gamma(k) * (1.0 + e_b))
    return U_BF16 * np.abs(ref) + c * absprod + k * 2.0 ** -126


def f32_gemm_bound(absprod: np.ndarray, k: int) -> np.ndarray:
    """Largest |got - ref| of an fp32 output accumulated in fp32 from k exact
    products of bf16 values (no output rounding beyond fp32): 2 gamma_k absprod
    (one fp32 ulp per addition, as in bf16_gemm_bound) plus one more fp32
    rounding of a value bounded by absprod."""
    return (2.0 * gamma(k) + U_F32) * absprod + k * 2.0 ** -126


def check_bound(name: str, got: np.ndarray, ref: np.ndarray, bound: np.ndarray) -> float:
    """Assert |got - ref| <= bound element by element; returns the largest
    ratio |got - ref| / bound (for the log)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= bound)                     # NaN counts as a violation
    if bad.any():
        idx = np.argwhere(bad)
        i = tuple(idx[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} elements outside the element-wise bound; "
                             f"first at {i}: got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, 0.0)
    return float(r.max()) if r.size else 0.0


def w_hat_exact(W, s, z, bits, group: int = 64, rows: int = 2048) -> np.ndarray:
    """The oracle's exact fake-quant W_hat [out, in] (fp64), computed in blocks
    of weight rows so that the oracle's per-element arrays stay small at the
    70B shapes."""
    out = W.shape[0]
    wh = np.empty(W.shape, np.float64)
    for r in range(0, out, rows):
        t = O.quantize(W[r:r + rows], s[r:r + rows], z[r:r + rows], bits, group)
        wh[r:r + rows] = O.dequantize_exact(t["q"], t["zr"], t["s"])
    return wh


def e2e_w_hat_exact(Wq, s, z, inp, bits, group: int = 64, rows: int = 2048) -> np.ndarray:
    """The oracle's E2E-QP W_hat = (q - z) s [out, in] (fp64), in blocks of rows."""
    out = Wq.shape[0]
    wh = np.empty((out, inp), np.float64)
    for r in range(0, out, rows):
        wh[r:r + rows] = O.e2e_w_hat(Wq[r:r + rows], s[r:r + rows], z[r:r + rows], inp, bits, group)
    return wh


def check_gemm_bf16(name: str, got_bits: np.ndarray, a_bits: np.ndarray, w_hat: np.ndarray,
                    frob: float = 2e-2) -> float:
    """got (bf16 bits [m, n]) against a_bits (bf16 bits [m, k]) times w_hat^T
    ([n, k], exact fp64): the element-wise bound of bf16_gemm_bound on every
    element, and the relative Frobenius gate beside it."""
    a = O.bf16_bits_to_f64(a_bits)
    ref = a @ w_hat.T
    absprod = np.abs(a) @ np.abs(w_hat).T
    got = O.bf16_bits_to_f64(got_bits)
    r = check_bound(name, got, ref, bf16_gemm_bound(ref, absprod, a.shape[1]))
    assert rel_fro(got, ref) < frob, name
    return r


def tile_samples(n: int, band: int, rng: np.random.Generator) -> np.ndarray:
    """One index drawn in every band of `band` consecutive indices of [0, n),
    plus the first and last index: a sampled row (or column) crosses every
    output tile of that band."""
    picks = [min(n - 1, b + int(rng.integers(0, band))) for b in range(0, n, band)]
    return np.unique(np.concatenate([[0, n - 1], picks]))


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def say(*a):
    print(*a, flush=True)
