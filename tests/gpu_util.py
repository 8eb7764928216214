"""Shared helpers of the GPU parity tests: tolerance checks against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_TOL = 2e-2       # max|gpu - ref| / max|ref| per tensor (bf16 / NVFP4 data, fp32 accumulation)
STAT_TOL = 1e-5      # |gpu - ref| <= STAT_TOL * max(1, |ref|) for fp32 softmax statistics and gates


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def max_abs_rel(gpu_bits, ref_bits) -> float:
    g = oracle.bf16_to_f64(gpu_bits)
    r = oracle.bf16_to_f64(ref_bits)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def assert_close_bf16(name, gpu_bits, ref_bits, tol=REL_TOL):
    assert gpu_bits.shape == ref_bits.shape, (name, gpu_bits.shape, ref_bits.shape)
    assert not np.any(gpu_bits == 0xFFFF), f"{name}: unwritten (poison) elements"
    err = max_abs_rel(gpu_bits, ref_bits)
    same = float(np.mean(gpu_bits == ref_bits))
    log(f"  {name}: max-abs-rel {err:.3e}, bit-identical fraction {same:.4f}")
    assert err <= tol, f"{name}: max-abs-rel {err} > {tol}"
    return err


def assert_stats(name, gpu, ref, tol=STAT_TOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref))
    log(f"  {name}: max scaled error {err.max():.3e}")
    assert err.max() <= tol, f"{name}: {err.max()} > {tol}"


def fp32_dot_bound(x_bits, w_bits) -> np.ndarray:
    """Rigorous bound on |fp32 dot - exact dot| for x . w^T with K terms: gamma_K * sum|x||w|,
    gamma_K = K u / (1 - K u), u = 2^-24 (any summation order)."""
    x = np.abs(oracle.bf16_to_f64(x_bits))
    w = np.abs(oracle.bf16_to_f64(w_bits))
    K = x.shape[1]
    u = 2.0 ** -24
    return (K * u / (1 - K * u)) * (x @ w.T)


# fp32 unit roundoff taken as 2^-23 (not 2^-24) so that the bounds below also hold if an
# accumulation step truncates instead of rounding to nearest
U32 = 2.0 ** -23
U64 = 2.0 ** -53
MISMATCH_CEILING = 0.005     # at most this fraction of an anchored stage's elements may differ


def rounding_band(x_bits, w_bits, residual_bits=None, extra_terms: int = 16):
    """Exact value v = x . W^T (+ residual) of a dense stage on bf16 inputs, and a rigorous
    bound B on |fp32 result - v| for any fp32 summation order: every product of two bf16
    values is exact in fp32, a sum of n terms is within gamma_n sum|x||w| (n = K plus
    `extra_terms` for partial sums combined afterwards), and the residual add rounds once
    more.  The fp64 evaluation of v adds its own (tiny) error bound."""
    x = oracle.bf16_to_f64(x_bits)
    w = oracle.bf16_to_f64(w_bits)
    v = x @ w.T
    if residual_bits is not None:
        v = v + oracle.bf16_to_f64(residual_bits)
    n = x.shape[1] + extra_terms
    g32 = n * U32 / (1 - n * U32)
    g64 = (n + 2) * U64 / (1 - (n + 2) * U64)
    mag = np.abs(x) @ np.abs(w).T
    B = (g32 + g64) * mag
    if residual_bits is not None:
        B = B + U32 * (np.abs(v) + B)
    B = B + 2.0 ** -50 * np.abs(v)
    return v, B


def assert_rounding_exact(name, gpu_bits, x_bits, w_bits, residual_bits=None, ceiling=MISMATCH_CEILING):
    """An anchored dense stage, bf16(x . W^T (+ residual)) with fp32 accumulation, against the
    exact value v.  With B the rigorous fp32 error bound (rounding_band), every GPU element
    must lie between bf16(v - B) and bf16(v + B): it equals the correctly rounded oracle value
    bit for bit unless v lies within B of a bf16 rounding boundary ("ambiguous"), and even
    then it is one of the two roundings.  The elements that differ from the oracle's
    rounding may be at most `ceiling` of the tensor (at least 2): a correct kernel differs
    only where its accumulation error crosses a boundary, a fraction of a percent."""
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    assert not np.any(gpu_bits == 0xFFFF), f"{name}: unwritten (poison) elements"
    v, B = rounding_band(x_bits, w_bits, residual_bits)
    assert gpu_bits.shape == v.shape, (name, gpu_bits.shape, v.shape)
    ref = oracle.bf16_round(v)
    lo = oracle.bf16_to_f64(oracle.bf16_round(v - B))
    hi = oracle.bf16_to_f64(oracle.bf16_round(v + B))
    g = oracle.bf16_to_f64(gpu_bits)
    outside = ~((g >= lo) & (g <= hi))
    ambiguous = int(np.count_nonzero(lo != hi))
    mismatch = int(np.count_nonzero(gpu_bits != ref))
    limit = max(2, int(ceiling * gpu_bits.size))
    log(f"  {name}: {gpu_bits.size - mismatch}/{gpu_bits.size} bit-equal to the oracle's rounding, "
        f"{mismatch} differ (limit {limit}), {ambiguous} within the fp32 bound of a rounding boundary, "
        f"{int(outside.sum())} outside the bound")
    assert not outside.any(), f"{name}: {int(outside.sum())} elements outside the rigorous fp32 band"
    assert mismatch <= limit, f"{name}: {mismatch} elements differ from the oracle's rounding (limit {limit})"
    return mismatch, ambiguous


def check_routing(gpu_logits, gpu_idx, gpu_gate, ref_logits64, bias, k, max_dlogit):
    """Routing parity: (i) indices equal the stable full sort of the GPU's own logits, always;
    (ii) equal the oracle's except where the oracle's k-th / (k+1)-th gap is within the
    logits' error (several correct answers); returns the number of such ambiguous tokens."""
    T, E = gpu_logits.shape
    for t in range(T):
        order = np.lexsort((np.arange(E), -gpu_logits[t].astype(np.float64)))[:k]
        assert list(gpu_idx[t]) == list(order), f"token {t}: idx not the sort of its own logits"
    z = ref_logits64.astype(np.float32)
    if bias is not None:
        z = (z + bias.astype(np.float32)).astype(np.float32)
    ambiguous = 0
    for t in range(T):
        ref_order = np.lexsort((np.arange(E), -z[t].astype(np.float64)))
        srt = np.sort(z[t].astype(np.float64))[::-1]
        gap = srt[k - 1] - srt[k] if E > k else np.inf
        if list(gpu_idx[t]) != list(ref_order[:k]):
            assert gap <= 2 * max_dlogit + 1e-6, f"token {t}: routing differs with gap {gap}"
            ambiguous += 1
        else:
            sel = z[t][gpu_idx[t]].astype(np.float64)
            g = np.exp(sel - sel.max())
            g /= g.sum()
            assert np.abs(g - gpu_gate[t]).max() <= STAT_TOL, f"token {t}: gates"
    log(f"  routing: {T - ambiguous}/{T} tokens identical to the oracle, {ambiguous} ambiguous")
    return ambiguous
