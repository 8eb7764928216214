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
