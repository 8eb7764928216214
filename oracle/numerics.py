"""Number formats used by the layer step (oracle side; test infrastructure only).

* bf16: 1 sign, 8 exponent, 7 stored mantissa bits.  Rounding here goes straight
  from fp64 to bf16, round to nearest, ties to even, subnormals kept, so there is
  no double rounding through fp32.
* NVFP4 (the pages store the routed experts "as 4-bit NVFP4" -- Muse Spark Open
  layer description, "where the kernel boundary sits"): E2M1 element codes, one
  E4M3 scale per 16 consecutive elements along K, and one fp32 scale per tensor.
  The pages give no more detail, so the format is taken from its public
  definition (OCP 8-bit floating point for E4M3 "FN": bias 7, no infinities,
  S.1111.111 is NaN, max 448; E2M1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).

Every quantisation decision below is an exact comparison of the input against a
midpoint of the target grid, scaled, so any two correct implementations agree to
the bit: the thresholds are products of at most 31 significant bits, exact in fp64.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16

def bf16_round(x) -> np.ndarray:
    """fp64 -> bf16 bit pattern (uint16), round to nearest even, directly from fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    # quantum of the bf16 grid at |x|: 2^(e-7) for normal |x| in [2^e, 2^(e+1)), 2^-133 below 2^-126
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one right at powers of two; fix with exact comparisons
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, -126)
    q = np.ldexp(1.0, (e - 7).astype(np.int64))
    out = np.rint(x / q) * q          # x/q is exact (power of two); rint = ties to even
    out = np.where(ax == 0, x, out)   # keep signed zero
    f32 = out.astype(np.float32)      # exact: out has <= 8 significant bits
    big = np.abs(out) > 3.3895313892515355e38
    f32 = np.where(big, np.copysign(np.float32(np.inf), out).astype(np.float32), f32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- E2M1 / E4M3

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_value(code) -> np.ndarray:
    """4-bit E2M1 code -> value: sign is bit 3, magnitude code in bits 0..2."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def e4m3_value(byte) -> np.ndarray:
    """OCP E4M3 'FN' byte -> value. E=0: (M/8)*2^-6; else (1+M/8)*2^(E-7); S.1111.111 = NaN."""
    b = np.asarray(byte, dtype=np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    E = (b >> 3) & 15
    M = b & 7
    mag = np.where(E == 0, (M / 8.0) * 2.0 ** -6, (1.0 + M / 8.0) * np.ldexp(1.0, E - 7))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return s * mag


# non-negative finite E4M3 values in increasing order; index == byte code 0..126
E4M3_POS = e4m3_value(np.arange(127))
_E4M3_MID = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2.0          # 126 midpoints, <= 5 significant bits
_E2M1_MID = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0        # 0.25 .75 1.25 1.75 2.5 3.5 5


def _rne_index(v: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point to each v >= 0 given the grid's midpoints,
    ties to the even index.  `v` and `mids` are compared exactly."""
    lo = np.searchsorted(mids, v, side="left")    # number of midpoints strictly below v
    hi = np.searchsorted(mids, v, side="right")   # number of midpoints <= v
    tie = hi > lo                                  # v equals midpoint `lo`
    # at a tie v sits between grid points lo and lo+1: take the even one
    return np.where(tie, np.where(lo % 2 == 0, lo, lo + 1), lo)


def e4m3_rne_scale(amax: np.ndarray, denom: np.ndarray) -> np.ndarray:
    """Byte code of RNE_e4m3(amax / denom), saturating at 448, for amax >= 0, denom > 0.
    Decided by comparing amax with denom*midpoint (exact in fp64)."""
    amax = np.asarray(amax, dtype=np.float64)
    denom = np.asarray(denom, dtype=np.float64)
    # compare amax/denom against midpoints <=> amax against denom*mid; do it per element
    thr = denom[..., None] * _E4M3_MID                       # exact products
    below = (thr < amax[..., None]).sum(-1)                  # midpoints strictly below
    equal = (thr == amax[..., None]).sum(-1)
    idx = np.where(equal > 0, np.where(below % 2 == 0, below, below + 1), below)
    return np.minimum(idx, 126).astype(np.uint8)


def _nvfp4_codes(x: np.ndarray, unit: np.ndarray) -> np.ndarray:
    """E2M1 codes of x on the grid {0,.5,...,6} * unit (unit > 0 per element), RNE with
    ties to the even code, saturating at +-6; a result of magnitude 0 is +0 (code 0)."""
    ax = np.abs(x)
    thr = unit[..., None] * _E2M1_MID                        # exact (<= 31 bits)
    below = (thr < ax[..., None]).sum(-1)
    equal = (thr == ax[..., None]).sum(-1)
    mag = np.where(equal > 0, np.where(below % 2 == 0, below, below + 1), below)
    mag = np.minimum(mag, 7)
    sign = np.where((x < 0) & (mag > 0), 8, 0)
    return (mag + sign).astype(np.uint8)


def nvfp4_pack(w) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Quantise one weight matrix w [N][K] (K % 16 == 0) to NVFP4.

    tensor scale ts = fp32(amax) / 2688 rounded to fp32 (2688 = 6 * 448, the largest
    E2M1 magnitude times the largest E4M3 scale), ts = 1 when amax = 0; block scale
    s = RNE_e4m3(amax_block / (6 ts)); code = RNE_e2m1(x / (s ts)), codes all +0 when
    s = 0.  Returns (codes uint8 [N][K/2] with element 2j in the low nibble,
    scales uint8 [N][K/16], ts)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % 16 == 0
    amax = np.float32(np.abs(w).max()) if w.size else np.float32(0)
    ts = np.float32(amax) / np.float32(2688.0) if amax > 0 else np.float32(1.0)
    ts = np.float32(ts)
    blocks = w.reshape(N, K // 16, 16)
    bmax = np.abs(blocks).max(-1)
    sb = e4m3_rne_scale(bmax, np.full(bmax.shape, 6.0 * np.float64(ts)))
    sval = E4M3_POS[sb]
    unit = np.repeat((sval * np.float64(ts))[..., None], 16, -1)
    codes = _nvfp4_codes(blocks, np.where(unit > 0, unit, 1.0))
    codes = np.where(unit > 0, codes, 0).astype(np.uint8).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb.astype(np.uint8), ts


def nvfp4_decode(codes, scales, ts) -> np.ndarray:
    """Decoded weights e2m1(code) * e4m3(scale) * ts as fp64 [N][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    lo = codes & 15
    hi = codes >> 4
    c = np.empty((N, codes.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    s = np.repeat(e4m3_value(np.asarray(scales)), 16, axis=1)
    return e2m1_value(c) * s * np.float64(ts)


def fp4_act_quant(a) -> tuple[np.ndarray, np.ndarray]:
    """NVFP4 requantisation of the SwiGLU intermediate before the second expert GEMM
    (the pages gather it "in fp4" after the first GEMM).  Tensor scale 1, one E4M3
    scale per 16 consecutive elements.  The decisions are taken on the value itself
    (fp64 here), compared exactly with 6*mid (scale) and mid*s (code): both thresholds
    have few significant bits and are exact in fp64 (and in fp32).
    Returns (codes uint8 [M][K/2], scales uint8 [M][K/16])."""
    a = np.asarray(a, dtype=np.float64)
    M, K = a.shape
    blocks = a.reshape(M, K // 16, 16)
    bmax = np.abs(blocks).max(-1)
    sb = e4m3_rne_scale(bmax, np.full(bmax.shape, 6.0))
    sval = E4M3_POS[sb]
    unit = np.repeat(sval[..., None], 16, -1)
    codes = _nvfp4_codes(blocks, np.where(unit > 0, unit, 1.0))
    codes = np.where(unit > 0, codes, 0).astype(np.uint8).reshape(M, K)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), sb.astype(np.uint8)
