"""One rank's share of the N-sharded expert layout, written out plainly in fp64 (test
infrastructure only).

The pages shard both expert GEMMs of the MoE on their output dimension N across the R
tensor-parallel ranks, which puts an all-gather after each: an fp4 all-gather of the
intermediate after the first GEMM and a bf16 all-gather of the expert output after the
second.  The authors prefer this to sharding the intermediate dimension (one all-reduce)
because the layout is bitwise-consistent with expert parallelism (orcarouter.ai write-up,
section "where the kernel boundary sits").  Receivers poll the payload against a sentinel
that no result can take (alphasignal.ai, "Four mechanisms keep work moving").

Reading of that passage (the pages give no shapes or index order):
  * a full expert has intermediate width R*I.  Rank r owns intermediate channels
    [r I, (r+1) I): its first GEMM is the full expert's gate rows and up rows of those
    channels, [2I][P];
  * its second GEMM is rows [r P/R, (r+1) P/R) of the full down projection, [P/R][R I],
    multiplied by the whole gathered intermediate (K = R I);
  * the combine over the k routed slots is local (each rank has every slot's columns); the
    bf16 all-gather then assembles y [T][P] from the ranks' column slices;
  * the gathered intermediate of a pair is the concatenation of the ranks' NVFP4 slices.
    With I a multiple of 16 no 16-element scale block straddles two ranks, so it equals the
    NVFP4 requantisation of the full-width intermediate row: the bitwise agreement with
    expert parallelism that the pages name.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64, nvfp4_decode, fp4_act_quant
from .layer import silu


def shard_w1(w1_full, I: int, r: int):
    """Rank r's GEMM1 weight [2I][P] from the full-width [2 R I][P]."""
    w1_full = np.asarray(w1_full)
    RI = w1_full.shape[0] // 2
    gate = w1_full[r * I:(r + 1) * I]
    up = w1_full[RI + r * I:RI + (r + 1) * I]
    return np.concatenate([gate, up], axis=0)


def shard_w2(w2_full, R: int, r: int):
    """Rank r's GEMM2 weight [P/R][R I]: rows r P/R .. (r+1) P/R of the full [P][R I]."""
    w2_full = np.asarray(w2_full)
    n = w2_full.shape[0] // R
    return w2_full[r * n:(r + 1) * n]


def intermediate_slice(xp_row, w1_rank_dec, I: int):
    """One pair's intermediate slice on rank r: a = silu(gate) * up of the rank's channels
    (fp64), requantised to NVFP4.  Returns (codes [I/2], scales [I/16])."""
    u = xp_row @ w1_rank_dec.T
    a = silu(u[:I]) * u[I:]
    codes, scales = fp4_act_quant(a[None, :])
    return codes[0], scales[0]


def gather_row(slices):
    """The gathered intermediate of one pair: the R ranks' (codes, scales) slices in rank
    order, concatenated."""
    return (np.concatenate([c for c, _ in slices]), np.concatenate([s for _, s in slices]))


def moe_rank(xp_bits, idx, gate, w1_rank: dict, w2_shard: dict, I: int, R: int, r: int,
             peer_codes, peer_scales):
    """Rank r's expert work and combine.

    xp_bits bf16 [T][P]; idx, gate [T][k]; w1_rank {e: (codes, scales, ts)} packed [2I][P];
    w2_shard {e: (codes, scales, ts)} packed [P/R][R I]; peer_codes uint8 [T k][R I / 2] and
    peer_scales uint8 [T k][R I / 16]: the gathered intermediate rows as the other ranks
    deliver them (pair p = t k + j; rank r's own slice in them is ignored, it is computed here).
    Returns y_own bf16 [T][P/R] (columns r P/R ..), and the gathered rows (codes, scales)
    with rank r's slice filled in."""
    xp = bf16_to_f64(xp_bits)
    T, k = np.asarray(idx).shape
    codes_all = np.array(peer_codes, dtype=np.uint8, copy=True)
    scales_all = np.array(peer_scales, dtype=np.uint8, copy=True)
    dec1, dec2 = {}, {}
    for e in set(np.asarray(idx).reshape(-1).tolist()):
        dec1[e] = nvfp4_decode(*w1_rank[e])
        dec2[e] = nvfp4_decode(*w2_shard[e])
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            p = t * k + j
            c, s = intermediate_slice(xp[t], dec1[e], I)
            codes_all[p, r * I // 2:(r + 1) * I // 2] = c
            scales_all[p, r * I // 16:(r + 1) * I // 16] = s
    return gemm2_rank(idx, gate, codes_all, scales_all, dec2), codes_all, scales_all


def gemm2_rank(idx, gate, codes_all, scales_all, w2_dec: dict):
    """Rank r's second GEMM and combine from the gathered rows as given: y_own[t] =
    sum over slots j (in slot order) of gate[t, j] * (decoded row of pair t k + j) . W2_e^T,
    with w2_dec {e: decoded [P/R][R I] fp64}; one bf16 rounding.  Returns bf16 [T][P/R]."""
    T, k = np.asarray(idx).shape
    n_own = next(iter(w2_dec.values())).shape[0]
    comb = np.zeros((T, n_own))
    for t in range(T):
        for j in range(k):
            p = t * k + j
            a_full = nvfp4_decode(codes_all[p][None, :], scales_all[p][None, :], 1.0)[0]
            comb[t] += gate[t, j] * (a_full @ w2_dec[int(idx[t, j])].T)
    return bf16_round(comb)


def gathered_y(y_peers_bits, y_own_bits, R: int, r: int):
    """The bf16 all-gather's result [T][P]: the peers' column slices with rank r's columns
    replaced by its own."""
    y = np.array(y_peers_bits, dtype=np.uint16, copy=True)
    n = y.shape[1] // R
    y[:, r * n:(r + 1) * n] = y_own_bits
    return y
