"""Pins of oracle/nshard.py (one rank's share of the N-sharded expert layout) against facts
that do not come from the module itself:

* one rank (R = 1) is the ordinary layer's expert step: moe_rank equals oracle.moe bit for bit;
* expert-parallel consistency: R ranks, each computing its own intermediate slice and its own
  output columns from row slices of one full-width expert, give exactly the full-width
  expert's output and intermediate (oracle.moe with inter = R I) -- this catches a wrong
  slice of either weight, a slice placed at the wrong rank offset, or a block that straddles
  two ranks;
* NVFP4 requantisation of a full row equals the concatenation of its rank slices;
* the bf16 all-gather places rank r's columns at r P/R.
"""
import numpy as np
import pytest

import oracle
from oracle import nshard
from oracle.numerics import nvfp4_pack, fp4_act_quant

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16(g, shape, scale):
    return oracle.bf16_round(g.standard_normal(shape) * scale)


def _routing(g, T, E, k):
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    z = g.standard_normal((T, k))
    gate = np.exp(z) / np.exp(z).sum(1, keepdims=True)
    return idx, gate


def _packed(mats):
    return {e: nvfp4_pack(oracle.bf16_to_f64(m)) for e, m in mats.items()}


def _slice_packed(packed, rows):
    c, s, ts = packed
    return c[rows], s[rows], ts


def test_one_rank_is_the_ordinary_expert_step():
    g = np.random.default_rng(101)
    T, P, E, k, I = 5, 64, 6, 3, 32
    xp = _bf16(g, (T, P), 1.0)
    idx, gate = _routing(g, T, E, k)
    w1 = {e: _bf16(g, (2 * I, P), 0.1) for e in range(E)}
    w2 = {e: _bf16(g, (P, I), 0.1) for e in range(E)}
    p1, p2 = _packed(w1), _packed(w2)
    y_ref, inter = oracle.moe(xp, idx, gate, {"fmt": "nvfp4", "w1": p1, "w2": p2}, I)
    empty_c = np.full((T * k, I // 2), 0xFF, np.uint8)
    empty_s = np.full((T * k, I // 16), 0xFF, np.uint8)
    y, codes, scales = nshard.moe_rank(xp, idx, gate, p1, p2, I, 1, 0, empty_c, empty_s)
    assert np.array_equal(y, y_ref)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(codes[t * k + j], inter[(t, j)][0])
            assert np.array_equal(scales[t * k + j], inter[(t, j)][1])


@pytest.mark.parametrize("R,I", [(4, 32), (8, 16)])
def test_ranks_together_equal_the_full_width_expert(R, I):
    g = np.random.default_rng(202 + R)
    T, P, E, k = 4, 64, 5, 2
    xp = _bf16(g, (T, P), 1.0)
    idx, gate = _routing(g, T, E, k)
    # full-width experts, packed as whole matrices (one tensor scale each), then sliced by rows
    w1f = {e: _bf16(g, (2 * R * I, P), 0.1) for e in range(E)}
    w2f = {e: _bf16(g, (P, R * I), 0.1) for e in range(E)}
    p1f, p2f = _packed(w1f), _packed(w2f)
    y_full, inter_full = oracle.moe(xp, idx, gate, {"fmt": "nvfp4", "w1": p1f, "w2": p2f}, R * I)
    RI = R * I
    w1r = [{e: _slice_packed(p1f[e], np.r_[r * I:(r + 1) * I, RI + r * I:RI + (r + 1) * I]) for e in range(E)}
           for r in range(R)]
    w2r = [{e: _slice_packed(p2f[e], np.arange(r * P // R, (r + 1) * P // R)) for e in range(E)} for r in range(R)]
    # the slices each rank sends: its own intermediate slice of every pair
    xpd = oracle.bf16_to_f64(xp)
    sent = {}
    for r in range(R):
        for t in range(T):
            for j in range(k):
                e = int(idx[t, j])
                dec = oracle.nvfp4_decode(*w1r[r][e])
                sent[(r, t * k + j)] = nshard.intermediate_slice(xpd[t], dec, I)
    peer_c = np.zeros((T * k, RI // 2), np.uint8)
    peer_s = np.zeros((T * k, RI // 16), np.uint8)
    for p in range(T * k):
        c, s = nshard.gather_row([sent[(r, p)] for r in range(R)])
        peer_c[p], peer_s[p] = c, s
    cols = []
    for r in range(R):
        # rank r's own slice is left as garbage in what it receives: it must compute it itself
        pc = peer_c.copy()
        pc[:, r * I // 2:(r + 1) * I // 2] ^= 0x5A
        y_own, codes, scales = nshard.moe_rank(xp, idx, gate, w1r[r], w2r[r], I, R, r, pc, peer_s)
        assert np.array_equal(codes, peer_c) and np.array_equal(scales, peer_s)
        cols.append(y_own)
    assert np.array_equal(np.concatenate(cols, axis=1), y_full)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(peer_c[t * k + j], inter_full[(t, j)][0])
            assert np.array_equal(peer_s[t * k + j], inter_full[(t, j)][1])


def test_requantisation_of_a_row_is_the_concatenation_of_its_rank_slices():
    g = np.random.default_rng(303)
    a = g.standard_normal((3, 8 * 48)) * np.exp(g.standard_normal((3, 8 * 48)))
    c_full, s_full = fp4_act_quant(a)
    parts = [fp4_act_quant(a[:, r * 48:(r + 1) * 48]) for r in range(8)]
    assert np.array_equal(c_full, np.concatenate([c for c, _ in parts], axis=1))
    assert np.array_equal(s_full, np.concatenate([s for _, s in parts], axis=1))


def test_gathered_y_places_the_own_columns():
    y_peers = np.arange(4 * 32, dtype=np.uint16).reshape(4, 32)
    own = np.full((4, 4), 7, np.uint16)
    y = nshard.gathered_y(y_peers, own, 8, 5)
    assert np.array_equal(y[:, 20:24], own)
    assert np.array_equal(np.delete(y, np.s_[20:24], axis=1), np.delete(y_peers, np.s_[20:24], axis=1))
