"""GPU parity of one rank's share of the N-sharded expert layout (mk_layer_step_nshard) against
the oracle (oracle/nshard.py), with the other ranks' parts delivered by the host into the two
receive buffers: seeded NVFP4 intermediate slices and y columns, as synth.nshard_inputs draws
them.  Also: the shared phases agree bit for bit with the ordinary launch, a withheld slot ends
in MK_ETIMEOUT instead of a hang, and the workspace runs normally afterwards."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import nshard
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt

from gpu_util import assert_close_bf16, assert_rounding_exact, log

R = 8
SMALL_NS = synth.LayerShape("small-ns-nvfp4", 256, 4, 1, 64, 256, 16, 4, 64, 128, 300, 16, True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Rank:
    """Rank r's device state: the layer's weights with its W2 rows packed in place of the
    ordinary W2, a step, and the two receive buffers as the other ranks leave them."""

    def __init__(self, shape, cfg_id, r, withhold_act=None, withhold_y=None):
        self.shape, self.r = shape, r
        self.inp = synth.make_layer_inputs(shape, cfg_id)
        self.ns = synth.nshard_inputs(shape, cfg_id, R, r)
        sh = shape
        E, P, I, T, k = sh.n_experts, sh.pooled, sh.expert_inter, sh.T, sh.top_k
        self.K2, self.N2 = R * I, P // R
        self.dw = dt.upload_weights(self.inp)
        u8 = dict(dtype=torch.uint8, device="cuda")
        self.dw.w2_codes = torch.empty((E, self.N2, self.K2 // 2), **u8)
        self.dw.w2_scales = torch.empty((E, self.N2, self.K2 // 16), **u8)
        self.dw.w2_ts = torch.empty(E, dtype=torch.float32, device="cuda")
        mk.mk_nvfp4_pack(dt.dev_u16(self.ns["w2_shard"]), 0, E, self.N2, self.K2, self.dw.w2_codes,
                         self.dw.w2_scales, self.dw.w2_ts)
        self.st = dt.make_step(self.inp)
        rec = dt.nvfp4_records(self.ns["peer_codes"], self.ns["peer_scales"])
        rec[:, r * I // 16:(r + 1) * I // 16, :] = 0xFFFFFFFF           # this rank's slice: not yet
        if withhold_act is not None:                                    # (pair, rank) never delivered
            p, q = withhold_act
            rec[p, q * I // 16:(q + 1) * I // 16, :] = 0xFFFFFFFF
        self.act_recv = torch.from_numpy(rec.view(np.int32)).cuda()
        yr = self.ns["peer_y"].copy()
        yr[:, r * self.N2:(r + 1) * self.N2] = 0xFFFF
        if withhold_y is not None:
            yr[:, withhold_y * self.N2:(withhold_y + 1) * self.N2] = 0xFFFF
        self.y_recv = torch.from_numpy(dt.tile_frag(yr, P).view(np.int16)).cuda()
        self.arg = mk.mk_nshard(r, R, self.act_recv.data_ptr(), self.y_recv.data_ptr())

    def run(self, spin_limit=0):
        mk.mk_layer_step_nshard(self.st.cfg, self.dw.struct(), self.st.struct(spin_limit=spin_limit), self.arg)
        torch.cuda.synchronize()

    def results(self):
        out = dt.outputs(self.st)
        rec = self.act_recv.cpu().numpy().view(np.uint32).reshape(self.shape.T * self.shape.top_k, self.K2 // 16, 4)
        codes, scales = dt.nvfp4_from_records(rec)
        y_full = dt.untile_frag(self.y_recv.cpu().numpy().view(np.uint16), self.shape.T, self.shape.pooled)
        return out, codes, scales, y_full


def _check(rk: Rank, out, codes, scales, y_full):
    sh, r, inp = rk.shape, rk.r, rk.inp
    I, T, k, P = sh.expert_inter, sh.T, sh.top_k, sh.pooled
    N2 = rk.N2
    assert out["status"] == mk.MK_OK, mk.mk_strerror(out["status"])
    # the other ranks' deliveries are read, never written
    own_c = np.s_[:, r * I // 2:(r + 1) * I // 2]
    own_s = np.s_[:, r * I // 16:(r + 1) * I // 16]
    mask_c = np.ones(codes.shape, bool)
    mask_c[own_c] = False
    mask_s = np.ones(scales.shape, bool)
    mask_s[own_s] = False
    assert np.array_equal(codes[mask_c], rk.ns["peer_codes"][mask_c])
    assert np.array_equal(scales[mask_s], rk.ns["peer_scales"][mask_s])
    other = np.ones(P, bool)
    other[r * N2:(r + 1) * N2] = False
    assert np.array_equal(y_full[:, other], rk.ns["peer_y"][:, other])
    # this rank's intermediate slice: the oracle's, on the GPU's pooled rows and routing (a
    # block whose value sits on a quantisation midpoint within fp32's error may differ)
    xp, idx, gate = out["xp"], out["idx"], out["gate"]
    used = sorted(set(idx.reshape(-1).tolist()))
    w1 = {e: oracle.nvfp4_pack(oracle.bf16_to_f64(inp.w1[e])) for e in used}
    xpd = oracle.bf16_to_f64(xp)
    ref_c = np.zeros((T * k, I // 2), np.uint8)
    ref_s = np.zeros((T * k, I // 16), np.uint8)
    for t in range(T):
        for j in range(k):
            ref_c[t * k + j], ref_s[t * k + j] = nshard.intermediate_slice(
                xpd[t], oracle.nvfp4_decode(*w1[int(idx[t, j])]), I)
    dc = np.count_nonzero(codes[own_c] != ref_c)
    ds = np.count_nonzero(scales[own_s] != ref_s)
    log(f"  own intermediate slice: {dc}/{ref_c.size} code bytes, {ds}/{ref_s.size} scales differ from the oracle")
    assert dc <= max(2, ref_c.size // 200) and ds <= max(1, ref_s.size // 200)
    # this rank's y columns: GEMM2 over the gathered rows the GPU read, combine, one rounding
    w2 = {e: oracle.nvfp4_decode(*oracle.nvfp4_pack(oracle.bf16_to_f64(rk.ns["w2_shard"][e]))) for e in used}
    y_ref = nshard.gemm2_rank(idx, gate, codes, scales, w2)
    y_own = y_full[:, r * N2:(r + 1) * N2]
    assert not np.any(y_own == 0xFFFF), "own y columns not written"
    assert_close_bf16("y (own columns)", y_own, y_ref)
    assert float(np.mean(y_own == y_ref)) >= 0.9
    # the unpooler over the gathered y, and the next layer's projection
    assert_rounding_exact("unpooler (gathered y)", out["h_out"], y_full, inp.w_unpool, out["h1"])
    qd = sh.n_q_heads * sh.head_dim
    assert_rounding_exact("q_next", out["q_next"], out["h_out"], inp.w_qkv_next[:qd])


@pytest.mark.parametrize("shape,cfg_id,r", [(SMALL_NS, 95, 3), (SMALL_NS, 96, 0), (SMALL_NS, 97, 7)])
def test_nshard_small_against_the_oracle(shape, cfg_id, r):
    log(f"nshard {shape.name} rank {r} of {R}")
    rk = Rank(shape, cfg_id, r)
    rk.run()
    _check(rk, *rk.results())


def test_nshard_shard_shape_against_the_oracle():
    """The layer's one-GPU shape (hidden 4096, pooled 2048, 256 experts top-8, local
    intermediate 192 of 1536): GEMM2 over K = 1536 for 256 of the 2048 output columns."""
    log(f"nshard {synth.CFG2.name} rank 3 of {R}")
    rk = Rank(synth.CFG2, 2, 3)
    rk.run()
    _check(rk, *rk.results())


def test_nshard_shared_phases_match_the_ordinary_launch():
    """Attention through routing run the same code in both layouts: pooled rows, logits and
    routing of an N-sharded launch equal the ordinary launch's bit for bit."""
    rk = Rank(SMALL_NS, 98, 2)
    rk.run()
    out_ns = dt.outputs(rk.st)
    dw = dt.upload_weights(rk.inp)
    st = dt.make_step(rk.inp)
    dt.run_step(dw, st)
    out = dt.outputs(st)
    for key in ("attn", "h1", "xp", "idx", "gate", "logits"):
        assert np.array_equal(out_ns[key], out[key]), key


@pytest.mark.parametrize("withhold", ["act", "y"])
def test_nshard_withheld_slot_times_out_and_the_workspace_recovers(withhold):
    """A slot another rank never delivers ends the launch with MK_ETIMEOUT (bounded polls, no
    hang); the same workspace then runs a complete launch normally."""
    kw = dict(withhold_act=(5, 6)) if withhold == "act" else dict(withhold_y=4)
    rk = Rank(SMALL_NS, 99, 1, **kw)
    rk.run(spin_limit=2000)
    assert mk.mk_read_status(rk.st.workspace) == mk.MK_ETIMEOUT
    good = Rank(SMALL_NS, 99, 1)
    good.st = rk.st                                     # the same workspace, not re-initialised
    good.st.hist.zero_()
    good.run()
    _check(good, *good.results())
