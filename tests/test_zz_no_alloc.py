"""The allocation-free entry point (mk_layer_step_noalloc): its static scratch against the
caller-workspace entry point (mk_layer_step), through the C ABI, on two calls in a row -- the
second on a smaller layer --, with two sequences per launch, and its rejection of a
configuration too large for the scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt

from gpu_util import log

# a small sliding-window layer with a ragged tree of 5 nodes (the second, smaller call)
SMALL_T5 = synth.LayerShape("small-t5-window-nvfp4", 256, 4, 1, 128, 256, 16, 2, 96, 40, 60, 5, True)
OUT_KEYS = ("h_out", "q_next", "k_cache_next", "v_cache_next", "idx", "gate", "logits", "stats", "hist")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _host_outputs(st) -> dict:
    torch.cuda.synchronize()
    return dict(h_out=dt.host_u16(st.h_out), q_next=dt.host_u16(st.q_next), k_cache_next=dt.host_u16(st.k_next),
                v_cache_next=dt.host_u16(st.v_next), idx=st.topk_idx.cpu().numpy(), gate=st.topk_gate.cpu().numpy(),
                logits=st.logits.cpu().numpy(), stats=st.stats.cpu().numpy(), hist=st.hist.cpu().numpy())


def test_noalloc_equals_layer_step_on_two_calls_in_a_row():
    for shape, cfg_id in ((synth.CFG2, 2), (SMALL_T5, 83)):
        log(f"[noalloc] {shape.name}")
        inp = synth.make_layer_inputs(shape, cfg_id)
        dw = dt.upload_weights(inp)
        ref_st = dt.make_step(inp)
        dt.run_step(dw, ref_st)
        ref = _host_outputs(ref_st)
        assert mk.mk_read_status(ref_st.workspace) == mk.MK_OK
        st = dt.make_step(inp)
        io = st.struct()
        io.workspace, io.workspace_bytes = None, 0
        assert mk.mk_layer_step_noalloc(st.cfg, dw.struct(), io) == mk.MK_OK
        got = _host_outputs(st)
        assert mk.mk_read_status(None) == mk.MK_OK
        for key in OUT_KEYS:
            assert np.array_equal(ref[key], got[key]), (shape.name, key)
        log(f"  outputs bit-identical to mk_layer_step ({len(np.unique(got['idx']))} experts routed)")


def test_noalloc_rejects_a_configuration_larger_than_its_scratch():
    inp = synth.make_layer_inputs(SMALL_T5, 83)
    st = dt.make_step(inp)
    dw = dt.upload_weights(inp)
    cfg = dt.layer_cfg(SMALL_T5)
    cfg.n_q_heads, cfg.n_kv_heads = 8, 8         # 8 kv heads of 128, global, over a long cache
    cfg.window, cfg.kv_capacity = 0, 1 << 20
    need = mk.mk_workspace_bytes(cfg, SMALL_T5.T)
    assert need > mk.MK_NOALLOC_SCRATCH_BYTES
    io = st.struct()
    io.workspace, io.workspace_bytes = None, 0
    assert mk.mk_layer_step_noalloc(cfg, dw.struct(), io, check=False) == mk.MK_ESCRATCH
    log(f"  a {need >> 20} MiB workspace is rejected: {mk.mk_strerror(mk.MK_ESCRATCH)}")


def test_noalloc_batch_two():
    """Two sequences per launch: bit-identical to mk_layer_step's batched launch at a small shape;
    at the shard shape the batched workspace exceeds the scratch and is rejected."""
    from test_gpu_batch import _two_sequences
    from test_gpu_parity import SMALL_I128
    seqs = _two_sequences(SMALL_I128, 124)
    dw = dt.upload_weights(seqs[0])
    ref_st = dt.make_step_batch(seqs)
    dt.run_step(dw, ref_st)
    ref = dt.outputs(ref_st)
    assert ref["status"] == mk.MK_OK
    st = dt.make_step_batch(seqs)
    io = st.struct()
    io.workspace, io.workspace_bytes = None, 0
    assert mk.mk_layer_step_noalloc(st.cfg, dw.struct(), io) == mk.MK_OK
    got = dt.outputs(st)
    assert mk.mk_read_status(None) == mk.MK_OK
    for key in ("h_out", "q_next", "k_cache_next", "v_cache_next", "idx", "gate", "logits", "stats"):
        assert np.array_equal(ref[key], got[key]), key
    log("  two sequences: outputs bit-identical to mk_layer_step")
    big = _two_sequences(synth.CFG2, 125)
    dwb = dt.upload_weights(big[0])
    stb = dt.make_step_batch(big)
    iob = stb.struct()
    iob.workspace, iob.workspace_bytes = None, 0
    assert mk.mk_layer_step_noalloc(stb.cfg, dwb.struct(), iob, check=False) == mk.MK_ESCRATCH
    log("  two sequences at the shard shape: rejected with MK_ESCRATCH")
