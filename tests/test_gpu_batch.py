"""GPU tests of two sequences verified in one launch (mk_step_io.batch = 2): every output of
the batched launch equals, bit for bit, the outputs of the two sequences launched one at a
time (every row's sums run in the same order whichever rows share an MFMA tile), and each
sequence passes the same oracle checks as a single launch."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt

from gpu_util import log
from test_gpu_parity import SMALL_I128, _check_layer

# a two-sequence shape with two K pieces per GEMM1 unit (pooled 1152: nine k-steps, 5 + 4), so
# that GEMM1's input rows are staged one K half at a time
SMALL_P1152_I128 = synth.LayerShape("small-p1152-i128-nvfp4", 256, 4, 1, 64, 1152, 16, 4, 128, 128, 300, 16, True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _two_sequences(shape, cfg_id):
    """Two sequences of one layer: the second draws its own tree, queries, residual and KV
    rows (another seed) and takes the first's weights."""
    s0 = synth.make_layer_inputs(shape, cfg_id)
    s1 = synth.make_layer_inputs(shape, cfg_id + 1000, step=1)
    weights = ("w_o", "w_pool", "w_router", "w_unpool", "w_qkv_next", "w1", "w2")
    s1 = dataclasses.replace(s1, **{w: getattr(s0, w) for w in weights})
    return [s0, s1]


def _sequence(out, b, shape):
    """Sequence b's part of a batched launch's outputs."""
    T, cap = shape.T, shape.kv_capacity
    o = {k: v[b * T:(b + 1) * T] for k, v in out.items()
         if k in ("h_out", "q_next", "idx", "gate", "logits", "stats", "attn", "h1", "xp", "y")}
    o["k_cache_next"] = out["k_cache_next"][b * cap:(b + 1) * cap]
    o["v_cache_next"] = out["v_cache_next"][b * cap:(b + 1) * cap]
    o["status"] = out["status"]
    o["hist"] = np.bincount(o["idx"].reshape(-1), minlength=shape.n_experts)
    return o


def _batched_and_single(shape, cfg_id):
    seqs = _two_sequences(shape, cfg_id)
    dw = dt.upload_weights(seqs[0])
    st = dt.make_step_batch(seqs)
    dt.run_step(dw, st)
    out = dt.outputs(st)
    singles = []
    for s in seqs:
        st1 = dt.make_step(s)
        dt.run_step(dw, st1)
        singles.append(dt.outputs(st1))
    return seqs, out, singles


# (global-ctx32768: 2 x 229 attention items, more than the grid, so the batched launch runs its
# items in two rounds while each single launch runs one)
@pytest.mark.parametrize("shape,cfg_id", [(SMALL_I128, 121), (SMALL_P1152_I128, 122), (synth.CFG2, 2),
                                           (synth.CFG3, 3)])
def test_batch2_equals_two_single_launches(shape, cfg_id):
    log(f"batch 2 {shape.name}")
    seqs, out, singles = _batched_and_single(shape, cfg_id)
    assert out["status"] == mk.MK_OK, mk.mk_strerror(out["status"])
    for b in range(2):
        ob, o1 = _sequence(out, b, shape), singles[b]
        for key in ("h_out", "q_next", "idx", "gate", "logits", "stats", "attn", "h1", "xp", "y",
                    "k_cache_next", "v_cache_next"):
            same = np.array_equal(ob[key], o1[key])
            if not same:
                diff = np.count_nonzero(ob[key] != o1[key])
                log(f"  sequence {b} {key}: {diff} of {ob[key].size} elements differ")
            assert same, (b, key)
    # the expert-usage histogram counts both sequences' pairs
    assert np.array_equal(out["hist"], singles[0]["hist"] + singles[1]["hist"])
    log("  both sequences bit-equal to their single launches")


def test_batch2_against_the_oracle():
    seqs, out, _ = _batched_and_single(SMALL_I128, 123)
    for b in range(2):
        log(f"  sequence {b}")
        _check_layer(seqs[b], _sequence(out, b, SMALL_I128))
