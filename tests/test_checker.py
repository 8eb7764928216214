"""The GPU parity checker itself, on the CPU: it must accept what a correct fp32-accumulating
kernel produces and reject a stage whose contribution is off by 10%, at the shard shape
(16 tokens, hidden 4096) where the residual stream dominates the stage outputs.

"Kernel" outputs here are made on the CPU: fp32 matrix products of the same bf16 inputs
(numpy's float32 GEMM, another summation order than the oracle's), the residual added in
fp32, and one fp32 -> bf16 rounding.  The perturbations are planted on this side, never in
a kernel."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import MISMATCH_CEILING, REL_TOL, assert_rounding_exact, max_abs_rel

T, H, HQD, P, QKV = 16, 4096, 1024, 2048, 1280


def _fp32_stage(x_bits, w_bits, residual_bits=None, scale=1.0):
    """bf16(fp32(scale * x . W^T) + residual) with fp32 accumulation."""
    x = oracle.bf16_to_f64(x_bits).astype(np.float32)
    w = oracle.bf16_to_f64(w_bits).astype(np.float32)
    acc = (x @ w.T) * np.float32(scale)
    if residual_bits is not None:
        acc = acc + oracle.bf16_to_f64(residual_bits).astype(np.float32)
    return synth.bf16_bits_from_f32(acc.astype(np.float32))


@pytest.fixture(scope="module")
def shard():
    g = np.random.default_rng(515)
    parent = synth.tree_parents(T, g)
    ctx = 8192
    q = synth.normal_bf16(g, (T, HQD), 1.0)
    K = synth.normal_bf16(g, (ctx + T, 1, 128), 1.0)
    V = synth.normal_bf16(g, (ctx + T, 1, 128), 1.0)
    # attention output of the sliding-window shard layer: its real magnitude
    attn, _ = oracle.attention(q, K, V, parent, ctx, 2048, 8, 1, 128)
    return dict(attn=attn, h_in=synth.normal_bf16(g, (T, H), 1.0), w_o=synth.normal_bf16(g, (H, HQD), 0.02),
                # combined expert output: about 0.1 per element at this shape
                y=synth.normal_bf16(g, (T, P), 0.1), w_u=synth.normal_bf16(g, (H, P), 0.02),
                w_qkv=synth.normal_bf16(g, (QKV, H), 0.02))


def test_checker_accepts_fp32_accumulation_of_every_anchored_stage(shard):
    s = shard
    h1 = _fp32_stage(s["attn"], s["w_o"], s["h_in"])
    assert_rounding_exact("o-proj", h1, s["attn"], s["w_o"], s["h_in"])
    h_out = _fp32_stage(s["y"], s["w_u"], h1)
    assert_rounding_exact("unpooler", h_out, s["y"], s["w_u"], h1)
    qkv = _fp32_stage(h_out, s["w_qkv"])
    assert_rounding_exact("qkv", qkv, h_out, s["w_qkv"])
    # the oracle's own rounding passes trivially
    assert assert_rounding_exact("o-proj (oracle)", oracle.dense(s["attn"], s["w_o"], s["h_in"]),
                                 s["attn"], s["w_o"], s["h_in"])[0] == 0


@pytest.mark.parametrize("scale", [0.9, 1.1])
def test_checker_rejects_an_oproj_off_by_ten_percent(shard, scale):
    s = shard
    bad = _fp32_stage(s["attn"], s["w_o"], s["h_in"], scale)
    # the residual-normalised tolerance cannot see it ...
    assert max_abs_rel(bad, oracle.dense(s["attn"], s["w_o"], s["h_in"])) <= REL_TOL
    # ... the rounding-aware check does
    with pytest.raises(AssertionError):
        assert_rounding_exact("o-proj x%.1f" % scale, bad, s["attn"], s["w_o"], s["h_in"])


@pytest.mark.parametrize("scale", [0.9, 1.1])
def test_checker_rejects_an_unpooler_off_by_ten_percent(shard, scale):
    s = shard
    h1 = oracle.dense(s["attn"], s["w_o"], s["h_in"])
    bad = _fp32_stage(s["y"], s["w_u"], h1, scale)
    assert max_abs_rel(bad, oracle.dense(s["y"], s["w_u"], h1)) <= REL_TOL
    with pytest.raises(AssertionError):
        assert_rounding_exact("unpooler x%.1f" % scale, bad, s["y"], s["w_u"], h1)


def test_checker_rejects_a_dropped_head_and_small_kv_errors(shard):
    s = shard
    attn = s["attn"].copy()
    attn[:, 3 * 128:4 * 128] = 0            # one head's output lost in the o-proj input
    bad = _fp32_stage(attn, s["w_o"], s["h_in"])
    with pytest.raises(AssertionError):
        assert_rounding_exact("o-proj without head 3", bad, s["attn"], s["w_o"], s["h_in"])
    # the KV write (k rows of the qkv projection): 1% too large is already caught
    h = oracle.dense(s["y"], s["w_u"], s["h_in"])
    wk = s["w_qkv"][HQD:HQD + 128]
    with pytest.raises(AssertionError):
        assert_rounding_exact("k x1.01", _fp32_stage(h, wk, None, 1.01), h, wk)


def test_checker_rejects_scattered_one_ulp_flips(shard):
    """One-ulp changes at random places beyond the mismatch ceiling fail, even though every
    flipped element stays within one rounding step of the exact value."""
    s = shard
    good = oracle.dense(s["attn"], s["w_o"], s["h_in"])
    g = np.random.default_rng(3)
    n = int(2 * MISMATCH_CEILING * good.size)
    pos = g.choice(good.size, n, replace=False)
    bad = good.copy().reshape(-1)
    bad[pos] = bad[pos] ^ np.uint16(1)
    with pytest.raises(AssertionError):
        assert_rounding_exact("o-proj with flips", bad.reshape(good.shape), s["attn"], s["w_o"], s["h_in"])
