"""The measurement's numerators, on the CPU: bench.py's algorithmic bytes and matrix-core work per
layer launch against the per-component figures of the hot-path table for the shard shape (dense
weights 53,477,376 B per layer; an NVFP4 expert slice 663,552 B, W1 442,368 + W2 221,184; the KV
rows a 16-token tree sees over a 2048 window at ctx 8192; dense / expert / attention work of
0.856 / 0.302 / 0.135 GFLOP at that shape), and against the definitions written out here."""
import numpy as np

import bench
import synth


def test_algorithmic_bytes_at_the_shard_shape():
    ab = bench.algorithmic_bytes(synth.CFG2, 102)
    assert ab["dense"] == 53_477_376
    assert ab["per_expert"] == 663_552 == 442_368 + 221_184
    assert ab["experts"] == 102 * 663_552
    # context rows ctx - (ctx - window + 1) = 2047, plus the 16 tree rows; K and V, bf16, d = 128
    assert ab["kv"] == (2047 + 16) * 1 * 128 * 2 * 2
    # h_in, h_out [16][4096] and q_in, q_next [16][1024], bf16
    assert ab["acts"] == 16 * (2 * 4096 + 2 * 1024) * 2
    assert ab["kv_write"] == 16 * 2 * 128 * 2
    assert ab["total"] == 122_551_808


def test_algorithmic_bytes_global_and_bf16_experts():
    ab = bench.algorithmic_bytes(synth.CFG3, 49)
    assert ab["kv"] == (32768 + 16) * 128 * 2 * 2          # every context row is visible
    assert ab["experts"] == 49 * 663_552
    t = bench.algorithmic_bytes(synth.CFG1, 2)             # bf16 experts: W1 [2I][P], W2 [P][I]
    I, P = synth.CFG1.expert_inter, synth.CFG1.pooled
    assert t["per_expert"] == 2 * (2 * I * P + P * I)


def test_algorithmic_flops_at_the_shard_shape():
    inp = synth.make_layer_inputs(synth.CFG2, 2)
    f = bench.algorithmic_flops(synth.CFG2, inp.parent)
    assert f["dense"] == 855_638_016
    assert f["experts"] == 301_989_888
    # attention: 2 (QK^T) x 2 (PV) x d x Hq x keys.  A node at position ctx + depth sees the
    # context rows within 2048 positions of it and its depth + 1 ancestors-or-self: 2048 keys
    # in all whatever its depth
    parent = np.asarray(inp.parent)
    depth = np.zeros(16, np.int64)
    for t in range(1, 16):
        depth[t] = depth[parent[t]] + 1
    keys = 0
    for t in range(16):
        pos = 8192 + int(depth[t])
        ctx_rows = 8192 - (pos - 2048 + 1)
        keys += ctx_rows + int(depth[t]) + 1
    assert keys == 16 * 2048
    assert f["attn"] == 4 * 128 * 8 * keys
    assert abs(f["attn"] / 1e9 - 0.135) < 0.001
