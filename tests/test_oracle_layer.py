"""Pins of the oracle's layer step against invariants, library routines, brute force
and the independent scalar-loop oracle (CPU only)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import scalar

TINY_NVFP4 = synth.LayerShape("tiny-tree-swa-nvfp4", 64, 2, 1, 32, 64, 8, 2, 32, 8, 24, 16, True)
TINY_GQA2 = synth.LayerShape("tiny-tree-gqa2-bf16", 64, 4, 2, 16, 32, 8, 3, 16, 0, 20, 16, False)


def _walk_closure(parent):
    T = len(parent)
    anc, depth = [], []
    for i in range(T):
        s, j, dd = 0, i, -1
        while j >= 0:
            s |= 1 << j
            j = parent[j]
            dd += 1
        anc.append(s)
        depth.append(dd)
    return anc, depth


@pytest.mark.parametrize("seed", range(5))
def test_tree_masks_are_transitive_closure(seed):
    parent = synth.tree_parents(16, np.random.default_rng(seed))
    anc, depth = oracle.tree_masks(parent)
    a2, d2 = _walk_closure(list(parent))
    assert [int(x) for x in anc] == a2 and list(depth) == d2
    assert max(depth) == 6 and all(parent[i] < i for i in range(1, 16))


def test_tree_masks_reject_malformed():
    with pytest.raises(ValueError):
        oracle.tree_masks([0, 0])
    with pytest.raises(ValueError):
        oracle.tree_masks([-1, 1])
    with pytest.raises(ValueError):
        oracle.tree_masks([-1, 0, 3, 1])


def _sdpa_causal_path(q_row, keys, vals, d):
    """Plain causal attention of the last query of a sequence (torch, fp64)."""
    q = torch.from_numpy(q_row)[None, None, None, :]
    k = torch.from_numpy(keys)[None, None]
    v = torch.from_numpy(vals)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1.0 / np.sqrt(d))[0, 0, 0].numpy()


@pytest.mark.parametrize("window", [0, 40])
def test_tree_attention_equals_per_branch_causal_attention(window):
    g = np.random.default_rng(11)
    T, ctx, Hq, Hkv, d = 16, 50, 4, 2, 16
    parent = synth.tree_parents(T, g)
    q = synth.normal_bf16(g, (T, Hq * d), 1.0)
    K = synth.normal_bf16(g, (ctx + T, Hkv, d), 1.0)
    V = synth.normal_bf16(g, (ctx + T, Hkv, d), 1.0)
    attn, stats = oracle.attention(q, K, V, parent, ctx, window, Hq, Hkv, d)
    _, depth = oracle.tree_masks(parent)
    qf, Kf, Vf = (oracle.bf16_to_f64(x) for x in (q, K, V))
    for i in range(T):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parent[j]
        path = path[::-1]                        # root .. i, positions ctx .. ctx+depth_i
        pos_i = ctx + depth[i]
        ctx_rows = [p for p in range(ctx) if window == 0 or pos_i - p < window]
        rows = ctx_rows + [ctx + n for n in path]
        for h in range(Hq):
            gh = h * Hkv // Hq
            ref = _sdpa_causal_path(qf[i, h * 16:(h + 1) * 16], Kf[rows, gh], Vf[rows, gh], d)
            got = oracle.bf16_to_f64(attn[i, h * 16:(h + 1) * 16])
            assert np.array_equal(got, oracle.bf16_to_f64(oracle.bf16_round(ref))) or \
                np.abs(got - ref).max() <= 2 ** -8 * np.abs(ref).max()


def test_swa_equals_global_when_window_covers_everything():
    g = np.random.default_rng(12)
    T, ctx, d = 16, 2041, 32
    parent = synth.tree_parents(T, g)
    q = synth.normal_bf16(g, (T, 2 * d), 1.0)
    K = synth.normal_bf16(g, (ctx + T, 1, d), 1.0)
    V = synth.normal_bf16(g, (ctx + T, 1, d), 1.0)
    a0, s0 = oracle.attention(q, K, V, parent, ctx, 0, 2, 1, d)
    a1, s1 = oracle.attention(q, K, V, parent, ctx, 2048, 2, 1, d)
    assert np.array_equal(a0, a1) and np.array_equal(s0, s1)
    # one more context row and the deepest node loses exactly the oldest row
    vis = oracle.visible_keys(parent, ctx + 1, 2048)
    _, depth = oracle.tree_masks(parent)
    for i in range(T):
        pos = ctx + 1 + depth[i]
        assert vis[i, 0] == (pos - 0 < 2048)


def test_swa_edge_positions():
    parent = np.array([-1, 0], np.int32)
    ctx, W = 3000, 2048
    vis = oracle.visible_keys(parent, ctx, W)
    # node 0 at position 3000 sees p with 3000 - p < 2048, i.e. p >= 953
    assert not vis[0, 952] and vis[0, 953]
    # node 1 at depth 1 (position 3001) sees p >= 954, plus both tree slots
    assert not vis[1, 953] and vis[1, 954] and vis[1, ctx] and vis[1, ctx + 1]
    assert not vis[0, ctx + 1]


def test_gqa_equals_mha_with_repeated_kv():
    g = np.random.default_rng(13)
    T, ctx, Hq, Hkv, d = 16, 30, 8, 2, 16
    parent = synth.tree_parents(T, g)
    q = synth.normal_bf16(g, (T, Hq * d), 1.0)
    K = synth.normal_bf16(g, (ctx + T, Hkv, d), 1.0)
    V = synth.normal_bf16(g, (ctx + T, Hkv, d), 1.0)
    a, s = oracle.attention(q, K, V, parent, ctx, 0, Hq, Hkv, d)
    Kr = np.repeat(K, Hq // Hkv, axis=1)
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    a2, s2 = oracle.attention(q, Kr, Vr, parent, ctx, 0, Hq, Hq, d)
    assert np.array_equal(a, a2) and np.array_equal(s, s2)


def test_single_root_is_plain_decode_and_rows_normalise():
    g = np.random.default_rng(14)
    ctx, d = 64, 32
    q = synth.normal_bf16(g, (1, d), 1.0)
    K = synth.normal_bf16(g, (ctx + 1, 1, d), 1.0)
    V = synth.normal_bf16(g, (ctx + 1, 1, d), 1.0)
    a, s = oracle.attention(q, K, V, np.array([-1]), ctx, 0, 1, 1, d)
    qf, Kf, Vf = (oracle.bf16_to_f64(x) for x in (q, K, V))
    ref = _sdpa_causal_path(qf[0], Kf[:, 0], Vf[:, 0], d)
    assert np.abs(oracle.bf16_to_f64(a[0]) - ref).max() <= 2 ** -8 * np.abs(ref).max()
    sc = (Kf[:, 0] @ qf[0]) / np.sqrt(d)
    assert s[0, 0, 0] == sc.max() and np.isclose(s[0, 0, 1], np.exp(sc - sc.max()).sum(), rtol=1e-14)
    ones = np.full_like(V, 0x3F80)                 # all-ones values: normalised weights give exactly 1
    a1, _ = oracle.attention(q, K, ones, np.array([-1]), ctx, 0, 1, 1, d)
    assert np.all(a1 == 0x3F80)


def test_router_topk_equals_stable_full_sort_and_gates():
    g = np.random.default_rng(15)
    xp = synth.normal_bf16(g, (16, 64), 1.0)
    wr = synth.normal_bf16(g, (32, 64), 0.02)
    wr[5] = wr[9]            # exact ties between experts 5 and 9
    bias = np.zeros((16, 32), np.float32)
    bias[3, 30] = 8.0
    logits64, z, idx, gate = oracle.router(xp, wr, bias, 8)
    for t in range(16):
        order = np.lexsort((np.arange(32), -z[t].astype(np.float64)))[:8]
        assert list(idx[t]) == list(order)
    assert np.allclose(gate.sum(1), 1.0, rtol=0, atol=1e-15)
    assert idx[3, 0] == 30
    # k = E: gates are the full softmax
    _, z2, idx2, gate2 = oracle.router(xp, wr, None, 32)
    full = torch.softmax(torch.from_numpy(z2.astype(np.float64)), dim=1).numpy()
    assert np.allclose(np.take_along_axis(full, idx2.astype(np.int64), 1), gate2, rtol=1e-14, atol=0)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 2001)
    assert np.allclose(oracle.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("shape,cfg_id", [(synth.CFG1, 1), (TINY_NVFP4, 91), (TINY_GQA2, 92)])
def test_moe_equals_dense_evaluation_of_all_experts(shape, cfg_id):
    inp = synth.make_layer_inputs(shape, cfg_id)
    ex = oracle.pack_experts(inp)
    ref = oracle.layer_step(inp, ex)
    xp, idx, gate = ref["xp"], ref["idx"], ref["gate"]
    T, E, I = shape.T, shape.n_experts, shape.expert_inter
    full_gate = np.zeros((T, E))
    for t in range(T):
        full_gate[t, idx[t]] = gate[t]
    comb = np.zeros((T, shape.pooled))
    xpf = oracle.bf16_to_f64(xp)
    for e in range(E):
        if shape.nvfp4:
            w1 = oracle.nvfp4_decode(*ex["w1"][e])
            w2 = oracle.nvfp4_decode(*ex["w2"][e])
        else:
            w1, w2 = oracle.bf16_to_f64(ex["w1"][e]), oracle.bf16_to_f64(ex["w2"][e])
        u = xpf @ w1.T
        a = u[:, :I] / (1 + np.exp(-u[:, :I])) * u[:, I:]
        if shape.nvfp4:
            aq = oracle.nvfp4_decode(*oracle.fp4_act_quant(a), 1.0)
        else:
            aq = oracle.bf16_to_f64(oracle.bf16_round(a))
        comb += full_gate[:, e:e + 1] * (aq @ w2.T)
    assert np.array_equal(oracle.bf16_round(comb), ref["y"])


@pytest.mark.parametrize("shape,cfg_id", [(synth.CFG1, 1), (TINY_NVFP4, 91), (TINY_GQA2, 92)])
def test_scalar_oracle_equals_vectorised_oracle(shape, cfg_id):
    inp = synth.make_layer_inputs(shape, cfg_id)
    ex = oracle.pack_experts(inp)
    a = oracle.layer_step(inp, ex)
    b = scalar.layer_step(inp, ex)
    for key in ("attn", "h1", "xp", "y", "h_out", "q_next"):
        assert np.array_equal(oracle.bf16_to_f64(a[key]), np.array(b[key])), key
    assert np.array_equal(oracle.bf16_to_f64(a["k_new"]).reshape(shape.T, -1), np.array(b["k_new"]))
    assert np.array_equal(oracle.bf16_to_f64(a["v_new"]).reshape(shape.T, -1), np.array(b["v_new"]))
    assert [list(r) for r in a["idx"]] == b["idx"]
    assert np.allclose(a["gate"], np.array(b["gate"]), rtol=1e-12, atol=0)
    st = np.array(b["stats"])
    assert np.allclose(a["stats"], st, rtol=1e-12, atol=0)


@pytest.mark.parametrize("shape,cfg_id", [(synth.CFG1, 1), (TINY_NVFP4, 91), (TINY_GQA2, 92)])
def test_layer_step_auto_equals_layer_step_with_every_expert_packed(shape, cfg_id):
    """layer_step_auto packs only the experts its own routing reaches; every output equals the
    step run with all E experts packed (routing does not depend on the experts)."""
    inp = synth.make_layer_inputs(shape, cfg_id)
    a = oracle.layer_step_auto(inp)
    b = oracle.layer_step(inp, oracle.pack_experts(inp))
    for key in ("attn", "stats", "h1", "xp", "logits64", "logits32", "idx", "gate", "y", "h_out", "q_next",
                "k_new", "v_new", "k_cache_next", "v_cache_next", "hist", "top14", "qkv64"):
        assert np.array_equal(a[key], b[key]), key
    assert a["inter_q"].keys() == b["inter_q"].keys()
    for k_ in a["inter_q"]:
        assert all(np.array_equal(x, y) for x, y in zip(a["inter_q"][k_], b["inter_q"][k_]))


def test_usage_top_is_count_desc_index_asc():
    idx = np.array([[3, 1], [1, 7], [7, 3], [2, 5]])
    hist, top = oracle.usage_top(idx, 10, 4)
    assert list(hist) == [0, 2, 1, 2, 0, 1, 0, 2, 0, 0]
    assert list(top) == [1, 3, 7, 2]
    _, top2 = oracle.usage_top(np.array([[0, 1]]), 10, 14)
    assert list(top2) == [0, 1]


def test_layer_kv_write_touches_only_tree_slots():
    inp = synth.make_layer_inputs(TINY_NVFP4, 91)
    out = oracle.layer_step(inp, oracle.pack_experts(inp))
    ctx, T = TINY_NVFP4.ctx, TINY_NVFP4.T
    kn = out["k_cache_next"]
    assert np.array_equal(kn[:ctx], inp.k_cache_next[:ctx]) and np.array_equal(kn[ctx + T:], inp.k_cache_next[ctx + T:])
    assert np.array_equal(kn[ctx:ctx + T], out["k_new"])


def test_zipf_routing_reaches_about_49_experts():
    # the pages' profiling reuses a measured 49 distinct experts per layer as synthetic routing
    counts = []
    for step in range(20):
        bias = synth.zipf_router_bias(synth.CFG3, synth.rng(synth.base_seed(3), 0, synth.T_BIAS, 0, step), synth.CFG3.zipf_s)
        counts.append(int((bias.max(0) > 0).sum()))
    assert 40 <= np.mean(counts) <= 58, counts


def test_qkv_project_matches_exact_per_element_dot_products():
    """qkv_project against every output written out one by one: an exactly rounded fp64 sum
    (math.fsum) of the bf16 products, rounded to bf16 by the scalar oracle's routine, and the
    query / key / value split checked by its row ranges."""
    import math
    from oracle import scalar
    g = np.random.default_rng(41)
    T, H, Hq, Hkv, d = 3, 64, 2, 1, 16
    h = synth.normal_bf16(g, (T, H), 1.0)
    w = synth.normal_bf16(g, ((Hq + 2 * Hkv) * d, H), 0.02)
    q, k, v, _ = oracle.qkv_project(h, w, Hq, Hkv, d)
    hf = [[scalar.bits_to_float(int(x)) for x in row] for row in h]
    wf = [[scalar.bits_to_float(int(x)) for x in row] for row in w]
    for t in range(T):
        for n in range((Hq + 2 * Hkv) * d):
            ref = scalar.bf16_of(math.fsum(hf[t][i] * wf[n][i] for i in range(H)))
            if n < Hq * d:
                got = q[t, n]
            elif n < (Hq + Hkv) * d:
                got = k[t].reshape(-1)[n - Hq * d]
            else:
                got = v[t].reshape(-1)[n - (Hq + Hkv) * d]
            assert scalar.bits_to_float(int(got)) == ref, (t, n)


def _accept_case(g, T, match_p):
    """A random tree whose siblings carry distinct drafted tokens, and target tokens that
    match one child with probability match_p."""
    parent = synth.tree_parents(T, g)
    draft = np.zeros(T, np.int64)
    target = g.integers(1000, 2000, T)
    for i in range(T):
        kids = [c for c in range(1, T) if parent[c] == i]
        toks = g.choice(np.arange(100, 200), size=len(kids), replace=False)
        draft[kids] = toks
        if kids and g.random() < match_p:
            target[i] = toks[g.integers(len(kids))]
    return parent, draft, target


def test_tree_accept_is_the_deepest_consistent_node():
    """Brute force: with distinct sibling tokens, the nodes whose every edge from the root
    matches (child's draft == target at its parent) form one chain; the accepted path is that
    chain, and the bonus is the target's token at its end."""
    g = np.random.default_rng(7)
    for trial in range(300):
        T = int(g.integers(1, 17))
        parent, draft, target = _accept_case(g, T, float(g.random()))
        def consistent(n):
            while n != 0:
                if draft[n] != target[parent[n]]:
                    return False
                n = parent[n]
            return True
        chain = [n for n in range(T) if consistent(n)]
        path, bonus = oracle.tree_accept(parent, draft, target)
        assert path == sorted(chain), (trial, path, chain)
        assert all(parent[b] == a for a, b in zip(path, path[1:]))
        assert bonus == target[path[-1]]


def test_tree_accept_special_cases():
    # a chain whose every draft matches: all of it, then the target after the leaf
    T = 7
    parent = np.arange(-1, T - 1)
    target = np.arange(10, 10 + T)
    draft = np.concatenate([[0], target[:-1]])
    path, bonus = oracle.tree_accept(parent, draft, target)
    assert path == list(range(T)) and bonus == target[-1]
    # nothing matches: the root alone, and its target token
    path, bonus = oracle.tree_accept(parent, draft + 1, target)
    assert path == [0] and bonus == target[0]
    # two siblings with the same token: the lower index is taken
    parent = np.array([-1, 0, 0])
    path, _ = oracle.tree_accept(parent, np.array([0, 5, 5]), np.array([5, 1, 2]))
    assert path == [0, 1]


def test_kv_commit_is_a_row_gather():
    g = np.random.default_rng(8)
    cap, ctx = 40, 20
    k = synth.normal_bf16(g, (cap, 2, 8), 1.0)
    v = synth.normal_bf16(g, (cap, 2, 8), 1.0)
    path = [0, 2, 5, 9]
    kc, vc = oracle.kv_commit(k, v, ctx, path)
    for j, node in enumerate(path):
        assert np.array_equal(kc[ctx + j], k[ctx + node]) and np.array_equal(vc[ctx + j], v[ctx + node])
    rest = np.ones(cap, bool)
    rest[ctx:ctx + len(path)] = False
    assert np.array_equal(kc[rest], k[rest]) and np.array_equal(vc[rest], v[rest])
