"""GPU tests of the stack mechanics: the last-layer launch mode, a stack of fused layers
(global every fourth layer, the last one without a next-layer projection) checked layer by
layer against the oracle and, run in one go by the stack runner, bit for bit against the
layer-by-layer chain, and the stack's verify step replayed as one HIP graph."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
import layer_persistent_amd as mk
from layer_persistent_amd import tensors as dt
from layer_persistent_amd.stack import Stack, is_global

from gpu_util import assert_close_bf16, log
from test_gpu_parity import SMALL_NVFP4, _check_layer

pytestmark = pytest.mark.gpu

SMALL_STACK = synth.LayerShape("small-stack-nvfp4", 256, 4, 1, 64, 256, 16, 4, 64, 128, 300, 16, True)
N_LAYERS = 6
CFG_ID = 90


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_last_layer_mode_ends_after_the_unpooler():
    inp = synth.make_layer_inputs(SMALL_NVFP4, 87)
    dw = dt.upload_weights(inp)
    st = dt.make_step(inp)
    dt.run_step(dw, st)
    full = dt.outputs(st)
    dw_last = dataclasses.replace(dw, w_qkv=None)
    st2 = dt.make_step(inp)
    dt.run_step(dw_last, st2)
    last = dt.outputs(st2)
    assert last["status"] == 0
    for key in ("h_out", "idx", "gate", "logits", "stats", "y", "xp", "h1", "attn"):
        assert np.array_equal(full[key], last[key]), key
    assert np.all(last["q_next"] == 0)                       # never written
    assert np.array_equal(last["k_cache_next"], inp.k_cache_next)
    assert np.array_equal(last["v_cache_next"], inp.v_cache_next)


def _host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _layer_inputs(L, step_in, prev) -> synth.LayerInputs:
    """Host inputs of stack layer L, drawn by the same device generators the stack uses; the
    tree rows, residual and queries come from the step inputs (L = 0) or from layer L-1."""
    sh = dataclasses.replace(SMALL_STACK, window=0 if is_global(L) else SMALL_STACK.window)
    w = synth.device_layer_weights(sh, CFG_ID, L, "cuda")
    kc, vc = synth.device_kv_context(sh, CFG_ID, L, "cuda")
    k_cache, v_cache = _host(kc), _host(vc)
    T, ctx = sh.T, sh.ctx
    if prev is None:
        h_in, q_in = step_in["h_in"], step_in["q_in"]
        k_cache[ctx:ctx + T], v_cache[ctx:ctx + T] = step_in["k_tree"], step_in["v_tree"]
    else:
        h_in, q_in = prev["h_out"], prev["q_next"]
        k_cache[ctx:ctx + T] = prev["k_cache_next"].reshape(k_cache.shape)[ctx:ctx + T]
        v_cache[ctx:ctx + T] = prev["v_cache_next"].reshape(v_cache.shape)[ctx:ctx + T]
    if L + 1 < N_LAYERS:
        shn = dataclasses.replace(SMALL_STACK, window=0 if is_global(L + 1) else SMALL_STACK.window)
        kn, vn = synth.device_kv_context(shn, CFG_ID, L + 1, "cuda")
        kn, vn = _host(kn), _host(vn)
    else:
        kn, vn = np.zeros_like(k_cache), np.zeros_like(v_cache)
    return synth.LayerInputs(sh, step_in["parent"].astype(np.int32), h_in, q_in, k_cache, v_cache, kn, vn,
                             _host(w["w_o"]), _host(w["w_pool"]), _host(w["w_router"]), _host(w["w_unpool"]),
                             _host(w["w_qkv_next"]), _host(w["w1"]), _host(w["w2"]), None)


def test_small_stack_layer_by_layer_and_in_one_go():
    step_in = synth.stack_step_inputs(SMALL_STACK, CFG_ID, 0)
    chain = []
    prev = None
    for L in range(N_LAYERS):
        log(f"[stack layer {L}] {'global' if is_global(L) else 'swa'}{' (last)' if L + 1 == N_LAYERS else ''}")
        inp = _layer_inputs(L, step_in, prev)
        dw = dt.upload_weights(inp)
        if L + 1 == N_LAYERS:
            dw = dataclasses.replace(dw, w_qkv=None)
        st = dt.make_step(inp)
        dt.run_step(dw, st)
        out = dt.outputs(st)
        if L + 1 < N_LAYERS:
            _check_layer(inp, out)
        else:
            assert out["status"] == 0
            ref = oracle.layer_step_auto(inp)
            assert_close_bf16("last layer h_out end-to-end", out["h_out"], ref["h_out"])
        chain.append(out)
        prev = out
    # the stack runner, all launches back to back on one stream
    stk = Stack(SMALL_STACK, CFG_ID, N_LAYERS)
    stk.set_step_inputs(step_in)
    stk.launch_step(stk.structs(False, False), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk.ws) == 0
    assert np.array_equal(_host(stk.h_out()), chain[-1]["h_out"])
    for L in range(N_LAYERS):
        assert np.array_equal(stk.layers[L].topk_idx.cpu().numpy(), chain[L]["idx"]), L
        if L + 1 < N_LAYERS:
            T, ctx = SMALL_STACK.T, SMALL_STACK.ctx
            kn = _host(stk.layers[L + 1].k_cache).reshape(SMALL_STACK.kv_capacity, -1)[ctx:ctx + T]
            vn = _host(stk.layers[L + 1].v_cache).reshape(SMALL_STACK.kv_capacity, -1)[ctx:ctx + T]
            cap = SMALL_STACK.kv_capacity
            assert np.array_equal(kn, chain[L]["k_cache_next"].reshape(cap, -1)[ctx:ctx + T]), L
            assert np.array_equal(vn, chain[L]["v_cache_next"].reshape(cap, -1)[ctx:ctx + T]), L
    log("  stack in one go: bit-identical to the layer-by-layer chain")


def _step_outputs(stk: Stack) -> dict:
    T, ctx, cap = SMALL_STACK.T, SMALL_STACK.ctx, SMALL_STACK.kv_capacity
    out = {"h_out": _host(stk.h_out())}
    for L, lay in enumerate(stk.layers):
        out[f"idx{L}"] = lay.topk_idx.cpu().numpy()
        out[f"k{L}"] = _host(lay.k_cache).reshape(cap, -1)[ctx:ctx + T].copy()
        out[f"v{L}"] = _host(lay.v_cache).reshape(cap, -1)[ctx:ctx + T].copy()
    return out


def test_stack_step_replayed_as_one_graph():
    """The step's launches captured once; over three steps with different trees and inputs (the
    inputs written eagerly, with a kernel launch, between replays) every replay equals the eager
    launches of the same step bit for bit, and the graph is replayed again after eager work."""
    stk = Stack(SMALL_STACK, CFG_ID, N_LAYERS)
    stream = torch.cuda.current_stream()
    structs = stk.structs(False, False)
    # warm launch (kernel attributes set, code loaded) before capture
    stk.set_step_inputs(synth.stack_step_inputs(SMALL_STACK, CFG_ID, 0))
    stk.launch_step(structs, stream.cuda_stream)
    torch.cuda.synchronize()
    g = stk.capture_step(structs)
    torch.cuda.synchronize()
    for s in (1, 2, 3, 1):
        step_in = synth.stack_step_inputs(SMALL_STACK, CFG_ID, s)
        log(f"[graph step inputs {s}]")
        stk.set_step_inputs(step_in)
        stk.launch_step(structs, stream.cuda_stream)
        torch.cuda.synchronize()
        assert mk.mk_read_status(stk.ws) == 0
        eager = _step_outputs(stk)
        # wipe what the step writes, so that a replay that wrote nothing cannot pass
        T, ctx, cap = SMALL_STACK.T, SMALL_STACK.ctx, SMALL_STACK.kv_capacity
        for t in stk.h + stk.q:
            t.zero_()
        for lay in stk.layers:
            lay.topk_idx.zero_()
            lay.k_cache.view(cap, -1)[ctx:ctx + T].zero_()
            lay.v_cache.view(cap, -1)[ctx:ctx + T].zero_()
        stk.set_step_inputs(step_in)
        g.replay()
        torch.cuda.synchronize()
        assert mk.mk_read_status(stk.ws) == 0
        replay = _step_outputs(stk)
        for key in eager:
            assert np.array_equal(eager[key], replay[key]), (s, key)
    log("  graph replays bit-identical to the eager launches")


def test_stack_step_from_embeddings_with_the_prologue():
    """A stack run with the first-layer prologue: layer 0's queries and tree K/V rows come
    from mk_qkv_prologue on the step tokens' embeddings (checked against the oracle), and the
    whole step, eager and replayed as one graph, equals the plain stack given those same
    prologue outputs as its step inputs, bit for bit."""
    sh = SMALL_STACK
    T, ctx, cap, H, Hq, Hkv, d = sh.T, sh.ctx, sh.kv_capacity, sh.hidden, sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    stream = torch.cuda.current_stream()
    stk_p = Stack(sh, CFG_ID, N_LAYERS, prologue=True)
    step_in = synth.stack_step_inputs(sh, CFG_ID, 4)
    # the prologue on its own
    q0 = torch.zeros((T, Hq * d), dtype=torch.int16, device="cuda")
    kc = torch.zeros((cap, Hkv, d), dtype=torch.int16, device="cuda")
    vc = torch.zeros((cap, Hkv, d), dtype=torch.int16, device="cuda")
    mk.mk_qkv_prologue(dt.dev_u16(step_in["h_in"]), stk_p.w_qkv0, T, H, Hq, Hkv, d, q0, kc, vc, cap, ctx)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, _ = oracle.qkv_project(step_in["h_in"], _host(stk_p.w_qkv0), Hq, Hkv, d)
    assert_close_bf16("prologue q", _host(q0), q_ref)
    assert_close_bf16("prologue k", _host(kc)[ctx:ctx + T], k_ref)
    assert_close_bf16("prologue v", _host(vc)[ctx:ctx + T], v_ref)
    # the plain stack given the prologue's outputs
    stk = Stack(sh, CFG_ID, N_LAYERS)
    stk.set_step_inputs(dict(step_in, q_in=_host(q0), k_tree=_host(kc)[ctx:ctx + T], v_tree=_host(vc)[ctx:ctx + T]))
    stk.launch_step(stk.structs(False, False), stream.cuda_stream)
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk.ws) == 0
    ref = _step_outputs(stk)
    # the prologue stack, eager, then replayed as one graph (prologue inside the graph)
    structs = stk_p.structs(False, False)
    stk_p.set_step_inputs(step_in)
    stk_p.launch_step(structs, stream.cuda_stream)
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk_p.ws) == 0
    got = _step_outputs(stk_p)
    for key in ref:
        assert np.array_equal(ref[key], got[key]), ("eager", key)
    g = stk_p.capture_step(structs)
    for t in stk_p.h + stk_p.q:
        t.zero_()
    for lay in stk_p.layers:
        lay.topk_idx.zero_()
        lay.k_cache.view(cap, -1)[ctx:ctx + T].zero_()
        lay.v_cache.view(cap, -1)[ctx:ctx + T].zero_()
    stk_p.set_step_inputs(step_in)
    g.replay()
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk_p.ws) == 0
    got = _step_outputs(stk_p)
    for key in ref:
        assert np.array_equal(ref[key], got[key]), ("graph", key)
    log("  step from embeddings: eager and graph replay bit-identical to the plain stack")


def test_stack_accept_and_commit_closes_the_step():
    """After a stack verify step, greedy acceptance with target tokens that follow one branch
    of the tree, then the KV commit in every layer: each layer's rows ctx..ctx+n-1 hold the
    accepted nodes' rows (as the step wrote them at ctx + node), the other rows are unchanged,
    and the path equals the oracle's."""
    sh = SMALL_STACK
    T, ctx, cap = sh.T, sh.ctx, sh.kv_capacity
    stream = torch.cuda.current_stream()
    stk = Stack(sh, CFG_ID, N_LAYERS)
    step_in = synth.stack_step_inputs(sh, CFG_ID, 5)
    stk.set_step_inputs(step_in)
    stk.launch_step(stk.structs(False, False), stream.cuda_stream)
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk.ws) == 0
    parent = step_in["parent"].astype(np.int32)
    g = np.random.default_rng(12)
    draft = g.integers(0, 1000, T).astype(np.int32)
    target = g.integers(1000, 2000, T).astype(np.int32)
    # the target follows the deepest-index child at every node along one branch
    node = 0
    while True:
        kids = [c for c in range(1, T) if parent[c] == node]
        if not kids:
            break
        target[node] = draft[kids[-1]]
        node = kids[-1]
    before = [(_host(l.k_cache).reshape(cap, -1).copy(), _host(l.v_cache).reshape(cap, -1).copy()) for l in stk.layers]
    stk.accept_and_commit(torch.from_numpy(draft).cuda(), torch.from_numpy(target).cuda(), stream.cuda_stream)
    torch.cuda.synchronize()
    ref_path, ref_bonus = oracle.tree_accept(parent, draft, target)
    n = int(stk.n_path.item())
    assert stk.path.cpu().numpy()[:n].tolist() == ref_path and int(stk.bonus.item()) == ref_bonus
    assert n >= 2
    for L, lay in enumerate(stk.layers):
        k0, v0 = before[L]
        ek, ev = oracle.kv_commit(k0, v0, ctx, ref_path)
        assert np.array_equal(_host(lay.k_cache).reshape(cap, -1), ek), L
        assert np.array_equal(_host(lay.v_cache).reshape(cap, -1), ev), L
    log(f"  accepted {n} of {T} nodes; committed in all {N_LAYERS} layers")
