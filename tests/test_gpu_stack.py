"""GPU tests of the stack mechanics: the last-layer launch mode, a stack of fused layers
(global every fourth layer, the last one without a next-layer projection) checked layer by
layer against the oracle and, run in one go by the stack runner, bit for bit against the
layer-by-layer chain, and the stack's verify step replayed as one HIP graph."""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
import layer_persistent_amd as mk
from layer_persistent_amd import _abi as abi
from layer_persistent_amd import tensors as dt
from layer_persistent_amd.stack import Stack, is_global

from gpu_util import assert_close_bf16, assert_rounding_exact, log
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
        _check_layer(inp, out, last=L + 1 == N_LAYERS)
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
    w0 = _host(stk_p.w_qkv0)
    assert_close_bf16("prologue q", _host(q0), q_ref)
    assert_rounding_exact("prologue q", _host(q0), step_in["h_in"], w0[:Hq * d])
    assert_rounding_exact("prologue k", _host(kc)[ctx:ctx + T].reshape(T, -1), step_in["h_in"], w0[Hq * d:(Hq + Hkv) * d])
    assert_rounding_exact("prologue v", _host(vc)[ctx:ctx + T].reshape(T, -1), step_in["h_in"], w0[(Hq + Hkv) * d:])
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


# ---------------------------------------------------------------- the 62-layer shard-shape stack

STACK62_CHECKED = (0, 1, 3, 61)


@pytest.fixture(scope="module")
def stack62_step0():
    """Step 0 of the 62-layer stack at one GPU's shard shape (46 SWA-2048 + 16 global layers,
    ctx 4096, NVFP4 experts), launched layer by layer on one stream as the stack runs it.  For
    the checked layers, the launch's inputs are copied out before it and its outputs and stage
    hand-off buffers after it (those launches also return gates, logits, softmax statistics and
    the usage histogram)."""
    sh, cfg_id, n_layers = synth.CFG4, 4, 62
    T, E, k, cap = sh.T, sh.n_experts, sh.top_k, sh.kv_capacity
    log(f"[stack62] building {n_layers} layers")
    stk = Stack(sh, cfg_id, n_layers)
    step_in = synth.stack_step_inputs(sh, cfg_id, 0)
    stk.set_step_inputs(step_in)
    structs = stk.structs(False, False)
    sp = torch.cuda.current_stream().cuda_stream
    f32 = dict(dtype=torch.float32, device="cuda")
    snaps = {}
    for L in range(n_layers):
        c, w, io = structs[L]
        lay = stk.layers[L]
        if L not in STACK62_CHECKED:
            assert stk.lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io), sp) == 0
            continue
        log(f"[stack62] layer {L}: launch and copy out")
        nxt = stk.layers[L + 1] if L + 1 < n_layers else None
        snap = dict(h_in=_host(stk.h[L % 2]), q_in=_host(stk.q[L % 2]), k_cache=_host(lay.k_cache),
                    v_cache=_host(lay.v_cache),
                    kn=_host(nxt.k_cache) if nxt else None, vn=_host(nxt.v_cache) if nxt else None)
        gate, logits = torch.zeros((T, k), **f32), torch.zeros((T, E), **f32)
        stats, hist = torch.zeros((T, sh.n_q_heads, 2), **f32), torch.zeros(E, dtype=torch.int32, device="cuda")
        io2 = abi.mk_step_io.from_buffer_copy(io)
        io2.topk_gate, io2.router_logits = gate.data_ptr(), logits.data_ptr()
        io2.attn_stats, io2.expert_hist = stats.data_ptr(), hist.data_ptr()
        assert stk.lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io2), sp) == 0
        torch.cuda.synchronize()
        lw = abi.mk_workspace_query(c, T)
        ws = stk.ws
        u16 = lambda off, n: ws[dt.stage_offset(ws, lw, off):dt.stage_offset(ws, lw, off) + 2 * n].cpu().numpy().view(np.uint16)
        Hqd = sh.n_q_heads * sh.head_dim
        snap["out"] = dict(
            status=mk.mk_read_status(ws), h_out=_host(stk.h[(L + 1) % 2]),
            q_next=_host(stk.q[(L + 1) % 2]) if nxt else None,
            k_cache_next=_host(nxt.k_cache) if nxt else None, v_cache_next=_host(nxt.v_cache) if nxt else None,
            idx=lay.topk_idx.cpu().numpy(), gate=gate.cpu().numpy(), logits=logits.cpu().numpy(),
            stats=stats.cpu().numpy(), hist=hist.cpu().numpy(),
            attn=dt.untile_frag(u16(lw.attn, 16 * Hqd), T, Hqd),
            h1=dt.untile_frag(u16(lw.h1, 16 * sh.hidden), T, sh.hidden),
            xp=dt.untile_frag(u16(lw.xp, 16 * sh.pooled), T, sh.pooled),
            y=dt.untile_frag(u16(lw.y, 16 * sh.pooled), T, sh.pooled))
        snaps[L] = snap
    torch.cuda.synchronize()
    assert mk.mk_read_status(stk.ws) == 0
    del stk
    torch.cuda.empty_cache()
    return snaps


@pytest.mark.parametrize("L", STACK62_CHECKED)
def test_stack62_shard_shape_layer_against_the_oracle(stack62_step0, L):
    """Layers 0, 1, 3 (sliding window) and 61 (the last: no next-layer projection) of step 0
    of the full 62-layer stack at the shard shape, each against the oracle fed that launch's
    own inputs: stage by stage (rounding-exact dense stages and KV write) and end to end."""
    sh0, cfg_id = synth.CFG4, 4
    sh = dataclasses.replace(sh0, window=0 if is_global(L) else sh0.window)
    snap = stack62_step0[L]
    log(f"[stack62 layer {L}] {'global' if is_global(L) else 'swa-2048'}, ctx {sh.ctx}")
    w = synth.device_layer_weights(sh, cfg_id, L, "cuda")
    hw = {key: _host(t) for key, t in w.items()}
    del w
    torch.cuda.empty_cache()
    last = L == 61
    kn = snap["kn"] if not last else np.zeros_like(snap["k_cache"])
    vn = snap["vn"] if not last else np.zeros_like(snap["v_cache"])
    parent = synth.stack_step_inputs(sh0, cfg_id, 0)["parent"].astype(np.int32)
    inp = synth.LayerInputs(sh, parent, snap["h_in"], snap["q_in"], snap["k_cache"], snap["v_cache"], kn, vn,
                            hw["w_o"], hw["w_pool"], hw["w_router"], hw["w_unpool"], hw["w_qkv_next"], hw["w1"],
                            hw["w2"], None)
    out = dict(snap["out"])
    if last:
        out["q_next"] = np.zeros((sh.T, sh.n_q_heads * sh.head_dim), np.uint16)
    _check_layer(inp, out, last=last)
    log(f"  distinct experts: {len(np.unique(out['idx']))}")
