"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle."""
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

from gpu_util import (assert_close_bf16, assert_rounding_exact, assert_stats, check_routing, fp32_dot_bound,
                      log, max_abs_rel)

SMALL_NVFP4 = synth.LayerShape("small-tree-swa-nvfp4", 256, 4, 1, 64, 256, 16, 4, 64, 128, 300, 16, True)
SMALL_GQA = synth.LayerShape("small-tree-gqa2-global-bf16", 256, 8, 2, 64, 128, 32, 3, 64, 0, 200, 16, False)
SMALL_T5 = synth.LayerShape("small-t5-window-nvfp4", 256, 4, 1, 128, 256, 16, 2, 96, 40, 60, 5, True)
# a long global context with 8 q heads of 64: on a 256-CU device its attention items hold
# four row tiles each, with two key groups per tile
SMALL_RW4 = synth.LayerShape("small-global-ctx8100-nvfp4", 256, 8, 1, 64, 256, 16, 4, 64, 0, 8100, 16, True)
# pooled 1152: nine 128-wide k-steps per W1 row, split 5 + 4 over two pieces (the second
# piece's scale bytes start at 40, not at half the row)
SMALL_P1152 = synth.LayerShape("small-p1152-nvfp4", 256, 4, 1, 64, 1152, 16, 4, 64, 128, 300, 16, True)
# hidden 1280 (40 k-steps of 32) with 24 qkv tiles: on a 256-CU device the next-layer qkv
# splits each tile's K over three workgroups, 16 + 16 + 8 k-steps
SMALL_H1280 = synth.LayerShape("small-h1280-splitk-nvfp4", 1280, 4, 1, 64, 256, 16, 4, 64, 128, 300, 16, True)
# local expert intermediates of 128 and 256: the register-fed GEMM2 path (I % 64 == 0, I >= 128)
SMALL_I128 = synth.LayerShape("small-i128-nvfp4", 256, 4, 1, 64, 256, 16, 4, 128, 128, 300, 16, True)
SMALL_I256 = synth.LayerShape("small-i256-t9-nvfp4", 256, 8, 2, 64, 512, 32, 8, 256, 0, 500, 9, True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_nvfp4_pack_bit_exact():
    g = np.random.default_rng(21)
    for is_fp32 in (0, 1):
        B, N, K = 3, 40, 96
        w = (g.standard_normal((B, N, K)) * 0.02).astype(np.float32)
        w[1, 3, :16] = 0
        w[2, 5, 7] = 1.5
        if is_fp32:
            wd = torch.from_numpy(w).cuda()
            ref_w = w.astype(np.float64)
        else:
            bits = synth.bf16_bits_from_f32(w)
            wd = dt.dev_u16(bits)
            ref_w = oracle.bf16_to_f64(bits)
        codes = torch.empty((B, N, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((B, N, K // 16), dtype=torch.uint8, device="cuda")
        ts = torch.empty(B, dtype=torch.float32, device="cuda")
        mk.mk_nvfp4_pack(wd, is_fp32, B, N, K, codes, scales, ts)
        torch.cuda.synchronize()
        for b in range(B):
            rc, rs, rt = oracle.nvfp4_pack(ref_w[b])
            assert np.array_equal(codes[b].cpu().numpy(), rc)
            assert np.array_equal(scales[b].cpu().numpy(), rs)
            assert ts[b].item() == rt
    log("  nvfp4 pack: bit-exact (bf16 and fp32 inputs)")


def _tile_w1_reference(codes, scales, K):
    """GEMM1's W1 operand order as include/mk.h states it, element by element."""
    B, N, _ = codes.shape
    L = K // 128
    p = 2 if L > 8 else 1
    S = 8 * ((L + p - 1) // p)
    ct = np.zeros((B, N // 16, L, 64, 16), dtype=np.uint8)
    st = np.zeros((B, N // 16, p, 16, S), dtype=np.uint8)
    for b in range(B):
        for t in range(N // 16):
            for s_ in range(L):
                for l in range(64):
                    ct[b, t, s_, l] = codes[b, 16 * t + l % 16, 64 * s_ + 16 * (l // 16):64 * s_ + 16 * (l // 16) + 16]
            for q in range(p):
                for r in range(16):
                    for i in range(S):
                        if q * S + i < K // 16:
                            st[b, t, q, r, i] = scales[b, 16 * t + r, q * S + i]
    return ct.reshape(-1), st.reshape(-1)


@pytest.mark.parametrize("K", [256, 1152, 2048])
def test_nvfp4_tile_w1_is_the_documented_permutation(K):
    g = np.random.default_rng(K)
    B, N = 2, 48
    codes = g.integers(0, 256, size=(B, N, K // 2), dtype=np.uint8)
    scales = g.integers(0, 256, size=(B, N, K // 16), dtype=np.uint8)
    nbytes = mk.mk_nvfp4_w1_scales_bytes(B, N, K)
    ct = torch.empty(B * N * K // 2, dtype=torch.uint8, device="cuda")
    st = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    mk.mk_nvfp4_tile_w1(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), B, N, K, ct, st)
    torch.cuda.synchronize()
    rc, rs = _tile_w1_reference(codes, scales, K)
    assert np.array_equal(ct.cpu().numpy(), rc)
    assert np.array_equal(st.cpu().numpy(), rs)
    log(f"  W1 operand order, K = {K}: bit-exact permutation")


def test_kv_append_bit_exact_and_untouched_rows():
    g = np.random.default_rng(22)
    cap, Hkv, d, pos, n = 64, 2, 64, 17, 9
    kc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
    vc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
    kn = synth.normal_bf16(g, (n, Hkv, d), 1.0)
    vn = synth.normal_bf16(g, (n, Hkv, d), 1.0)
    K, V, KN, VN = (dt.dev_u16(x) for x in (kc, vc, kn, vn))
    mk.mk_kv_append(K, V, cap, Hkv, d, pos, KN, VN, n)
    torch.cuda.synchronize()
    ek, ev = kc.copy(), vc.copy()
    ek[pos:pos + n] = kn
    ev[pos:pos + n] = vn
    assert np.array_equal(dt.host_u16(K), ek) and np.array_equal(dt.host_u16(V), ev)
    assert mk.mk_kv_append(K, V, cap, Hkv, d, cap - 2, KN, VN, n, check=False) == mk.MK_ECAPACITY


@pytest.mark.parametrize("T,H,Hq,Hkv,d,cap,pos", [(16, 4096, 8, 1, 128, 8208, 8192),   # the shard shape
                                                      (16, 256, 4, 1, 64, 320, 300),
                                                      (5, 256, 8, 2, 64, 64, 59),        # ragged T, GQA
                                                      (1, 128, 2, 1, 64, 8, 0)])
def test_qkv_prologue_against_the_oracle(T, H, Hq, Hkv, d, cap, pos):
    """First-layer prologue: q, and the k / v rows at pos..pos+T-1, against the oracle's qkv
    projection (fp64, one rounding); every other cache row untouched."""
    log(f"[qkv prologue T={T} H={H} Hq={Hq} Hkv={Hkv} d={d} pos={pos}]")
    g = np.random.default_rng(24 + T)
    h = synth.normal_bf16(g, (T, H), 1.0)
    w = synth.normal_bf16(g, ((Hq + 2 * Hkv) * d, H), 0.02)
    kc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
    vc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
    q_out = torch.zeros((T, Hq * d), dtype=torch.int16, device="cuda")
    K, V = dt.dev_u16(kc), dt.dev_u16(vc)
    mk.mk_qkv_prologue(dt.dev_u16(h), dt.dev_u16(w), T, H, Hq, Hkv, d, q_out, K, V, cap, pos)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, _ = oracle.qkv_project(h, w, Hq, Hkv, d)
    kg, vg = dt.host_u16(K), dt.host_u16(V)
    qd, kd = Hq * d, Hkv * d
    assert_close_bf16("prologue q", dt.host_u16(q_out), q_ref)
    assert_rounding_exact("prologue q", dt.host_u16(q_out), h, w[:qd])
    assert_rounding_exact("prologue k", kg[pos:pos + T].reshape(T, -1), h, w[qd:qd + kd])
    assert_rounding_exact("prologue v", vg[pos:pos + T].reshape(T, -1), h, w[qd + kd:])
    rest = np.ones(cap, bool)
    rest[pos:pos + T] = False
    assert np.array_equal(kg[rest], kc[rest]) and np.array_equal(vg[rest], vc[rest])


def test_tree_accept_and_kv_commit_against_the_oracle():
    """Greedy acceptance on seeded trees (the verification tree generator, tokens drawn so
    that the walk stops at every depth) equals the oracle's path and bonus exactly, and the
    KV commit of that path equals the oracle's row moves bit for bit with every other row
    untouched; n_path is read on the device.  A malformed tree accepts nothing."""
    g = np.random.default_rng(31)
    cap, Hkv, d, ctx = 96, 1, 128, 70
    dev_i32 = lambda a: torch.from_numpy(np.asarray(a, np.int32)).cuda()
    path = torch.empty(16, dtype=torch.int32, device="cuda")
    n_path = torch.empty(1, dtype=torch.int32, device="cuda")
    bonus = torch.empty(1, dtype=torch.int32, device="cuda")
    depths = set()
    for trial in range(40):
        T = 16 if trial % 4 else int(g.integers(1, 17))
        parent = synth.tree_parents(T, g) if T > 1 else np.array([-1], np.int32)
        draft = g.integers(100, 110, T).astype(np.int32)
        target = g.integers(100, 110, T).astype(np.int32)
        # make the walk go deep in some trials: copy each first child's token to its parent
        if trial % 3 == 0:
            for i in range(T):
                kids = [c for c in range(1, T) if parent[c] == i]
                if kids:
                    target[i] = draft[kids[-1]]
        mk.mk_tree_accept(dev_i32(parent), dev_i32(draft), dev_i32(target), T, path, n_path, bonus)
        kc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
        vc = synth.normal_bf16(g, (cap, Hkv, d), 1.0)
        K, V = dt.dev_u16(kc), dt.dev_u16(vc)
        mk.mk_kv_commit(K, V, cap, Hkv, d, ctx, path, n_path, T)
        torch.cuda.synchronize()
        ref_path, ref_bonus = oracle.tree_accept(parent, draft, target)
        n = int(n_path.item())
        assert n == len(ref_path), (trial, n, ref_path)
        gp = path.cpu().numpy()[:T]
        assert gp[:n].tolist() == ref_path and np.all(gp[n:] == -1), (trial, gp, ref_path)
        assert int(bonus.item()) == ref_bonus
        ek, ev = oracle.kv_commit(kc, vc, ctx, ref_path)
        assert np.array_equal(dt.host_u16(K), ek) and np.array_equal(dt.host_u16(V), ev), trial
        depths.add(n)
    log(f"  accepted path lengths seen: {sorted(depths)}")
    assert len(depths) >= 4
    bad = np.array([-1, 0, 3, 1], np.int32)
    mk.mk_tree_accept(dev_i32(bad), dev_i32([1, 2, 3, 4]), dev_i32([2, 3, 4, 5]), 4, path, n_path, bonus)
    torch.cuda.synchronize()
    assert int(n_path.item()) == 0 and int(bonus.item()) == -1 and np.all(path.cpu().numpy()[:4] == -1)


def test_route_topk_standalone():
    g = np.random.default_rng(23)
    T, P, E, k = 16, 2048, 256, 8
    x = synth.normal_bf16(g, (T, P), 1.0)
    w = synth.normal_bf16(g, (E, P), 0.02)
    bias = np.zeros((T, E), np.float32)
    bias[2, 77] = 8.0
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    mk.mk_route_topk(dt.dev_u16(x), dt.dev_u16(w), torch.from_numpy(bias).cuda(), T, P, E, k, idx, gate, logits)
    torch.cuda.synchronize()
    l64, _, _, _ = oracle.router(x, w, None, k)
    gl = logits.cpu().numpy()
    bound = fp32_dot_bound(x, w)
    assert np.all(np.abs(gl - bias - l64) <= bound + 1e-6)
    check_routing(gl, idx.cpu().numpy(), gate.cpu().numpy(), l64, bias, k, float(bound.max()))
    assert idx[2, 0].item() == 77


@pytest.mark.parametrize("n_words,blocks", [(4 * (1 << 20) + 4 * 37, 256), (4 * 1000 + 4, 3), (4, 2048)])
def test_stream_read_reads_every_byte_once(n_words, blocks):
    """The streaming-read probe XORs every 32-bit word it reads into the sink: on random data
    the result equals the host's XOR of the whole buffer (a piece skipped or read twice would
    change it), and a second call XORs the same value in again, back to zero."""
    g = np.random.default_rng(31)
    w = g.integers(0, 1 << 32, n_words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(w.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mk.mk_stream_read(src, 4 * n_words, blocks, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(w)), (n_words, blocks)
    mk.mk_stream_read(src, 4 * n_words, blocks, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == 0


def _run(inp, timestamps=False, st=None, dw=None):
    dw = dw or dt.upload_weights(inp)
    st = st or dt.make_step(inp, timestamps=timestamps)
    dt.run_step(dw, st)
    out = dt.outputs(st)
    return dw, st, out


def _pack_used(inp, gpu_idx):
    """The layer's experts in storage format, packed by the oracle for every expert that the
    GPU's routing or the oracle's own (end-to-end) routing selects; the others stay None.
    oracle.layer_step on these equals oracle.layer_step_auto (which packs the oracle's set)."""
    sh = inp.shape
    if not sh.nvfp4:
        return oracle.pack_experts(inp)
    attn, _ = oracle.attention(inp.q_in, inp.k_cache, inp.v_cache, inp.parent, sh.ctx, sh.window, sh.n_q_heads,
                               sh.n_kv_heads, sh.head_dim)
    xp = oracle.dense(oracle.dense(attn, inp.w_o, inp.h_in), inp.w_pool)
    _, _, idx, _ = oracle.router(xp, inp.w_router, inp.router_bias, sh.top_k)
    return oracle.pack_experts(inp, sorted(set(np.unique(idx).tolist()) | set(np.unique(gpu_idx).tolist())))


def _end_to_end_reference(inp, out, ex, logit_bound: float) -> dict:
    """The oracle's layer step from the launch's own inputs, for the end-to-end comparison.

    Upstream roundings (attention's softmax, then each bf16 stage) make the GPU's xp differ
    from the oracle's in a few low bits, so the two routers' logits differ by at most delta
    per token (the change those xp differences can cause, plus the fp32 bound).  Where a
    token's logits are that close, more than one selection (or order of it) is correct.  Rank
    statistics move by at most delta when every value does, so a correct GPU selection
    satisfies, at every rank j, |z(gpu's j-th expert) - z(oracle's j-th expert)| <= 2 delta on
    the oracle's logits z; every token that differs must pass that.  For them the reference
    takes the GPU's selection (the oracle step anchored on the GPU's indices and gates); every
    other token's selection is the oracle's own, which the GPU's equals."""
    sh = inp.shape
    ref = oracle.layer_step(inp, ex)
    flip = [t for t in range(sh.T) if list(ref["idx"][t]) != list(out["idx"][t])]
    dxp = oracle.bf16_to_f64(out["xp"]) - oracle.bf16_to_f64(ref["xp"])
    dlog = np.abs(dxp) @ np.abs(oracle.bf16_to_f64(inp.w_router)).T
    log(f"  end-to-end: xp differs from the oracle's in {int(np.count_nonzero(dxp))} of {dxp.size} elements; "
        f"{len(flip)} token(s) routed differently from the oracle's own routing")
    for t in flip:
        z = ref["logits32"][t].astype(np.float64)
        delta = dlog[t].max() + logit_bound
        worst = float(np.abs(z[out["idx"][t]] - z[ref["idx"][t]]).max())
        log(f"    token {t}: gpu {out['idx'][t].tolist()} oracle {ref['idx'][t].tolist()}, "
            f"largest rank-wise logit difference {worst:.3e} <= 2 delta = {2 * delta:.3e}")
        assert worst <= 2 * delta, f"token {t}: routing differs end-to-end by {worst} > {2 * delta}"
    if flip:
        ref = oracle.layer_step(inp, ex, anchors={"idx": out["idx"], "gate": out["gate"].astype(np.float64)})
    for key in ("h1", "xp", "y"):
        log(f"  {key} end-to-end: max-abs-rel {max_abs_rel(out[key], ref[key]):.3e}")
    return ref


def _check_layer(inp, out, last: bool = False):
    """Stage-local parity (each stage's oracle fed the GPU's own stage inputs) and end-to-end.

    The dense stages (o-proj, pooler, unpooler, next-layer q / k / v and the KV write) are
    checked rounding-exact (assert_rounding_exact): their bf16 outputs equal the oracle's
    correctly rounded values except where the exact value lies within the rigorous fp32 bound
    of a rounding boundary, and only a fraction of a percent may differ at all.  The residual
    stream's magnitude therefore hides no error in the o-proj or unpooler contributions.
    `last`: the stack's last layer, which ends after the unpooler (no next-layer q / k / v)."""
    sh = inp.shape
    T, ctx = sh.T, sh.ctx
    assert out["status"] == 0, mk.mk_strerror(out["status"])
    attn, stats = oracle.attention(inp.q_in, inp.k_cache, inp.v_cache, inp.parent, ctx, sh.window,
                                   sh.n_q_heads, sh.n_kv_heads, sh.head_dim)
    assert_close_bf16("attn", out["attn"], attn)
    assert_stats("attn stats m", out["stats"][..., 0], stats[..., 0])
    assert_stats("attn stats l", out["stats"][..., 1], stats[..., 1])
    assert_rounding_exact("h1 = o-proj + residual (anchored on gpu attn)", out["h1"], out["attn"], inp.w_o, inp.h_in)
    assert_rounding_exact("xp = pooler (anchored on gpu h1)", out["xp"], out["h1"], inp.w_pool)
    l64, _, _, _ = oracle.router(out["xp"], inp.w_router, None, sh.top_k)
    bias = inp.router_bias
    bound = fp32_dot_bound(out["xp"], inp.w_router)
    dl = np.abs(out["logits"] - (bias if bias is not None else 0) - l64)
    log(f"  logits: max |gpu - fp64| {dl.max():.3e} (rigorous fp32 bound {bound.max():.3e})")
    assert np.all(dl <= bound + 1e-6)
    check_routing(out["logits"], out["idx"], out["gate"], l64, bias, sh.top_k, float(bound.max()))
    hist = np.bincount(out["idx"].reshape(-1), minlength=sh.n_experts)
    assert np.array_equal(out["hist"], hist)
    # the experts packed once, for both the anchored check and the end-to-end step: those the
    # GPU routed to and those the oracle's own routing reaches
    ex = _pack_used(inp, out["idx"])
    y_ref, _ = oracle.moe(out["xp"], out["idx"], out["gate"].astype(np.float64), ex, sh.expert_inter)
    assert_close_bf16("y (anchored on gpu xp, routing)", out["y"], y_ref)
    assert_rounding_exact("h_out = unpooler + residual (anchored on gpu y, h1)", out["h_out"], out["y"], inp.w_unpool,
                          out["h1"])
    ref = _end_to_end_reference(inp, out, ex, float(bound.max()))
    if last:
        assert_close_bf16("h_out end-to-end", out["h_out"], ref["h_out"])
        return
    qd, kd = sh.n_q_heads * sh.head_dim, sh.n_kv_heads * sh.head_dim
    wq = inp.w_qkv_next
    kn = out["k_cache_next"].reshape(sh.kv_capacity, -1)
    vn = out["v_cache_next"].reshape(sh.kv_capacity, -1)
    assert_rounding_exact("q_next (anchored on gpu h_out)", out["q_next"], out["h_out"], wq[:qd])
    # the KV write: rounding-exact against the oracle re-anchored on the GPU's h_out
    assert_rounding_exact("k_new, KV write (anchored on gpu h_out)", kn[ctx:ctx + T], out["h_out"], wq[qd:qd + kd])
    assert_rounding_exact("v_new, KV write (anchored on gpu h_out)", vn[ctx:ctx + T], out["h_out"], wq[qd + kd:])
    # every other row of the next layer's cache is untouched, bit for bit
    k0 = inp.k_cache_next.reshape(sh.kv_capacity, -1)
    v0 = inp.v_cache_next.reshape(sh.kv_capacity, -1)
    assert np.array_equal(kn[:ctx], k0[:ctx]) and np.array_equal(kn[ctx + T:], k0[ctx + T:])
    assert np.array_equal(vn[:ctx], v0[:ctx]) and np.array_equal(vn[ctx + T:], v0[ctx + T:])
    # end to end, no anchoring
    assert_close_bf16("h_out end-to-end", out["h_out"], ref["h_out"])
    assert_close_bf16("q_next end-to-end", out["q_next"], ref["q_next"])
    assert_close_bf16("k_new end-to-end", kn[ctx:ctx + T], ref["k_new"].reshape(T, -1))
    assert_close_bf16("v_new end-to-end", vn[ctx:ctx + T], ref["v_new"].reshape(T, -1))


@pytest.mark.parametrize("shape,cfg_id", [(synth.CFG1, 1), (SMALL_NVFP4, 81), (SMALL_GQA, 82), (SMALL_T5, 83),
                                           (SMALL_RW4, 84), (SMALL_P1152, 85), (SMALL_H1280, 88),
                                           (SMALL_I128, 93), (SMALL_I256, 94)])
def test_layer_small_shapes(shape, cfg_id):
    log(f"[layer parity] {shape.name}")
    inp = synth.make_layer_inputs(shape, cfg_id)
    _, _, out = _run(inp)
    _check_layer(inp, out)


def test_layer_router_ties():
    """Router weight rows repeated in threes (experts 3j, 3j+1, 3j+2 share a row), so every
    logit occurs three times and ties fall inside the top-k and across its k-th / (k+1)-th
    boundary.  The published selection must be the stable sort (logit desc, expert index asc)
    of the GPU's own logits -- the tie rule of the routing -- and the rest of the layer must
    pass the usual checks."""
    log("[layer parity] router rows tied in threes")
    inp = synth.make_layer_inputs(SMALL_NVFP4, 95)
    assert inp.router_bias is None
    wr = inp.w_router.copy()
    for e in range(wr.shape[0]):
        wr[e] = wr[3 * (e // 3)]
    inp = dataclasses.replace(inp, w_router=wr)
    _, _, out = _run(inp)
    lg, k = out["logits"], SMALL_NVFP4.top_k
    for e in range(lg.shape[1]):
        assert np.array_equal(lg[:, e], lg[:, 3 * (e // 3)]), f"expert {e}: tied logits differ"
    srt = -np.sort(-lg.astype(np.float64), axis=1)
    boundary = int(np.sum(srt[:, k - 1] == srt[:, k]))
    log(f"  {boundary}/{lg.shape[0]} tokens with a tie across the top-{k} boundary")
    assert boundary > 0
    _check_layer(inp, out)


@pytest.fixture(scope="module")
def cfg2_inputs():
    return synth.make_layer_inputs(synth.CFG2, 2)


def test_layer_cfg2_full_size(cfg2_inputs):
    log("[layer parity] cfg2 full size: SWA-2048 over ctx 8192, 16-token tree, NVFP4 experts")
    dw, st, out = _run(cfg2_inputs)
    _check_layer(cfg2_inputs, out)
    log(f"  distinct experts: {len(np.unique(out['idx']))}")


def test_layer_cfg3_full_size():
    log("[layer parity] cfg3 full size: global over ctx 32768, Zipf routing")
    inp = synth.make_layer_inputs(synth.CFG3, 3)
    _, _, out = _run(inp)
    _check_layer(inp, out)
    log(f"  distinct experts: {len(np.unique(out['idx']))}")


def test_deterministic_and_timing_build_identical():
    inp = synth.make_layer_inputs(SMALL_NVFP4, 84)
    dw = dt.upload_weights(inp)
    outs = []
    for ts in (False, False, True):
        st = dt.make_step(inp, timestamps=ts)
        dt.run_step(dw, st)
        outs.append(dt.outputs(st))
    for key in ("h_out", "q_next", "k_cache_next", "v_cache_next", "idx", "gate", "logits", "stats", "y", "xp"):
        assert np.array_equal(outs[0][key], outs[1][key]), key
        assert np.array_equal(outs[0][key], outs[2][key]), key


@pytest.mark.parametrize("shape,cfg_id,n", [(SMALL_NVFP4, 86, 16), (synth.CFG2, 2, 14)])
def test_expert_prefetch_lists_and_changes_no_output(shape, cfg_id, n):
    """The kernel's next-step prefetch list equals the most-used experts of its own routing
    (count desc, index asc, -1 past the used ones), and a launch that prefetches -- a real
    list, or one with ids outside [0, E) -- returns bit-identical outputs."""
    log(f"[prefetch] {shape.name}")
    inp = synth.make_layer_inputs(shape, cfg_id)
    dw = dt.upload_weights(inp)
    st = dt.make_step(inp)
    st.prefetch_next = torch.full((16,), -7, dtype=torch.int32, device="cuda")
    st.n_prefetch_next = n
    dt.run_step(dw, st)
    base = dt.outputs(st)
    _, top = oracle.usage_top(base["idx"], shape.n_experts, n)
    want = np.full(n, -1, dtype=np.int32)
    want[:len(top)] = top
    got = st.prefetch_next.cpu().numpy()
    assert np.array_equal(got[:n], want), (got[:n], want)
    assert np.all(got[n:] == -7)
    lists = [st.prefetch_next[:n].clone(),
             torch.tensor([-1, shape.n_experts, 1 << 20, 0, shape.n_experts - 1], dtype=torch.int32, device="cuda")]
    for lst in lists:
        st2 = dt.make_step(inp)
        st2.prefetch, st2.n_prefetch = lst, lst.numel()
        dt.run_step(dw, st2)
        out = dt.outputs(st2)
        for key in ("h_out", "q_next", "k_cache_next", "v_cache_next", "idx", "gate", "logits", "stats", "y", "xp"):
            assert np.array_equal(base[key], out[key]), key
    log(f"  prefetch list {got[:n].tolist()}")


@pytest.mark.parametrize("shape,cfg_id", [(SMALL_NVFP4, 85), (SMALL_H1280, 89)])
def test_repeated_steps_on_one_workspace(shape, cfg_id):
    """Successive launches on one workspace (as layer after layer / step after step); the
    hidden-1280 shape splits the next-layer qkv over workgroups, whose arrival counters must
    start every launch at zero."""
    log(f"[repeated steps] {shape.name}")
    dw = None
    st = None
    for step in range(4):
        inp = synth.make_layer_inputs(shape, cfg_id, step=step)
        if dw is None:
            dw = dt.upload_weights(inp)
            st = dt.make_step(inp)
        else:
            # refresh the step inputs in place, keep the workspace
            st.q_in.copy_(dt.dev_u16(inp.q_in)); st.h_in.copy_(dt.dev_u16(inp.h_in))
            st.k_cache.copy_(dt.dev_u16(inp.k_cache)); st.v_cache.copy_(dt.dev_u16(inp.v_cache))
            st.parent.copy_(torch.from_numpy(inp.parent).cuda())
            st.k_next.copy_(dt.dev_u16(inp.k_cache_next)); st.v_next.copy_(dt.dev_u16(inp.v_cache_next))
            st.hist.zero_()
        dt.run_step(dw, st)
        out = dt.outputs(st)
        ref = oracle.layer_step_auto(inp)
        assert out["status"] == 0
        assert_close_bf16(f"step {step} h_out", out["h_out"], ref["h_out"])
        assert_close_bf16(f"step {step} q_next", out["q_next"], ref["q_next"])
        ctx, T = shape.ctx, shape.T
        kn = out["k_cache_next"].reshape(shape.kv_capacity, -1)
        vn = out["v_cache_next"].reshape(shape.kv_capacity, -1)
        assert_close_bf16(f"step {step} k_new", kn[ctx:ctx + T], ref["k_new"].reshape(T, -1))
        assert_close_bf16(f"step {step} v_new", vn[ctx:ctx + T], ref["v_new"].reshape(T, -1))


def test_bad_tree_reports_status_and_does_not_outlive_its_launch():
    """A malformed tree sets MK_EBADTREE for that launch; the next launch on the same workspace
    (no re-initialisation) runs normally, matches the oracle, and reports MK_OK -- also with a
    short spin limit, so that any wait that polls the status word sees the stale code."""
    inp = synth.make_layer_inputs(SMALL_NVFP4, 86)
    bad = inp.parent.copy()
    bad[5] = 9   # parent after child
    dw = dt.upload_weights(inp)
    st = dt.make_step(inp)
    st.parent.copy_(torch.from_numpy(bad).cuda())
    dt.run_step(dw, st)
    assert mk.mk_read_status(st.workspace) == mk.MK_EBADTREE
    st.parent.copy_(torch.from_numpy(inp.parent.astype(np.int32)).cuda())
    dt.run_step(dw, st, spin_limit=4096)
    out = dt.outputs(st)
    assert out["status"] == mk.MK_OK and mk.mk_read_status(st.workspace) == mk.MK_OK
    _check_layer(inp, out)


def test_stalled_workgroup_times_out_instead_of_hanging():
    """A workgroup that never signals (host-set test hook) makes every bounded wait expire; the
    next launches on the same workspace, with no re-initialisation, run normally."""
    inp = synth.make_layer_inputs(SMALL_H1280, 87)
    dw = dt.upload_weights(inp)
    st = dt.make_step(inp)
    dt.run_step(dw, st, spin_limit=2000, skip_wg=5)
    assert mk.mk_read_status(st.workspace) == mk.MK_ETIMEOUT
    for _ in range(2):
        st.hist.zero_()                     # the usage histogram accumulates over launches
        dt.run_step(dw, st)
        out = dt.outputs(st)
        assert out["status"] == mk.MK_OK
        _check_layer(inp, out)
