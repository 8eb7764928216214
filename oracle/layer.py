"""One decoder-layer launch, written out plainly in fp64 (test infrastructure only).

The pages (LMSYS / SGLang megakernel for Muse Spark Open; the orcarouter.ai
write-up, section "where the kernel boundary sits") fix the unit of work: one
launch runs attention of layer L and continues through the next layer's query /
key / value projection and KV-cache write; in between sit the output projection,
a pooler that compresses each token vector before the experts, a router that
sends each token to 8 of 256 experts stored as NVFP4, and an unpooler that
restores the vector.  46 layers attend over the most recent 2,048 tokens and 16
attend globally; the verify step checks a 16-token tree proposed by the draft
model ("the draft model also got faster" section).

Readings where the pages are silent (each is listed in the design notes):
  * residual adds after the output projection and after the unpooler; no norms,
    no rotary embedding, no biases, no shared expert; attention scale 1/sqrt(d);
  * tree node 0 is the root at depth 0, parent[i] < i, node i has position
    ctx + depth_i and sits in KV slot ctx + i;
  * sliding window: a key at position p is visible from position P iff P - p < W;
  * bf16 rounding at attn, h1, xp, y, h_out and the next q/k/v; fp32 logits;
  * routing: top-k by (logit desc, index asc) on fp32 logits, gates = softmax over
    the k selected logits;
  * GEMM1 rows [0, I) are the gate projection and rows [I, 2I) the up projection;
    a = silu(gate) * up, requantised to NVFP4 (tensor scale 1) when the experts are
    NVFP4, else rounded to bf16; the combine sums gate * expert output in slot order.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64, nvfp4_decode, fp4_act_quant


def tree_masks(parent) -> tuple[np.ndarray, np.ndarray]:
    """Ancestor-or-self bitmask and depth of every tree node.  Raises on a malformed
    tree (parent[0] != -1 or parent[i] not in [0, i))."""
    parent = np.asarray(parent, dtype=np.int64)
    T = len(parent)
    if T < 1 or T > 32 or parent[0] != -1:
        raise ValueError("bad tree root")
    anc = np.zeros(T, dtype=np.uint64)
    depth = np.zeros(T, dtype=np.int64)
    anc[0] = 1
    for i in range(1, T):
        p = parent[i]
        if not (0 <= p < i):
            raise ValueError(f"bad parent for node {i}")
        anc[i] = anc[p] | (np.uint64(1) << np.uint64(i))
        depth[i] = depth[p] + 1
    return anc, depth


def visible_keys(parent, ctx: int, window: int) -> np.ndarray:
    """Boolean [T][ctx+T]: which KV rows token i attends to (context rows then tree slots)."""
    anc, depth = tree_masks(parent)
    T = len(anc)
    vis = np.zeros((T, ctx + T), dtype=bool)
    for i in range(T):
        pos = ctx + depth[i]
        lo = max(0, pos - window + 1) if window > 0 else 0
        vis[i, lo:ctx] = True
        for j in range(T):
            if (int(anc[i]) >> j) & 1:
                vis[i, ctx + j] = True
    return vis


def attention(q_in, k_cache, v_cache, parent, ctx: int, window: int, n_q_heads: int,
              n_kv_heads: int, head_dim: int):
    """Tree-masked grouped-query attention.  q_in bf16 [T][Hq*d]; caches bf16
    [cap][Hkv][d] with the tree's own rows already at slots ctx..ctx+T-1.
    Returns attn bf16 [T][Hq*d] and stats fp64 [T][Hq][2] = (m, l): the row max of
    the scaled scores and the sum of exp(score - m)."""
    T = len(parent)
    d, Hq, Hkv = head_dim, n_q_heads, n_kv_heads
    G = Hq // Hkv
    vis = visible_keys(parent, ctx, window)
    q = bf16_to_f64(q_in).reshape(T, Hq, d)
    K = bf16_to_f64(k_cache[:ctx + T]).reshape(ctx + T, Hkv, d)
    V = bf16_to_f64(v_cache[:ctx + T]).reshape(ctx + T, Hkv, d)
    out = np.zeros((T, Hq, d))
    stats = np.zeros((T, Hq, 2))
    for h in range(Hq):
        g = h // G
        s = (q[:, h, :] @ K[:, g, :].T) / np.sqrt(d)          # [T][keys]
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ V[:, g, :]) / l
        stats[:, h, 0] = m[:, 0]
        stats[:, h, 1] = l[:, 0]
    return bf16_round(out.reshape(T, Hq * d)), stats


def dense(x_bits, w_bits, residual_bits=None):
    """bf16(residual + x . W^T) with fp64 accumulation and a single rounding.
    x bf16 [T][K], W bf16 [N][K] (PyTorch Linear layout), residual bf16 [T][N]."""
    acc = bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T
    if residual_bits is not None:
        acc = acc + bf16_to_f64(residual_bits)
    return bf16_round(acc)


def router(xp_bits, wr_bits, bias, top_k: int):
    """Router logits (fp64 and fp32), top-k indices and softmax gates.
    The selection is taken on fp32 logits (the kernel's precision): order by value
    descending, then expert index ascending."""
    logits64 = bf16_to_f64(xp_bits) @ bf16_to_f64(wr_bits).T
    z = logits64.astype(np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    T, E = z.shape
    idx = np.zeros((T, top_k), dtype=np.int32)
    for t in range(T):
        taken = np.zeros(E, dtype=bool)
        for j in range(top_k):
            best = -1
            for e in range(E):
                if taken[e]:
                    continue
                if best < 0 or z[t, e] > z[t, best]:
                    best = e
            idx[t, j] = best
            taken[best] = True
    sel = np.take_along_axis(z.astype(np.float64), idx, axis=1)
    g = np.exp(sel - sel.max(axis=1, keepdims=True))
    gate = g / g.sum(axis=1, keepdims=True)
    return logits64, z, idx, gate


def silu(x):
    return x / (1.0 + np.exp(-x))


def moe(xp_bits, idx, gate, experts: dict, inter: int):
    """Routed experts and their combine.  experts: {"fmt": "bf16", "w1", "w2"} with
    bf16 [E][2I][P] / [E][P][I], or {"fmt": "nvfp4", "w1": [(codes, scales, ts)]*E,
    "w2": [...]}.  Returns y bf16 [T][P] and the per-pair intermediate codes/values."""
    T, k = idx.shape
    xp = bf16_to_f64(xp_bits)
    P = xp.shape[1]
    comb = np.zeros((T, P))
    decoded = {}

    def dec(e):
        if e not in decoded:
            if experts["fmt"] == "nvfp4":
                c1, s1, t1 = experts["w1"][e]
                c2, s2, t2 = experts["w2"][e]
                decoded[e] = (nvfp4_decode(c1, s1, t1), nvfp4_decode(c2, s2, t2))
            else:
                decoded[e] = (bf16_to_f64(experts["w1"][e]), bf16_to_f64(experts["w2"][e]))
        return decoded[e]

    inter_q = {}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            w1, w2 = dec(e)
            u = xp[t] @ w1.T
            a = silu(u[:inter]) * u[inter:]
            if experts["fmt"] == "nvfp4":
                codes, scales = fp4_act_quant(a[None, :])
                a_q = nvfp4_decode(codes, scales, 1.0)[0]
                inter_q[(t, j)] = (codes[0], scales[0])
            else:
                a_q = bf16_to_f64(bf16_round(a))
            comb[t] += gate[t, j] * (a_q @ w2.T)
    return bf16_round(comb), inter_q


def usage_top(idx, n_experts: int, n: int = 14):
    """Expert-usage histogram of one step and its n most-used experts ordered by
    (count desc, index asc); experts with count 0 are never listed (the pages'
    speculative prefetch takes the previous step's 14 most-used experts)."""
    hist = np.bincount(np.asarray(idx).reshape(-1), minlength=n_experts).astype(np.int64)
    order = sorted(range(n_experts), key=lambda e: (-hist[e], e))
    top = [e for e in order[:n] if hist[e] > 0]
    return hist, np.array(top, dtype=np.int32)


def qkv_project(h_bits, w_qkv_bits, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """The next layer's query / key / value projection (the launch's last step, and on its own
    the first layer's prologue: the pages' first launch has no earlier launch to produce its
    inputs): qkv = h . W^T in fp64, each part rounded once to bf16.  h bf16 [T][H]; W bf16
    [(Hq + 2 Hkv) d][H], query rows, then key rows, then value rows.  Returns q [T][Hq d] and
    k, v [T][Hkv][d] (bit patterns) and the fp64 products."""
    qkv = bf16_to_f64(h_bits) @ bf16_to_f64(w_qkv_bits).T
    T = qkv.shape[0]
    qd, kd = n_q_heads * head_dim, n_kv_heads * head_dim
    q = bf16_round(qkv[:, :qd])
    k = bf16_round(qkv[:, qd:qd + kd]).reshape(T, n_kv_heads, head_dim)
    v = bf16_round(qkv[:, qd + kd:]).reshape(T, n_kv_heads, head_dim)
    return q, k, v, qkv


def layer_step(inp, experts: dict, anchors: dict | None = None) -> dict:
    """The whole launch.  `inp` is a synth.LayerInputs.  `anchors` may replace a
    stage's input by another implementation's value (stage-local checks): keys
    "attn", "h1", "xp", "idx", "gate", "y", "h_out"."""
    sh = inp.shape
    a = anchors or {}
    T, ctx = sh.T, sh.ctx
    attn, stats = attention(inp.q_in, inp.k_cache, inp.v_cache, inp.parent, ctx, sh.window,
                            sh.n_q_heads, sh.n_kv_heads, sh.head_dim)
    attn_in = a.get("attn", attn)
    h1 = dense(attn_in, inp.w_o, inp.h_in)
    h1_in = a.get("h1", h1)
    xp = dense(h1_in, inp.w_pool)
    xp_in = a.get("xp", xp)
    logits64, z, idx, gate = router(xp_in, inp.w_router, inp.router_bias, sh.top_k)
    idx_in = a.get("idx", idx)
    gate_in = a.get("gate", gate)
    y, inter_q = moe(xp_in, idx_in, gate_in, experts, sh.expert_inter)
    y_in = a.get("y", y)
    h_out = dense(y_in, inp.w_unpool, h1_in)
    h_out_in = a.get("h_out", h_out)
    q_next, k_new, v_new, qkv = qkv_project(h_out_in, inp.w_qkv_next, sh.n_q_heads, sh.n_kv_heads, sh.head_dim)
    k_next = inp.k_cache_next.copy()
    v_next = inp.v_cache_next.copy()
    k_next[ctx:ctx + T] = k_new
    v_next[ctx:ctx + T] = v_new
    hist, top = usage_top(idx, sh.n_experts)
    return dict(attn=attn, stats=stats, h1=h1, xp=xp, logits64=logits64, logits32=z, idx=idx,
                gate=gate, y=y, h_out=h_out, q_next=q_next, k_new=k_new, v_new=v_new,
                k_cache_next=k_next, v_cache_next=v_next, hist=hist, top14=top, inter_q=inter_q,
                qkv64=qkv)


def pack_experts(inp, which=None) -> dict:
    """Experts in the layer's storage format: NVFP4 (packed here by the oracle's own
    packer) or bf16.  `which` limits packing to a set of expert ids (others None)."""
    from .numerics import nvfp4_pack
    sh = inp.shape
    if not sh.nvfp4:
        return {"fmt": "bf16", "w1": inp.w1, "w2": inp.w2}
    E = sh.n_experts
    ids = range(E) if which is None else which
    w1 = [None] * E
    w2 = [None] * E
    for e in ids:
        w1[e] = nvfp4_pack(bf16_to_f64(inp.w1[e]))
        w2[e] = nvfp4_pack(bf16_to_f64(inp.w2[e]))
    return {"fmt": "nvfp4", "w1": w1, "w2": w2}


def used_experts(inp, anchors=None) -> set:
    """The experts the step's routing reaches: attention, o-proj, pooler and router as in
    layer_step (routing does not depend on the experts), with the same anchors."""
    sh = inp.shape
    a = anchors or {}
    attn, _ = attention(inp.q_in, inp.k_cache, inp.v_cache, inp.parent, sh.ctx, sh.window,
                        sh.n_q_heads, sh.n_kv_heads, sh.head_dim)
    h1 = dense(a.get("attn", attn), inp.w_o, inp.h_in)
    xp = dense(a.get("h1", h1), inp.w_pool)
    _, _, idx, _ = router(a.get("xp", xp), inp.w_router, inp.router_bias, sh.top_k)
    return set(np.unique(np.asarray(a.get("idx", idx))).tolist())


def layer_step_auto(inp, anchors=None) -> dict:
    """Layer step that packs only the experts the routing reaches (the full pack of
    256 experts is slow in plain NumPy)."""
    if not inp.shape.nvfp4:
        return layer_step(inp, pack_experts(inp), anchors)
    return layer_step(inp, pack_experts(inp, used_experts(inp, anchors)), anchors)
