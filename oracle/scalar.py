"""Second oracle: the same layer written as pure-Python scalar loops (test
infrastructure only).  It shares no helper with oracle.numerics / oracle.layer --
its own bf16 rounding (exact rational arithmetic), its own E2M1 / E4M3 decoding
from the bit fields, its own NVFP4 requantisation and its own attention -- so that
agreement of the two on small shapes pins both against slips in either.
Only for tiny shapes (it is O(minutes) at real shard sizes)."""
from __future__ import annotations

import math
from fractions import Fraction


def bf16_of(x: float) -> float:
    """Nearest bf16 value to x (ties to even), computed with exact rationals."""
    if x == 0.0 or math.isinf(x) or math.isnan(x):
        return x
    f = Fraction(x)
    a = abs(f)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = abs(f) / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * q)
    return -v if x < 0 else v


def bits_to_float(b: int) -> float:
    """bf16 bit pattern -> value, from the bit fields."""
    s = -1.0 if b & 0x8000 else 1.0
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return s * m * 2.0 ** -133
    return s * (1 + m / 128.0) * 2.0 ** (e - 127)


def e2m1(c: int) -> float:
    s = -1.0 if c & 8 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        return s * 0.5 * m
    return s * (1 + 0.5 * m) * 2.0 ** (e - 1)


def e4m3(b: int) -> float:
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 15
    m = b & 7
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1 + m / 8.0) * 2.0 ** (e - 7)


def _nearest(v: float, grid: list[float]) -> int:
    """Index of the grid value nearest to v (grid increasing, v >= 0); ties -> even index;
    beyond the end -> last index."""
    best = 0
    for i in range(1, len(grid)):
        if abs(grid[i] - v) < abs(grid[best] - v):
            best = i
        elif abs(grid[i] - v) == abs(grid[best] - v) and i % 2 == 0:
            best = i
    return best


def act_quant_dequant(a: list[float]) -> list[float]:
    """NVFP4 (tensor scale 1) round trip of one intermediate row, block size 16.
    Decisions on the values as given, compared exactly (Fractions)."""
    vals = list(a)
    e4 = [e4m3(b) for b in range(127)]
    g2 = [e2m1(c) for c in range(8)]
    out = []
    for b0 in range(0, len(vals), 16):
        blk = vals[b0:b0 + 16]
        amax = max(abs(x) for x in blk)
        si = _nearest_frac(Fraction(amax) / 6, e4)
        s = e4[si]
        for x in blk:
            if s == 0:
                out.append(0.0)
                continue
            ci = _nearest_frac(abs(Fraction(x)) / Fraction(s), g2)
            v = g2[ci] * s
            out.append(-v if (x < 0 and v != 0) else v)
    return out


def _nearest_frac(v: Fraction, grid: list[float]) -> int:
    best = 0
    for i in range(1, len(grid)):
        di, db = abs(Fraction(grid[i]) - v), abs(Fraction(grid[best]) - v)
        if di < db or (di == db and i % 2 == 0):
            best = i
    return best


def nvfp4_weight(codes, scales, ts, n: int, k: int) -> float:
    byte = int(codes[n][k // 2])
    c = (byte >> 4) if (k & 1) else (byte & 15)
    return e2m1(c) * e4m3(int(scales[n][k // 16])) * float(ts)


def layer_step(inp, experts) -> dict:
    """Scalar-loop statement of the layer (same readings as oracle.layer)."""
    sh = inp.shape
    T, ctx, W = sh.T, sh.ctx, sh.window
    H, Hq, Hkv, d, P, E, k, I = (sh.hidden, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.pooled,
                                 sh.n_experts, sh.top_k, sh.expert_inter)
    G = Hq // Hkv
    par = [int(p) for p in inp.parent]
    # ancestors by walking parents; depth by counting steps
    anc = []
    depth = []
    for i in range(T):
        s, j, dpt = set(), i, 0
        while j >= 0:
            s.add(j)
            j = par[j]
            dpt += 1
        anc.append(s)
        depth.append(dpt - 1)
    bf = bits_to_float
    attn = [[0.0] * (Hq * d) for _ in range(T)]
    stats = [[(0.0, 0.0)] * Hq for _ in range(T)]
    for i in range(T):
        pos = ctx + depth[i]
        keys = [p for p in range(ctx) if (W == 0 or pos - p < W)] + [ctx + j for j in sorted(anc[i])]
        for h in range(Hq):
            g = h // G
            sc = []
            for r in keys:
                acc = 0.0
                for c in range(d):
                    acc += bf(int(inp.q_in[i][h * d + c])) * bf(int(inp.k_cache[r][g][c]))
                sc.append(acc / math.sqrt(d))
            m = max(sc)
            ws = [math.exp(s - m) for s in sc]
            l = sum(ws)
            for c in range(d):
                acc = 0.0
                for w_, r in zip(ws, keys):
                    acc += w_ * bf(int(inp.v_cache[r][g][c]))
                attn[i][h * d + c] = bf16_of(acc / l)
            stats[i][h] = (m, l)

    def lin(x, w, n_out, n_in, res=None):
        out = []
        for t in range(len(x)):
            row = []
            for n in range(n_out):
                acc = 0.0
                for c in range(n_in):
                    acc += x[t][c] * bf(int(w[n][c]))
                if res is not None:
                    acc += res[t][n]
                row.append(acc)
            out.append(row)
        return out

    h_in = [[bf(int(v)) for v in row] for row in inp.h_in]
    h1 = [[bf16_of(v) for v in row] for row in lin(attn, inp.w_o, H, Hq * d, h_in)]
    xp = [[bf16_of(v) for v in row] for row in lin(h1, inp.w_pool, P, H)]
    import numpy as _np  # only for fp32 rounding of the logits, as the kernel holds them
    logits = lin(xp, inp.w_router, E, P)
    idx, gate = [], []
    for t in range(T):
        z = [float(_np.float32(v)) for v in logits[t]]
        if inp.router_bias is not None:
            z = [float(_np.float32(_np.float32(z[e]) + _np.float32(inp.router_bias[t][e]))) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-z[e], e))[:k]
        mx = max(z[e] for e in order)
        ex = [math.exp(z[e] - mx) for e in order]
        sm = sum(ex)
        idx.append(order)
        gate.append([v / sm for v in ex])
    y = []
    for t in range(T):
        comb = [0.0] * P
        for j in range(k):
            e = idx[t][j]
            if experts["fmt"] == "nvfp4":
                c1, s1, t1 = experts["w1"][e]
                c2, s2, t2 = experts["w2"][e]
                w1 = lambda n, c: nvfp4_weight(c1, s1, t1, n, c)
                w2 = lambda n, c: nvfp4_weight(c2, s2, t2, n, c)
            else:
                w1 = lambda n, c: bf(int(experts["w1"][e][n][c]))
                w2 = lambda n, c: bf(int(experts["w2"][e][n][c]))
            u = [sum(xp[t][c] * w1(n, c) for c in range(P)) for n in range(2 * I)]
            a = [(u[n] / (1 + math.exp(-u[n]))) * u[I + n] for n in range(I)]
            aq = act_quant_dequant(a) if experts["fmt"] == "nvfp4" else [bf16_of(v) for v in a]
            for n in range(P):
                comb[n] += gate[t][j] * sum(aq[c] * w2(n, c) for c in range(I))
        y.append([bf16_of(v) for v in comb])
    h_out = [[bf16_of(v) for v in row] for row in lin(y, inp.w_unpool, H, P, h1)]
    qkv = lin(h_out, inp.w_qkv_next, (Hq + 2 * Hkv) * d, H)
    q_next = [[bf16_of(v) for v in row[:Hq * d]] for row in qkv]
    k_new = [[bf16_of(v) for v in row[Hq * d:(Hq + Hkv) * d]] for row in qkv]
    v_new = [[bf16_of(v) for v in row[(Hq + Hkv) * d:]] for row in qkv]
    return dict(attn=attn, stats=stats, h1=h1, xp=xp, idx=idx, gate=gate, y=y, h_out=h_out,
                q_next=q_next, k_new=k_new, v_new=v_new)
