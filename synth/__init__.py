"""Seeded synthetic inputs for the fused decode-layer step.

This module is shared by the CPU oracle and by the GPU tests / benchmark.  It
holds workload shapes and random draws only -- none of the layer's arithmetic:
no attention, projections, routing, codec or rounding of intermediate values.
The one numeric conversion here, turning a random fp32 draw into a bf16 bit
pattern, is how an input tensor is *stored*; both sides receive the same bits.

The pages (LMSYS "Muse Spark Open" megakernel write-ups) measure one GSM8K
request at batch one with a 16-token verification tree and ~49 distinct experts
per layer.  Neither the dataset nor the trained weights exist here, so every
tensor below is drawn from seeded generators with the shapes of one GPU's share
of a layer: N(0, 0.02) weights, N(0, 1) activations and KV rows, a seeded
depth-6 tree, and (for the routing-locality workloads) an injected router bias.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# tensor ids for np.random.default_rng([base, layer, tensor_id, expert])
T_HIN, T_QIN, T_KCTX, T_VCTX, T_KTREE, T_VTREE = 0, 1, 2, 3, 4, 5
T_WO, T_WP, T_WR, T_WU, T_WQKV = 10, 11, 12, 13, 14
T_WQKV0 = 15        # layer 0's own qkv projection (the embedding prologue of a stack)
T_W1, T_W2 = 20, 21
T_TREE, T_BIAS, T_MARKOV, T_KNEXT = 30, 31, 32, 33
T_W2SHARD, T_PEER_CODES, T_PEER_SCALES, T_PEER_Y = 40, 41, 42, 43


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One GPU's share of one decoder layer (names follow the pages' vocabulary)."""
    name: str
    hidden: int          # H
    n_q_heads: int       # Hq
    n_kv_heads: int      # Hkv
    head_dim: int        # d
    pooled: int          # P, pooler output width
    n_experts: int       # E
    top_k: int           # k
    expert_inter: int    # I, local expert intermediate width
    window: int          # sliding window length, 0 = global attention
    ctx: int             # KV rows cached before the tree
    T: int               # tree nodes verified this step
    nvfp4: bool          # experts stored as NVFP4 (else bf16)
    routing: str = "weights"   # "weights" | "zipf" | "markov"
    zipf_s: float = 1.41

    @property
    def kv_capacity(self) -> int:
        return self.ctx + 16

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


# The five workloads.  Shapes: one tiny all-bf16 layer, then one GPU's 1/8 shard of
# the model described on the pages (8 of 64 q heads, 1 of 8 kv heads, 1/8 of the
# 1536-wide expert intermediate).
CFG1 = LayerShape("tiny-global-bf16", 256, 4, 1, 64, 128, 16, 2, 128, 0, 128, 1, False)
CFG2 = LayerShape("swa2048-ctx8192-nvfp4", 4096, 8, 1, 128, 2048, 256, 8, 192, 2048, 8192, 16, True)
CFG3 = LayerShape("global-ctx32768-zipf49", 4096, 8, 1, 128, 2048, 256, 8, 192, 0, 32768, 16, True, "zipf")
CFG4 = LayerShape("stack62-ctx4096", 4096, 8, 1, 128, 2048, 256, 8, 192, 2048, 4096, 16, True)
CFG5 = LayerShape("stack62-ctx4096-markov80", 4096, 8, 1, 128, 2048, 256, 8, 192, 2048, 4096, 16, True, "markov")
CONFIGS = {1: CFG1, 2: CFG2, 3: CFG3, 4: CFG4, 5: CFG5}


def base_seed(cfg_id: int) -> int:
    return 20261105 + cfg_id


def rng(base: int, layer: int, tensor_id: int, expert: int = 0, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([base, layer, tensor_id, expert, step])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Storage conversion of an fp32 draw to a bf16 bit pattern (round to nearest even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)  # finite draws only: no NaN / overflow handling needed


def normal_bf16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return bf16_bits_from_f32(x)


def tree_parents(T: int, seed_rng: np.random.Generator) -> np.ndarray:
    """Seeded verification tree: node 0 is the root (the last accepted token); nodes
    1..6 form a chain so the depth is 6; every later node picks a uniformly random
    earlier node of depth <= 5 as its parent.  parent[i] < i always."""
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int32)
    for i in range(1, T):
        if i <= 6:
            p = i - 1
        else:
            cand = [j for j in range(i) if depth[j] <= 5]
            p = cand[int(seed_rng.integers(len(cand)))]
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def zipf_router_bias(shape: LayerShape, g: np.random.Generator, s: float, margin: float = 8.0) -> np.ndarray:
    """Per token, 8 distinct experts drawn by Gumbel-top-k over Zipf(s) weights on a
    random permutation of expert ids; the chosen experts get +margin.  The margin is
    far above any rounding difference, so the routing is unambiguous by construction."""
    E, k, T = shape.n_experts, shape.top_k, shape.T
    perm = g.permutation(E)
    logw = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    bias = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        gum = logw - np.log(-np.log(g.random(E)))
        pick = np.argsort(-gum, kind="stable")[:k]
        bias[t, perm[pick]] = margin
    return bias


def markov_router_bias(shape: LayerShape, g: np.random.Generator, prev_idx: np.ndarray | None,
                       reuse: float, s: float = 1.41, margin: float = 8.0) -> np.ndarray:
    """Routing-locality stand-in: each (token, slot) reuses, with probability `reuse`,
    an expert from the previous step's multiset (count-weighted, no repeat within a
    token); otherwise it draws a fresh Zipf expert."""
    E, k, T = shape.n_experts, shape.top_k, shape.T
    if prev_idx is None:
        return zipf_router_bias(shape, g, s, margin)
    counts = np.bincount(prev_idx.reshape(-1), minlength=E).astype(np.float64)
    logw = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    zw = np.exp(logw - logw.max())
    zw /= zw.sum()
    perm = g.permutation(E)
    bias = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        chosen: list[int] = []
        while len(chosen) < k:
            if g.random() < reuse and counts.sum() > 0:
                w = counts.copy()
                w[chosen] = 0
                if w.sum() == 0:
                    continue
                e = int(g.choice(E, p=w / w.sum()))
            else:
                e = int(perm[g.choice(E, p=zw)])
            if e not in chosen:
                chosen.append(e)
        bias[t, chosen] = margin
    return bias


@dataclasses.dataclass
class LayerInputs:
    """Everything one layer step consumes, as host arrays (bf16 as uint16 bits)."""
    shape: LayerShape
    parent: np.ndarray          # int32 [T]
    h_in: np.ndarray            # bf16 [T][H]
    q_in: np.ndarray            # bf16 [T][Hq*d]
    k_cache: np.ndarray         # bf16 [cap][Hkv][d], rows [0, ctx+T) valid
    v_cache: np.ndarray
    k_cache_next: np.ndarray    # next layer's cache before the step (arbitrary contents)
    v_cache_next: np.ndarray
    w_o: np.ndarray             # bf16 [H][Hq*d]
    w_pool: np.ndarray          # bf16 [P][H]
    w_router: np.ndarray        # bf16 [E][P]
    w_unpool: np.ndarray        # bf16 [H][P]
    w_qkv_next: np.ndarray      # bf16 [(Hq+2Hkv)d][H]
    w1: np.ndarray              # bf16 [E][2I][P]  (master weights; NVFP4 layers pack them)
    w2: np.ndarray              # bf16 [E][P][I]
    router_bias: np.ndarray | None  # fp32 [T][E] or None


def make_layer_inputs(shape: LayerShape, cfg_id: int, layer: int = 0, step: int = 0,
                      prev_idx: np.ndarray | None = None, reuse: float = 0.8) -> LayerInputs:
    b = base_seed(cfg_id)
    H, Hq, Hkv, d, P, E, I, T = (shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                                 shape.pooled, shape.n_experts, shape.expert_inter, shape.T)
    cap, ctx = shape.kv_capacity, shape.ctx
    parent = tree_parents(T, rng(b, layer, T_TREE, 0, step)) if T > 1 else np.array([-1], np.int32)
    h_in = normal_bf16(rng(b, layer, T_HIN, 0, step), (T, H), 1.0)
    q_in = normal_bf16(rng(b, layer, T_QIN, 0, step), (T, Hq * d), 1.0)
    k_cache = np.zeros((cap, Hkv, d), np.uint16)
    v_cache = np.zeros((cap, Hkv, d), np.uint16)
    k_cache[:ctx] = normal_bf16(rng(b, layer, T_KCTX), (ctx, Hkv, d), 1.0)
    v_cache[:ctx] = normal_bf16(rng(b, layer, T_VCTX), (ctx, Hkv, d), 1.0)
    k_cache[ctx:ctx + T] = normal_bf16(rng(b, layer, T_KTREE, 0, step), (T, Hkv, d), 1.0)
    v_cache[ctx:ctx + T] = normal_bf16(rng(b, layer, T_VTREE, 0, step), (T, Hkv, d), 1.0)
    kn = normal_bf16(rng(b, layer + 1, T_KNEXT, 0), (2, cap, Hkv, d), 1.0)
    w = lambda tid, shp, e=0: normal_bf16(rng(b, layer, tid, e), shp, 0.02)
    w1 = np.stack([w(T_W1, (2 * I, P), e) for e in range(E)])
    w2 = np.stack([w(T_W2, (P, I), e) for e in range(E)])
    bias = None
    if shape.routing == "zipf":
        bias = zipf_router_bias(shape, rng(b, layer, T_BIAS, 0, step), shape.zipf_s)
    elif shape.routing == "markov":
        bias = markov_router_bias(shape, rng(b, layer, T_MARKOV, 0, step), prev_idx, reuse, shape.zipf_s)
    return LayerInputs(shape, parent, h_in, q_in, k_cache, v_cache, kn[0].copy(), kn[1].copy(),
                       w(T_WO, (H, Hq * d)), w(T_WP, (P, H)), w(T_WR, (E, P)), w(T_WU, (H, P)),
                       w(T_WQKV, (shape.qkv_out, H)), w1, w2, bias)


# ---------------------------------------------------------------- device-side draws (stacks)
#
# A 62-layer stack holds ~14 GB of weights; drawing them with NumPy would take minutes, so
# the stack workloads draw on the device with torch's counter-based CUDA generator, seeded per
# (workload, layer, tensor).  The same bits are then copied to the host wherever the oracle
# needs them, so both sides still consume identical inputs.

def _torch_gen(device, base: int, layer: int, tensor_id: int, step: int = 0):
    import torch
    g = torch.Generator(device=device)
    seed = int(np.random.SeedSequence([base, layer, tensor_id, step]).generate_state(1, np.uint64)[0])
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def device_normal_bf16(shape, std: float, device, base: int, layer: int, tensor_id: int, step: int = 0):
    """N(0, std) draw stored as bf16 (torch tensor, bfloat16, round to nearest even)."""
    import torch
    g = _torch_gen(device, base, layer, tensor_id, step)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return x.to(torch.bfloat16)


def device_layer_weights(shape: LayerShape, cfg_id: int, layer: int, device) -> dict:
    """One layer's weights drawn on the device (bf16 torch tensors): the dense matrices and
    the expert masters w1 [E][2I][P], w2 [E][P][I] (NVFP4 layers pack these)."""
    b = base_seed(cfg_id)
    H, Hq, d, P, E, I = shape.hidden, shape.n_q_heads, shape.head_dim, shape.pooled, shape.n_experts, shape.expert_inter
    w = lambda tid, shp: device_normal_bf16(shp, 0.02, device, b, layer, tid)
    return dict(w_o=w(T_WO, (H, Hq * d)), w_pool=w(T_WP, (P, H)), w_router=w(T_WR, (E, P)),
                w_unpool=w(T_WU, (H, P)), w_qkv_next=w(T_WQKV, (shape.qkv_out, H)),
                w1=w(T_W1, (E, 2 * I, P)), w2=w(T_W2, (E, P, I)))


def device_first_qkv_weight(shape: LayerShape, cfg_id: int, device):
    """Layer 0's own qkv projection [qkv_out][H] bf16, drawn on the device: what a stack's
    prologue applies to the step tokens' embeddings."""
    return device_normal_bf16((shape.qkv_out, shape.hidden), 0.02, device, base_seed(cfg_id), 0, T_WQKV0)


def device_kv_context(shape: LayerShape, cfg_id: int, layer: int, device):
    """A layer's KV cache [cap][Hkv][d] bf16 with rows [0, ctx) drawn N(0, 1), the rest zero."""
    import torch
    b = base_seed(cfg_id)
    cap, ctx, Hkv, d = shape.kv_capacity, shape.ctx, shape.n_kv_heads, shape.head_dim
    k = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.zeros((cap, Hkv, d), dtype=torch.bfloat16, device=device)
    k[:ctx] = device_normal_bf16((ctx, Hkv, d), 1.0, device, b, layer, T_KCTX)
    v[:ctx] = device_normal_bf16((ctx, Hkv, d), 1.0, device, b, layer, T_VCTX)
    return k, v


def stack_step_inputs(shape: LayerShape, cfg_id: int, step: int) -> dict:
    """Per-step host inputs of a stack: the tree, layer 0's residual and queries, and layer
    0's own tree K/V rows (what the step's first launch consumes)."""
    b = base_seed(cfg_id)
    H, Hq, Hkv, d, T = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.T
    return dict(parent=tree_parents(T, rng(b, 0, T_TREE, 0, step)),
                h_in=normal_bf16(rng(b, 0, T_HIN, 0, step), (T, H), 1.0),
                q_in=normal_bf16(rng(b, 0, T_QIN, 0, step), (T, Hq * d), 1.0),
                k_tree=normal_bf16(rng(b, 0, T_KTREE, 0, step), (T, Hkv, d), 1.0),
                v_tree=normal_bf16(rng(b, 0, T_VTREE, 0, step), (T, Hkv, d), 1.0))


def stack_router_biases(shape: LayerShape, cfg_id: int, n_layers: int, n_steps: int, reuse: float) -> np.ndarray:
    """Router biases [steps][layers][T][E] of the routing-locality workload: per layer a
    Markov chain over steps where each (token, slot) reuses the previous step's experts with
    probability `reuse` (the bias margin fixes the routing, so the chain is known in advance)."""
    b = base_seed(cfg_id)
    out = np.zeros((n_steps, n_layers, shape.T, shape.n_experts), np.float32)
    for L in range(n_layers):
        prev = None
        for s in range(n_steps):
            bias = markov_router_bias(shape, rng(b, L, T_MARKOV, 0, s), prev, reuse, shape.zipf_s)
            out[s, L] = bias
            prev = np.stack([np.flatnonzero(bias[t]) for t in range(shape.T)])
    return out


# ---------------------------------------------------------------- N-sharded expert layout

def nshard_inputs(shape: LayerShape, cfg_id: int, R: int, r: int) -> dict:
    """What rank r of R needs beyond the layer's inputs in the N-sharded expert layout, drawn
    at random: its rows of the full down projections, w2_shard bf16 [E][P/R][R I] (N(0, 0.02)
    like every weight); what the other ranks deliver -- the gathered intermediate rows as
    NVFP4 codes uint8 [T k][R I / 2] (any byte) and E4M3 scale bytes [T k][R I / 16] (0x10 ..
    0x30: 2^-5 .. 2^-1, so that decoded values stay below 3, near the size of a real
    intermediate), and y columns bf16 [T][P] (N(0, 0.1)).  Rank r's own parts of the last two
    are filled in by whoever computes them; their draws here are discarded."""
    b = base_seed(cfg_id)
    P, E, I, T, k = shape.pooled, shape.n_experts, shape.expert_inter, shape.T, shape.top_k
    w2 = np.stack([normal_bf16(rng(b, r, T_W2SHARD, e), (P // R, R * I), 0.02) for e in range(E)])
    g = rng(b, r, T_PEER_CODES, 0)
    codes = g.integers(0, 256, (T * k, R * I // 2), dtype=np.uint8)
    scales = rng(b, r, T_PEER_SCALES, 0).integers(0x10, 0x31, (T * k, R * I // 16), dtype=np.uint8)
    y = normal_bf16(rng(b, r, T_PEER_Y, 0), (T, P), 0.1)
    return dict(w2_shard=w2, peer_codes=codes, peer_scales=scales, peer_y=y)
