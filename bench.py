#!/usr/bin/env python3
"""Benchmark of the fused decode-layer step on one MI355X.

One "step" is one launch of mk_layer_step: a whole decoder layer (16-token tree verify) of
the sliding-window-2048 layer at one GPU's shard shape over a KV context of 8192 rows, NVFP4
experts -- the workload the headline metric is quoted on.  Inputs are seeded synthetic
tensors already resident in HBM.  To keep the 256 MB MALL from serving a layer's weights
from an earlier launch, launches rotate over R full replicas of weights, KV and step inputs
(R * ~120 MB read per launch between two uses of a replica).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0           # dense bf16 / fp16 matrix-core peak
HERE = os.path.dirname(os.path.abspath(__file__))
# sources that decide what the layer kernel reads and writes
KERNEL_SOURCES = ["layer_persistent_amd/csrc/mk_layer.hip", "layer_persistent_amd/csrc/mk_device.h",
                  "layer_persistent_amd/csrc/mk_internal.h", "layer_persistent_amd/csrc/mk_api.hip"]
COPY_CALIB_ELEMS = 1 << 26          # fp32 elements of the copy-calibration kernel (256 MiB each way)


# timestamp events the layer kernel records (index, name): phase ends, hand-off ends, and the
# points inside the routing and expert phases
PHASE_EVENTS = [(1, "setup"), (2, "attn_work"), (3, "attn_handoff"), (61, "merge_loaded"),
                (63, "merge_reduced"), (4, "merge_work"), (5, "oproj_weights_issued"),
                (6, "oproj_work"), (7, "oproj_handoff"), (8, "pool_work"), (9, "pool_handoff"), (10, "router_work"),
                (11, "xs_built"), (51, "route_logits_in"), (52, "route_published"), (46, "route_in"),
                (18, "route_tables"),
                (49, "gemm1_first_loads"), (45, "gemm1_round1"), (12, "gemm1_work"), (13, "w2_first_issued"),
                (42, "gemm2_staged"), (48, "gemm2_batch0"), (43, "gemm2_experts"), (14, "gemm2_work"),
                (15, "gemm2_handoff"), (16, "unpool_work"), (17, "qkv_weights_issued"), (19, "qkv_end")]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload: str):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counters (copy-kernel
    calibrated), read from the committed counter summary -- but only if that summary was taken
    on the current kernel sources; otherwise None."""
    path = os.path.join(HERE, "profiles", f"layer_kernel_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not tb or sha.group(1) != kernel_source_sha():
        return None
    return int(tb.group(1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(shape, n_active: int) -> dict:
    """Compulsory HBM bytes of one layer launch: weights read once, KV rows the tree can see,
    the step's activations in and out, the KV rows written."""
    H, Hq, Hkv, d, P, E, I, T = (shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                                 shape.pooled, shape.n_experts, shape.expert_inter, shape.T)
    lo = max(0, shape.ctx - shape.window + 1) if shape.window > 0 else 0
    kv = (shape.ctx - lo + T) * Hkv * d * 2 * 2
    dense = 2 * (H * Hq * d + P * H + E * P + H * P + shape.qkv_out * H)
    if shape.nvfp4:     # codes and E4M3 block scales of W1 [2I][P] and W2 [P][I]
        per_expert = (2 * I * P // 2 + 2 * I * P // 16) + (P * I // 2 + P * I // 16)
    else:               # bf16 W1 and W2
        per_expert = 2 * (2 * I * P + P * I)
    experts = n_active * per_expert
    acts = T * (2 * H + 2 * Hq * d) * 2
    kv_write = T * 2 * Hkv * d * 2
    return dict(kv=kv, dense=dense, experts=experts, per_expert=per_expert, acts=acts, kv_write=kv_write,
                total=kv + dense + experts + acts + kv_write)


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def batch_bytes(shape, n_active: int, B: int) -> int:
    """Compulsory bytes of a launch of B sequences: the weights and the active experts once,
    each sequence's visible KV rows, activations and KV writes."""
    ab = algorithmic_bytes(shape, n_active)
    return ab["dense"] + ab["experts"] + B * (ab["kv"] + ab["acts"] + ab["kv_write"])


def cpu_baseline(inputs: dict, reps: int = 3) -> dict:
    """The oracle (fp64 NumPy) on the host: full layer steps of the single-layer workloads,
    each timed `reps` times with BLAS limited to one thread and with every thread it has, the
    median reported.  Expert packing is weight preparation (the GPU side does it with
    mk_nvfp4_pack outside the timed region) and is done once per workload, untimed.  `inputs`
    maps a workload id to its inputs; the first one is the headline workload."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    all_threads = _blas_threads()
    runs = []
    for cfg, inp in inputs.items():
        t0 = time.time()
        ex = oracle.pack_experts(inp, oracle.used_experts(inp))
        prep = time.time() - t0
        for threads in (1, all_threads):
            ts = []
            with threadpool_limits(limits=threads):
                for _ in range(reps):
                    t1 = time.perf_counter()
                    oracle.layer_step(inp, ex)
                    ts.append(time.perf_counter() - t1)
            runs.append({"workload": inp.shape.name, "blas_threads": threads, "median_us": round(float(np.median(ts)) * 1e6, 1),
                         "all_us": [round(t * 1e6, 1) for t in ts]})
            log(f"cpu baseline: {inp.shape.name}, {threads} BLAS thread(s): oracle layer step median "
                f"{np.median(ts) * 1e3:.1f} ms of {reps} (prep {prep:.1f} s)")
    head = [r for r in runs if r["workload"] == next(iter(inputs.values())).shape.name]
    best = min(head, key=lambda r: r["median_us"])
    return {"value": best["median_us"], "unit": "us", "cores": int(best["blas_threads"]), "kind": "oracle",
            "sample": f"one full layer step of each of {', '.join(i.shape.name for i in inputs.values())}, "
                      f"fp64 NumPy, median of {reps}, with BLAS at 1 thread and at all {all_threads}; value = the "
                      f"headline workload's faster median; expert packing excluded; {cores} host cores visible",
            "runs": runs}


def algorithmic_flops(shape, parent) -> dict:
    """Multiply-add work of one layer launch (2 flops each): the dense projections at T rows,
    attention over the keys each (token, head) can see, and the experts' two GEMMs per routed
    (token, slot) pair.  All of it runs on the matrix cores (bf16, and fp16 for the experts)."""
    H, Hq, Hkv, d, P, E, I, T = (shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                                 shape.pooled, shape.n_experts, shape.expert_inter, shape.T)
    dense = 2 * T * (H * Hq * d + P * H + E * P + H * P + shape.qkv_out * H)
    depth = np.zeros(T, np.int64)
    for t in range(1, T):
        depth[t] = depth[parent[t]] + 1
    keys = 0
    for t in range(T):
        pos = shape.ctx + int(depth[t])
        lo = max(0, pos - shape.window + 1) if shape.window > 0 else 0
        keys += (shape.ctx - min(lo, shape.ctx)) + int(depth[t]) + 1
    attn = 2 * 2 * d * Hq * keys
    experts = T * shape.top_k * (2 * 2 * I * P + 2 * P * I)
    return dict(dense=dense, attn=attn, experts=experts, total=dense + attn + experts)


def stream_read_gbs(torch, lib_mod, stream) -> dict:
    """Read rate of the library's plain streaming-read kernel (mk_stream_read) over 2 GiB that
    no other work touches, for a few grid sizes; best of 5 timed passes per size.  `stream` is
    the torch stream object (events record on it; the library takes its handle)."""
    nbytes = 2 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(0x01020304)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for blocks in (1024, 2048, 4096, 8192):
        lib_mod.mk_stream_read(buf, nbytes, blocks, sink, stream.cuda_stream)
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib_mod.mk_stream_read(buf, nbytes, blocks, sink, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0
            best = us if best is None else min(best, us)
        out[blocks] = round(nbytes / (best * 1e-6) / 1e9, 1)
    del buf
    return out


def stack_bytes(shape, n_active_per_layer) -> int:
    """Algorithmic bytes of one verify step of the stack: every layer's dense weights, its
    active experts, the KV rows it can see (global every fourth layer), activations."""
    import dataclasses
    from layer_persistent_amd.stack import is_global
    tot = 0
    for L, na in enumerate(n_active_per_layer):
        lsh = dataclasses.replace(shape, window=0 if is_global(L) else shape.window)
        ab = algorithmic_bytes(lsh, na)
        if L + 1 == len(n_active_per_layer):        # the last layer has no next-layer projection
            ab["total"] -= 2 * shape.qkv_out * shape.hidden + ab["kv_write"]
        tot += ab["total"]
    return tot


def bench_stack(args) -> dict:
    """Configs 4 and 5: a stack of fused layers (62 by default), one launch per layer per
    verify step; per-step time is the median over the timed steps (each step is a new tree,
    residual and layer-0 queries); config 5 adds Markov routing (expert reuse between steps)
    and the speculative expert prefetch."""
    import torch
    import synth
    from layer_persistent_amd.stack import Stack, is_global
    shape = synth.CONFIGS[args.config]
    n_layers = args.layers
    t0 = time.time()
    stk = Stack(shape, args.config, n_layers)
    log(f"stack of {n_layers} layers built in {time.time() - t0:.1f} s "
        f"({sum(l.w.nbytes() for l in stk.layers) / 1e9:.2f} GB of weights)")
    n_steps = args.warmup + args.steps
    ins = [synth.stack_step_inputs(shape, args.config, s) for s in range(n_steps)]
    if args.config == 5:
        return bench_reuse(args, stk, ins)
    # the step as given (layer 0's queries and tree K/V rows supplied), and the step from the
    # tokens' embeddings with the first-layer prologue in front of layer 0
    variants = [("stack", None, False, False), ("stack_from_embeddings", None, False, True),
                ("decode_step", None, False, True)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    res = {}
    n_active = None
    for name, biases, pf, prologue in variants:
        if prologue and stk.w_qkv0 is None:
            stk.w_qkv0 = synth.device_first_qkv_weight(shape, args.config, "cuda").view(torch.int16)
        stk.prologue = prologue
        structs = [stk.structs(pf, biases is not None, parity) for parity in (0, 1)]
        # the whole decode step: prologue, layers, then greedy acceptance and the KV commit of the
        # accepted path in every layer.  The target tokens would come from an LM head (outside
        # this library); synthetic ones accept the tree's chain of depth 6 (7 nodes).
        accept = None
        if name == "decode_step":
            T = shape.T
            draft = torch.arange(100, 100 + T, dtype=torch.int32, device="cuda")
            target = torch.full((T,), 999, dtype=torch.int32, device="cuda")
            target[:6] = draft[1:7]
            accept = (draft, target)
        step_us, layer_us = [], []
        for s in range(n_steps):
            stk.set_step_inputs(ins[s], None if biases is None else biases[s])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            stk.launch_step(structs[s % 2], sp, accept)
            e1.record(stream)
            torch.cuda.synchronize()
            if s >= args.warmup:
                step_us.append(e0.elapsed_time(e1) * 1000.0)
        # per-layer split: the same steps again with an event after every launch (the records
        # add ~3 us per launch of their own)
        for s in range(args.warmup, n_steps):
            stk.set_step_inputs(ins[s], None if biases is None else biases[s])
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_layers + 1)]
            st = structs[s % 2]
            if stk.prologue:
                stk.launch_step([], sp)          # the prologue alone, outside the per-layer split
            ev[0].record(stream)
            for L in range(n_layers):
                c, w, io = st[L]
                rc = stk.lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io), sp)
                if rc != 0:
                    raise RuntimeError(f"mk_layer_step: {rc}")
                ev[L + 1].record(stream)
            torch.cuda.synchronize()
            layer_us.append([ev[L].elapsed_time(ev[L + 1]) * 1000.0 for L in range(n_layers)])
        # the same steps with each step's launches replayed as one HIP graph (one graph per
        # prefetch-list parity); the last step's output must equal its eager launches bit for bit
        graph_us = []
        if not args.no_graph:
            graphs = [stk.capture_step(structs[parity], accept) for parity in (0, 1)]
            for s in range(n_steps):
                stk.set_step_inputs(ins[s], None if biases is None else biases[s])
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                graphs[s % 2].replay()
                e1.record(stream)
                torch.cuda.synchronize()
                if s >= args.warmup:
                    graph_us.append(e0.elapsed_time(e1) * 1000.0)
            h_graph = stk.h_out().clone()
            s = n_steps - 1
            stk.set_step_inputs(ins[s], None if biases is None else biases[s])
            stk.launch_step(structs[s % 2], sp, accept)
            torch.cuda.synchronize()
            if not torch.equal(h_graph, stk.h_out()):
                raise RuntimeError("stack graph replay differs from the eager launches")
            del graphs
        st0 = mk_read_status_ok(stk)
        lu = np.array(layer_us)
        glob = [L for L in range(n_layers) if is_global(L)]
        swa = [L for L in range(n_layers) if not is_global(L)]
        if accept is not None and int(stk.n_path.item()) != 7:
            raise RuntimeError(f"decode step accepted {int(stk.n_path.item())} nodes, expected the chain of 7")
        if n_active is None:
            n_active = [int(len(torch.unique(l.topk_idx))) for l in stk.layers]
        res[name] = dict(step_us_median=round(float(np.median(step_us)), 1),
                         step_us_p10=round(float(np.percentile(step_us, 10)), 1),
                         step_us_p90=round(float(np.percentile(step_us, 90)), 1),
                         layer_us_mean=round(float(np.median(step_us)) / n_layers, 2),
                         layer_us_evented_mean=round(float(lu.mean()), 2),
                         swa_layer_us_mean=round(float(lu[:, swa].mean()), 2),
                         global_layer_us_mean=round(float(lu[:, glob].mean()), 2) if glob else None,
                         last_layer_us_mean=round(float(lu[:, -1].mean()), 2), status=st0,
                         graph_step_us_median=round(float(np.median(graph_us)), 1) if graph_us else None)
        log(f"{name}: step median {res[name]['step_us_median']} us, layer mean {res[name]['layer_us_mean']} us "
            f"(SWA {res[name]['swa_layer_us_mean']}, global {res[name]['global_layer_us_mean']}); "
            f"replayed as one graph: step median {res[name]['graph_step_us_median']} us")
    return dict(results=res, n_active_last_step=n_active, n_layers=n_layers)


def routing_stats(stk) -> dict:
    """Distinct experts and the largest number of (token, slot) pairs on one expert, per layer,
    from the topk_idx every launch of the last step wrote."""
    import torch
    n_act, max_pairs = [], []
    for lay in stk.layers:
        idx = lay.topk_idx.reshape(-1).to(torch.int64)
        cnt = torch.bincount(idx, minlength=stk.shape.n_experts)
        n_act.append(int((cnt > 0).sum()))
        max_pairs.append(int(cnt.max()))
    return dict(n_active_mean=round(float(np.mean(n_act)), 2), n_active_min=int(min(n_act)),
                n_active_max=int(max(n_act)), max_pairs_mean=round(float(np.mean(max_pairs)), 2),
                max_pairs_max=int(max(max_pairs))), n_act


def bench_reuse(args, stk, ins) -> dict:
    """Config 5: the stack under Markov routing (each (token, slot) keeps the previous step's
    expert with probability 0.8, or 0) with and without the speculative expert prefetch.  The
    four variants run in blocks of warmup + steps verify steps, in the order A B C D D C B A,
    args.abba rounds of it, so that a drift over the run (clocks, caches, memory placement)
    weighs on every variant alike; each block reports its median step and the routing it saw."""
    import torch
    import synth
    shape, n_layers = stk.shape, stk.n_layers
    n_steps = args.warmup + args.steps
    biases = {r: synth.stack_router_biases(shape, args.config, n_layers, n_steps, r) for r in (0.8, 0.0)}
    variants = [("reuse80_noprefetch", 0.8, False), ("reuse80_prefetch", 0.8, True),
                ("reuse0_noprefetch", 0.0, False), ("reuse0_prefetch", 0.0, True)]
    structs = {n: [stk.structs(pf, True, parity) for parity in (0, 1)] for n, _, pf in variants}
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    steps = {n: [] for n, _, _ in variants}
    blocks = {n: [] for n, _, _ in variants}
    routing, per_layer = {}, {}
    order = (variants + variants[::-1]) * args.abba
    for name, reuse, _ in order:
        b = biases[reuse]
        times = []
        for s in range(n_steps):
            stk.set_step_inputs(ins[s], b[s])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            stk.launch_step(structs[name][s % 2], sp)
            e1.record(stream)
            torch.cuda.synchronize()
            if s >= args.warmup:
                times.append(e0.elapsed_time(e1) * 1000.0)
        mk_read_status_ok(stk)
        steps[name] += times
        blocks[name].append(round(float(np.median(times)), 1))
        routing[name], per_layer[name] = routing_stats(stk)
        log(f"{name}: block median {blocks[name][-1]} us; routing {routing[name]}")
    res = {}
    for name, _, _ in variants:
        res[name] = dict(step_us_median=round(float(np.median(steps[name])), 1),
                         step_us_p10=round(float(np.percentile(steps[name], 10)), 1),
                         step_us_p90=round(float(np.percentile(steps[name], 90)), 1),
                         layer_us_mean=round(float(np.median(steps[name])) / n_layers, 2),
                         block_medians_us=blocks[name], **routing[name])
    # the prefetch's effect, block by block: the two blocks of one ABBA round sit symmetrically
    # around its middle, so their mean difference cancels a linear drift
    for r in ("reuse80", "reuse0"):
        d = np.array(blocks[f"{r}_noprefetch"]) - np.array(blocks[f"{r}_prefetch"])
        res[f"{r}_prefetch_saving_us"] = dict(mean=round(float(d.mean()), 1), per_block=[round(float(x), 1) for x in d])
    log("reuse workload: " + json.dumps(res))
    return dict(results=res, n_active_last_step=per_layer["reuse80_prefetch"], n_layers=n_layers)


def bench_nshard(inp, args, R: int = 8, r: int = 3) -> dict:
    """The same layer in the pages' N-sharded expert layout (rank r of R; mk_layer_step_nshard):
    the other ranks' intermediate slices and y columns are delivered by the host into a fresh
    pair of receive buffers per launch before the timed region (so that every launch polls
    real arrivals, not leftovers), and the K launches run back to back."""
    import torch
    import synth
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt
    sh = inp.shape
    E, P, I, T, k = sh.n_experts, sh.pooled, sh.expert_inter, sh.T, sh.top_k
    K2, N2 = R * I, P // R
    ns = synth.nshard_inputs(sh, args.config, R, r)
    dw = dt.upload_weights(inp)
    u8 = dict(dtype=torch.uint8, device="cuda")
    dw.w2_codes = torch.empty((E, N2, K2 // 2), **u8)
    dw.w2_scales = torch.empty((E, N2, K2 // 16), **u8)
    dw.w2_ts = torch.empty(E, dtype=torch.float32, device="cuda")
    mk.mk_nvfp4_pack(dt.dev_u16(ns["w2_shard"]), 0, E, N2, K2, dw.w2_codes, dw.w2_scales, dw.w2_ts)
    st = dt.make_step(inp)
    rec = dt.nvfp4_records(ns["peer_codes"], ns["peer_scales"])
    rec[:, r * I // 16:(r + 1) * I // 16, :] = 0xFFFFFFFF
    yr = ns["peer_y"].copy()
    yr[:, r * N2:(r + 1) * N2] = 0xFFFF
    n = args.warmup + args.steps
    act = torch.from_numpy(rec.view(np.int32)).cuda().unsqueeze(0).repeat(n, 1, 1, 1).contiguous()
    yrv = torch.from_numpy(dt.tile_frag(yr, P).view(np.int16)).cuda().unsqueeze(0).repeat(n, 1).contiguous()
    lib = mk.lib()
    stream = torch.cuda.current_stream()
    cfg, w, io = st.cfg, dw.struct(), st.struct()
    args_ns = [mk.mk_nshard(r, R, act[i].data_ptr(), yrv[i].data_ptr()) for i in range(n)]
    call = lambda i: lib.mk_layer_step_nshard(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io),
                                              ctypes.byref(args_ns[i]), stream.cuda_stream)
    for i in range(args.warmup):
        if call(i) != 0:
            raise RuntimeError("mk_layer_step_nshard failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, n):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    s_ = mk.mk_read_status(st.workspace)
    if s_ != 0:
        raise RuntimeError(f"nshard in-kernel status {mk.mk_strerror(s_)}")
    us = e0.elapsed_time(e1) * 1000.0 / args.steps
    log(f"N-sharded expert layout (rank {r} of {R}, GEMM2 K = {K2} -> {N2} columns): {us:.2f} us per launch")
    return {"us_per_launch": round(us, 2), "ranks": R, "rank": r, "gemm2_k": K2, "gemm2_n": N2,
            "launches": args.steps}


def bench_batch2(inp, args, n_rep: int = 3) -> dict:
    """Two sequences verified in one launch (mk_step_io.batch = 2): the workload's sequence and a
    second one with its own tree, queries, residual and KV rows (another seed) over the same
    weights; `n_rep` replicas of weights and steps rotate so that a launch's weights are not
    served from the previous launch's cache."""
    import dataclasses
    import torch
    import synth
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt
    sh = inp.shape
    s1 = synth.make_layer_inputs(sh, args.config + 1000, step=1)
    weights = ("w_o", "w_pool", "w_router", "w_unpool", "w_qkv_next", "w1", "w2")
    s1 = dataclasses.replace(s1, **{w: getattr(inp, w) for w in weights})
    reps = []
    for _ in range(n_rep):
        dw = dt.upload_weights(inp)
        st = dt.make_step_batch([inp, s1])
        reps.append((dw, st, st.cfg, dw.struct(), st.struct()))
    lib = mk.lib()
    stream = torch.cuda.current_stream()
    call = lambda i: lib.mk_layer_step(ctypes.byref(reps[i % n_rep][2]), ctypes.byref(reps[i % n_rep][3]),
                                       ctypes.byref(reps[i % n_rep][4]), stream.cuda_stream)
    for i in range(args.warmup):
        if call(i) != 0:
            raise RuntimeError("mk_layer_step (batch 2) failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        call(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    for _, st, _, _, _ in reps:
        s_ = mk.mk_read_status(st.workspace)
        if s_ != 0:
            raise RuntimeError(f"batch 2 in-kernel status {mk.mk_strerror(s_)}")
    us = e0.elapsed_time(e1) * 1000.0 / args.steps
    n_active = int(len(np.unique(reps[0][1].topk_idx.cpu().numpy())))
    log(f"two sequences per launch (32 tokens, {n_active} active experts): {us:.2f} us per launch")
    return {"us_per_launch": round(us, 2), "sequences": 2, "tokens": 2 * sh.T, "active_experts": n_active,
            "bytes_per_launch": batch_bytes(sh, n_active, 2),
            "launches": args.steps}


def mk_read_status_ok(stk) -> int:
    import layer_persistent_amd as mk
    s = mk.mk_read_status(stk.ws)
    if s != 0:
        raise RuntimeError(f"in-kernel status {mk.mk_strerror(s)}")
    return s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--config", type=int, default=2,
                    help="workload id (2: SWA layer ctx 8192, 3: global layer ctx 32768, "
                         "4: 62-layer stack ctx 4096, 5: stack with expert reuse and prefetch)")
    ap.add_argument("--layers", type=int, default=62, help="stack depth for configs 4 and 5")
    ap.add_argument("--abba", type=int, default=2, help="config 5: rounds of the A B C D D C B A variant order")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true")
    ap.add_argument("--dump-timestamps", default=None,
                    help="save the timing build's per-workgroup event ticks ([n_wg][64] int64, .npy)")
    ap.add_argument("--no-nshard", action="store_true", help="skip the N-sharded expert layout's timing")
    ap.add_argument("--no-batch2", action="store_true", help="skip the two-sequence launch's timing")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing of the same K launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain elementwise copy of 256 MiB three times "
                         "(the known-size kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (the layer kernel needs no collectives); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import layer_persistent_amd as mk
    from layer_persistent_amd import tensors as dt

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.config in (4, 5):
        out = bench_stack(args)
        main_name = "stack" if args.config == 4 else "reuse80_prefetch"
        r = out["results"][main_name]
        shape = synth.CONFIGS[args.config]
        nbytes = stack_bytes(shape, out["n_active_last_step"])
        achieved = nbytes / (r["step_us_median"] * 1e-6) / 1e9
        print(json.dumps({
            "metric": "us per verify step (stack of fused decoder layers, 16-token tree, 1 GPU)",
            "value": r["step_us_median"], "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["step_us_median"] / 1000.0, 4), "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": shape.name, "layers": out["n_layers"], "global_every": 4, "T": shape.T,
                       "ctx": shape.ctx, "window": shape.window, "launches_per_step": out["n_layers"]},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_step": nbytes},
            "results": out["results"], "n_active_per_layer": out["n_active_last_step"],
            "cpu_baseline": None}), flush=True)
        return
    shape = synth.CONFIGS[args.config]
    log(f"workload {shape.name}: generating inputs")
    t0 = time.time()
    inp = synth.make_layer_inputs(shape, args.config)
    log(f"  inputs ready in {time.time() - t0:.1f} s; uploading + packing {args.replicas} replicas")
    reps = []
    for r in range(args.replicas):
        dw = dt.upload_weights(inp)
        st = dt.make_step(inp)
        reps.append((dw, st))
    ts_step = dt.make_step(inp, timestamps=True)
    stream = torch.cuda.current_stream()
    lib = mk.lib()
    import ctypes
    # argument structs built once, kept alive for the whole run
    structs = [(st.cfg, dw.struct(), st.struct()) for dw, st in reps]
    sp = stream.cuda_stream

    def launch(i):
        c, w, io = structs[i % len(structs)]
        rc = lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io), sp)
        if rc != 0:
            raise RuntimeError(f"mk_layer_step: {mk.mk_strerror(rc)}")

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    for _, st in reps:
        s = mk.mk_read_status(st.workspace)
        if s != 0:
            raise RuntimeError(f"in-kernel status {mk.mk_strerror(s)}")
    out = dt.outputs(reps[0][1])
    n_active = int(len(np.unique(out["idx"])))
    ab = algorithmic_bytes(shape, n_active)

    # timed region: K launches back to back on the launch stream, one event pair around all
    # of them; value = elapsed / K (the inter-launch gap counts, per-launch event records do not)
    K = args.steps
    wall0 = torch.cuda.Event(enable_timing=True)
    wall1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0.record(stream)
    for i in range(K):
        launch(args.warmup + i)
    wall1.record(stream)
    torch.cuda.synchronize()
    wall_us = wall0.elapsed_time(wall1) * 1000.0
    ms_per_step = wall_us / K / 1000.0
    kern_us = wall_us / K
    # spread: a second, untimed pass with an event pair around every launch (those records
    # add ~3 us per launch of their own)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        launch(args.warmup + K + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])     # us per launch
    med_us = float(np.median(per))
    log(f"per launch: {kern_us:.2f} us over {K} back-to-back launches; with an event pair around each launch: "
        f"median {med_us:.2f} p10 {np.percentile(per, 10):.2f} p90 {np.percentile(per, 90):.2f}")
    # the same K launches captured once in a HIP graph and replayed (the pages replay each
    # verify step as one graph); outputs after the replays must equal the eager ones bit for bit
    graph = None
    if not args.no_graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            gsp = torch.cuda.current_stream().cuda_stream
            for i in range(K):
                c, w, io = structs[i % len(structs)]
                rc = lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io), gsp)
                if rc != 0:
                    raise RuntimeError(f"mk_layer_step (capture): {mk.mk_strerror(rc)}")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        reps_us = []
        for _ in range(3):
            g0.record(stream)
            g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            reps_us.append(g0.elapsed_time(g1) * 1000.0 / K)
        for _, st in reps:
            s = mk.mk_read_status(st.workspace)
            if s != 0:
                raise RuntimeError(f"in-kernel status after graph replay {mk.mk_strerror(s)}")
        outg = dt.outputs(reps[0][1])
        same = all(np.array_equal(outg[k], out[k]) for k in ("h_out", "q_next", "idx", "gate"))
        if not same:
            raise RuntimeError("graph replay outputs differ from the eager launch")
        graph = {"us_per_launch_best": round(min(reps_us), 2), "us_per_launch_all": [round(x, 2) for x in reps_us],
                 "launches_per_graph": K, "outputs_equal_eager": same}
        log(f"graph replay of {K} launches: {min(reps_us):.2f} us per launch (best of 3)")
        del g
    # MALL-warm, labelled apart: the same number of launches on one replica, whose touched
    # weights and KV (about 122 MB here) stay in the 256 MB memory-side cache between launches.
    # The timed region above rotates replicas whose touched bytes together exceed that cache.
    c0, w0, io0 = structs[0]

    def launch0():
        rc = lib.mk_layer_step(ctypes.byref(c0), ctypes.byref(w0), ctypes.byref(io0), sp)
        if rc != 0:
            raise RuntimeError(f"mk_layer_step: {mk.mk_strerror(rc)}")

    for _ in range(3):
        launch0()
    m0 = torch.cuda.Event(enable_timing=True)
    m1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    m0.record(stream)
    for _ in range(K):
        launch0()
    m1.record(stream)
    torch.cuda.synchronize()
    warm_us = m0.elapsed_time(m1) * 1000.0 / K
    mall_warm = {"us_per_launch": round(warm_us, 2), "replicas": 1, "launches": K}
    log(f"MALL-warm (one replica relaunched): {warm_us:.2f} us per launch")
    achieved = ab["total"] / (kern_us * 1e-6) / 1e9
    log(f"algorithmic bytes {ab['total'] / 1e6:.2f} MB ({n_active} active experts) -> {achieved:.0f} GB/s "
        f"= {achieved / HBM_PEAK_GBS:.3f} of {HBM_PEAK_GBS:.0f} GB/s")

    # matrix-core work per launch against the bf16/fp16 dense peak
    fl = algorithmic_flops(shape, inp.parent)
    tflops = fl["total"] / (kern_us * 1e-6) / 1e12
    mfma = {"flops_per_launch": int(fl["total"]), "dense": int(fl["dense"]), "attn": int(fl["attn"]),
            "experts": int(fl["experts"]), "achieved_tflops": round(tflops, 2), "peak_tflops": MFMA_PEAK_TFLOPS,
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 5)}
    log(f"matrix-core work {fl['total'] / 1e9:.3f} GFLOP per launch -> {tflops:.1f} TFLOP/s "
        f"= {tflops / MFMA_PEAK_TFLOPS:.4f} of {MFMA_PEAK_TFLOPS:.0f}")

    # achievable streaming-read rate in this run: the library's plain read kernel over 2 GiB
    sweep = stream_read_gbs(torch, mk, stream)
    read_gbs = max(sweep.values())
    log(f"streaming read (mk_stream_read over 2 GiB), GB/s by workgroup count: {sweep}")

    if args.copy_calibration:
        src = torch.ones(COPY_CALIB_ELEMS, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x torch.neg over {COPY_CALIB_ELEMS * 4} B read + {COPY_CALIB_ELEMS * 4} B written")
        del src, dst

    # (both need NVFP4 experts; two sequences need trees of 16 and a local intermediate of
    # 128..192, a multiple of 64)
    sh = inp.shape
    nshard_res = None if args.no_nshard or not sh.nvfp4 else bench_nshard(inp, args)
    batch2_ok = sh.nvfp4 and sh.T == 16 and sh.expert_inter % 64 == 0 and 128 <= sh.expert_inter <= 192
    batch2_res = None if args.no_batch2 or not batch2_ok else bench_batch2(inp, args)

    phases = None
    if not args.no_phases:
        dw0 = reps[0][0]
        for _ in range(3):
            dt.run_step(dw0, ts_step)
        torch.cuda.synchronize()
        tsv = ts_step.timestamps.cpu().numpy().astype(np.int64)
        if args.dump_timestamps:
            np.save(args.dump_timestamps, tsv)
        # timestamp events (ticks of the 100 MHz wall clock, per workgroup), in launch order
        t0 = tsv[:, 0].min()
        phases = {}
        for ev, name in PHASE_EVENTS:
            m = tsv[:, ev] > 0
            if m.any():
                v = (tsv[m, ev] - t0) / 100.0
                phases[name] = [round(float(np.median(v)), 2), round(float(v.max()), 2)]
        # the four grid hand-offs left (flag waits): last arrival to last release
        for p, n in ((1, "attn"), (3, "oproj"), (4, "pool"), (7, "gemm2")):
            phases[n + "_handoff_us"] = round(float((tsv[:, 2 * p + 1].max() - tsv[:, 2 * p].max()) / 100.0), 2)
        starts = (tsv[:, 0] - t0) / 100.0
        phases["wg_start_spread"] = round(float(starts.max()), 2)
        # first workgroup start to last workgroup end of the timestamped launch, next to the
        # per-launch time from HIP events (the rest is dispatch and end-of-kernel work)
        phases["launch_span_us"] = round(float((tsv[:, 19].max() - t0) / 100.0), 2)
        d = lambda e1, e0, m: round(float(((tsv[m, e1] - tsv[m, e0]) / 100.0).max()), 2)
        items = tsv[:, 37] > 0
        if items.any():
            phases["attn_stage_us_max"] = d(37, 1, items)
            phases["attn_compute_us_max"] = d(38, 37, items)
        mg = tsv[:, 63] > 0
        if mg.any():
            phases["merge_reduce_us_max"] = d(63, 61, mg)
        rtm = tsv[:, 46] > 0
        if rtm.any():
            phases["route_wait_us_max"] = d(46, 11, rtm)
            phases["route_tables_us_max"] = d(18, 46, rtm)
        pub = tsv[:, 52] > 0
        if pub.any():
            phases["route_topk_us_max"] = d(52, 51, pub)
        phases["gemm1_us_p50_max"] = [round(float(np.median((tsv[:, 12] - tsv[:, 18]) / 100.0)), 2), d(12, 18, tsv[:, 12] > 0)]
        g2 = tsv[:, 43] > 0
        if g2.any():
            phases["gemm2_us_p50_max"] = [round(float(np.median((tsv[g2, 43] - tsv[g2, 13]) / 100.0)), 2), d(43, 13, g2)]
        log("event times, [median, max] over workgroups in us after the first workgroup starts "
            "(timestamp build): " + json.dumps(phases))

    cpu = None
    if not args.no_cpu_baseline:
        inputs = {args.config: inp}
        if args.config == 2:                      # the global-attention and the tiny layers as well
            inputs[3] = synth.make_layer_inputs(synth.CONFIGS[3], 3)
            inputs[1] = synth.make_layer_inputs(synth.CONFIGS[1], 1)
        cpu = cpu_baseline(inputs)

    res = {
        "metric": "us per fused decoder layer (16-token verify, 1 GPU)",
        "value": round(kern_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "ctx": shape.ctx, "window": shape.window,
                   "hidden": shape.hidden, "q_heads": shape.n_q_heads, "kv_heads": shape.n_kv_heads,
                   "head_dim": shape.head_dim, "pooled": shape.pooled, "experts": shape.n_experts,
                   "top_k": shape.top_k, "expert_inter": shape.expert_inter, "expert_format": "nvfp4" if shape.nvfp4 else "bf16",
                   "active_experts": n_active, "replicas": args.replicas, "launches_per_layer": 1},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counted_traffic(shape.name),
                     "bytes_per_launch": ab["total"], "achievable_read_gbs": round(read_gbs, 1),
                     "frac_of_achievable": round(achieved / read_gbs, 4), "stream_read_sweep_gbs": sweep},
        "mfma": mfma,
        "evented_launch_us": {"median": round(med_us, 2), "p10": round(float(np.percentile(per, 10)), 2),
                              "p90": round(float(np.percentile(per, 90)), 2),
                              "note": "an event pair around every launch adds ~3 us per launch"},
        "graph_replay": graph,
        "mall_warm": mall_warm,
        # 62 launches of this layer per verify step (46 of the pages' layers use this sliding-window
        # shape; their 16 global layers are slower): a projection, next to the stack workload's
        # measured step (bench.py --config 4)
        "projected_62_layer_step_us": round(62 * kern_us, 1),
        "phases_end_us": phases,
        "nshard_layout": nshard_res,
        "batch2": batch2_res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
