"""A decoder stack of fused layer launches: one mk_layer_step launch per layer, all on one
stream, as the verify step of the pages' system runs its layers (one kernel per decoder
layer: orcarouter.ai write-up, "where the kernel boundary sits").

Layer L's launch reads its own KV cache and writes the tree rows of layer L+1's cache, so the
next launch finds them in place; h_out / q_next of layer L are h_in / q_in of layer L+1.
Every fourth layer (0, 4, ..., 60) attends globally and the rest over a 2048-token window
(46 + 16 of 62).  The last layer has no next-layer projection.  Layer 0's inputs come either
from the caller (queries, residual and its tree K/V rows) or, with the prologue, from the step
tokens' embeddings alone: a first launch (mk_qkv_prologue) computes layer 0's queries and
tree K/V rows, as the pages' first launch differs from the others.

This module only places tensors in HBM and fills the C-ABI structs; all arithmetic runs in
libmk.so.
"""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import torch

import synth
from . import _abi as abi
from .tensors import DeviceWeights, layer_cfg, tile_w1


@dataclasses.dataclass
class StackLayer:
    cfg: abi.mk_layer_cfg
    w: DeviceWeights
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    prefetch: list                  # two lists: a step reads one and writes the other
    topk_idx: torch.Tensor


def is_global(layer: int) -> bool:
    return layer % 4 == 0


class Stack:
    def __init__(self, shape: synth.LayerShape, cfg_id: int, n_layers: int = 62, device: str = "cuda",
                 n_prefetch: int = 14, prologue: bool = False):
        """With `prologue`, a step starts from the step tokens' embeddings: before layer 0's
        launch, mk_qkv_prologue computes layer 0's queries and tree K/V rows from them with
        layer 0's own qkv projection.  Without it the caller supplies those (stand-ins)."""
        self.shape, self.cfg_id, self.n_layers, self.device = shape, cfg_id, n_layers, device
        self.n_prefetch = n_prefetch
        self.prologue = prologue
        self.w_qkv0 = synth.device_first_qkv_weight(shape, cfg_id, device).view(torch.int16) if prologue else None
        sh = shape
        E, I, P, T, k = sh.n_experts, sh.expert_inter, sh.pooled, sh.T, sh.top_k
        u8 = dict(dtype=torch.uint8, device=device)
        self.layers: list[StackLayer] = []
        for L in range(n_layers):
            lsh = dataclasses.replace(sh, window=0 if is_global(L) else sh.window)
            wd = synth.device_layer_weights(lsh, cfg_id, L, device)
            asi16 = lambda t: t.view(torch.int16)
            dw = DeviceWeights(asi16(wd["w_o"]), asi16(wd["w_pool"]), asi16(wd["w_router"]),
                               asi16(wd["w_unpool"]), asi16(wd["w_qkv_next"]) if L + 1 < n_layers else None)
            dw.w1_codes = torch.empty((E, 2 * I, P // 2), **u8)
            dw.w1_scales = torch.empty((E, 2 * I, P // 16), **u8)
            dw.w2_codes = torch.empty((E, P, I // 2), **u8)
            dw.w2_scales = torch.empty((E, P, I // 16), **u8)
            dw.w1_ts = torch.empty(E, dtype=torch.float32, device=device)
            dw.w2_ts = torch.empty(E, dtype=torch.float32, device=device)
            abi.mk_nvfp4_pack(wd["w1"], 0, E, 2 * I, P, dw.w1_codes, dw.w1_scales, dw.w1_ts)
            abi.mk_nvfp4_pack(wd["w2"], 0, E, P, I, dw.w2_codes, dw.w2_scales, dw.w2_ts)
            tile_w1(dw, E, I, P)
            torch.cuda.synchronize()
            del wd
            kc, vc = synth.device_kv_context(lsh, cfg_id, L, device)
            self.layers.append(StackLayer(layer_cfg(lsh), dw, kc.view(torch.int16), vc.view(torch.int16),
                                          [torch.full((16,), -1, dtype=torch.int32, device=device) for _ in range(2)],
                                          torch.zeros((T, k), dtype=torch.int32, device=device)))
        # one workspace serves every launch (launches on one stream run one after another)
        self.ws_bytes = max(abi.mk_workspace_bytes(l.cfg, T) for l in self.layers[:2])
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        abi.mk_workspace_init(self.ws, self.ws_bytes)
        i16 = dict(dtype=torch.int16, device=device)
        self.h = [torch.zeros((T, sh.hidden), **i16) for _ in range(2)]
        self.q = [torch.zeros((T, sh.n_q_heads * sh.head_dim), **i16) for _ in range(2)]
        self.parent = torch.zeros(T, dtype=torch.int32, device=device)
        self.bias = None
        self.lib = abi.lib()
        self._structs = None

    def set_step_inputs(self, step_in: dict, bias: np.ndarray | None = None) -> None:
        """Layer 0's inputs for a step (host arrays from synth.stack_step_inputs), written into
        place: the tree and h_in (the step tokens' embeddings), and unless the stack runs the
        prologue, q_in and layer 0's tree K/V rows; router biases [L][T][E]."""
        sh = self.shape
        self.parent.copy_(torch.from_numpy(step_in["parent"].astype(np.int32)))
        self.h[0].copy_(torch.from_numpy(step_in["h_in"].view(np.int16)))
        if not self.prologue:
            self.q[0].copy_(torch.from_numpy(step_in["q_in"].view(np.int16)))
            k0 = torch.from_numpy(step_in["k_tree"].view(np.int16)).to(self.device)
            v0 = torch.from_numpy(step_in["v_tree"].view(np.int16)).to(self.device)
            l0 = self.layers[0]
            abi.mk_kv_append(l0.k_cache, l0.v_cache, sh.kv_capacity, sh.n_kv_heads, sh.head_dim, sh.ctx, k0, v0,
                             sh.T)
        if bias is not None:
            if self.bias is None:
                self.bias = torch.empty(bias.shape, dtype=torch.float32, device=self.device)
            self.bias.copy_(torch.from_numpy(bias))
        torch.cuda.synchronize()

    def structs(self, prefetch: bool, use_bias: bool, parity: int = 0):
        """The argument structs of one step's launches (kept alive by the caller).  Every
        launch writes its layer's most-used experts into list 1 - parity; with `prefetch` it
        prefetches the experts of list `parity` (the previous step's), so steps alternate."""
        sh = self.shape
        if use_bias and self.bias is None:
            # the structs hold the bias buffer's address: it must exist before they are built
            self.bias = torch.zeros((self.n_layers, sh.T, sh.n_experts), dtype=torch.float32, device=self.device)
        out = []
        for L, lay in enumerate(self.layers):
            nxt = self.layers[L + 1] if L + 1 < self.n_layers else None
            hi, ho = self.h[L % 2], self.h[(L + 1) % 2]
            qi, qo = self.q[L % 2], self.q[(L + 1) % 2]
            p = lambda t: None if t is None else t.data_ptr()
            io = abi.mk_step_io(
                sh.T, sh.ctx, p(self.parent), p(qi), p(hi), p(lay.k_cache), p(lay.v_cache),
                p(nxt.k_cache) if nxt else None, p(nxt.v_cache) if nxt else None, p(ho), p(qo) if nxt else None,
                p(lay.topk_idx), None, None, None, None,
                p(lay.prefetch[parity]) if prefetch else None, self.n_prefetch if prefetch else 0,
                p(lay.prefetch[1 - parity]), self.n_prefetch,
                p(self.bias[L]) if use_bias else None,
                p(self.ws), self.ws_bytes, None, 0, -1)
            out.append((lay.cfg, lay.w.struct(), io))
        return out

    def launch_step(self, structs, stream_ptr, accept=None) -> None:
        """One verify step: [the prologue,] every layer's launch, and with `accept` = (draft,
        target) the acceptance and KV commit after the last layer."""
        self._launch_layers(structs, stream_ptr)
        if accept is not None:
            self.accept_and_commit(accept[0], accept[1], stream_ptr)

    def _launch_layers(self, structs, stream_ptr) -> None:
        if self.prologue:
            sh, l0 = self.shape, self.layers[0]
            rc = self.lib.mk_qkv_prologue(self.h[0].data_ptr(), self.w_qkv0.data_ptr(), sh.T, sh.hidden,
                                          sh.n_q_heads, sh.n_kv_heads, sh.head_dim, self.q[0].data_ptr(),
                                          l0.k_cache.data_ptr(), l0.v_cache.data_ptr(), sh.kv_capacity, sh.ctx,
                                          stream_ptr)
            if rc != 0:
                raise abi.MKError(rc, "mk_qkv_prologue")
        for c, w, io in structs:
            rc = self.lib.mk_layer_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(io), stream_ptr)
            if rc != 0:
                raise abi.MKError(rc, "mk_layer_step")

    def accept_and_commit(self, draft: torch.Tensor, target: torch.Tensor, stream_ptr) -> None:
        """After a verify step: greedy acceptance along the step's tree (mk_tree_accept; draft
        and target are int32 [T] device tensors, target being the target model's greedy token
        after each node, which an LM head outside this library produces), then the accepted
        nodes' K/V rows moved to positions ctx + depth in every layer's cache (mk_kv_commit_layers,
        one launch for all layers).
        The path, its length and the bonus token stay on the device (self.path, self.n_path,
        self.bonus), so the calls can sit in the step's graph."""
        sh = self.shape
        if not hasattr(self, "path"):
            self.path = torch.full((sh.T,), -1, dtype=torch.int32, device=self.device)
            self.n_path = torch.zeros(1, dtype=torch.int32, device=self.device)
            self.bonus = torch.zeros(1, dtype=torch.int32, device=self.device)
        rc = self.lib.mk_tree_accept(self.parent.data_ptr(), draft.data_ptr(), target.data_ptr(), sh.T,
                                     self.path.data_ptr(), self.n_path.data_ptr(), self.bonus.data_ptr(), stream_ptr)
        if rc != 0:
            raise abi.MKError(rc, "mk_tree_accept")
        if not hasattr(self, "kv_ptrs"):
            # device arrays of every layer's cache pointers, for the one-launch commit
            self.kv_ptrs = [torch.tensor([getattr(l, f).data_ptr() for l in self.layers], dtype=torch.int64,
                                         device=self.device) for f in ("k_cache", "v_cache")]
        rc = self.lib.mk_kv_commit_layers(self.kv_ptrs[0].data_ptr(), self.kv_ptrs[1].data_ptr(), self.n_layers,
                                          sh.kv_capacity, sh.n_kv_heads, sh.head_dim, sh.ctx, self.path.data_ptr(),
                                          self.n_path.data_ptr(), sh.T, stream_ptr)
        if rc != 0:
            raise abi.MKError(rc, "mk_kv_commit_layers")

    def capture_step(self, structs, accept=None) -> torch.cuda.CUDAGraph:
        """One step's launches captured once as a HIP graph (the pages switch the stack on per
        server flag and replay each verify step as one graph: orcarouter.ai write-up, "where the
        5.9 ms still goes").  A replay runs the same launches on the stream it is replayed on;
        the step's inputs are written into place (set_step_inputs) before each replay, and the
        kernels keep their epoch in the workspace, so replays need no host-side state."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        if accept is not None and not hasattr(self, "path"):
            self.accept_and_commit(accept[0], accept[1], torch.cuda.current_stream().cuda_stream)   # buffers
            torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            self.launch_step(structs, torch.cuda.current_stream().cuda_stream, accept)
        torch.cuda.current_stream().wait_stream(side)
        return g

    def h_out(self) -> torch.Tensor:
        return self.h[self.n_layers % 2]
