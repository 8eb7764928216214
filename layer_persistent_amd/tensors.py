"""Device-buffer plumbing around the C ABI: puts one layer's weights and step tensors in HBM
(PyTorch tensors, used only as memory), packs NVFP4 experts with mk_nvfp4_pack, and fills the
mk_* argument structs.  No layer arithmetic happens here."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import _abi as abi


def dev_u16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device tensor (int16 storage)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def layer_cfg(shape) -> abi.mk_layer_cfg:
    return abi.mk_layer_cfg(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.pooled,
                            shape.n_experts, shape.top_k, shape.expert_inter, shape.window,
                            abi.MK_W_NVFP4 if shape.nvfp4 else abi.MK_W_BF16, shape.kv_capacity)


@dataclasses.dataclass
class DeviceWeights:
    w_o: torch.Tensor
    w_pool: torch.Tensor
    w_router: torch.Tensor
    w_unpool: torch.Tensor
    w_qkv: torch.Tensor | None              # None: the stack's last layer (no next-layer q/k/v)
    w1: torch.Tensor | None = None          # bf16 experts
    w2: torch.Tensor | None = None
    w1_codes: torch.Tensor | None = None    # NVFP4 experts
    w1_scales: torch.Tensor | None = None
    w2_codes: torch.Tensor | None = None
    w2_scales: torch.Tensor | None = None
    w1_ts: torch.Tensor | None = None
    w2_ts: torch.Tensor | None = None

    def struct(self) -> abi.mk_layer_weights:
        p = lambda t: None if t is None else t.data_ptr()
        return abi.mk_layer_weights(p(self.w_o), p(self.w_pool), p(self.w_router), p(self.w_unpool), p(self.w_qkv),
                                    p(self.w1), p(self.w2), p(self.w1_codes), p(self.w1_scales), p(self.w2_codes),
                                    p(self.w2_scales), p(self.w1_ts), p(self.w2_ts))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in dataclasses.asdict(self).values() if t is not None)


def upload_weights(inp, device="cuda", stream=None) -> DeviceWeights:
    sh = inp.shape
    dw = DeviceWeights(dev_u16(inp.w_o, device), dev_u16(inp.w_pool, device), dev_u16(inp.w_router, device),
                       dev_u16(inp.w_unpool, device), dev_u16(inp.w_qkv_next, device))
    w1 = dev_u16(inp.w1, device)
    w2 = dev_u16(inp.w2, device)
    if not sh.nvfp4:
        dw.w1, dw.w2 = w1, w2
        return dw
    E, I, P = sh.n_experts, sh.expert_inter, sh.pooled
    u8 = dict(dtype=torch.uint8, device=device)
    dw.w1_codes = torch.empty((E, 2 * I, P // 2), **u8)
    dw.w1_scales = torch.empty((E, 2 * I, P // 16), **u8)
    dw.w2_codes = torch.empty((E, P, I // 2), **u8)
    dw.w2_scales = torch.empty((E, P, I // 16), **u8)
    dw.w1_ts = torch.empty(E, dtype=torch.float32, device=device)
    dw.w2_ts = torch.empty(E, dtype=torch.float32, device=device)
    abi.mk_nvfp4_pack(w1, 0, E, 2 * I, P, dw.w1_codes, dw.w1_scales, dw.w1_ts, stream)
    abi.mk_nvfp4_pack(w2, 0, E, P, I, dw.w2_codes, dw.w2_scales, dw.w2_ts, stream)
    tile_w1(dw, E, I, P, stream)
    torch.cuda.synchronize()
    del w1, w2
    return dw


def tile_w1(dw, E: int, I: int, P: int, stream=None) -> None:
    """Replace dw.w1_codes / dw.w1_scales (row-major, as mk_nvfp4_pack writes them) by their
    GEMM1 operand order (mk_nvfp4_tile_w1)."""
    codes_t = torch.empty_like(dw.w1_codes)
    scales_t = torch.empty(abi.mk_nvfp4_w1_scales_bytes(E, 2 * I, P), dtype=torch.uint8, device=dw.w1_codes.device)
    abi.mk_nvfp4_tile_w1(dw.w1_codes, dw.w1_scales, E, 2 * I, P, codes_t, scales_t, stream)
    torch.cuda.synchronize()
    dw.w1_codes, dw.w1_scales = codes_t, scales_t


@dataclasses.dataclass
class DeviceStep:
    """Step inputs, outputs and workspace of one layer launch."""
    cfg: abi.mk_layer_cfg
    T: int
    ctx: int
    parent: torch.Tensor
    q_in: torch.Tensor
    h_in: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_next: torch.Tensor
    v_next: torch.Tensor
    h_out: torch.Tensor
    q_next: torch.Tensor
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    logits: torch.Tensor
    stats: torch.Tensor
    hist: torch.Tensor
    bias: torch.Tensor | None
    workspace: torch.Tensor
    layout: abi.mk_workspace_layout
    timestamps: torch.Tensor | None = None
    batch: int = 1                          # sequences of T tokens (rows: batch * T)
    prefetch: torch.Tensor | None = None
    n_prefetch: int = 0
    prefetch_next: torch.Tensor | None = None
    n_prefetch_next: int = 0

    def struct(self, spin_limit: int = 0, skip_wg: int = -1) -> abi.mk_step_io:
        p = lambda t: None if t is None else t.data_ptr()
        return abi.mk_step_io(self.T, self.ctx, p(self.parent), p(self.q_in), p(self.h_in), p(self.k_cache),
                              p(self.v_cache), p(self.k_next), p(self.v_next), p(self.h_out), p(self.q_next),
                              p(self.topk_idx), p(self.topk_gate), p(self.logits), p(self.stats), p(self.hist),
                              p(self.prefetch), self.n_prefetch, p(self.prefetch_next), self.n_prefetch_next,
                              p(self.bias), p(self.workspace),
                              self.workspace.numel(), p(self.timestamps), spin_limit, skip_wg, self.batch)

    def ws_u16(self, off: int, n: int) -> np.ndarray:
        return self.workspace[off:off + 2 * n].cpu().numpy().view(np.uint16)

    def ws_f32(self, off: int, n: int) -> np.ndarray:
        return self.workspace[off:off + 4 * n].cpu().numpy().view(np.float32)


def make_step(inp, device="cuda", timestamps: bool = False, stream=None) -> DeviceStep:
    sh = inp.shape
    cfg = layer_cfg(sh)
    T, E, k = sh.T, sh.n_experts, sh.top_k
    f32 = dict(dtype=torch.float32, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    lay = abi.mk_workspace_query(cfg, T)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=device)
    abi.mk_workspace_init(ws, lay.total, stream)
    st = DeviceStep(cfg, T, sh.ctx, torch.from_numpy(inp.parent.astype(np.int32)).to(device),
                    dev_u16(inp.q_in, device), dev_u16(inp.h_in, device), dev_u16(inp.k_cache, device),
                    dev_u16(inp.v_cache, device), dev_u16(inp.k_cache_next, device), dev_u16(inp.v_cache_next, device),
                    torch.zeros((T, sh.hidden), dtype=torch.int16, device=device),
                    torch.zeros((T, sh.n_q_heads * sh.head_dim), dtype=torch.int16, device=device),
                    torch.full((T, k), -1, **i32), torch.zeros((T, k), **f32), torch.zeros((T, E), **f32),
                    torch.zeros((T, sh.n_q_heads, 2), **f32), torch.zeros(E, **i32),
                    None if inp.router_bias is None else torch.from_numpy(inp.router_bias).to(device),
                    ws, lay)
    if timestamps:
        st.timestamps = torch.zeros((lay.n_wg, abi.MK_TS_EVENTS), dtype=torch.int64, device=device)
    return st


def make_step_batch(inps, device="cuda") -> DeviceStep:
    """Two sequences in one launch: their trees, queries, residuals, caches and outputs stacked
    (sequence b on rows 16 b .., its caches at b * capacity rows).  The sequences must share the
    layer's weights and shape (T = 16, same ctx)."""
    sh = inps[0].shape
    B = len(inps)
    assert B == 2 and sh.T == 16 and all(i.shape == sh for i in inps)
    cfg = layer_cfg(sh)
    T, E, k = sh.T, sh.n_experts, sh.top_k
    R = B * T
    f32 = dict(dtype=torch.float32, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    lay = abi.mk_workspace_query(cfg, T)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=device)
    abi.mk_workspace_init(ws, lay.total, None)
    cat = lambda name: np.concatenate([getattr(i, name) for i in inps], axis=0)
    bias = None if inps[0].router_bias is None else torch.from_numpy(cat("router_bias")).to(device)
    return DeviceStep(cfg, T, sh.ctx, torch.from_numpy(cat("parent").astype(np.int32)).to(device),
                      dev_u16(cat("q_in"), device), dev_u16(cat("h_in"), device), dev_u16(cat("k_cache"), device),
                      dev_u16(cat("v_cache"), device), dev_u16(cat("k_cache_next"), device),
                      dev_u16(cat("v_cache_next"), device),
                      torch.zeros((R, sh.hidden), dtype=torch.int16, device=device),
                      torch.zeros((R, sh.n_q_heads * sh.head_dim), dtype=torch.int16, device=device),
                      torch.full((R, k), -1, **i32), torch.zeros((R, k), **f32), torch.zeros((R, E), **f32),
                      torch.zeros((R, sh.n_q_heads, 2), **f32), torch.zeros(E, **i32), bias, ws, lay, None, B)


def run_step(dw: DeviceWeights, st: DeviceStep, stream=None, spin_limit: int = 0, skip_wg: int = -1) -> int:
    io = st.struct(spin_limit, skip_wg)
    return abi.mk_layer_step(st.cfg, dw.struct(), io, stream)


def untile_frag(buf: np.ndarray, T: int, K: int) -> np.ndarray:
    """[16][K] bf16 held in MFMA fragment order (element (t, c) at ((c//32)*64 + (c//8)%4*16 + t)*8
    + c%8) back to row-major [T][K]."""
    return buf.reshape(K // 32, 4, 16, 8).transpose(2, 0, 1, 3).reshape(16, K)[:T].copy()


def tile_frag(rows: np.ndarray, K: int) -> np.ndarray:
    """Row-major [T <= 16][K] bf16 into MFMA fragment order [16 * K] (rows >= T all ones, the
    hand-off sentinel): the inverse of untile_frag."""
    full = np.full((16, K), 0xFFFF, np.uint16)
    full[:rows.shape[0]] = rows
    return full.reshape(16, K // 32, 4, 8).transpose(1, 2, 0, 3).reshape(-1).copy()


def nvfp4_records(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """NVFP4 rows (codes uint8 [M][K/2], element 2j in the low nibble; E4M3 scales uint8
    [M][K/16]) as the kernel's 16-byte intermediate records, uint32 [M][K/16][4]: the 4 code
    bytes of elements 0-7, the scale byte, the 4 code bytes of elements 8-15, the scale byte."""
    M, K2 = codes.shape[0], codes.shape[1] * 2
    c = np.ascontiguousarray(codes).reshape(M, K2 // 16, 2, 4).view(np.uint32).reshape(M, K2 // 16, 2)
    rec = np.empty((M, K2 // 16, 4), np.uint32)
    rec[:, :, 0] = c[:, :, 0]
    rec[:, :, 2] = c[:, :, 1]
    rec[:, :, 1] = scales
    rec[:, :, 3] = scales
    return rec


def nvfp4_from_records(rec: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of nvfp4_records: (codes uint8 [M][K/2], scales uint8 [M][K/16])."""
    M, nb = rec.shape[0], rec.shape[1]
    c = np.stack([rec[:, :, 0], rec[:, :, 2]], axis=2).astype(np.uint32).view(np.uint8).reshape(M, nb * 8)
    return c.copy(), (rec[:, :, 1] & 0xFF).astype(np.uint8)


def stage_offset(workspace: torch.Tensor, layout, off: int) -> int:
    """Byte offset of a stage buffer of the workspace's last launch: copy (epoch & 1) of the
    launch's epoch, which is one less than the epoch slot of workgroup 0 afterwards."""
    epoch = int(workspace[layout.epoch:layout.epoch + 4].cpu().numpy().view(np.uint32)[0]) - 1
    return off + (epoch & 1) * layout.stage_copy


def outputs(st: DeviceStep) -> dict:
    """Copy a step's outputs and stage hand-off buffers (those of its last launch) to the host
    (stage buffers: one 16-row fragment tile per sequence, rows stacked)."""
    torch.cuda.synchronize()
    sh_T = st.T
    lay = st.layout
    c = st.cfg

    class _L:      # the stage offsets of the last launch's copy
        attn, h1, xp, y = (stage_offset(st.workspace, lay, o) for o in (lay.attn, lay.h1, lay.xp, lay.y))
        status = lay.status
    L = _L

    def tiles(off, K):
        return np.concatenate([untile_frag(st.ws_u16(off + 2 * b * 16 * K, 16 * K), sh_T, K) for b in range(st.batch)])
    if st.batch > 1:
        return dict(
            h_out=host_u16(st.h_out), q_next=host_u16(st.q_next),
            k_cache_next=host_u16(st.k_next), v_cache_next=host_u16(st.v_next),
            idx=st.topk_idx.cpu().numpy(), gate=st.topk_gate.cpu().numpy(), logits=st.logits.cpu().numpy(),
            stats=st.stats.cpu().numpy(), hist=st.hist.cpu().numpy(),
            attn=tiles(L.attn, c.n_q_heads * c.head_dim), h1=tiles(L.h1, c.hidden), xp=tiles(L.xp, c.pooled),
            y=tiles(L.y, c.pooled), status=abi.mk_read_status(st.workspace))
    return dict(
        h_out=host_u16(st.h_out), q_next=host_u16(st.q_next),
        k_cache_next=host_u16(st.k_next), v_cache_next=host_u16(st.v_next),
        idx=st.topk_idx.cpu().numpy(), gate=st.topk_gate.cpu().numpy(), logits=st.logits.cpu().numpy(),
        stats=st.stats.cpu().numpy(), hist=st.hist.cpu().numpy(),
        attn=untile_frag(st.ws_u16(L.attn, 16 * c.n_q_heads * c.head_dim), sh_T, c.n_q_heads * c.head_dim),
        h1=untile_frag(st.ws_u16(L.h1, 16 * c.hidden), sh_T, c.hidden),
        xp=untile_frag(st.ws_u16(L.xp, 16 * c.pooled), sh_T, c.pooled),
        y=untile_frag(st.ws_u16(L.y, 16 * c.pooled), sh_T, c.pooled),
        status=abi.mk_read_status(st.workspace),
    )
