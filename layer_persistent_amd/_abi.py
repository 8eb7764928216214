"""ctypes binding of include/mk.h: the same names, argument marshalling only.

Every computation runs in the HIP kernels of libmk.so.  Device memory and streams come
from PyTorch (tensors' data_ptr() and torch.cuda streams); the library sees plain pointers.
If libmk.so is missing, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK, MK_EINVAL, MK_ESHAPE, MK_EALIGN, MK_ECAPACITY, MK_EHIP, MK_ETIMEOUT, MK_EBADTREE = 0, -1, -2, -3, -4, -5, -6, -7
MK_ESCRATCH = -8
MK_NOALLOC_SCRATCH_BYTES = 24 << 20
MK_W_BF16, MK_W_NVFP4 = 0, 1
MK_TS_EVENTS = 64

EXPORTED = ["mk_workspace_bytes", "mk_workspace_query", "mk_workspace_init", "mk_layer_step", "mk_layer_step_noalloc",
            "mk_layer_step_nshard",
            "mk_kv_append", "mk_qkv_prologue", "mk_tree_accept", "mk_kv_commit", "mk_kv_commit_layers", "mk_route_topk", "mk_nvfp4_pack", "mk_nvfp4_tile_w1", "mk_nvfp4_w1_scales_bytes",
            "mk_stream_read", "mk_read_status", "mk_strerror"]


class mk_nshard(C.Structure):
    _fields_ = [("rank", C.c_int), ("n_ranks", C.c_int), ("act_recv", C.c_void_p), ("y_recv", C.c_void_p)]


class mk_layer_cfg(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_q_heads", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("pooled", C.c_int), ("n_experts", C.c_int), ("top_k", C.c_int), ("expert_inter", C.c_int),
                ("window", C.c_int), ("expert_fmt", C.c_int), ("kv_capacity", C.c_int)]


class mk_layer_weights(C.Structure):
    _fields_ = [("w_o", C.c_void_p), ("w_pool", C.c_void_p), ("w_router", C.c_void_p),
                ("w_unpool", C.c_void_p), ("w_qkv_next", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p),
                ("w1_codes", C.c_void_p), ("w1_scales", C.c_void_p), ("w2_codes", C.c_void_p),
                ("w2_scales", C.c_void_p), ("w1_tscale", C.c_void_p), ("w2_tscale", C.c_void_p)]


class mk_step_io(C.Structure):
    _fields_ = [("T", C.c_int), ("ctx_len", C.c_int), ("tree_parent", C.c_void_p), ("q_in", C.c_void_p),
                ("h_in", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("k_cache_next", C.c_void_p), ("v_cache_next", C.c_void_p), ("h_out", C.c_void_p),
                ("q_next", C.c_void_p), ("topk_idx", C.c_void_p), ("topk_gate", C.c_void_p),
                ("router_logits", C.c_void_p), ("attn_stats", C.c_void_p), ("expert_hist", C.c_void_p),
                ("prefetch_experts", C.c_void_p), ("n_prefetch", C.c_int),
                ("prefetch_next", C.c_void_p), ("n_prefetch_next", C.c_int), ("router_bias", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("timestamps", C.c_void_p),
                ("spin_limit", C.c_int), ("debug_skip_signal_wg", C.c_int), ("batch", C.c_int)]


class mk_workspace_layout(C.Structure):
    _fields_ = [("status", C.c_size_t), ("attn", C.c_size_t), ("h1", C.c_size_t), ("xp", C.c_size_t),
                ("logits", C.c_size_t), ("y", C.c_size_t), ("total", C.c_size_t), ("n_wg", C.c_int),
                ("attn_items", C.c_int), ("stage_copy", C.c_size_t), ("epoch", C.c_size_t)]


_lib = None


def lib() -> C.CDLL:
    """Load libmk.so once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m layer_persistent_amd.build` "
                               "(there is no non-HIP fallback)")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.mk_workspace_bytes.argtypes = [C.POINTER(mk_layer_cfg), C.c_int]
        L.mk_workspace_bytes.restype = C.c_size_t
        L.mk_workspace_query.argtypes = [C.POINTER(mk_layer_cfg), C.c_int, C.POINTER(mk_workspace_layout)]
        L.mk_workspace_init.argtypes = [P, C.c_size_t, P]
        L.mk_layer_step.argtypes = [C.POINTER(mk_layer_cfg), C.POINTER(mk_layer_weights), C.POINTER(mk_step_io), P]
        L.mk_layer_step_noalloc.argtypes = [C.POINTER(mk_layer_cfg), C.POINTER(mk_layer_weights),
                                            C.POINTER(mk_step_io), P]
        L.mk_layer_step_nshard.argtypes = [C.POINTER(mk_layer_cfg), C.POINTER(mk_layer_weights),
                                           C.POINTER(mk_step_io), C.POINTER(mk_nshard), P]
        L.mk_kv_append.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, C.c_int, P]
        L.mk_qkv_prologue.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, C.c_int,
                                      C.c_int, P]
        L.mk_tree_accept.argtypes = [P, P, P, C.c_int, P, P, P, P]
        L.mk_kv_commit.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, C.c_int, P]
        L.mk_kv_commit_layers.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, C.c_int, P]
        L.mk_route_topk.argtypes = [P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.mk_nvfp4_pack.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.mk_nvfp4_tile_w1.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P, P, P]
        L.mk_nvfp4_w1_scales_bytes.argtypes = [C.c_int, C.c_int, C.c_int]
        L.mk_nvfp4_w1_scales_bytes.restype = C.c_size_t
        L.mk_stream_read.argtypes = [P, C.c_size_t, C.c_int, P, P]
        L.mk_read_status.argtypes = [P, P]
        L.mk_strerror.argtypes = [C.c_int]
        L.mk_strerror.restype = C.c_char_p
        for name in ("mk_workspace_query", "mk_workspace_init", "mk_layer_step", "mk_layer_step_noalloc",
                     "mk_layer_step_nshard",
                     "mk_kv_append", "mk_qkv_prologue",
                     "mk_tree_accept", "mk_kv_commit", "mk_kv_commit_layers",
                     "mk_route_topk", "mk_nvfp4_pack", "mk_nvfp4_tile_w1", "mk_stream_read", "mk_read_status"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _ptr(x) -> int | None:
    """Device (or host) pointer of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


class MKError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {mk_strerror(status)} ({status})")
        self.status = status


def _check(rc: int, what: str) -> int:
    if rc != MK_OK:
        raise MKError(rc, what)
    return rc


def mk_strerror(status: int) -> str:
    return lib().mk_strerror(status).decode()


def mk_workspace_bytes(cfg: mk_layer_cfg, T: int) -> int:
    return lib().mk_workspace_bytes(C.byref(cfg), T)


def mk_workspace_query(cfg: mk_layer_cfg, T: int) -> mk_workspace_layout:
    out = mk_workspace_layout()
    _check(lib().mk_workspace_query(C.byref(cfg), T, C.byref(out)), "mk_workspace_query")
    return out


def mk_workspace_init(workspace, nbytes: int, stream=None) -> int:
    return _check(lib().mk_workspace_init(_ptr(workspace), nbytes, _stream(stream)), "mk_workspace_init")


def mk_layer_step(cfg: mk_layer_cfg, w: mk_layer_weights, io: mk_step_io, stream=None, check=True) -> int:
    rc = lib().mk_layer_step(C.byref(cfg), C.byref(w), C.byref(io), _stream(stream))
    return _check(rc, "mk_layer_step") if check else rc


def mk_qkv_prologue(h, w_qkv, T, hidden, n_q_heads, n_kv_heads, head_dim, q_out, k_cache, v_cache, capacity,
                    pos, stream=None, check=True):
    rc = lib().mk_qkv_prologue(_ptr(h), _ptr(w_qkv), T, hidden, n_q_heads, n_kv_heads, head_dim, _ptr(q_out),
                               _ptr(k_cache), _ptr(v_cache), capacity, pos, _stream(stream))
    return _check(rc, "mk_qkv_prologue") if check else rc


def mk_tree_accept(parent, draft, target, T, path, n_path, bonus, stream=None, check=True):
    rc = lib().mk_tree_accept(_ptr(parent), _ptr(draft), _ptr(target), T, _ptr(path), _ptr(n_path), _ptr(bonus),
                              _stream(stream))
    return _check(rc, "mk_tree_accept") if check else rc


def mk_kv_commit(k_cache, v_cache, capacity, n_kv_heads, head_dim, ctx, path, n_path, T, stream=None, check=True):
    rc = lib().mk_kv_commit(_ptr(k_cache), _ptr(v_cache), capacity, n_kv_heads, head_dim, ctx, _ptr(path),
                            _ptr(n_path), T, _stream(stream))
    return _check(rc, "mk_kv_commit") if check else rc


def mk_kv_commit_layers(k_caches, v_caches, n_layers, capacity, n_kv_heads, head_dim, ctx, path, n_path, T,
                        stream=None, check=True):
    rc = lib().mk_kv_commit_layers(_ptr(k_caches), _ptr(v_caches), n_layers, capacity, n_kv_heads, head_dim, ctx,
                                   _ptr(path), _ptr(n_path), T, _stream(stream))
    return _check(rc, "mk_kv_commit_layers") if check else rc


def mk_kv_append(k_cache, v_cache, capacity, n_kv_heads, head_dim, pos, k_new, v_new, n, stream=None, check=True):
    rc = lib().mk_kv_append(_ptr(k_cache), _ptr(v_cache), capacity, n_kv_heads, head_dim, pos, _ptr(k_new),
                            _ptr(v_new), n, _stream(stream))
    return _check(rc, "mk_kv_append") if check else rc


def mk_route_topk(x, w_router, bias, T, P, E, k, idx, gate, logits=None, stream=None, check=True):
    rc = lib().mk_route_topk(_ptr(x), _ptr(w_router), _ptr(bias), T, P, E, k, _ptr(idx), _ptr(gate),
                             _ptr(logits), _stream(stream))
    return _check(rc, "mk_route_topk") if check else rc


def mk_nvfp4_pack(w, w_is_fp32, batch, N, K, codes, scales, tensor_scale, stream=None, check=True):
    rc = lib().mk_nvfp4_pack(_ptr(w), int(w_is_fp32), batch, N, K, _ptr(codes), _ptr(scales),
                             _ptr(tensor_scale), _stream(stream))
    return _check(rc, "mk_nvfp4_pack") if check else rc


def mk_nvfp4_tile_w1(codes, scales, batch, N, K, codes_t, scales_t, stream=None, check=True):
    rc = lib().mk_nvfp4_tile_w1(_ptr(codes), _ptr(scales), batch, N, K, _ptr(codes_t), _ptr(scales_t),
                                _stream(stream))
    return _check(rc, "mk_nvfp4_tile_w1") if check else rc


def mk_nvfp4_w1_scales_bytes(batch, N, K) -> int:
    return int(lib().mk_nvfp4_w1_scales_bytes(batch, N, K))


def mk_layer_step_noalloc(cfg: mk_layer_cfg, w: mk_layer_weights, io: mk_step_io, stream=None,
                          check=True) -> int:
    rc = lib().mk_layer_step_noalloc(C.byref(cfg), C.byref(w), C.byref(io), _stream(stream))
    return _check(rc, "mk_layer_step_noalloc") if check else rc


def mk_stream_read(src, nbytes, n_blocks, sink, stream=None, check=True) -> int:
    rc = lib().mk_stream_read(_ptr(src), nbytes, n_blocks, _ptr(sink), _stream(stream))
    return _check(rc, "mk_stream_read") if check else rc


def mk_layer_step_nshard(cfg: mk_layer_cfg, w: mk_layer_weights, io: mk_step_io, ns: mk_nshard, stream=None,
                         check=True) -> int:
    rc = lib().mk_layer_step_nshard(C.byref(cfg), C.byref(w), C.byref(io), C.byref(ns), _stream(stream))
    return _check(rc, "mk_layer_step_nshard") if check else rc


def mk_read_status(workspace, stream=None) -> int:
    return lib().mk_read_status(_ptr(workspace), _stream(stream))
