"""MI355X-native persistent fused MoE decode-layer step.

The compute path is libmk.so (hand-written HIP kernels for gfx950) behind the C ABI in
include/mk.h; this package is its ctypes binding plus device-buffer plumbing.
"""
from ._abi import (MK_OK, MK_EINVAL, MK_ESHAPE, MK_EALIGN, MK_ECAPACITY, MK_EHIP, MK_ETIMEOUT,
                   MK_EBADTREE, MK_ESCRATCH, MK_NOALLOC_SCRATCH_BYTES, MK_W_BF16, MK_W_NVFP4, MK_TS_EVENTS, EXPORTED, LIB_PATH, MKError,
                   mk_layer_cfg, mk_layer_weights, mk_step_io, mk_workspace_layout, mk_nshard, lib,
                   mk_strerror, mk_workspace_bytes, mk_workspace_query, mk_workspace_init,
                   mk_layer_step, mk_layer_step_noalloc, mk_layer_step_nshard, mk_kv_append, mk_qkv_prologue, mk_tree_accept, mk_kv_commit, mk_kv_commit_layers,
                   mk_route_topk, mk_nvfp4_pack, mk_nvfp4_tile_w1,
                   mk_nvfp4_w1_scales_bytes, mk_stream_read, mk_read_status)
