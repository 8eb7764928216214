"""C ABI checks that need no GPU: the library loads, exports every function include/mk.h
declares, and rejects bad arguments on the host before any HIP call."""
import os
import re

import pytest

import layer_persistent_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GOOD = 0x10000       # fake, 16-byte aligned "device pointers": never dereferenced on the host
BAD = 0x10008


def _declared():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 9
    L = mk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(mk.EXPORTED)


def test_strerror():
    assert mk.mk_strerror(mk.MK_ETIMEOUT) == "in-kernel wait timed out"
    assert mk.mk_strerror(mk.MK_EBADTREE) == "malformed tree_parent"
    assert mk.mk_strerror(12345) == "unknown status"


def _cfg(**kw):
    base = dict(hidden=4096, n_q_heads=8, n_kv_heads=1, head_dim=128, pooled=2048, n_experts=256, top_k=8,
                expert_inter=192, window=2048, expert_fmt=mk.MK_W_NVFP4, kv_capacity=8208)
    base.update(kw)
    return mk.mk_layer_cfg(*[base[f] for f, _ in mk.mk_layer_cfg._fields_])


def _weights(ptr=GOOD):
    return mk.mk_layer_weights(*([ptr] * len(mk.mk_layer_weights._fields_)))


def _io(T=16, ctx=8192, ptr=GOOD, **kw):
    io = mk.mk_step_io()
    for f, _ in mk.mk_step_io._fields_:
        if f not in ("T", "ctx_len", "n_prefetch", "n_prefetch_next", "workspace_bytes", "spin_limit",
                     "debug_skip_signal_wg", "batch"):
            setattr(io, f, ptr)
    io.T, io.ctx_len, io.workspace_bytes, io.debug_skip_signal_wg = T, ctx, 1 << 30, -1
    io.prefetch_experts = None
    io.prefetch_next = None
    for k, v in kw.items():
        setattr(io, k, v)
    return io


@pytest.mark.parametrize("field", ["tree_parent", "q_in", "h_in", "k_cache", "v_cache", "k_cache_next",
                                   "v_cache_next", "h_out", "q_next", "workspace"])
def test_layer_step_rejects_null_inputs(field):
    assert mk.mk_layer_step(_cfg(), _weights(), _io(**{field: None}), check=False) == mk.MK_EINVAL


@pytest.mark.parametrize("kw", [dict(hidden=4000), dict(head_dim=96), dict(n_q_heads=12, n_kv_heads=8),
                                dict(n_experts=300), dict(top_k=9), dict(expert_inter=100), dict(window=-1),
                                dict(n_q_heads=16)])
def test_layer_step_rejects_bad_shapes(kw):
    assert mk.mk_layer_step(_cfg(**kw), _weights(), _io(), check=False) == mk.MK_ESHAPE


def test_batch_is_validated_on_host():
    ok = dict(check=False)
    assert mk.mk_layer_step(_cfg(), _weights(), _io(batch=3), **ok) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(batch=-1), **ok) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(batch=2, T=9), **ok) == mk.MK_ESHAPE       # trees of 16
    assert mk.mk_layer_step(_cfg(expert_fmt=mk.MK_W_BF16), _weights(), _io(batch=2), **ok) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(expert_inter=256), _weights(), _io(batch=2), **ok) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(expert_inter=96), _weights(), _io(batch=2), **ok) == mk.MK_ESHAPE
    ns = mk.mk_nshard(3, 8, GOOD, GOOD)
    assert mk.mk_layer_step_nshard(_cfg(), _weights(), _io(batch=2), ns, check=False) == mk.MK_ESHAPE


def test_layer_step_rejects_bad_T_capacity_alignment_and_enum():
    assert mk.mk_layer_step(_cfg(), _weights(), _io(T=17), check=False) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(T=0), check=False) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(ctx=8193), check=False) == mk.MK_ECAPACITY
    assert mk.mk_layer_step(_cfg(), _weights(), _io(ctx=-1), check=False) == mk.MK_ECAPACITY
    assert mk.mk_layer_step(_cfg(), _weights(), _io(h_out=BAD), check=False) == mk.MK_EALIGN
    assert mk.mk_layer_step(_cfg(), _weights(BAD), _io(), check=False) == mk.MK_EALIGN
    assert mk.mk_layer_step(_cfg(expert_fmt=7), _weights(), _io(), check=False) == mk.MK_EINVAL
    assert mk.mk_layer_step(_cfg(), _weights(), _io(n_prefetch=17), check=False) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(n_prefetch=3), check=False) == mk.MK_EINVAL
    assert mk.mk_layer_step(_cfg(), _weights(), _io(n_prefetch_next=17), check=False) == mk.MK_ESHAPE
    assert mk.mk_layer_step(_cfg(), _weights(), _io(n_prefetch_next=14), check=False) == mk.MK_EINVAL
    w = _weights()
    w.w1_codes = None
    assert mk.mk_layer_step(_cfg(), w, _io(), check=False) == mk.MK_EINVAL


def test_noalloc_layer_step_validates_like_layer_step_and_ignores_the_workspace():
    step = mk.mk_layer_step_noalloc
    for field in ("tree_parent", "q_in", "h_in", "k_cache", "v_cache", "h_out", "q_next"):
        assert step(_cfg(), _weights(), _io(**{field: None}), check=False) == mk.MK_EINVAL, field
    assert step(_cfg(hidden=4000), _weights(), _io(workspace=None), check=False) == mk.MK_ESHAPE
    assert step(_cfg(), _weights(), _io(T=17, workspace=None), check=False) == mk.MK_ESHAPE
    assert step(_cfg(), _weights(), _io(ctx=8193, workspace=None), check=False) == mk.MK_ECAPACITY
    assert step(_cfg(), _weights(), _io(h_out=BAD, workspace=None), check=False) == mk.MK_EALIGN
    # the workspace fields are not used: with no workspace the checks go on to the alignment of
    # the other pointers (mk_layer_step stops at the missing workspace)
    assert mk.mk_layer_step(_cfg(), _weights(), _io(workspace=None, h_out=BAD), check=False) == mk.MK_EINVAL
    assert step(_cfg(), _weights(), _io(workspace=None, h_out=BAD), check=False) == mk.MK_EALIGN
    assert mk.mk_strerror(mk.MK_ESCRATCH).startswith("configuration needs a larger workspace")


def test_small_entry_points_validate_on_host():
    assert mk.mk_kv_append(None, GOOD, 64, 1, 64, 0, GOOD, GOOD, 4, check=False) == mk.MK_EINVAL
    assert mk.mk_kv_append(GOOD, GOOD, 64, 1, 64, 62, GOOD, GOOD, 4, check=False) == mk.MK_ECAPACITY
    assert mk.mk_kv_append(GOOD, GOOD, 64, 1, 60, 0, GOOD, GOOD, 4, check=False) == mk.MK_ESHAPE
    assert mk.mk_kv_append(GOOD, BAD, 64, 1, 64, 0, GOOD, GOOD, 4, check=False) == mk.MK_EALIGN
    # first-layer prologue: h, w_qkv, T, hidden, Hq, Hkv, d, q_out, k_cache, v_cache, capacity, pos
    assert mk.mk_qkv_prologue(None, GOOD, 16, 4096, 8, 1, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_EINVAL
    assert mk.mk_qkv_prologue(GOOD, GOOD, 17, 4096, 8, 1, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_ESHAPE
    assert mk.mk_qkv_prologue(GOOD, GOOD, 0, 4096, 8, 1, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_ESHAPE
    assert mk.mk_qkv_prologue(GOOD, GOOD, 16, 4080, 8, 1, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_ESHAPE
    assert mk.mk_qkv_prologue(GOOD, GOOD, 16, 4096, 8, 3, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_ESHAPE
    assert mk.mk_qkv_prologue(GOOD, GOOD, 16, 4096, 8, 1, 128, GOOD, GOOD, GOOD, 64, 49, check=False) == mk.MK_ECAPACITY
    assert mk.mk_qkv_prologue(GOOD, BAD, 16, 4096, 8, 1, 128, GOOD, GOOD, GOOD, 64, 0, check=False) == mk.MK_EALIGN
    assert mk.mk_tree_accept(None, GOOD, GOOD, 16, GOOD, GOOD, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_tree_accept(GOOD, GOOD, GOOD, 65, GOOD, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_tree_accept(GOOD, GOOD, GOOD, 0, GOOD, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_kv_commit(GOOD, GOOD, 64, 1, 128, 0, None, GOOD, 16, check=False) == mk.MK_EINVAL
    assert mk.mk_kv_commit(GOOD, GOOD, 64, 1, 128, 50, GOOD, GOOD, 16, check=False) == mk.MK_ECAPACITY
    assert mk.mk_kv_commit(GOOD, GOOD, 64, 1, 60, 0, GOOD, GOOD, 16, check=False) == mk.MK_ESHAPE
    assert mk.mk_kv_commit(GOOD, GOOD, 4096, 8, 1024, 0, GOOD, GOOD, 16, check=False) == mk.MK_ESHAPE
    assert mk.mk_kv_commit(BAD, GOOD, 64, 1, 128, 0, GOOD, GOOD, 16, check=False) == mk.MK_EALIGN
    assert mk.mk_kv_commit_layers(None, GOOD, 62, 64, 1, 128, 0, GOOD, GOOD, 16, check=False) == mk.MK_EINVAL
    assert mk.mk_kv_commit_layers(GOOD, GOOD, 0, 64, 1, 128, 0, GOOD, GOOD, 16, check=False) == mk.MK_ESHAPE
    assert mk.mk_kv_commit_layers(GOOD, GOOD, 62, 64, 1, 128, 60, GOOD, GOOD, 16, check=False) == mk.MK_ECAPACITY
    assert mk.mk_route_topk(GOOD, GOOD, None, 16, 2048, 256, 9, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_route_topk(GOOD, GOOD, None, 65, 2048, 256, 8, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_route_topk(BAD, GOOD, None, 16, 2048, 256, 8, GOOD, GOOD, check=False) == mk.MK_EALIGN
    assert mk.mk_route_topk(GOOD, GOOD, None, 16, 2048, 256, 8, None, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_nvfp4_pack(GOOD, 0, 1, 16, 40, GOOD, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_nvfp4_pack(GOOD, 2, 1, 16, 32, GOOD, GOOD, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_nvfp4_pack(GOOD, 0, 1, 16, 32, BAD, GOOD, GOOD, check=False) == mk.MK_EALIGN
    assert mk.mk_nvfp4_pack(None, 0, 1, 16, 32, GOOD, GOOD, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_nvfp4_tile_w1(None, GOOD, 1, 16, 128, GOOD, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_nvfp4_tile_w1(GOOD, GOOD, 1, 24, 128, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_nvfp4_tile_w1(GOOD, GOOD, 1, 16, 192, GOOD, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_nvfp4_tile_w1(GOOD, GOOD, 1, 16, 128, BAD, GOOD, check=False) == mk.MK_EALIGN
    assert mk.mk_stream_read(None, 16, 256, GOOD, check=False) == mk.MK_EINVAL
    assert mk.mk_stream_read(GOOD, 16, 256, None, check=False) == mk.MK_EINVAL
    assert mk.mk_stream_read(GOOD, 16, -1, GOOD, check=False) == mk.MK_ESHAPE
    assert mk.mk_stream_read(GOOD, 24, 256, GOOD, check=False) == mk.MK_EALIGN
    assert mk.mk_stream_read(BAD, 16, 256, GOOD, check=False) == mk.MK_EALIGN
    assert mk.mk_stream_read(GOOD, 0, 256, GOOD, check=False) == mk.MK_OK      # nothing to read: no launch


def test_nshard_entry_validates_on_host():
    c, w, io = _cfg(), _weights(), _io()
    ns = lambda **kw: mk.mk_nshard(*[kw.get(f, d) for f, d in (("rank", 3), ("n_ranks", 8), ("act_recv", GOOD),
                                                                  ("y_recv", GOOD))])
    call = lambda cfg, n: mk.mk_layer_step_nshard(cfg, w, io, n, check=False)
    assert call(_cfg(expert_fmt=mk.MK_W_BF16), ns()) == mk.MK_EINVAL
    assert call(c, ns(n_ranks=1, rank=0)) == mk.MK_ESHAPE
    assert call(c, ns(n_ranks=9)) == mk.MK_ESHAPE
    assert call(c, ns(rank=8)) == mk.MK_ESHAPE
    assert call(c, ns(rank=-1)) == mk.MK_ESHAPE
    assert call(c, ns(n_ranks=3)) == mk.MK_ESHAPE                     # 2048 % 24 != 0
    assert call(c, ns(n_ranks=2)) == mk.MK_ESHAPE                     # 2 * 192 % 256 != 0
    assert call(c, ns(act_recv=None)) == mk.MK_EINVAL
    assert call(c, ns(y_recv=BAD)) == mk.MK_EALIGN
    assert mk.lib().mk_layer_step_nshard(ctypes_byref(c), ctypes_byref(w), ctypes_byref(io), None, None) == mk.MK_EINVAL


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)


def test_w1_scale_bytes_follow_the_piece_rule():
    # L = K/128 k-steps; 2 pieces when L > 8; 8 * ceil(L / pieces) bytes per piece and row
    assert mk.mk_nvfp4_w1_scales_bytes(1, 16, 2048) == 16 * 128       # L = 16: 2 x 64 = K/16
    assert mk.mk_nvfp4_w1_scales_bytes(3, 32, 256) == 3 * 32 * 16      # L = 2: one piece of 16
    assert mk.mk_nvfp4_w1_scales_bytes(1, 16, 1152) == 16 * 80         # L = 9: 2 x 40 > K/16 = 72
    assert mk.mk_nvfp4_w1_scales_bytes(1, 16, 1000) == 0


def test_c_host_caller_compiles_against_header(tmp_path):
    """A plain C program that includes mk.h and calls the validation paths links and runs."""
    import subprocess
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include "mk.h"
#include <stdio.h>
int main(void) {
  mk_layer_cfg c = {4096, 8, 1, 128, 2048, 256, 8, 192, 2048, MK_W_NVFP4, 8208};
  mk_layer_weights w = {0};
  mk_step_io io = {0};
  io.T = 16;
  int rc = mk_layer_step(&c, &w, &io, 0);
  printf("%d %s\n", rc, mk_strerror(rc));
  return rc == MK_EINVAL ? 0 : 1;
}
''')
    exe = tmp_path / "caller"
    lib_dir = os.path.dirname(mk.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", lib_dir, "-lmk", f"-Wl,-rpath,{lib_dir}"], capture_output=True, text=True)
    if r.returncode != 0 and "-lmk" in r.stderr:
        pytest.skip("linker could not resolve libmk by name")
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr


def test_fragment_order_untile_matches_the_documented_index():
    """The hand-off activations' layout as include/mk.h states it, element by element, against
    the reshape that tensors.untile_frag uses to read them back."""
    import numpy as np
    from layer_persistent_amd.tensors import untile_frag
    with open(os.path.join(ROOT, "include", "mk.h")) as f:
        assert "((c / 32) * 64 + ((c / 8) % 4) * 16 + t) * 8 + c % 8" in f.read()
    rng = np.random.default_rng(5)
    for T, K in ((16, 256), (5, 64), (1, 4096)):
        x = rng.integers(0, 1 << 16, size=(T, K), dtype=np.uint16)
        buf = np.zeros(16 * K, dtype=np.uint16)
        for t in range(T):
            for c in range(K):
                buf[((c // 32) * 64 + ((c // 8) % 4) * 16 + t) * 8 + c % 8] = x[t, c]
        assert np.array_equal(untile_frag(buf, T, K), x)
