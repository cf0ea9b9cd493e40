"""The C ABI without a GPU: the library loads, exports every function that
include/dv.h declares, sizes workspaces, and rejects bad arguments on the host
before anything is enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from contextual_sparsity_mlp_amd import dv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dv.h")

# Fake, never dereferenced device addresses: aligned and misaligned.
P = 0x7f0000000000
BAD = P + 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = dv.lib()
    names = declared_functions()
    assert set(names) == set(dv.EXPORTS), f"header {names} vs binding {dv.EXPORTS}"
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert lib.dv_version() == 104


def test_library_has_gfx950_code():
    # the shared object carries a gfx950 code object (offload bundle)
    blob = open(dv.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def ws_bytes(op, **kw):
    return dv.workspace_bytes(op, **kw)


def test_workspace_sizes_c4():
    b1 = ws_bytes(dv.OP_DECODE_LAYER, batch=1, d=12288, F=49152, h=96, dh=128, n_ctx=2048, r=1000,
                  max_count_m=4915, max_count_a=19)
    b16 = ws_bytes(dv.OP_DECODE_LAYER, batch=16, d=12288, F=49152, h=96, dh=128, n_ctx=2048,
                   r=1000, max_count_m=49152, max_count_a=96)
    assert 1 << 20 < b1 < 64 << 20
    assert b1 < b16 < 2 << 30
    assert ws_bytes(dv.OP_SELECT_TOPK, batch=4, N=49152) >= 4 * 49152 // 8
    assert ws_bytes(dv.OP_SPARSE_MLP, batch=1, d=256, max_count_m=0) > 0


def test_workspace_bad_shape():
    with pytest.raises(dv.DvError):
        ws_bytes(dv.OP_SPARSE_MLP, batch=0, d=256, max_count_m=3)
    with pytest.raises(dv.DvError):
        ws_bytes(99, batch=1)
    assert dv.lib().dv_workspace_bytes(dv.OP_PREDICT, None) == 0


def call_mlp(**over):
    a = dict(y=P, batch=1, d=256, W1t=P, W2t=P, F=1024, wdt=dv.DV_BF16, idx=P, count=P,
             max_count=10, out=P + 4096, acc=0, act=dv.DV_ACT_RELU, ws=P, ws_bytes=1 << 30,
             stream=None)
    a.update(over)
    return dv.lib().dv_sparse_mlp(a["y"], a["batch"], a["d"], a["W1t"], a["W2t"], a["F"], a["wdt"],
                                  a["idx"], a["count"], a["max_count"], a["out"], a["acc"], a["act"],
                                  a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(y=None), dv.DV_EINVAL), (dict(W2t=None), dv.DV_EINVAL), (dict(count=None), dv.DV_EINVAL),
    (dict(batch=0), dv.DV_EINVAL), (dict(F=0), dv.DV_EINVAL), (dict(max_count=-1), dv.DV_EINVAL),
    (dict(max_count=1025), dv.DV_EINVAL), (dict(wdt=7), dv.DV_EINVAL),
    (dict(d=260), dv.DV_EALIGN), (dict(d=0), dv.DV_EINVAL), (dict(d=20000), dv.DV_EUNSUPPORTED),
    (dict(W1t=BAD), dv.DV_EALIGN), (dict(out=BAD), dv.DV_EALIGN), (dict(idx=BAD), dv.DV_EALIGN),
    (dict(ws=None), dv.DV_EWORKSPACE), (dict(ws_bytes=100), dv.DV_EWORKSPACE),
    (dict(ws=BAD), dv.DV_EALIGN), (dict(out=P), dv.DV_EINVAL),
    (dict(act=2), dv.DV_EINVAL), (dict(act=-1), dv.DV_EINVAL),
    (dict(wdt=dv.DV_FP8), dv.DV_EUNSUPPORTED),
])
def test_sparse_mlp_rejects(over, code):
    assert call_mlp(**over) == code
    assert dv.last_error().startswith("dv_sparse_mlp")


def call_mha(**over):
    a = dict(y=P, batch=2, d=256, h=4, dh=64, Wq=P, Wo=P, wdt=dv.DV_BF16, K=P, V=P, n_ctx=32,
             kvdt=dv.DV_BF16, heads=P, count=P, max_count=2, scale=1.0, out=P + 4096, acc=0, ws=P,
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    return dv.lib().dv_sparse_mha(*[a[k] for k in ("y", "batch", "d", "h", "dh", "Wq", "Wo", "wdt",
                                                   "K", "V", "n_ctx", "kvdt", "heads", "count",
                                                   "max_count", "scale", "out", "acc", "ws",
                                                   "ws_bytes", "stream")])


@pytest.mark.parametrize("over,code", [
    (dict(K=None), dv.DV_EINVAL), (dict(n_ctx=0), dv.DV_EINVAL), (dict(h=0), dv.DV_EINVAL),
    (dict(max_count=5), dv.DV_EINVAL), (dict(dh=48), dv.DV_EUNSUPPORTED),
    (dict(dh=512), dv.DV_EUNSUPPORTED), (dict(n_ctx=(1 << 20) + 1), dv.DV_EUNSUPPORTED),
    (dict(V=BAD), dv.DV_EALIGN), (dict(kvdt=3), dv.DV_EINVAL), (dict(scale=float("nan")), dv.DV_EINVAL),
    (dict(ws_bytes=16), dv.DV_EWORKSPACE), (dict(d=12), dv.DV_EALIGN),
])
def test_sparse_mha_rejects(over, code):
    assert call_mha(**over) == code
    assert dv.last_error().startswith("dv_sparse_mha")


@pytest.mark.parametrize("args,code", [
    (dict(k=-1), dv.DV_EINVAL), (dict(k=1001), dv.DV_EINVAL), (dict(N=0), dv.DV_EINVAL),
    (dict(batch=0), dv.DV_EINVAL), (dict(scores=None), dv.DV_EINVAL), (dict(idx=BAD), dv.DV_EALIGN),
    (dict(ws=None), dv.DV_EWORKSPACE),
])
def test_select_topk_rejects(args, code):
    a = dict(scores=P, batch=3, N=1000, k=10, union=1, idx=P, count=P, ws=P, ws_bytes=1 << 20)
    a.update(args)
    rc = dv.lib().dv_select_topk(a["scores"], a["batch"], a["N"], a["k"], a["union"], a["idx"],
                                 a["count"], a["ws"], a["ws_bytes"] if a["ws"] else 0, None)
    assert rc == code
    assert dv.last_error().startswith("dv_select_topk")


@pytest.mark.parametrize("args,code", [
    (dict(A=None), dv.DV_EINVAL), (dict(r=0), dv.DV_EINVAL), (dict(N=-3), dv.DV_EINVAL),
    (dict(Bm=BAD), dv.DV_EALIGN), (dict(ws_bytes=8), dv.DV_EWORKSPACE), (dict(d=100), dv.DV_EALIGN),
])
def test_predict_rejects(args, code):
    a = dict(y=P, batch=1, d=256, A=P, Bm=P, r=64, N=1024, wdt=dv.DV_F32, scores=P, ws=P,
             ws_bytes=1 << 30)
    a.update(args)
    rc = dv.lib().dv_predict(a["y"], a["batch"], a["d"], a["A"], a["Bm"], a["r"], a["N"], a["wdt"],
                             a["scores"], a["ws"], a["ws_bytes"], None)
    assert rc == code
    assert dv.last_error().startswith("dv_predict")


def _layer(**over):
    s = dv.LayerStruct(d=256, F=1024, h=4, dh=64, n_ctx=32, r=64, k_m=154, k_a=2, wdt=dv.DV_BF16,
                       kvdt=dv.DV_BF16, scale=1.0, W1t=P, W2t=P, Wq=P, Wo=P, K=P, V=P, A_M=P,
                       B_M=P, A_A=P, B_A=P)
    for k, v in over.items():
        setattr(s, k, v)
    return s


@pytest.mark.parametrize("lo,no,args,code", [
    (dict(), dict(), dict(), None),
    (dict(W1t=None), dict(), dict(), dv.DV_EINVAL),
    (dict(dh=100), dict(), dict(), dv.DV_EUNSUPPORTED),
    (dict(), dict(d=512), dict(), dv.DV_EINVAL),
    (dict(), dict(k_m=2000), dict(), dv.DV_EINVAL),
    (dict(), dict(B_M=None), dict(), dv.DV_EINVAL),
    (dict(), dict(pwdt=7), dict(), dv.DV_EINVAL),
    (dict(wdt=dv.DV_FP8), dict(), dict(), dv.DV_EINVAL),                  # fp8 without scales
    (dict(wdt=dv.DV_FP8, d=264, W1s=P, W2s=P, Wqs=P, Wos=P), dict(d=264), dict(), dv.DV_EALIGN),
    (dict(wdt=dv.DV_FP8, W1s=P, W2s=BAD, Wqs=P, Wos=P), dict(), dict(), dv.DV_EALIGN),
    (dict(), dict(), dict(next_idx_m=None), dv.DV_EINVAL),
    (dict(), dict(), dict(max_count_a=9), dv.DV_EINVAL),
    (dict(K=BAD), dict(), dict(), dv.DV_EALIGN),
    (dict(), dict(), dict(ws_bytes=64), dv.DV_EWORKSPACE),
    (dict(n_ctx=0), dict(), dict(), dv.DV_EINVAL),
    (dict(act=5), dict(), dict(), dv.DV_EINVAL),
    # the KV append: both W^K and W^V, a cache row to append to, aligned pointers
    (dict(Wk=P), dict(), dict(), dv.DV_EINVAL),
    (dict(Wk=P, Wv=P), dict(), dict(), dv.DV_EINVAL),                     # kv_cap 0 = n_ctx: no room
    (dict(Wk=P, Wv=P, kv_cap=32), dict(), dict(), dv.DV_EINVAL),
    (dict(Wk=P, Wv=P, kv_cap=33, n_ctx=-1), dict(), dict(), dv.DV_EINVAL),
    (dict(Wk=P, Wv=BAD, kv_cap=33), dict(), dict(), dv.DV_EALIGN),
    (dict(wdt=dv.DV_FP8, W1s=P, W2s=P, Wqs=P, Wos=P, Wk=P, Wv=P, kv_cap=33), dict(), dict(),
     dv.DV_EINVAL),                                                         # fp8 W^K without scales
    (dict(kv_cap=16), dict(), dict(), dv.DV_EINVAL),                      # cache smaller than n_ctx
    (dict(kv_cap=-1), dict(), dict(), dv.DV_EINVAL),
])
def test_decode_layer_rejects(lo, no, args, code):
    a = dict(batch=1, y_in=P, y_out=P, idx_m=P, count_m=P, max_count_m=154, idx_a=P, count_a=P,
             max_count_a=2, next_idx_m=P, next_count_m=P, next_idx_a=P, next_count_a=P, ws=P,
             ws_bytes=1 << 30)
    a.update(args)
    if code is None:
        return  # the valid call would launch; covered by the GPU tests
    L, N = _layer(**lo), _layer(**no)
    rc = dv.lib().dv_decode_layer(ctypes.byref(L), ctypes.byref(N), a["batch"], a["y_in"],
                                  a["y_out"], a["idx_m"], a["count_m"], a["max_count_m"],
                                  a["idx_a"], a["count_a"], a["max_count_a"], a["next_idx_m"],
                                  a["next_count_m"], a["next_idx_a"], a["next_count_a"], a["ws"],
                                  a["ws_bytes"], None)
    assert rc == code, dv.last_error()
    assert dv.last_error().startswith("dv_decode_layer")


def test_decode_layer_noalloc_rejects_oversized():
    """The allocation-free entry point refuses shapes whose workspace exceeds the
    library's scratch (OPT-175B at batch 4 with the look-ahead predictor) on the host,
    and runs every other argument check of dv_decode_layer first."""
    lib = dv.lib()
    assert lib.dv_noalloc_scratch_bytes() == 64 << 20
    big = dict(d=12288, F=49152, h=96, dh=128, n_ctx=2048, r=1000, k_m=4915, k_a=19,
               pwdt=dv.DV_BF16)
    B = 4
    need = dv.workspace_bytes(dv.OP_DECODE_LAYER, batch=B, d=12288, F=49152, h=96, dh=128,
                              n_ctx=2048, r=1000, max_count_m=B * 4915, max_count_a=B * 19)
    assert need > lib.dv_noalloc_scratch_bytes()
    L, N = _layer(**big), _layer(**big)

    def call(L, N, max_m, max_a):
        return lib.dv_decode_layer_noalloc(ctypes.byref(L), ctypes.byref(N), B, P, P, P, P, max_m,
                                           P, P, max_a, P, P, P, P, None)
    assert call(L, N, B * 4915, min(96, B * 19)) == dv.DV_EWORKSPACE
    assert "scratch" in dv.last_error() and dv.last_error().startswith("dv_decode_layer_noalloc")
    # the shared argument checks come first
    assert call(_layer(**dict(big, W1t=None)), N, B * 4915, min(96, B * 19)) == dv.DV_EINVAL
    assert call(_layer(**dict(big, K=BAD)), N, B * 4915, min(96, B * 19)) == dv.DV_EALIGN


def test_timing_read_empty():
    ms, cnt = dv.timing_read(4)
    assert ms == [] and cnt == []


def test_step_path_selector():
    """dv_set_step_path takes the three plans and rejects anything else (no launch)."""
    lib = dv.lib()
    for p in (dv.PATH_ONE_LAUNCH, dv.PATH_TWO_LAUNCH, dv.PATH_AUTO):
        assert lib.dv_set_step_path(p) == dv.DV_OK
    for bad in (-1, 3, 99):
        assert lib.dv_set_step_path(bad) == dv.DV_EINVAL
        assert "dv_set_step_path" in dv.last_error()
    assert lib.dv_set_step_path(dv.PATH_AUTO) == dv.DV_OK


def test_wait_limits_hook():
    """dv_debug_wait_limits sets and restores the in-launch wait limits (no launch)."""
    lib = dv.lib()
    assert lib.dv_debug_wait_limits(64, 1) == dv.DV_OK
    assert lib.dv_debug_wait_limits(0, 0) == dv.DV_OK
