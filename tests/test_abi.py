"""The C-ABI library without a GPU: it loads, exports every symbol the headers
declare, and rejects bad arguments before launching anything."""
import ctypes
import glob
import os
import re

import pytest

import paged_kv_cache_448_amd as pkv
from paged_kv_cache_448_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, E_NULL, E_SHAPE, E_UNSUPPORTED, E_WORKSPACE = 0, -1, -2, -3, -4


def declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        names.update(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 20
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for n in sorted(names):
        assert hasattr(handle, n), f"{n} declared but not exported"
    assert names == set(_lib.PROTOTYPES), names ^ set(_lib.PROTOTYPES)


def test_status_strings():
    L = pkv.lib()
    for s in range(-8, 1):
        assert L.pkv_status_str(s)
    assert L.pkv_status_str(-99) == b"unknown status"


NULL = None


def _decode(**kw):
    a = dict(q=16, kc=16, vc=16, bt=16, mb=4, cl=16, mcl=64, scale=0.125, out=16, B=2, Hq=4, Hkv=2, D=64, bs=16,
             N=8, dt=0, ws=NULL, wsb=0, pt=0, impl=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_paged_attn_decode_ex(p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]),
                                              a["mcl"], ctypes.c_float(a["scale"]), p(a["out"]), a["B"], a["Hq"],
                                              a["Hkv"], a["D"], a["bs"], a["N"], a["dt"], p(a["ws"]),
                                              ctypes.c_size_t(a["wsb"]), a["pt"], a["impl"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), E_NULL), (dict(out=NULL), E_NULL), (dict(bt=NULL), E_NULL),
    (dict(Hq=6, Hkv=4), E_SHAPE), (dict(mcl=65), E_SHAPE), (dict(B=-1), E_SHAPE), (dict(N=0), E_SHAPE),
    (dict(pt=24), E_SHAPE), (dict(q=8), E_SHAPE),
    (dict(D=96), E_UNSUPPORTED), (dict(bs=24), E_UNSUPPORTED), (dict(bs=2048, mcl=64), E_UNSUPPORTED),
    (dict(dt=5), E_UNSUPPORTED), (dict(impl=9), E_UNSUPPORTED), (dict(Hq=6, Hkv=2), E_UNSUPPORTED),
    (dict(pt=16), E_WORKSPACE), (dict(pt=16, ws=256, wsb=10), E_WORKSPACE), (dict(B=0), OK),
])
def test_decode_rejects_bad_arguments_before_launch(kw, status):
    assert _decode(**kw) == status


def _append(**kw):
    a = dict(k=16, v=16, sm=16, T=3, kc=16, vc=16, N=4, bs=16, Hkv=2, D=64, dt=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_kv_append(p(a["k"]), p(a["v"]), p(a["sm"]), a["T"], p(a["kc"]), p(a["vc"]), a["N"],
                                   a["bs"], a["Hkv"], a["D"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=NULL), E_NULL), (dict(sm=NULL), E_NULL), (dict(T=-1), E_SHAPE), (dict(N=0), E_SHAPE),
    (dict(k=24), E_SHAPE), (dict(D=12), E_UNSUPPORTED), (dict(bs=8), E_UNSUPPORTED), (dict(dt=2), E_UNSUPPORTED),
    (dict(T=0, k=NULL), OK),
])
def test_append_rejects_bad_arguments_before_launch(kw, status):
    assert _append(**kw) == status


def test_workspace_and_plan():
    # the Llama-3.2-1B batch shape: 64 sequences x 8 kv heads, contexts up to 2048 -> one pass, no workspace
    assert pkv.plan_partition(64, 8, 16, 2048) == 0
    assert pkv.decode_workspace_bytes(64, 32, 8, 64, 16, 2048) == 0
    # the long-context shape: 16 x 8 units cannot fill 256 compute units -> 1536-token partitions
    pt = pkv.plan_partition(16, 8, 256, 8192)
    assert pt == 1536
    assert pkv.decode_workspace_bytes(16, 32, 8, 64, 256, 8192) >= 16 * 32 * 4 * (64 + 2) * 4
    # a forced split sizes the workspace for its partitions
    assert pkv.decode_workspace_bytes(64, 32, 8, 64, 16, 2048, partition_tokens=512) >= 64 * 32 * 4 * (64 + 2) * 4
    # a context that fits one partition needs no workspace
    assert pkv.decode_workspace_bytes(64, 32, 8, 64, 16, 2048, partition_tokens=4096) == 0
    assert pkv.decode_workspace_bytes(2, 4, 2, 64, 16, 37) == 0
    # partitions never exceed 8192 tokens, whatever is asked for
    assert pkv.plan_partition(4, 8, 16, 100000) <= 8192
    assert pkv.decode_workspace_bytes(4, 32, 8, 64, 16, 100000, partition_tokens=100000) >= 4 * 32 * 13 * (64 + 2) * 4
    assert pkv.decode_supported("simt", "bf16", 64, 4)
    assert not pkv.decode_supported("simt", "bf16", 96, 4)


def _fused(**kw):
    a = dict(q=16, kn=16, vn=16, sm=16, kc=16, vc=16, bt=16, mb=4, cl=16, mcl=64, scale=0.125, out=16, B=2, Hq=4,
             Hkv=2, D=64, bs=16, N=8, dt=0, ws=NULL, wsb=0, pt=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_append_paged_attn_decode(
        p(a["q"]), p(a["kn"]), p(a["vn"]), p(a["sm"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]),
        a["mcl"], ctypes.c_float(a["scale"]), p(a["out"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["N"],
        a["dt"], p(a["ws"]), ctypes.c_size_t(a["wsb"]), a["pt"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(sm=NULL), E_NULL), (dict(kn=NULL), E_NULL), (dict(vn=NULL), E_NULL), (dict(q=NULL), E_NULL),
    (dict(kn=24), E_SHAPE), (dict(Hq=6, Hkv=4), E_SHAPE), (dict(D=96), E_UNSUPPORTED), (dict(dt=3), E_UNSUPPORTED),
    (dict(Hq=64, Hkv=2), E_UNSUPPORTED), (dict(B=0, sm=NULL), OK),
])
def test_fused_append_decode_rejects_bad_arguments_before_launch(kw, status):
    assert _fused(**kw) == status


def _append_fp8(**kw):
    a = dict(k=16, v=16, sm=16, T=3, kc=16, vc=16, N=4, bs=16, Hkv=2, D=64, dt=0, ks=0.5, vs=0.25)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_kv_append_fp8(p(a["k"]), p(a["v"]), p(a["sm"]), a["T"], p(a["kc"]), p(a["vc"]), a["N"],
                                       a["bs"], a["Hkv"], a["D"], a["dt"], ctypes.c_float(a["ks"]),
                                       ctypes.c_float(a["vs"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=NULL), E_NULL), (dict(vc=NULL), E_NULL), (dict(T=-1), E_SHAPE), (dict(kc=8), E_SHAPE),
    (dict(ks=0.0), E_SHAPE), (dict(vs=-1.0), E_SHAPE), (dict(ks=float("inf")), E_SHAPE), (dict(vs=float("nan")), E_SHAPE),
    (dict(D=12), E_UNSUPPORTED), (dict(bs=8), E_UNSUPPORTED), (dict(dt=2), E_UNSUPPORTED), (dict(T=0, k=NULL), OK),
])
def test_append_fp8_rejects_bad_arguments_before_launch(kw, status):
    assert _append_fp8(**kw) == status


def _decode_fp8(**kw):
    a = dict(q=16, kc=16, vc=16, bt=16, mb=4, cl=16, mcl=64, scale=0.125, ks=0.5, vs=0.25, out=16, B=2, Hq=4, Hkv=2,
             D=64, bs=16, N=8, dt=0, ws=NULL, wsb=0, pt=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_paged_attn_decode_fp8(
        p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]), a["mcl"], ctypes.c_float(a["scale"]),
        ctypes.c_float(a["ks"]), ctypes.c_float(a["vs"]), p(a["out"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"],
        a["N"], a["dt"], p(a["ws"]), ctypes.c_size_t(a["wsb"]), a["pt"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), E_NULL), (dict(kc=NULL), E_NULL), (dict(out=NULL), E_NULL),
    (dict(ks=0.0), E_SHAPE), (dict(vs=float("inf")), E_SHAPE), (dict(ks=float("nan")), E_SHAPE),
    (dict(Hq=6, Hkv=4), E_SHAPE), (dict(mcl=65), E_SHAPE), (dict(pt=24), E_SHAPE), (dict(vc=8), E_SHAPE),
    (dict(D=96), E_UNSUPPORTED), (dict(dt=4), E_UNSUPPORTED), (dict(Hq=64, Hkv=2), E_UNSUPPORTED),
    (dict(pt=16), E_WORKSPACE), (dict(B=0), OK),
])
def test_decode_fp8_rejects_bad_arguments_before_launch(kw, status):
    assert _decode_fp8(**kw) == status


def _prefill(**kw):
    a = dict(q=16, kc=16, vc=16, bt=16, mb=4, cl=16, qs=16, T=8, mql=8, mcl=64, scale=0.125, out=16, B=2, Hq=4,
             Hkv=2, D=64, bs=16, N=8, dt=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_paged_prefill(p(a["q"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]), p(a["qs"]),
                                       a["T"], a["mql"], a["mcl"], ctypes.c_float(a["scale"]), p(a["out"]), a["B"],
                                       a["Hq"], a["Hkv"], a["D"], a["bs"], a["N"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), E_NULL), (dict(qs=NULL), E_NULL), (dict(out=NULL), E_NULL), (dict(cl=NULL), E_NULL),
    (dict(T=-1), E_SHAPE), (dict(mql=-1), E_SHAPE), (dict(mcl=65), E_SHAPE), (dict(Hq=6, Hkv=4), E_SHAPE),
    (dict(scale=0.0), E_SHAPE), (dict(scale=-0.5), E_SHAPE), (dict(scale=float("nan")), E_SHAPE), (dict(q=8), E_SHAPE),
    (dict(D=96), E_UNSUPPORTED), (dict(dt=3), E_UNSUPPORTED), (dict(Hq=6, Hkv=2), E_UNSUPPORTED),
    (dict(bs=24), E_UNSUPPORTED), (dict(B=0), OK), (dict(T=0, q=NULL), OK), (dict(mql=0), OK),
])
def test_prefill_rejects_bad_arguments_before_launch(kw, status):
    assert _prefill(**kw) == status


def _fused_fp8(**kw):
    a = dict(q=16, kn=16, vn=16, sm=16, kc=16, vc=16, bt=16, mb=4, cl=16, mcl=64, scale=0.125, ks=0.5, vs=0.25, out=16,
             B=2, Hq=4, Hkv=2, D=64, bs=16, N=8, dt=0, ws=NULL, wsb=0, pt=0)
    a.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return pkv.lib().pkv_append_paged_attn_decode_fp8(
        p(a["q"]), p(a["kn"]), p(a["vn"]), p(a["sm"]), p(a["kc"]), p(a["vc"]), p(a["bt"]), a["mb"], p(a["cl"]),
        a["mcl"], ctypes.c_float(a["scale"]), ctypes.c_float(a["ks"]), ctypes.c_float(a["vs"]), p(a["out"]), a["B"],
        a["Hq"], a["Hkv"], a["D"], a["bs"], a["N"], a["dt"], p(a["ws"]), ctypes.c_size_t(a["wsb"]), a["pt"], None,
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(sm=NULL), E_NULL), (dict(kn=NULL), E_NULL), (dict(vn=NULL), E_NULL), (dict(q=NULL), E_NULL),
    (dict(kn=24), E_SHAPE), (dict(ks=0.0), E_SHAPE), (dict(vs=float("nan")), E_SHAPE), (dict(Hq=6, Hkv=4), E_SHAPE),
    (dict(D=96), E_UNSUPPORTED), (dict(dt=3), E_UNSUPPORTED), (dict(Hq=64, Hkv=2), E_UNSUPPORTED),
    (dict(pt=16), E_WORKSPACE), (dict(B=0, sm=NULL), OK),
])
def test_fused_fp8_rejects_bad_arguments_before_launch(kw, status):
    assert _fused_fp8(**kw) == status


def test_workspace_query_covers_every_shorter_bound():
    """The automatic plan may cut a shorter longest context into more partitions;
    the workspace query at a bound covers every bound below it."""
    for B, Hkv in ((3, 8), (7, 8), (14, 2), (16, 8), (64, 1), (256, 8)):
        for mc in (512, 4096, 8192):
            top = pkv.decode_workspace_bytes(B, 4 * Hkv, Hkv, 64, 16, mc)
            for m in range(16, mc + 1, 16):
                assert pkv.decode_workspace_bytes(B, 4 * Hkv, Hkv, 64, 16, m) <= top, (B, Hkv, mc, m)


def test_noalloc_refuses_plans_beyond_its_scratch_before_touching_the_device():
    # 4096 sequences up to 8192 tokens, 32 q / 8 kv heads of 128 dims: the split
    # plan's partial states need far more than the 16 MiB device scratch
    p = ctypes.c_void_p(256)
    st = pkv.lib().pkv_paged_attn_decode_noalloc(p, p, p, p, 32, p, 8192, ctypes.c_float(0.1), p, 4096, 32, 8, 128,
                                                 256, 1 << 16, 0, None)
    assert st == E_WORKSPACE
