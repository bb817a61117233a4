"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fa.h declares, and rejects bad arguments with the documented status
before anything is launched (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import exact_attention_forward_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_fp8", "fa_fwd_varlen", "fa_fwd_kvcache", "fa_fwd_kvcache_append", "fa_combine",
            "fa_kvcache_workspace_size", "fa_kvcache_num_splits", "fa_bwd", "fa_bwd_workspace_size",
            "fa_status_string", "fa_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libfa.so"


def test_status_strings(lib):
    for code, name in enumerate(["FA_OK", "FA_ERR_INVALID_ARGUMENT", "FA_ERR_UNSUPPORTED",
                                 "FA_ERR_WORKSPACE_TOO_SMALL", "FA_ERR_HIP"]):
        assert lib.fa_status_string(code).decode() == name


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced: validation fails first


def _opts(**kw):
    o = fa._Opts(kw.get("scale", 0.0), kw.get("causal", 0), kw.get("wl", -1), kw.get("wr", -1),
                 kw.get("softcap", 0.0), None)
    return ctypes.byref(o), o


def fwd(lib, dtype=0, B=1, Sq=8, Sk=8, Hq=2, Hkv=2, D=64, ptrs=None, strides=None, **o):
    ob, keep = _opts(**o)
    p = ptrs or [FAKE] * 5
    s = strides or [None] * 4
    return lib.fa_fwd(dtype, *p, B, Sq, Sk, Hq, Hkv, D, *s, ob, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 1),
    (dict(Hq=3, Hkv=2), 1),
    (dict(Hkv=0), 1),
    (dict(D=0), 1),
    (dict(D=80), 2),
    (dict(D=512), 2),
    (dict(B=-1), 1),
    (dict(Sk=-3), 1),
    (dict(wl=-2), 1),
    (dict(wr=-5), 1),
    (dict(softcap=-1.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(ptrs=[FAKE, None, FAKE, FAKE, FAKE]), 1),
    (dict(ptrs=[ctypes.c_void_p((1 << 20) + 2)] + [FAKE] * 4), 2),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_fwd_stride_checks(lib):
    bad = (ctypes.c_int64 * 3)(1000, 12, 64)          # 12 not a multiple of 8
    assert fwd(lib, strides=[bad, None, None, None]) == 2
    neg = (ctypes.c_int64 * 3)(-8, 128, 64)
    assert fwd(lib, strides=[None, neg, None, None]) == 1


def test_noop_sizes_return_ok(lib):
    assert fwd(lib, B=0, ptrs=[None] * 5) == 0
    assert fwd(lib, Sq=0, ptrs=[None] * 5) == 0


def test_varlen_rejects(lib):
    ob, keep = _opts()
    f = lambda **k: lib.fa_fwd_varlen(k.get("dtype", 0), FAKE, FAKE, FAKE, FAKE, FAKE, k.get("cu", FAKE), FAKE,
                                      k.get("B", 2), 16, 16, 32, 32, k.get("Hq", 4), 2, k.get("D", 64),
                                      None, None, None, None, ob, None)
    assert f(cu=None) == 1
    assert f(Hq=3) == 1
    assert f(D=80) == 2
    assert f(B=-1) == 1


def test_kvcache_workspace_and_rejects(lib):
    # out partials, lse partials, schedule order (b, len) pairs; each padded to 256 bytes
    assert lib.fa_kvcache_workspace_size(64, 1, 32, 128, 16) == 64 * 32 * 16 * 128 * 4 + 64 * 32 * 16 * 4 + 512
    assert lib.fa_kvcache_workspace_size(1, 1, 1, 64, 3) == 768 + 256 + 256
    assert lib.fa_kvcache_num_splits(64, 8, 16384, 16) == 16
    assert 1 <= lib.fa_kvcache_num_splits(64, 8, 16384, 0) <= 64
    assert lib.fa_kvcache_num_splits(1, 1, 100, 0) == 1
    ob, keep = _opts()

    def kv(ws=FAKE, wsb=1 << 30, ns=16, Hq=32, Hkv=8, Sq=1, bt=FAKE, page=256, bts=64):
        return lib.fa_fwd_kvcache(1, FAKE, FAKE, FAKE, FAKE, bt, bts, page, 100, ns, ws, wsb, FAKE, FAKE,
                                  4, Sq, Hq, Hkv, 128, ob, None)
    assert kv(wsb=100) == 3
    assert kv(ws=None) == 1
    assert kv(ws=ctypes.c_void_p((1 << 20) + 16)) == 2
    assert kv(ns=65) == 2
    assert kv(ns=-1) == 1
    assert kv(Hq=8, Hkv=8, Sq=17) == 2        # 17 query positions per kv head > 16 (heads split, positions not)
    assert kv(Hq=32, Hkv=1, Sq=17) == 2
    assert kv(page=0) == 1
    # q of more than 2^31 bytes: B * Sq * Hq * D * 2 = 2^20 * 16 * 8 * 128 * 2
    assert lib.fa_fwd_kvcache(1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 100, 16, FAKE, 1 << 40, FAKE, FAKE,
                              1 << 20, 16, 8, 8, 128, ob, None) == 2
    assert lib.fa_fwd_kvcache(1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 100, 16, FAKE, 1 << 30, FAKE, FAKE,
                              4, 1, 32, 8, 80, ob, None) == 2   # head dim 80: not built
    assert kv(bts=0) == 1


def test_kvcache_append_rejects(lib):
    """Every argument error of the append variant is reported before any launch."""
    ob, keep = _opts()
    FAKE16 = ctypes.c_void_p(1 << 20)

    def ap(kn=FAKE16, vn=FAKE16, S=3, kst=None, nb=100, ws=FAKE, wsb=1 << 30, Sq=1, bt=FAKE):
        return lib.fa_fwd_kvcache_append(1, FAKE, FAKE, FAKE, FAKE, bt, 64, 256, nb, 16, kn, vn, S, kst, None,
                                         ws, wsb, FAKE, FAKE, 4, Sq, 32, 8, 128, ob, None)
    assert ap(S=-1) == 1                      # negative number of new tokens
    assert ap(kn=None) == 1                   # new keys missing
    assert ap(vn=None) == 1
    assert ap(kn=ctypes.c_void_p((1 << 20) + 2)) == 2             # not 16-byte aligned
    assert ap(kst=(ctypes.c_int64 * 3)(3 * 8 * 128, 8 * 128, 100)) == 2   # stride not a multiple of 8
    assert ap(kst=(ctypes.c_int64 * 3)(-8, 8 * 128, 128)) == 1
    assert ap(nb=0) == 1                      # no room: empty cache
    assert ap(wsb=100) == 3                   # decode workspace checked before the append runs
    assert ap(ws=None) == 1
    assert ap(S=0, Sq=0) == 0                 # nothing to do
    assert lib.fa_fwd_kvcache_append(1, None, None, None, None, None, 0, 0, 0, 0, None, None, 0, None, None,
                                     None, 0, None, None, 0, 1, 32, 8, 128, ob, None) == 0   # B = 0


def test_fp8_rejects(lib):
    ob, keep = _opts()

    def f8(D=64, dq=1.0, dk=1.0, dv=1.0, B=1):
        return lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, B, 8, 8, 2, 2, D, None, None, None, None,
                              dq, dk, dv, ob, None)
    assert f8(D=96) == 2                      # fp8: D 64 or 128
    assert f8(D=256) == 2
    assert f8(dq=0.0) == 1
    assert f8(dk=-1.0) == 1
    assert f8(dv=float("inf")) == 1
    assert f8(dv=float("nan")) == 1
    assert f8(B=0) == 0                       # no work


def test_bwd_workspace_size(lib):
    assert lib.fa_bwd_workspace_size(4, 4096, 32) == 4 * 32 * 4096 * 4
    assert lib.fa_bwd_workspace_size(1, 3, 5) == 256           # 60 bytes padded to 256
    assert lib.fa_bwd_workspace_size(0, 8, 8) == 0
    assert lib.fa_bwd_workspace_size(2, 0, 8) == 0


def test_bwd_rejects(lib):
    """Every argument error of the backward is reported before any launch."""
    ob, keep = _opts()
    WS = ctypes.c_void_p(1 << 21)

    def bw(dtype=0, B=1, Sq=8, Sk=8, Hq=2, Hkv=2, D=64, ws=WS, wsb=1 << 20, ptrs=None, strides=None, o=None):
        p = ptrs or [FAKE] * 9          # dout, q, k, v, out, lse, dq, dk, dv
        s = strides or [None] * 5
        return lib.fa_bwd(dtype, *p, B, Sq, Sk, Hq, Hkv, D, *s, o if o is not None else ob, ws, wsb, None)
    assert bw(dtype=3) == 1
    assert bw(Hq=3, Hkv=2) == 1
    assert bw(D=48) == 2                      # D 32, 64, 96, 128 or 256
    assert bw(D=80) == 2
    assert bw(Sq=-1) == 1
    assert bw(wsb=100) == 3                   # 2*2*8*4 = 128 -> 256 bytes needed
    assert bw(ws=None) == 1
    assert bw(ws=ctypes.c_void_p((1 << 21) + 4)) == 2
    assert bw(ptrs=[None] + [FAKE] * 8) == 1  # dout
    assert bw(ptrs=[FAKE] * 8 + [None]) == 1  # dv
    assert bw(ptrs=[FAKE, ctypes.c_void_p((1 << 20) + 8)] + [FAKE] * 7) == 2   # q misaligned
    assert bw(strides=[(ctypes.c_int64 * 3)(8 * 128, 128, 60)] + [None] * 4) == 2
    assert bw(strides=[None] * 4 + [(ctypes.c_int64 * 3)(-8, 128, 64)]) == 1  # dout stride
    o2, keep2 = _opts(wl=-2)
    assert bw(o=o2) == 1
    o3, keep3 = _opts(softcap=-1.0)
    assert bw(o=o3) == 1
    assert bw(B=0) == 0                       # nothing to do
    assert bw(Sq=0, Sk=0) == 0
    assert bw(Sq=0, ws=None, wsb=0, ptrs=[None, None, FAKE, FAKE, None, None, None, FAKE, None]) == 1
    # (Sq = 0 still writes dk = dv = 0, so dv must be given)


def test_bwd_varlen_rejects(lib):
    ob, keep = _opts()
    WS = ctypes.c_void_p(1 << 21)

    def bv(B=2, mq=8, mk=8, tq=12, tk=12, D=64, ws=WS, wsb=1 << 20, cu=FAKE, ptrs=None):
        p = ptrs or [FAKE] * 9
        return lib.fa_bwd_varlen(0, *p, cu, cu, B, mq, mk, tq, tk, 2, 2, D, None, None, None, None, None, ob,
                                 ws, wsb, None)
    assert bv(D=80) == 2
    assert bv(tq=-1) == 1
    assert bv(cu=None) == 1
    assert bv(wsb=16) == 3                    # 2 heads * 12 rows * 4 bytes -> 256 needed
    assert bv(ptrs=[FAKE] * 8 + [None]) == 1  # dv
    assert bv(B=0) == 0
    assert bv(tq=0, tk=0) == 0


def test_combine_rejects(lib):
    f = lambda **k: lib.fa_combine(FAKE, FAKE, 1, 1, 1, k.get("D", 64), k.get("ns", 4), None, None,
                                   k.get("dt", 0), k.get("out", FAKE), None, None, None)
    assert f(ns=0) == 1
    assert f(ns=65) == 2
    assert f(dt=5) == 1
    assert f(out=None) == 1
    assert f(D=0) == 1


def test_python_layer_rejects_unsupported_kwargs():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q, dropout_p=0.1)
    with pytest.raises(NotImplementedError):
        fa.fwd(q, q, q, return_attn_probs=True)
    with pytest.raises(NotImplementedError):
        fa.fwd_kvcache(q, q, q, torch.zeros(1, dtype=torch.int32), cache_leftpad=q)
    with pytest.raises(ValueError):          # new keys without new values
        fa.fwd_kvcache(q, q, q, torch.zeros(1, dtype=torch.int32), k=q)
    with pytest.raises(ValueError):          # CPU tensors: no fallback path exists
        fa.fwd(q, q, q)


def test_negative_scale_rejected(lib):
    """softmax_scale 0 selects 1/sqrt(D); a negative scale is an error, not a silent default."""
    assert fwd(lib, scale=-0.5) == 1
    assert "negative" in lib.fa_last_error().decode()
    assert fwd(lib, scale=-0.5, ptrs=[None] * 5, B=0) == 1      # checked even when there is no work


def test_dispatch_work_item_bound(lib):
    """One dispatch holds at most 2^32 - 1 work-items (workgroups x threads); larger
    grids are FA_ERR_UNSUPPORTED before anything is launched, for every kernel."""
    # prefill: 33 query tiles x 64 heads x 4096 batches = 8.65M workgroups of 512 threads > 2^32
    assert fwd(lib, B=4096, Sq=33 * 256, Sk=8, Hq=64, Hkv=64) == 2
    assert "2^32" in lib.fa_last_error().decode()
    assert fwd(lib, B=4096, Sq=31 * 256, Sk=8, Hq=64, Hkv=64) != 2 or "2^32" not in lib.fa_last_error().decode()
    ob, keep = _opts()
    # KV append: B * S_new * Hkv * D/8 = 2^16 * 2^10 * 8 * 16 = 2^33 copy lanes
    assert lib.fa_fwd_kvcache_append(1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 100, 16, FAKE, FAKE, 1 << 10,
                                     None, None, FAKE, 1 << 30, FAKE, FAKE, 1 << 16, 1, 8, 8, 128, ob, None) == 2
    assert "2^32" in lib.fa_last_error().decode()
    # combine: B * S * H = 2^27 rows, 4 per 256-thread workgroup = 2^33 work-items
    assert lib.fa_combine(FAKE, FAKE, 1 << 14, 1 << 7, 1 << 6, 64, 4, None, None, 0, FAKE, None, None, None) == 2
    assert "2^32" in lib.fa_last_error().decode()
    # backward: 8.65M dQ workgroups
    WS = ctypes.c_void_p(1 << 21)
    assert lib.fa_bwd(0, *([FAKE] * 9), 4096, 33 * 256, 8, 64, 64, 64, None, None, None, None, None, ob, WS,
                      1 << 40, None) == 2
    assert "2^32" in lib.fa_last_error().decode()


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.float16)


def test_python_layer_checks_shapes_before_anything_runs():
    """The binding validates what the C ABI cannot see (tensor sizes) before any
    launch: mismatched caches, tables, lengths, outputs and slopes raise ValueError
    (checked here on CPU tensors, where the shape check comes first)."""
    import torch
    i32 = torch.int32
    q = _cpu(2, 1, 8, 64)
    kc = _cpu(10, 16, 2, 64)                       # page pool [P, page, Hkv, D]
    lens = torch.ones(2, dtype=i32)
    bt = torch.zeros(2, 4, dtype=i32)
    cases = [
        (dict(cache_seqlens=torch.ones(3, dtype=i32)), "cache_seqlens"),
        (dict(block_table=torch.zeros(3, 4, dtype=i32)), "block_table"),
        (dict(v_cache=_cpu(10, 16, 2, 32)), "one shape"),
        (dict(k_cache=_cpu(10, 16, 2, 32), v_cache=_cpu(10, 16, 2, 32)), "head_dim"),
        (dict(block_table=None, k_cache=_cpu(3, 16, 2, 64), v_cache=_cpu(3, 16, 2, 64)), "batch"),
        (dict(out=_cpu(2, 1, 8, 32)), "out must be"),
        (dict(out=_cpu(2, 1, 8, 64, dtype=torch.bfloat16)), "out must be"),
        (dict(lse=torch.zeros(2, 8, 2)), "lse must be"),
        (dict(k=_cpu(2, 1, 3, 64), v=_cpu(2, 1, 3, 64)), "S_new"),
    ]
    for over, match in cases:
        args = dict(q=q, k_cache=kc, v_cache=kc, cache_seqlens=lens, block_table=bt)
        args.update(over)
        with pytest.raises(ValueError, match=match):
            fa.fwd_kvcache(**args)
    qd, kd = _cpu(1, 8, 4, 64), _cpu(1, 8, 2, 64)
    with pytest.raises(ValueError, match="out must be"):
        fa.fwd(qd, kd, kd, out=_cpu(1, 8, 4, 32))
    with pytest.raises(ValueError, match="lse must be"):
        fa.fwd(qd, kd, kd, lse=torch.zeros(1, 4, 7))
    with pytest.raises(ValueError, match="lse must be"):
        fa.fwd(qd, kd, kd, lse=torch.zeros(1, 4, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="batch / head_dim"):
        fa.fwd(qd, _cpu(2, 8, 2, 64), _cpu(2, 8, 2, 64))
    cu = torch.tensor([0, 8], dtype=i32)
    with pytest.raises(ValueError, match="lse must be"):
        fa.fwd_varlen(qd[0], kd[0], kd[0], cu, cu, 8, 8, lse=torch.zeros(4, 9))
    with pytest.raises(ValueError, match="head_dim"):
        fa.fwd_varlen(qd[0], kd[0, :, :, :32], kd[0, :, :, :32], cu, cu, 8, 8)
    op, lp = torch.zeros(1, 1, 2, 64, 3), torch.zeros(1, 1, 2, 3)
    with pytest.raises(ValueError, match="out must be"):
        fa.combine(op, lp, out=_cpu(1, 1, 2, 32))
    with pytest.raises(ValueError, match="lse must be"):
        fa.combine(op, lp, lse=torch.zeros(1, 1, 3))


def test_noalloc_rejects_beyond_its_static_workspace(lib):
    """fa_fwd_kvcache_noalloc: a decode whose workspace exceeds the static array
    is FA_ERR_UNSUPPORTED before anything touches the GPU; other errors are those
    of fa_fwd_kvcache."""
    ob, keep = _opts()
    cap = lib.fa_kvcache_noalloc_max_bytes()
    assert cap == 32 << 20
    f = lambda B=64, Sq=1, Hq=32, Hkv=8, D=128, ns=64: lib.fa_fwd_kvcache_noalloc(
        1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 100, ns, FAKE, FAKE, B, Sq, Hq, Hkv, D, ob, None)
    assert lib.fa_kvcache_workspace_size(64, 1, 32, 128, 64) > cap
    assert f() == 2 and "static scratch" in lib.fa_last_error().decode()
    assert f(D=80) == 2                     # head dim not built
    assert f(Hq=30) == 1                    # Hkv must divide Hq
    assert f(ns=-1) == 1
    assert f(B=0) == 0                      # no work: nothing touched
