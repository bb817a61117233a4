"""Seeded random sweep of small problems through every call, each checked
against the oracle with the same bars as the hand-written cases.  The shapes
are drawn so that head counts, lengths and window sides are often odd (head
counts not divisible by 8, lengths off tile boundaries, Sq > Sk), which the
fixed cases cover only in part."""

import numpy as np
import pytest
import torch

import exact_attention_forward_fa_amd as fa
from exact_attention_forward_fa_amd import inputs
from oracle import ref

from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HEAD_DIMS = [32, 64, 96, 128, 256]
U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def draw(seed):
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2, 3]))
    G = int(r.choice([1, 2, 3, 4]))
    o = dict(causal=bool(r.random() < 0.6))
    if r.random() < 0.3:
        o["window"] = (int(r.integers(-1, 90)), int(r.integers(-1, 90)))
    if r.random() < 0.3:
        o["softcap"] = float(r.uniform(1.0, 20.0))
    if r.random() < 0.3:
        o["alibi"] = True
    if r.random() < 0.2:
        o["softmax_scale"] = float(r.uniform(0.05, 0.3))
    return dict(B=int(r.integers(1, 4)), Sq=int(r.integers(1, 300)), Sk=int(r.integers(1, 300)), Hkv=Hkv, Hq=Hkv * G,
                D=int(r.choice(HEAD_DIMS)), dt=torch.float16 if r.random() < 0.5 else torch.bfloat16, o=o)


def kw_of(c):
    o = c["o"]
    slopes = inputs.alibi_slopes(c["Hq"]) if o.get("alibi") else None
    return slopes, dict(softmax_scale=o.get("softmax_scale"), causal=o["causal"], window_size=o.get("window", (-1, -1)),
                        softcap=o.get("softcap", 0.0))


def oracle_kw(c, slopes):
    o = c["o"]
    return dict(softmax_scale=o.get("softmax_scale"), causal=o["causal"], window=o.get("window", (-1, -1)),
                softcap=o.get("softcap", 0.0), alibi_slopes=slopes)


@pytest.mark.parametrize("seed", range(48))
def test_random_dense_forward_and_backward(seed):
    c = draw(7000 + seed)
    print("case", seed, c, flush=True)
    q, k, v = inputs.dense_qkv(c["B"], c["Sq"], c["Sk"], c["Hq"], c["Hkv"], c["D"], c["dt"], seed=7100 + seed)
    slopes, kw = kw_of(c)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    sd = None if slopes is None else slopes.to(DEV)
    out, lse = fa.fwd(qd, kd, vd, alibi_slopes=sd, **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention(q, k, v, **oracle_kw(c, slopes))
    check(out.cpu(), lse.cpu(), ro, rl, c["dt"], f"random fwd {seed}")
    g = inputs.randn(torch.Generator().manual_seed(7200 + seed), q.shape, c["dt"])
    dq, dk, dv = fa.bwd(g.to(DEV), qd, kd, vd, out, lse, alibi_slopes=sd, **kw)
    torch.cuda.synchronize()
    want = ref.attention_backward(q, k, v, g, **oracle_kw(c, slopes))
    u = U[c["dt"]]
    floor = max(float(np.abs(w).max(initial=0.0)) for w in want)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        x = got.cpu().double().numpy()
        assert np.isfinite(x).all(), (seed, name)
        err = float(np.abs(x - w).max(initial=0.0))
        scale = float(np.abs(w).max(initial=0.0)) or floor
        assert err <= 4 * u * max(scale, 1e-30) + 1e-30, (seed, name, err, scale)


@pytest.mark.parametrize("seed", range(16))
def test_random_varlen_forward(seed):
    r = np.random.default_rng(7300 + seed)
    n = int(r.integers(1, 5))
    lq = [int(x) for x in r.integers(0, 200, n)]
    lk = [int(x) for x in r.integers(0, 200, n)]
    c = draw(7400 + seed)
    if sum(lq) == 0:
        lq[0] = 1
    print("case", seed, lq, lk, c, flush=True)
    q, k, v, cq, ck = inputs.varlen_pack(lq, lk, c["Hq"], c["Hkv"], c["D"], c["dt"], seed=7500 + seed)
    slopes, kw = kw_of(c)
    out, lse = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), max(lq), max(max(lk), 1),
                             alibi_slopes=None if slopes is None else slopes.to(DEV), **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention_varlen(q, k, v, cq, ck, **oracle_kw(c, slopes))
    check(out.cpu(), lse.cpu(), ro, rl, c["dt"], f"random varlen {seed}")


@pytest.mark.parametrize("seed", range(32))
def test_random_kvcache(seed):
    r = np.random.default_rng(7600 + seed)
    c = draw(7700 + seed)
    B = c["B"]
    Sq = int(r.integers(1, 5))
    page = int(r.choice([0, 16, 64, 256]))
    lens = [int(x) for x in r.integers(Sq, 700, B)]
    print("case", seed, Sq, page, lens, c, flush=True)
    pc = inputs.paged_cache(B, Sq, c["Hq"], c["Hkv"], c["D"], c["dt"], seed=7800 + seed, page_size=page or 64,
                            lengths=lens, tail_fill="nan")
    slopes, kw = kw_of(c)
    sd = None if slopes is None else slopes.to(DEV)
    ns = int(r.integers(0, 9))
    if page:
        out, lse = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV),
                                  block_table=pc.block_table.to(DEV), num_splits=ns, alibi_slopes=sd, **kw)
    else:
        kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
        vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
        out, lse = fa.fwd_kvcache(pc.q.to(DEV), kd.to(DEV), vd.to(DEV), pc.cache_seqlens.to(DEV), num_splits=ns,
                                  alibi_slopes=sd, **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page or 64,
                                   **oracle_kw(c, slopes))
    check(out.cpu(), lse.cpu(), ro, rl, c["dt"], f"random kvcache {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_kvcache_adjacent_heads(seed):
    """Seeded sweep over the shapes whose decode, with finite_cache=True, reads
    2, 4 or 8 adjacent kv heads as one work item (D = 32 and 64, kv head counts 2, 4 and 8, few query
    rows per kv head), with random options, pages and splits."""
    r = np.random.default_rng(8100 + seed)
    c = draw(8200 + seed)
    Hkv = int(r.choice([2, 4, 8]))
    G = int(r.choice([1, 2]))
    D = int(r.choice([32, 64]))
    B = int(r.integers(1, 5))
    Sq = int(r.integers(1, 3))
    page = int(r.choice([16, 64, 256]))
    lens = [int(x) for x in r.integers(Sq, 900, B)]
    print("case", seed, B, Sq, Hkv * G, Hkv, D, page, lens, c["dt"], c["o"], flush=True)
    pc = inputs.paged_cache(B, Sq, Hkv * G, Hkv, D, c["dt"], seed=8300 + seed, page_size=page, lengths=lens,
                            tail_fill="nan")
    c = dict(c, Hq=Hkv * G)
    slopes, kw = kw_of(c)
    sd = None if slopes is None else slopes.to(DEV)
    ns = int(r.integers(0, 9))
    out, lse = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV),
                              block_table=pc.block_table.to(DEV), num_splits=ns, alibi_slopes=sd,
                              finite_cache=True, **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page,
                                   **oracle_kw(c, slopes))
    check(out.cpu(), lse.cpu(), ro, rl, c["dt"], f"random kvcache adjacent heads {seed}")
