"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every workload is compared element by element in full: the full-size ones
(configs 3 and 4, the fp8 leg) with the oracle run over all (batch, head)
pairs in parallel worker processes (tests/oracle_pool.py).  Paged vs dense-cache decode and varlen vs per-sequence
dense are compared bit for bit on the GPU.
"""

import numpy as np
import pytest
import torch

import exact_attention_forward_fa_amd as fa
from exact_attention_forward_fa_amd import inputs
from oracle import ref

import oracle_pool
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def run_dense(c):
    q, k, v = gpu(c["q"], c["k"], c["v"])
    slopes = c.get("alibi_slopes")
    out, lse = fa.fwd(q, k, v, softmax_scale=c.get("softmax_scale"), causal=c.get("causal", False),
                      window_size=c.get("window", (-1, -1)), softcap=c.get("softcap", 0.0),
                      alibi_slopes=None if slopes is None else slopes.to(DEV))
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def oracle_dense(c, rows=None):
    return ref.attention(c["q"], c["k"], c["v"], softmax_scale=c.get("softmax_scale"),
                         causal=c.get("causal", False), window=c.get("window", (-1, -1)),
                         softcap=c.get("softcap", 0.0), alibi_slopes=c.get("alibi_slopes"), rows=rows)


# ---------------------------------------------------------------- full compares

@pytest.mark.parametrize("name", ["c1_noncausal", "c1_causal", "c1_decode", "c2_causal", "c2_noncausal"])
def test_dense_small_full(name):
    print("case", name, flush=True)
    c = inputs.case(name)
    out, lse = run_dense(c)
    ro, rl = oracle_dense(c)
    check(out, lse, ro, rl, c["q"].dtype, name)


def test_c1_decode_causal_flag_irrelevant():
    c = inputs.case("c1_decode")
    a = run_dense(dict(c, causal=True))
    b = run_dense(dict(c, causal=False))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_c2_varlen_full_and_bitexact_vs_dense():
    print("case c2_varlen", flush=True)
    c = inputs.case("c2_varlen")
    q, k, v, cq, ck = gpu(c["q"], c["k"], c["v"], c["cu_seqlens_q"], c["cu_seqlens_k"])
    out, lse = fa.fwd_varlen(q, k, v, cq, ck, c["max_seqlen_q"], c["max_seqlen_k"], causal=True)
    torch.cuda.synchronize()
    ro, rl = ref.attention_varlen(c["q"], c["k"], c["v"], c["cu_seqlens_q"], c["cu_seqlens_k"], causal=True)
    check(out.cpu(), lse.cpu(), ro, rl, torch.float16, "c2_varlen")
    # each packed sequence equals the dense call on that sequence alone, bit for bit
    cu = c["cu_seqlens_q"].tolist()
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        od, ld = fa.fwd(q[None, a:e], k[None, a:e], v[None, a:e], causal=True)
        assert torch.equal(od[0], out[a:e]), f"seq {b} out differs from dense"
        assert torch.equal(ld[0], lse[:, a:e]), f"seq {b} lse differs from dense"


# ---------------------------------------------------------------- full-size workloads, every row

@pytest.mark.parametrize("name", ["c3_causal", "c3_win256_0", "c3_win256_256", "c4_gqa"])
def test_full_size_all_rows(name):
    """Configs 3 and 4 at full size, in the launch configuration the benchmark
    times, against the oracle on every row of every (batch, head)."""
    print("case", name, flush=True)
    c = inputs.case(name)
    out, lse = run_dense(c)
    ro, rl = oracle_pool.dense_full(c["q"], c["k"], c["v"], softmax_scale=c.get("softmax_scale"),
                                    causal=c.get("causal", False), window=c.get("window", (-1, -1)),
                                    softcap=c.get("softcap", 0.0), alibi_slopes=c.get("alibi_slopes"))
    check(out, lse, ro, rl, c["q"].dtype, name)
    # determinism: a second run is bit-identical
    out2, lse2 = run_dense(c)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


# ---------------------------------------------------------------- paged split-KV decode

@pytest.fixture(scope="module")
def c5():
    return inputs.case("c5_paged")


def run_paged(c, block_table=True, num_splits=None, dense=None, **opts):
    q = c["q"].to(DEV)
    lens = c["cache_seqlens"].to(DEV)
    ns = c.get("num_splits", 0) if num_splits is None else num_splits
    if block_table:
        out, lse = fa.fwd_kvcache(q, c["k_pool"].to(DEV), c["v_pool"].to(DEV), lens,
                                  block_table=c["block_table"].to(DEV), num_splits=ns, **opts)
    else:
        kd, vd = dense
        out, lse = fa.fwd_kvcache(q, kd.to(DEV), vd.to(DEV), lens, num_splits=ns, **opts)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def test_c5_paged_decode_full(c5):
    print("case c5_paged", flush=True)
    out, lse = run_paged(c5)
    ro, rl = ref.attention_kvcache(c5["q"], c5["k_pool"], c5["v_pool"], c5["cache_seqlens"],
                                   c5["block_table"], c5["page_size"])
    check(out, lse, ro, rl, torch.bfloat16, "c5_paged")
    out2, lse2 = run_paged(c5)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_c5_decode_with_one_token_append(c5):
    """Config 5 in the form the benchmark times with an append: each sequence's
    last token is written again from k=, v= (its own values) at position
    cache_seqlens - 1 and attended with the rest.  The pool must be unchanged and
    the result equal, bit for bit, the plain decode of the full cache."""
    print("case c5_append", flush=True)
    page = c5["page_size"]
    last = c5["cache_seqlens"].long() - 1
    pages = c5["block_table"][torch.arange(last.numel()), last // page].long()
    kn = c5["k_pool"][pages, last % page].unsqueeze(1).contiguous()
    vn = c5["v_pool"][pages, last % page].unsqueeze(1).contiguous()
    kp, vp = c5["k_pool"].to(DEV), c5["v_pool"].to(DEV)
    out, lse = fa.fwd_kvcache(c5["q"].to(DEV), kp, vp, (c5["cache_seqlens"] - 1).to(DEV),
                              block_table=c5["block_table"].to(DEV), num_splits=c5.get("num_splits", 0),
                              k=kn.to(DEV), v=vn.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kp.cpu(), c5["k_pool"]) and torch.equal(vp.cpu(), c5["v_pool"])
    ro, rl = run_paged(c5)
    assert torch.equal(out.cpu(), ro) and torch.equal(lse.cpu(), rl)


def test_c5_paged_equals_dense_cache_bitexact(c5):
    """The paged gather equals the dense cache bit for bit.  At D = 128 the paged
    call runs the decode form that loads K straight into MFMA operand registers
    and the dense call the form that stages K in LDS, so this also checks that
    the two forms compute the same products in the same order."""
    kd = inputs.dense_cache_from_pool(c5["k_pool"], c5["block_table"], c5["cache_seqlens"])
    vd = inputs.dense_cache_from_pool(c5["v_pool"], c5["block_table"], c5["cache_seqlens"])
    a = run_paged(c5)
    b = run_paged(c5, block_table=False, dense=(kd, vd))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------- edge cases (small, full compare)

EDGE = [
    # (B, Sq, Sk, Hq, Hkv, D, dtype, opts)
    (1, 77, 200, 2, 2, 64, torch.float16, dict()),
    (2, 77, 200, 4, 2, 64, torch.float16, dict(causal=True)),
    (1, 200, 77, 2, 1, 64, torch.float16, dict(causal=True)),          # Sq > Sk: leading rows empty
    (1, 200, 77, 2, 2, 128, torch.bfloat16, dict()),
    (2, 130, 130, 4, 1, 128, torch.bfloat16, dict(causal=True)),        # MQA
    (1, 257, 257, 2, 2, 64, torch.float16, dict(window=(0, 0))),
    (1, 257, 300, 2, 2, 64, torch.float16, dict(window=(17, 5))),
    (1, 300, 300, 2, 2, 128, torch.float16, dict(causal=True, window=(64, 64))),
    (1, 190, 190, 4, 2, 64, torch.bfloat16, dict(softcap=3.0, causal=True)),
    (1, 190, 250, 4, 4, 64, torch.float16, dict(alibi=True)),
    (1, 190, 250, 4, 2, 128, torch.bfloat16, dict(alibi=True, softcap=20.0, window=(40, 10))),
    (3, 1, 333, 8, 2, 128, torch.float16, dict(causal=True)),            # decode shape via prefill
    (1, 64, 1, 2, 2, 64, torch.float16, dict(causal=True)),              # Sk = 1
    (1, 33, 33, 2, 2, 64, torch.float16, dict(softmax_scale=0.3)),
    (2, 300, 300, 4, 4, 128, torch.float16, dict()),                     # plain D=128 fp16, non-causal
    (1, 260, 200, 4, 2, 64, torch.bfloat16, dict(alibi=True, window=(50, 20))),
    (1, 220, 150, 4, 1, 64, torch.float16, dict(alibi=True, softcap=10.0, causal=True)),
    # head dims 32 and 96
    (1, 200, 300, 4, 2, 32, torch.float16, dict(causal=True)),
    (2, 130, 130, 4, 4, 32, torch.bfloat16, dict(window=(20, 5), softcap=5.0)),
    (1, 257, 300, 4, 2, 96, torch.float16, dict()),
    (1, 300, 200, 2, 1, 96, torch.bfloat16, dict(causal=True, alibi=True)),
    (1, 190, 250, 4, 2, 96, torch.float16, dict(softcap=10.0, window=(60, 0))),
    (2, 520, 520, 2, 2, 32, torch.float16, dict(causal=True)),              # several q-tiles, ragged tail
    # head dim 256
    (1, 300, 333, 2, 1, 256, torch.bfloat16, dict(causal=True)),
    (1, 130, 200, 4, 2, 256, torch.float16, dict(softcap=20.0, alibi=True, window=(64, 16))),
    (2, 77, 77, 2, 2, 256, torch.float16, dict()),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"B{c[0]}q{c[1]}k{c[2]}h{c[3]}/{c[4]}d{c[5]}{'bf' if c[6] == torch.bfloat16 else 'f'}{sorted(c[7])}")
def test_dense_edge_cases(case):
    B, Sq, Sk, Hq, Hkv, D, dt, opts = case
    print("case", case, flush=True)
    q, k, v = inputs.dense_qkv(B, Sq, Sk, Hq, Hkv, D, dt, seed=4242 + Sq + Sk + D)
    slopes = inputs.alibi_slopes(Hq) if opts.get("alibi") else None
    kw = dict(causal=opts.get("causal", False), softcap=opts.get("softcap", 0.0))
    out, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), softmax_scale=opts.get("softmax_scale"),
                      window_size=opts.get("window", (-1, -1)),
                      alibi_slopes=None if slopes is None else slopes.to(DEV), **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention(q, k, v, softmax_scale=opts.get("softmax_scale"), window=opts.get("window", (-1, -1)),
                           alibi_slopes=slopes, **kw)
    check(out.cpu(), lse.cpu(), ro, rl, dt, str(case))


def test_strided_inputs_match_contiguous():
    q, k, v = inputs.dense_qkv(2, 150, 170, 4, 2, 64, torch.float16, seed=31)
    big_q = torch.zeros(2, 150, 6, 64, dtype=torch.float16)
    big_q[:, :, 1:5] = q
    qs = big_q.to(DEV)[:, :, 1:5]                 # non-contiguous head/batch strides
    kv = torch.stack([k, v], dim=3).to(DEV)       # [B, Sk, Hkv, 2, D]: k and v interleaved
    ks, vs = kv[:, :, :, 0], kv[:, :, :, 1]
    a = fa.fwd(qs, ks, vs, causal=True)
    b = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].cpu(), b[0].cpu()) and torch.equal(a[1].cpu(), b[1].cpu())


def test_varlen_ragged_with_empty_sequences():
    lq, lk = [5, 0, 130, 1, 64], [9, 3, 100, 0, 64]
    q, k, v, cq, ck = inputs.varlen_pack(lq, lk, 4, 2, 64, torch.bfloat16, seed=71)
    qd, kd, vd, cqd, ckd = gpu(q, k, v, cq, ck)
    for opts in (dict(causal=True), dict(window=(3, 2)), dict()):
        gopts = dict(causal=opts.get("causal", False), window_size=opts.get("window", (-1, -1)))
        out, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), **gopts)
        torch.cuda.synchronize()
        ro, rl = ref.attention_varlen(q, k, v, cq, ck, **opts)
        check(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, f"varlen {opts}")


@pytest.mark.parametrize("page,lens,ns,sq,fill,D,dt", [
    (16, [1, 15, 16, 17, 100, 333], 4, 1, "nan", 128, torch.bfloat16),
    (48, [47, 48, 49, 500, 3], 7, 1, "nan", 64, torch.float16),       # page size not a power of two
    (256, [1024, 3000, 257], 16, 1, "nan", 128, torch.float16),
    (64, [10, 200, 64], 64, 1, "nan", 64, torch.bfloat16),            # more splits than chunks: empty splits
    (32, [90, 31, 200], 0, 1, "zero", 128, torch.bfloat16),           # library split heuristic
    (32, [90, 31, 200], 3, 3, "nan", 128, torch.float16),             # 3 new queries per sequence, causal
    (32, [90, 31, 200], 2, 2, "nan", 64, torch.bfloat16),
])
def test_paged_decode_edge_cases(page, lens, ns, sq, fill, D, dt):
    print("paged case", page, lens, ns, sq, fill, D, dt, flush=True)
    Hq, Hkv = 8, 2
    pc = inputs.paged_cache(len(lens), sq, Hq, Hkv, D, dt, seed=page + ns, page_size=page,
                            lengths=lens, tail_fill=fill)
    c = dict(q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool, block_table=pc.block_table,
             cache_seqlens=pc.cache_seqlens, page_size=page)
    out, lse = run_paged(c, num_splits=ns, causal=True)
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page, causal=True)
    check(out, lse, ro, rl, dt, f"paged p{page} ns{ns} sq{sq} D{D}")
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    b = run_paged(c, block_table=False, dense=(kd, vd), num_splits=ns, causal=True)
    assert torch.equal(out, b[0]) and torch.equal(lse, b[1])


@pytest.mark.parametrize("D,dt", [(32, torch.bfloat16), (96, torch.float16)])
def test_varlen_head_dims_32_96(D, dt):
    q, k, v, cq, ck = inputs.varlen_pack([300, 1, 517], [400, 90, 517], 4, 2, D, dt, seed=830 + D)
    out, lse = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), 517, 517, causal=True)
    torch.cuda.synchronize()
    ro, rl = ref.attention_varlen(q, k, v, cq, ck, causal=True)
    check(out.cpu(), lse.cpu(), ro, rl, dt, f"varlen D={D}")


def test_varlen_options_d128():
    lq, lk = [40, 1, 300, 97], [60, 50, 300, 128]
    q, k, v, cq, ck = inputs.varlen_pack(lq, lk, 8, 2, 128, torch.bfloat16, seed=73)
    qd, kd, vd, cqd, ckd = gpu(q, k, v, cq, ck)
    slopes = inputs.alibi_slopes(8)
    for opts in (dict(causal=True, softcap=15.0), dict(alibi=True, window=(30, 0), causal=True), dict(softcap=5.0, alibi=True)):
        gopts = dict(causal=opts.get("causal", False), window_size=opts.get("window", (-1, -1)),
                     softcap=opts.get("softcap", 0.0), alibi_slopes=slopes.to(DEV) if opts.get("alibi") else None)
        out, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), **gopts)
        torch.cuda.synchronize()
        ro, rl = ref.attention_varlen(q, k, v, cq, ck, causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
                                      softcap=opts.get("softcap", 0.0), alibi_slopes=slopes if opts.get("alibi") else None)
        check(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, f"varlen D128 {opts}")


@pytest.mark.parametrize("page,Hq,Hkv,sq,D,dt,ns,opts", [
    (100, 8, 2, 1, 128, torch.bfloat16, 3, dict()),                                   # pages >= 64, not a power of two
    (64, 32, 4, 2, 128, torch.bfloat16, 4, dict(causal=True)),                        # 16 query rows per kv head
    (128, 8, 2, 2, 128, torch.bfloat16, 5, dict(causal=True, window=(90, 0), softcap=30.0, alibi=True)),
    (16, 8, 4, 3, 64, torch.float16, 2, dict(causal=True, window=(20, 0), alibi=True)),
    (256, 8, 2, 1, 128, torch.bfloat16, 1, dict(softcap=7.0)),                        # one split
])
def test_paged_decode_options(page, Hq, Hkv, sq, D, dt, ns, opts):
    print("paged options", page, Hq, Hkv, sq, D, dt, ns, opts, flush=True)
    lens = [300, 1, 777, 64, 129]
    pc = inputs.paged_cache(len(lens), sq, Hq, Hkv, D, dt, seed=page + 7 * sq, page_size=page, lengths=lens,
                            tail_fill="nan")
    slopes = inputs.alibi_slopes(Hq) if opts.get("alibi") else None
    c = dict(q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool, block_table=pc.block_table,
             cache_seqlens=pc.cache_seqlens, page_size=page)
    gkw = dict(causal=opts.get("causal", False), window_size=opts.get("window", (-1, -1)),
               softcap=opts.get("softcap", 0.0), alibi_slopes=None if slopes is None else slopes.to(DEV))
    out, lse = run_paged(c, num_splits=ns, **gkw)
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page,
                                   causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
                                   softcap=opts.get("softcap", 0.0), alibi_slopes=slopes)
    check(out, lse, ro, rl, dt, f"paged options p{page} sq{sq} {opts}")
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    b = run_paged(c, block_table=False, dense=(kd, vd), num_splits=ns, **gkw)
    assert torch.equal(out, b[0]) and torch.equal(lse, b[1])


@pytest.mark.parametrize("D,dt,page,paged", [(32, torch.float16, 64, True), (32, torch.bfloat16, 0, False),
                                             (256, torch.bfloat16, 256, True), (256, torch.float16, 16, True),
                                             (256, torch.bfloat16, 0, False), (96, torch.bfloat16, 64, True),
                                             (96, torch.float16, 256, True), (96, torch.float16, 0, False),
                                             (96, torch.bfloat16, 16, True)])
def test_decode_head_dims_32_96_256(D, dt, page, paged):
    print("case decode D", D, dt, page, paged, flush=True)
    lens = [700, 33, 1500]
    pc = inputs.paged_cache(3, 2, 8, 2, D, dt, seed=900 + D + page, page_size=page or 64, lengths=lens,
                            tail_fill="nan")
    if paged:
        out, lse = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV),
                                  block_table=pc.block_table.to(DEV), num_splits=5, causal=True)
    else:
        kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
        vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
        out, lse = fa.fwd_kvcache(pc.q.to(DEV), kd.to(DEV), vd.to(DEV), pc.cache_seqlens.to(DEV), num_splits=5,
                                  causal=True)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page or 64,
                                   causal=True)
    check(out.cpu(), lse.cpu(), ro, rl, dt, f"decode D={D} page={page} paged={paged}")


@pytest.mark.parametrize("D,Hq,Hkv,Sq,dt,opts", [
    (32, 8, 8, 2, torch.float16, dict(causal=True)),                      # 8 kv heads per work item, 16 rows
    (64, 8, 4, 2, torch.bfloat16, dict(causal=True, softcap=5.0)),        # 4 per item
    (64, 6, 6, 1, torch.float16, dict(window=(300, 0), alibi=True)),      # 2 per item (6 = 2 * 3)
    (32, 12, 4, 1, torch.bfloat16, dict()),                               # 4 per item, 3 query heads each
])
def test_decode_adjacent_heads_per_item(D, Hq, Hkv, Sq, dt, opts):
    """With finite_cache=True, small head dims read 2, 4 or 8 adjacent kv heads
    as one work item; every query must still see exactly its own head's keys,
    and a paged cache and its dense equivalent give the same bits."""
    print("case decode heads per item", D, Hq, Hkv, Sq, dt, opts, flush=True)
    lens = [700, 33, 1500, 260]
    pc = inputs.paged_cache(4, Sq, Hq, Hkv, D, dt, seed=950 + D + Hq + Sq, page_size=64, lengths=lens,
                            tail_fill="nan")
    slopes = inputs.alibi_slopes(Hq) if opts.get("alibi") else None
    kw = dict(causal=opts.get("causal", False), window_size=opts.get("window", (-1, -1)),
              softcap=opts.get("softcap", 0.0), alibi_slopes=None if slopes is None else slopes.to(DEV),
              finite_cache=True)
    out, lse = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV),
                              block_table=pc.block_table.to(DEV), num_splits=3, **kw)
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    out2, lse2 = fa.fwd_kvcache(pc.q.to(DEV), kd.to(DEV), vd.to(DEV), pc.cache_seqlens.to(DEV), num_splits=3, **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 64,
                                   causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
                                   softcap=opts.get("softcap", 0.0), alibi_slopes=slopes)
    check(out.cpu(), lse.cpu(), ro, rl, dt, f"decode heads per item D={D} Hq={Hq} Hkv={Hkv} Sq={Sq}")
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("D,dt", [(32, torch.float16), (64, torch.bfloat16)])
def test_decode_nonfinite_value_stays_in_its_head(D, dt):
    """Without finite_cache every query head reads its own kv head only: an Inf
    in kv head 1's K and a NaN in its V leave every other head's out and lse
    bit-identical to the decode of the finite cache (8 kv heads of one query
    row each, the shape that finite_cache would read 4-8 heads at a time)."""
    print("case nonfinite head", D, dt, flush=True)
    pc = inputs.paged_cache(3, 1, 8, 8, D, dt, seed=960 + D, page_size=64, lengths=[300, 130, 77])
    kp, vp = pc.k_pool.clone(), pc.v_pool.clone()
    for b, t in ((0, 5), (1, 129), (2, 40)):
        page = int(pc.block_table[b, t // 64])
        kp[page, t % 64, 1, 3] = float("inf")
        vp[page, (t + 1) % 64, 1, 0] = float("nan")
    args = dict(block_table=pc.block_table.to(DEV), num_splits=2, causal=True)
    a = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV), **args)
    b = fa.fwd_kvcache(pc.q.to(DEV), kp.to(DEV), vp.to(DEV), pc.cache_seqlens.to(DEV), **args)
    torch.cuda.synchronize()
    others = [h for h in range(8) if h != 1]
    assert torch.equal(a[0][:, :, others], b[0][:, :, others])
    assert torch.equal(a[1][:, others], b[1][:, others])
    assert not torch.isfinite(b[0][:, :, 1]).all()        # the planted head itself is affected
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 64, causal=True)
    check(a[0].cpu(), a[1].cpu(), ro, rl, dt, f"nonfinite head D={D} (finite cache)")


def test_c5_default_splits_paged_equals_dense_bitexact(c5):
    """num_splits = 0 resolves from the cache capacity; a dense cache of the
    paged cache's capacity (block-table width x page size) takes the same split
    count and gives the same bits."""
    cap = c5["block_table"].shape[1] * c5["page_size"]
    kd = inputs.dense_cache_from_pool(c5["k_pool"], c5["block_table"], c5["cache_seqlens"], smax=cap)
    vd = inputs.dense_cache_from_pool(c5["v_pool"], c5["block_table"], c5["cache_seqlens"], smax=cap)
    a = run_paged(c5, num_splits=0)
    b = run_paged(c5, block_table=False, dense=(kd, vd), num_splits=0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_paged_decode_many_sequences():
    # more than 64 sequences: the schedule order comes from its own kernel
    lens = [int(x) for x in np.random.default_rng(80).integers(0, 400, 80)]
    lens[3] = 0
    pc = inputs.paged_cache(80, 1, 8, 2, 64, torch.bfloat16, seed=80, page_size=32, lengths=lens, tail_fill="nan")
    c = dict(q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool, block_table=pc.block_table,
             cache_seqlens=pc.cache_seqlens, page_size=32)
    out, lse = run_paged(c, num_splits=3)
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 32)
    check(out, lse, ro, rl, torch.bfloat16, "paged B=80")
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    b = run_paged(c, block_table=False, dense=(kd, vd), num_splits=3)
    assert torch.equal(out, b[0]) and torch.equal(lse, b[1])


def test_paged_decode_pool_beyond_4gib():
    # the same pages placed past the first 4 GiB of a larger pool take the
    # 64-bit addressing path; results must not change at all
    lens = [700, 1, 300, 512]
    page, Hkv, D = 256, 8, 128
    pc = inputs.paged_cache(len(lens), 1, 32, Hkv, D, torch.bfloat16, seed=44, page_size=page, lengths=lens)
    c = dict(q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool, block_table=pc.block_table,
             cache_seqlens=pc.cache_seqlens, page_size=page)
    small = run_paged(c, num_splits=3)
    n = pc.k_pool.shape[0]
    page_bytes = page * Hkv * D * 2
    first = (4 << 30) // page_bytes + 3                 # first page index past 4 GiB
    big_k = torch.zeros((first + n, page, Hkv, D), dtype=torch.bfloat16, device=DEV)
    big_v = torch.zeros_like(big_k)
    big_k[first:] = pc.k_pool.to(DEV)
    big_v[first:] = pc.v_pool.to(DEV)
    bt = pc.block_table.clone()
    bt[bt >= 0] += first
    out, lse = fa.fwd_kvcache(pc.q.to(DEV), big_k, big_v, pc.cache_seqlens.to(DEV), block_table=bt.to(DEV),
                              num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), small[0]) and torch.equal(lse.cpu(), small[1])
    del big_k, big_v
    torch.cuda.empty_cache()


def test_kvcache_options_match_oracle():
    pc = inputs.paged_cache(3, 1, 8, 8, 64, torch.float16, seed=9, page_size=64, lengths=[700, 64, 1000])
    slopes = inputs.alibi_slopes(8)
    c = dict(q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool, block_table=pc.block_table,
             cache_seqlens=pc.cache_seqlens, page_size=64)
    for opts in (dict(window=(100, 0)), dict(softcap=5.0), dict(alibi=True), dict(softmax_scale=0.05)):
        kw = {kk: vv for kk, vv in opts.items() if kk not in ("alibi", "window")}
        gkw = dict(kw, window_size=opts.get("window", (-1, -1)))
        out, lse = run_paged(c, num_splits=5, alibi_slopes=slopes.to(DEV) if opts.get("alibi") else None, **gkw)
        kw["window"] = opts.get("window", (-1, -1))
        ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 64,
                                       alibi_slopes=slopes if opts.get("alibi") else None, **kw)
        check(out, lse, ro, rl, torch.float16, f"kvcache {opts}")


def _combine_case(seed, B, S, H, D, n, nan_rows=True):
    rng = np.random.default_rng(seed)
    op = rng.standard_normal((B, S, H, D, n)).astype(np.float32)
    lp = (rng.standard_normal((B, S, H, n)) * 3).astype(np.float32)
    if nan_rows:
        lp[0, 0, 0, :] = -np.inf               # a row with no keys anywhere
        op[0, 0, 0] = np.nan
        if n > 1:
            lp[-1, -1, -1, ::2] = -np.inf      # some empty splits
            op[-1, -1, -1, :, ::2] = np.nan    # whose partials must not be read
    return op, lp


@pytest.mark.parametrize("B,S,H,D,n", [(2, 3, 4, 128, 6), (2, 1, 3, 128, 1), (1, 2, 5, 64, 64), (3, 1, 2, 64, 3)])
def test_combine_standalone(B, S, H, D, n):
    op, lp = _combine_case(B * 100 + n, B, S, H, D, n)
    lpd = torch.from_numpy(lp).to(DEV)
    ro, rl = ref.combine(np.nan_to_num(op), lp)
    # the pages' [B,S,H,D,n] order (any-stride kernel) ...
    out, lse = fa.combine(torch.from_numpy(op).to(DEV), lpd, out_dtype=torch.float16)
    torch.cuda.synchronize()
    check(out.cpu(), lse.cpu(), ro, rl, torch.float16, f"combine [B,S,H,D,n] n={n}")
    # ... and a [B,S,H,n,D] buffer seen through a transposed view (the decode
    # workspace order, row kernel): same result up to summation order
    opt = torch.from_numpy(np.ascontiguousarray(op.transpose(0, 1, 2, 4, 3))).to(DEV).transpose(3, 4)
    out2, lse2 = fa.combine(opt, lpd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check(out2.cpu(), lse2.cpu(), ro, rl, torch.bfloat16, f"combine [B,S,H,n,D] n={n}")
    out3, _ = fa.combine(opt, lpd, out_dtype=torch.float16)
    torch.cuda.synchronize()
    d = (out3.cpu().float() - out.cpu().float()).abs()
    ulp = torch.maximum(out.cpu().float().abs(), torch.tensor(6.1e-5)) * 2.0 ** -10
    assert bool((d <= ulp + 1e-7).all()), f"row kernel vs any-stride kernel differ by {d.max().item()}"


def test_empty_batch_is_noop():
    q = torch.empty(0, 16, 2, 64, dtype=torch.float16, device=DEV)
    out, lse = fa.fwd(q, q, q)
    assert out.shape == q.shape and lse.shape == (0, 2, 16)


# ------------------------------------------------- running-max stress (rescale paths)

def _ramped_qkv(B, Sq, Sk, H, D, dt, seed, profile):
    """q with a common direction u and keys whose component along u follows a
    profile over the key index, so the row max moves by several units (log2)
    per 64-key tile: "rise" climbs steadily, "jump" has one block of keys far
    above the rest, "fall" puts the largest scores first."""
    g = torch.Generator().manual_seed(seed)
    u = torch.ones(D, dtype=torch.float64) / D ** 0.5
    q = torch.randn(B, Sq, H, D, generator=g, dtype=torch.float64) + 3.0 * u
    j = torch.arange(Sk, dtype=torch.float64)
    if profile == "rise":
        a = 0.3 * j
    elif profile == "jump":
        a = torch.where((j >= Sk // 2) & (j < Sk // 2 + 40), torch.full_like(j, 60.0), torch.zeros_like(j))
    else:
        a = 0.3 * (Sk - 1 - j)
    k = torch.randn(B, Sk, H, D, generator=g, dtype=torch.float64) * 0.5 + a[None, :, None, None] * u
    v = torch.randn(B, Sk, H, D, generator=g, dtype=torch.float64)
    return q.to(dt), k.to(dt), v.to(dt)


@pytest.mark.parametrize("profile", ["rise", "jump", "fall"])
@pytest.mark.parametrize("D,dt,causal", [(64, torch.float16, False), (64, torch.bfloat16, True),
                                         (128, torch.float16, True), (128, torch.bfloat16, False)])
def test_prefill_running_max_stress(profile, D, dt, causal):
    print("case", profile, D, dt, causal, flush=True)
    q, k, v = _ramped_qkv(1, 300, 700, 2, D, dt, 77 + D, profile)
    out, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ro, rl = ref.attention(q, k, v, causal=causal)
    check(out.cpu(), lse.cpu(), ro, rl, dt, f"prefill {profile} D{D} {dt} causal={causal}")


@pytest.mark.parametrize("profile", ["rise", "jump", "fall"])
def test_decode_running_max_stress(profile):
    print("case decode", profile, flush=True)
    B, Smax, Hkv, Hq, D = 2, 1500, 2, 4, 128
    q, k, v = _ramped_qkv(B, 1, Smax, Hkv, D, torch.bfloat16, 91, profile)
    q = q.repeat_interleave(Hq // Hkv, dim=2).contiguous()
    lens = torch.tensor([1500, 1100], dtype=torch.int32)
    out, lse = fa.fwd_kvcache(q.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV), num_splits=3)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(q, k, v, lens)
    check(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, f"decode {profile}")


# ------------------------------------------------- KV append (new keys and values)

APPEND = [
    # (paged, page, B, final lengths, S_new, Sq, Hq, Hkv, D, dtype, causal)
    (True, 256, 3, [1000, 257, 4097], 1, 1, 8, 2, 128, torch.bfloat16, True),
    (True, 64, 2, [130, 70], 5, 5, 4, 2, 64, torch.float16, True),        # the new block crosses a page
    (True, 64, 2, [64, 3], 3, 1, 4, 4, 128, torch.float16, False),        # starts on a page boundary
    (False, 0, 2, [900, 33], 4, 4, 8, 2, 128, torch.bfloat16, True),
    (False, 0, 2, [17, 300], 6, 0, 4, 4, 64, torch.float16, False),       # Sq = 0: append only
    (True, 64, 2, [130, 70], 2, 2, 4, 2, 256, torch.bfloat16, True),
    (False, 0, 2, [40, 9], 3, 1, 4, 4, 32, torch.float16, False),
    (True, 64, 2, [130, 70], 3, 3, 8, 2, 96, torch.bfloat16, True),
    (False, 0, 2, [300, 65], 1, 1, 4, 1, 96, torch.float16, False),
]


@pytest.mark.parametrize("case", APPEND, ids=lambda c: f"{'paged' + str(c[1]) if c[0] else 'dense'}-S{c[4]}-q{c[5]}-d{c[8]}")
def test_kvcache_append(case):
    paged, page, B, final, S, Sq, Hq, Hkv, D, dt, causal = case
    print("case", case, flush=True)
    pc = inputs.paged_cache(B, max(Sq, 1), Hq, Hkv, D, dt, seed=600 + sum(final), page_size=page or 64,
                            lengths=final, tail_fill="nan")
    g = torch.Generator().manual_seed(601 + S)
    kn = torch.randn(B, S, Hkv, D, generator=g).to(dt)
    vn = torch.randn(B, S, Hkv, D, generator=g).to(dt)
    lens = (pc.cache_seqlens - S).to(torch.int32)
    q = pc.q[:, :Sq].contiguous()
    if paged:
        kc, vc, bt = pc.k_pool, pc.v_pool, pc.block_table
    else:
        smax = max(final) + 5
        kc = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens, smax=smax)
        vc = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens, smax=smax)
        kc[:, max(final):] = float("nan")              # rows past every final length
        vc[:, max(final):] = float("nan")
        bt = None
    kg, vg, lg = kc.to(DEV), vc.to(DEV), lens.to(DEV)
    res = fa.fwd_kvcache(q.to(DEV), kg, vg, lg, block_table=None if bt is None else bt.to(DEV),
                         k=kn.to(DEV), v=vn.to(DEV), causal=causal, num_splits=3)
    torch.cuda.synchronize()
    k2, v2 = ref.kvcache_append(kc, vc, kn, vn, lens, bt, page if paged else None)
    # the caches after the call: bit for bit, NaN (rows past the lengths) matching any NaN
    want_k = torch.from_numpy(k2).to(dt)
    want_v = torch.from_numpy(v2).to(dt)
    for name, got, want in (("k", kg.cpu(), want_k), ("v", vg.cpu(), want_v)):
        bad = ((got.view(torch.int16) != want.view(torch.int16)) & ~(got.isnan() & want.isnan())).nonzero()
        assert bad.shape[0] == 0, (f"{name} cache after append: {bad.shape[0]} elements differ, first at "
                                   f"{bad[:4].tolist()}: got {[float(got[tuple(i)]) for i in bad[:4].tolist()]} "
                                   f"want {[float(want[tuple(i)]) for i in bad[:4].tolist()]}")
    assert torch.equal(lg.cpu(), lens), "cache_seqlens must not change"
    if Sq:
        out, lse = res
        ro, rl = ref.attention_kvcache(q, k2, v2, pc.cache_seqlens, bt, page if paged else None, causal=causal)
        check(out.cpu(), lse.cpu(), ro, rl, dt, f"append {case}")


def test_kvcache_append_then_decode_equals_prefilled_cache():
    """Two steps of generation with appends give the same result, bit for bit, as
    decoding against a cache that already holds those tokens."""
    B, Hq, Hkv, D, dt = 2, 8, 2, 128, torch.bfloat16
    final = [700, 1300]
    pc = inputs.paged_cache(B, 1, Hq, Hkv, D, dt, seed=777, page_size=64, lengths=final)
    kg0, vg0 = pc.k_pool.to(DEV), pc.v_pool.to(DEV)
    bt = pc.block_table.to(DEV)
    # reference: the full cache, decoding step 2 (lengths final)
    ref_out, ref_lse = fa.fwd_kvcache(pc.q.to(DEV), kg0, vg0, pc.cache_seqlens.to(DEV), block_table=bt,
                                      num_splits=4)
    # the same pool with the last two tokens blanked, then appended one at a time
    kg, vg = kg0.clone(), vg0.clone()
    for b, n in enumerate(final):
        for t in (n - 2, n - 1):
            page = int(pc.block_table[b, t // 64])
            kg[page, t % 64] = 0
            vg[page, t % 64] = 0
    for step in (2, 1):
        lens = (pc.cache_seqlens - step).to(DEV)
        kn = torch.stack([kg0[int(pc.block_table[b, (n - step) // 64]), (n - step) % 64] for b, n in enumerate(final)])
        vn = torch.stack([vg0[int(pc.block_table[b, (n - step) // 64]), (n - step) % 64] for b, n in enumerate(final)])
        out, lse = fa.fwd_kvcache(pc.q.to(DEV), kg, vg, lens, block_table=bt, k=kn[:, None].contiguous(),
                                  v=vn[:, None].contiguous(), num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(kg, kg0) and torch.equal(vg, vg0)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


# ------------------------------------------------- fp8 e4m3 inputs

FP8 = [
    # (B, Sq, Sk, Hq, Hkv, D, descales (q, k, v), opts)
    (2, 300, 300, 4, 2, 64, (1.0, 1.0, 1.0), dict(causal=True)),
    (1, 257, 400, 4, 4, 64, (0.5, 2.0, 0.25), dict()),
    (1, 200, 333, 4, 1, 128, (1.0, 1.0, 1.0), dict(causal=True)),
    (2, 130, 130, 2, 2, 128, (0.125, 0.5, 2.0), dict(softcap=15.0, alibi=True, window=(40, 8))),
    (1, 520, 520, 2, 2, 64, (1.0, 1.0, 1.0), dict(causal=True, window=(100, 0))),
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: f"B{c[0]}q{c[1]}k{c[2]}d{c[5]}{sorted(c[7])}-{c[6]}")
def test_fp8_prefill(case):
    B, Sq, Sk, Hq, Hkv, D, (dq, dk, dv), opts = case
    print("case fp8", case, flush=True)
    q16, k16, v16 = inputs.dense_qkv(B, Sq, Sk, Hq, Hkv, D, torch.float32, seed=1700 + Sq + D)
    # fp8 codes of values spread over e4m3's range; the descales give the real values
    q8 = (q16 / dq).to(torch.float8_e4m3fn)
    k8 = (k16 / dk).to(torch.float8_e4m3fn)
    v8 = (v16 / dv).to(torch.float8_e4m3fn)
    slopes = inputs.alibi_slopes(Hq) if opts.get("alibi") else None
    kw = dict(causal=opts.get("causal", False), softcap=opts.get("softcap", 0.0))
    out, lse = fa.fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), window_size=opts.get("window", (-1, -1)),
                      alibi_slopes=None if slopes is None else slopes.to(DEV), q_descale=dq, k_descale=dk,
                      v_descale=dv, **kw)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    deq = lambda t, s: (t.double() * s)
    ro, rl = ref.attention(deq(q8, dq), deq(k8, dk), deq(v8, dv), window=opts.get("window", (-1, -1)),
                           alibi_slopes=slopes, **kw)
    check(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, f"fp8 {case}")


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_rows_8_byte_aligned_equal_contiguous(D):
    """fp8 q, k and v whose rows start only 8 bytes apart from a 16-byte boundary
    (head stride D + 8 bytes): the 32-byte Q operands are read in 8-byte pieces
    and K is staged 8 bytes at a time, so the bits equal those of contiguous
    copies."""
    print("case fp8 8-byte rows", D, flush=True)
    q, k, v = inputs.dense_qkv(2, 140, 200, 4, 2, D, torch.float32, seed=1750 + D)
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))

    def padded(t):
        B, S, H, _ = t.shape
        store = torch.zeros(B, S, H, D + 8, dtype=torch.uint8)
        store[..., :D] = t.view(torch.uint8)
        return store.to(DEV).view(torch.float8_e4m3fn)[..., :D]

    a = fa.fwd(padded(q8), padded(k8), padded(v8), causal=True)
    b = fa.fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].cpu(), b[0].cpu()) and torch.equal(a[1].cpu(), b[1].cpu())


def test_fp8_prefill_full_size_all_rows():
    """The fp8 prefill at the size and in the launch configuration the benchmark
    times (B=4, S=4096, H=32, D=64 causal, the fp16 inputs converted to e4m3,
    descales 1), checked on every row against the oracle on the e4m3 values."""
    print("case fp8 c3_causal", flush=True)
    c = inputs.case("c3_causal")
    q8, k8, v8 = (c[x].to(torch.float8_e4m3fn) for x in ("q", "k", "v"))
    out, lse = fa.fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ro, rl = oracle_pool.dense_full(q8, k8, v8, causal=True)
    check(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, "fp8 c3_causal")


@pytest.mark.parametrize("opts", [dict(causal=True), dict(window=(100, 20)), dict(window=(600, 20)),
                                  dict(causal=True, softcap=8.0), dict(causal=True, window=(100, 0), softcap=8.0)])
def test_prefill_same_bits_for_any_workgroup_rows(opts):
    """A small grid runs 64-row workgroups and a large one 256-row workgroups
    (128 rows under a window of at most 512 keys besides the row's own); each
    wave owns the same 32 rows and walks the same tiles either way, so the
    results of one (batch, head) agree bit for bit."""
    q, k, v = inputs.dense_qkv(1, 512, 600, 2, 2, 64, torch.float16, seed=4711)
    small = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=opts.get("causal", False),
                   window_size=opts.get("window", (-1, -1)), softcap=opts.get("softcap", 0.0))
    rep = lambda t: t.expand(128, -1, -1, -1).contiguous().to(DEV)
    large = fa.fwd(rep(q), rep(k), rep(v), causal=opts.get("causal", False),
                   window_size=opts.get("window", (-1, -1)), softcap=opts.get("softcap", 0.0))
    torch.cuda.synchronize()
    assert torch.equal(small[0][0], large[0][0]) and torch.equal(small[0][0], large[0][127])
    assert torch.equal(small[1][0], large[1][0])


def test_huge_window_equals_unbounded():
    """A window side of 2^31 - 1 reaches every key: the same bits as -1, in the
    prefill (causal and not) and in the KV-cache decode."""
    print("case huge window", flush=True)
    big = 2 ** 31 - 1
    q, k, v = inputs.dense_qkv(1, 300, 333, 4, 2, 64, torch.float16, seed=4900)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    for causal in (False, True):
        a = fa.fwd(qd, kd, vd, causal=causal, window_size=(big, big))
        b = fa.fwd(qd, kd, vd, causal=causal, window_size=(-1, -1))
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    pc = inputs.paged_cache(3, 2, 8, 2, 128, torch.bfloat16, seed=4901, page_size=64, lengths=[300, 5, 129])
    kv = [t.to(DEV) for t in (pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table)]
    a = fa.fwd_kvcache(kv[0], kv[1], kv[2], kv[3], block_table=kv[4], num_splits=3, causal=True,
                       window_size=(big, big))
    b = fa.fwd_kvcache(kv[0], kv[1], kv[2], kv[3], block_table=kv[4], num_splits=3, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("D,dt", [(64, torch.float16), (128, torch.bfloat16), (64, torch.float8_e4m3fn)])
def test_dense_no_keys(D, dt):
    """Sk = 0: every row has no allowed key, so out = 0 and lse = -inf (k and v
    may be empty tensors without storage)."""
    print("case no keys", D, dt, flush=True)
    q, k, v = inputs.dense_qkv(2, 70, 0, 4, 2, D, torch.float32, seed=4990)
    qd, kd, vd = (t.to(dt).to(DEV) for t in (q, k, v))
    out, lse = fa.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0
    assert torch.isneginf(lse).all()


SPLIT_HEADS = [
    # (B, Sq, Hq, Hkv, D, dtype, page, lengths, options): (Hq/Hkv)*Sq > 16 query rows per kv head
    (3, 1, 32, 1, 128, torch.bfloat16, 64, [300, 1, 1000], dict(causal=True)),           # MQA decode
    (2, 5, 8, 2, 64, torch.float16, 16, [130, 77], dict(causal=True, softcap=5.0)),       # 20 rows
    (2, 3, 16, 1, 128, torch.float16, 0, [500, 40], dict(causal=True, alibi=True)),       # 48 rows
    (2, 1, 64, 2, 64, torch.bfloat16, 256, [700, 2000], dict(window=(100, 0))),           # 32 rows
]


@pytest.mark.parametrize("case", SPLIT_HEADS, ids=lambda c: f"B{c[0]}-sq{c[1]}-h{c[2]}/{c[3]}-d{c[4]}-p{c[6]}")
def test_kvcache_more_than_16_rows_per_kv_head(case):
    """The query heads of a kv head are split into groups of at most 16 rows
    that read the same cache; results match the oracle, paged equals dense."""
    B, Sq, Hq, Hkv, D, dt, page, lens, o = case
    print("case split heads", case[:7], flush=True)
    pc = inputs.paged_cache(B, Sq, Hq, Hkv, D, dt, seed=5000 + Hq + Sq, page_size=page or 64, lengths=lens,
                            tail_fill="nan")
    slopes = inputs.alibi_slopes(Hq) if o.get("alibi") else None
    kw = dict(causal=o.get("causal", False), window_size=o.get("window", (-1, -1)), softcap=o.get("softcap", 0.0),
              alibi_slopes=None if slopes is None else slopes.to(DEV))
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    dense = fa.fwd_kvcache(pc.q.to(DEV), kd.to(DEV), vd.to(DEV), pc.cache_seqlens.to(DEV), num_splits=3, **kw)
    torch.cuda.synchronize()
    ro, rl = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, page or 64,
                                   causal=kw["causal"], window=kw["window_size"], softcap=kw["softcap"],
                                   alibi_slopes=slopes)
    check(dense[0].cpu(), dense[1].cpu(), ro, rl, dt, f"split heads dense {case[:7]}")
    if page:
        paged = fa.fwd_kvcache(pc.q.to(DEV), pc.k_pool.to(DEV), pc.v_pool.to(DEV), pc.cache_seqlens.to(DEV),
                               block_table=pc.block_table.to(DEV), num_splits=3, **kw)
        torch.cuda.synchronize()
        assert torch.equal(paged[0], dense[0]) and torch.equal(paged[1], dense[1])
