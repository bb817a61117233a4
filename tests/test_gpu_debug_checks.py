"""FA_DEBUG=1: the device-side index data a caller promises to keep consistent
(cu_seqlens, cache_seqlens, block_table) is copied back and checked before
anything is launched.  Each inconsistent input below is chosen so that, even
unchecked, every access would stay inside allocated memory (the declared pool
or totals are smaller than the allocations behind them)."""

import ctypes

import pytest
import torch

import exact_attention_forward_fa_amd as fa
from exact_attention_forward_fa_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("FA_DEBUG", "1")


def _varlen(lengths):
    q, k, v, cq, ck = inputs.varlen_pack(lengths, lengths, 2, 2, 64, torch.float16, seed=4800)
    return [t.to(DEV) for t in (q, k, v, cq, ck)]


def test_valid_calls_unchanged_under_debug(monkeypatch):
    print("case debug valid", flush=True)
    q, k, v, cq, ck = _varlen([100, 60, 37])
    a = fa.fwd_varlen(q, k, v, cq, ck, 100, 100, causal=True)
    pc = inputs.paged_cache(3, 1, 4, 2, 128, torch.bfloat16, seed=4801, page_size=64, lengths=[300, 1, 129])
    kv = [t.to(DEV) for t in (pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table)]
    c = fa.fwd_kvcache(kv[0], kv[1], kv[2], kv[3], block_table=kv[4], num_splits=3)
    monkeypatch.setenv("FA_DEBUG", "1")
    b = fa.fwd_varlen(q, k, v, cq, ck, 100, 100, causal=True)
    d = fa.fwd_kvcache(kv[0], kv[1], kv[2], kv[3], block_table=kv[4], num_splits=3)
    torch.cuda.synchronize()
    for x, y in zip(a + c, b + d):
        assert torch.equal(x, y)


def test_decreasing_cu_seqlens_rejected(debug):
    print("case debug cu decreasing", flush=True)
    q, k, v, cq, ck = _varlen([100, 60, 37])
    bad = torch.tensor([0, 100, 50, 197], dtype=torch.int32, device=DEV)   # sequence 1 would be empty
    out = torch.full_like(q, float("nan"))
    with pytest.raises(ValueError, match="FA_DEBUG: cu_seqlens decrease"):
        fa.fwd_varlen(q, k, v, bad, ck, 100, 100, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()                                        # nothing was launched


def test_sequence_longer_than_max_seqlen_rejected(debug):
    print("case debug max_seqlen", flush=True)
    q, k, v, cq, ck = _varlen([100, 60, 37])
    with pytest.raises(ValueError, match="above max_seqlen"):
        fa.fwd_varlen(q, k, v, cq, ck, 64, 100)                          # sequence 0 has 100 rows


def test_cu_seqlens_beyond_total_rejected_forward_and_backward(debug):
    print("case debug beyond total", flush=True)
    q, k, v, cq, ck = _varlen([100, 60, 40])                             # 200 rows allocated
    out, lse = fa.fwd_varlen(q, k, v, cq, ck, 100, 100, causal=True)
    lib = fa.load_library()
    ob, keep = fa._opts(None, True, (-1, -1), 0.0, None, q.device, q.shape[1])
    lse_big = torch.empty((2, 200), dtype=torch.float32, device=DEV)
    # declare 150 rows while cu_seqlens end at 200
    st = lib.fa_fwd_varlen(0, fa._ptr(q), fa._ptr(k), fa._ptr(v), fa._ptr(out), fa._ptr(lse_big), fa._ptr(cq),
                           fa._ptr(ck), 3, 100, 100, 150, 150, 2, 2, 64, None, None, None, None, ob,
                           fa._stream(q.device))
    assert st == 1 and b"beyond total" in lib.fa_last_error()
    g = torch.randn_like(q)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws = torch.empty(fa.bwd_workspace_size(1, 200, 2), dtype=torch.uint8, device=DEV)
    st = lib.fa_bwd_varlen(0, fa._ptr(g), fa._ptr(q), fa._ptr(k), fa._ptr(v), fa._ptr(out), fa._ptr(lse),
                           fa._ptr(dq), fa._ptr(dk), fa._ptr(dv), fa._ptr(cq), fa._ptr(ck), 3, 100, 100, 150, 150,
                           2, 2, 64, None, None, None, None, None, ob, fa._ptr(ws), ws.numel(),
                           fa._stream(q.device))
    assert st == 1 and b"beyond total" in lib.fa_last_error()


def test_block_table_entry_outside_pool_rejected(debug):
    print("case debug block table", flush=True)
    pc = inputs.paged_cache(3, 1, 4, 2, 128, torch.bfloat16, seed=4802, page_size=64, lengths=[300, 1, 129])
    q, kp, vp, lens, bt = (t.to(DEV) for t in (pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table))
    P = kp.shape[0]
    small_k, small_v = kp[:P - 1], vp[:P - 1]                            # declare one page fewer
    bt2 = bt.clone()
    bt2[0, 0] = P - 1                                                     # allocated, but outside the declared pool
    with pytest.raises(ValueError, match="outside the pool"):
        fa.fwd_kvcache(q, small_k, small_v, lens, block_table=bt2, num_splits=2)


def test_cache_seqlens_beyond_cache_rejected(debug):
    print("case debug cache length", flush=True)
    pc = inputs.paged_cache(2, 1, 4, 2, 128, torch.bfloat16, seed=4803, page_size=64, lengths=[70, 50])
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens, smax=80).to(DEV)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens, smax=80).to(DEV)
    lens = torch.tensor([90, 50], dtype=torch.int32, device=DEV)         # sequence 0 past Smax = 80
    with pytest.raises(ValueError, match="the cache holds 80"):
        fa.fwd_kvcache(pc.q.to(DEV), kd, vd, lens, num_splits=2)
    neg = torch.tensor([10, -1], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="is negative"):
        fa.fwd_kvcache(pc.q.to(DEV), kd, vd, neg, num_splits=2)
