"""Seeded synthetic inputs for the attention-forward workloads.

This module only draws random tensors and lays them out (packing, page pools,
block tables); it holds none of the attention arithmetic.  Both the HIP path
and the CPU oracle are fed from it.

Recipe: a CPU ``torch.Generator`` seeded per case draws float32 values (normal
N(0,1), times a scale when the workload asks for one) in the order q, k, v,
then any extras; the values are rounded to float16/bfloat16 (round to nearest
even).  The same host tensors go to the device and, upcast exactly, to the
oracle.  The pages' own examples build their inputs the same way, with
``torch.randn`` of the [batch, seqlen, heads, head_dim] shape
("FlashAttention 常用接口简单介绍", §3.1-§3.3).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


def seed_for(config: int, variant: int = 0) -> int:
    return 1000 + config + 10 * variant


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def randn(gen: torch.Generator, shape, dtype: torch.dtype, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def dense_qkv(B, Sq, Sk, Hq, Hkv, D, dtype, seed, scale=1.0):
    """q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] on the CPU."""
    g = _gen(seed)
    q = randn(g, (B, Sq, Hq, D), dtype, scale)
    k = randn(g, (B, Sk, Hkv, D), dtype, scale)
    v = randn(g, (B, Sk, Hkv, D), dtype, scale)
    return q, k, v


def alibi_slopes_closed_form(H: int) -> torch.Tensor:
    """Slopes 2^(-8(i+1)/H) for head i, float32."""
    return torch.tensor([2.0 ** (-8.0 * (i + 1) / H) for i in range(H)], dtype=torch.float32)


def alibi_slopes(H: int) -> torch.Tensor:
    """ALiBi slopes built the way "FlashAttention 常用接口简单介绍", §5.1 describes.

    For a power of two n the slopes form a geometric sequence whose first term
    and ratio are both 2^(-8/n).  Otherwise the slopes of the largest power of
    two p below H are followed by every other slope of the 2p sequence, up to
    H slopes in total.
    """
    def pow2(n):
        start = 2.0 ** (-(2.0 ** -(math.log2(n) - 3)))
        return [start ** (i + 1) for i in range(n)]

    if math.log2(H).is_integer():
        s = pow2(H)
    else:
        p = 2 ** int(math.floor(math.log2(H)))
        s = pow2(p) + pow2(2 * p)[0::2][: H - p]
    return torch.tensor(s, dtype=torch.float32)


def varlen_pack(lengths_q, lengths_k, Hq, Hkv, D, dtype, seed, scale=1.0):
    """Packed q [total_q,Hq,D], k/v [total_k,Hkv,D] plus int32 cu_seqlens [B+1]."""
    g = _gen(seed)
    cq = torch.tensor([0] + list(lengths_q), dtype=torch.int64).cumsum(0).to(torch.int32)
    ck = torch.tensor([0] + list(lengths_k), dtype=torch.int64).cumsum(0).to(torch.int32)
    q = randn(g, (int(cq[-1]), Hq, D), dtype, scale)
    k = randn(g, (int(ck[-1]), Hkv, D), dtype, scale)
    v = randn(g, (int(ck[-1]), Hkv, D), dtype, scale)
    return q, k, v, cq, ck


def pad_varlen_to_dense(x: torch.Tensor, cu: torch.Tensor, smax: int) -> torch.Tensor:
    """[total, H, D] packed -> [B, smax, H, D] zero-padded (layout only)."""
    B = cu.numel() - 1
    out = torch.zeros((B, smax) + tuple(x.shape[1:]), dtype=x.dtype)
    for b in range(B):
        a, e = int(cu[b]), int(cu[b + 1])
        out[b, : e - a] = x[a:e]
    return out


@dataclass
class PagedCache:
    q: torch.Tensor              # [B, Sq, Hq, D]
    k_pool: torch.Tensor         # [P, page_size, Hkv, D]
    v_pool: torch.Tensor
    block_table: torch.Tensor    # int32 [B, max_pages], -1 past each sequence's pages
    cache_seqlens: torch.Tensor  # int32 [B]
    page_size: int
    extra: dict = field(default_factory=dict)


def paged_cache(B, Sq, Hq, Hkv, D, dtype, seed, page_size=256, len_lo=1024, len_hi=16384,
                max_pages=None, lengths=None, tail_fill="randn", scale=1.0) -> PagedCache:
    """Decode inputs over a paged KV pool with a randomly permuted block table.

    Draw order: sequence lengths (uniform integers in [len_lo, len_hi] unless
    given), a permutation of the P = Σ ceil(len_b / page_size) pages, then q,
    then the K pool, then the V pool.  Sequence b's pages are consecutive
    entries of the permutation.  Rows of a sequence's last page past its length
    are filled per ``tail_fill`` ("randn", "zero" or "nan"), so a kernel that
    reads them is caught.
    """
    g = _gen(seed)
    if lengths is None:
        lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    else:
        lens = torch.tensor(list(lengths), dtype=torch.int64)
    npages = [(int(n) + page_size - 1) // page_size for n in lens]
    P = sum(npages)
    perm = torch.randperm(max(P, 1), generator=g)[:P]
    if max_pages is None:
        max_pages = max(1, max(npages) if npages else 1)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32)
    pos = 0
    for b in range(B):
        bt[b, : npages[b]] = perm[pos: pos + npages[b]].to(torch.int32)
        pos += npages[b]
    q = randn(g, (B, Sq, Hq, D), dtype, scale)
    kp = randn(g, (max(P, 1), page_size, Hkv, D), dtype, scale)
    vp = randn(g, (max(P, 1), page_size, Hkv, D), dtype, scale)
    if tail_fill != "randn":
        fill = 0.0 if tail_fill == "zero" else float("nan")
        for b in range(B):
            n = int(lens[b])
            if n % page_size and npages[b]:
                last = int(bt[b, npages[b] - 1])
                kp[last, n % page_size:] = fill
                vp[last, n % page_size:] = fill
    return PagedCache(q=q, k_pool=kp, v_pool=vp, block_table=bt,
                      cache_seqlens=lens.to(torch.int32), page_size=page_size)


def dense_cache_from_pool(pool: torch.Tensor, block_table: torch.Tensor, lens: torch.Tensor,
                          smax: int | None = None) -> torch.Tensor:
    """Dense cache [B, smax, Hkv, D] holding each sequence's tokens gathered from the pool.

    Token t of sequence b is pool[block_table[b, t // page], t % page]; positions
    at or past the length are zero.  Layout only (used to build the dense twin
    of a paged workload).
    """
    page = pool.shape[1]
    B = block_table.shape[0]
    if smax is None:
        smax = int(lens.max()) if B else 0
    out = torch.zeros((B, smax) + tuple(pool.shape[2:]), dtype=pool.dtype)
    for b in range(B):
        n = int(lens[b])
        npg = (n + page - 1) // page
        if npg:
            pages = pool[block_table[b, :npg].long()]              # [npg, page, H, D]
            out[b, :n] = pages.reshape((npg * page,) + tuple(pool.shape[2:]))[:n]
    return out


# ---------------------------------------------------------------------------
# The five workloads.  Each case returns a dict with the tensors and options.
# ---------------------------------------------------------------------------

def case(name: str) -> dict:
    """Inputs of one named workload case (all CPU tensors)."""
    if name.startswith("c1"):
        # B=1, Hq=Hkv=2, Sq=Sk=128, D=64, fp16 N(0,1), scale 1/8
        if name == "c1_decode":
            q, k, v = dense_qkv(1, 1, 128, 2, 2, 64, torch.float16, seed_for(1, 2))
        else:
            q, k, v = dense_qkv(1, 128, 128, 2, 2, 64, torch.float16, seed_for(1))
        causal = name in ("c1_causal", "c1_decode")
        return dict(kind="dense", q=q, k=k, v=v, softmax_scale=0.125, causal=causal)
    if name in ("c2_causal", "c2_noncausal"):
        q, k, v = dense_qkv(2, 1024, 1024, 8, 8, 64, torch.float16, seed_for(2))
        return dict(kind="dense", q=q, k=k, v=v, causal=name == "c2_causal")
    if name == "c2_varlen":
        q, k, v, cq, ck = varlen_pack([512, 1024, 768], [512, 1024, 768], 8, 8, 64,
                                      torch.float16, seed_for(2, 1))
        return dict(kind="varlen", q=q, k=k, v=v, cu_seqlens_q=cq, cu_seqlens_k=ck,
                    max_seqlen_q=1024, max_seqlen_k=1024, causal=True)
    if name.startswith("c3"):
        q, k, v = dense_qkv(4, 4096, 4096, 32, 32, 64, torch.float16, seed_for(3))
        if name == "c3_causal":
            return dict(kind="dense", q=q, k=k, v=v, causal=True)
        if name == "c3_win256_0":
            return dict(kind="dense", q=q, k=k, v=v, causal=True, window=(256, 0))
        if name == "c3_win256_256":
            return dict(kind="dense", q=q, k=k, v=v, causal=False, window=(256, 256))
    if name == "c4_gqa":
        q, k, v = dense_qkv(2, 8192, 8192, 32, 8, 128, torch.bfloat16, seed_for(4), scale=0.5)
        return dict(kind="dense", q=q, k=k, v=v, causal=True, softcap=50.0,
                    alibi_slopes=alibi_slopes_closed_form(32))
    if name == "c5_paged":
        pc = paged_cache(64, 1, 32, 8, 128, torch.bfloat16, seed_for(5), page_size=256,
                         len_lo=1024, len_hi=16384, max_pages=64)
        return dict(kind="paged", q=pc.q, k_pool=pc.k_pool, v_pool=pc.v_pool,
                    block_table=pc.block_table, cache_seqlens=pc.cache_seqlens,
                    page_size=256, num_splits=16)
    raise KeyError(name)


CASES = ["c1_noncausal", "c1_causal", "c1_decode", "c2_causal", "c2_noncausal", "c2_varlen",
         "c3_causal", "c3_win256_0", "c3_win256_256", "c4_gqa", "c5_paged"]
