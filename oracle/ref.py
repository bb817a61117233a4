"""numpy float64 oracle for exact attention, forward and backward (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the ``cpu_baseline`` leg of the
benchmark may use this module; the product path never does.

What it computes is the plain definition of attention: three separate steps,
scores = Q Kᵀ, softmax over each score row, then the softmax weights times V
("optimizing-attention-flash" skill page, §3 workflow one, the hand-written
standard attention it replaces; the same three steps in "FlashAttention重大更新",
§1.2).  The pages stress that the fused method is exact, not an
approximation ("FlashAttention 常用接口简单介绍", §1 overview), so the oracle
is that definition written out, with no tiling and no online softmax: every
score row is materialised in full.

Options, and where each is defined:

* ``softmax_scale`` -- multiplies Q Kᵀ; ``None`` means 1/sqrt(head_dim)
  ("FlashAttention 常用接口简单介绍", §3.1 flash_attn_func).
* ``softcap`` -- tanh saturation of the scaled score, ``c * tanh(s / c)``, which
  keeps every score inside [-c, c]; 0 disables it (Flash-Attention v2.0–v2.7
  update notes, v2.6 Softcapping; "FlashAttention 常用接口简单介绍", §5.2).
* ``alibi_slopes`` -- a per-query-head linear distance penalty (update notes,
  v2.4 ALiBi; "FlashAttention 常用接口简单介绍", §5.1 gives the slopes).  The
  bias form is not printed; reading: ``-slope[h] * |i' - j|``.
* ``causal`` -- aligned to the bottom-right corner of the Sq x Sk matrix
  (update notes, the causal-mask change between v2.0.x and v2.1): query row i
  sits at key position ``i' = i + Sk - Sq``; key j is allowed iff ``j <= i'``.
* ``window=(left, right)`` -- local attention; -1 means unbounded on that side
  ("FlashAttention 常用接口简单介绍", §3.1 window_size; "optimizing-attention-flash",
  §3 workflow two, (-1,-1) is global).  Reading: inclusive
  ``i' - left <= j <= i' + right`` with the same alignment as causal.
* GQA / MQA -- query head h reads key/value head ``h // (Hq // Hkv)``
  ("FlashAttention 常用接口简单介绍", §4.2 FlashGQA; the skill page, §2).
* Rows with no allowed key: out = 0, lse = -inf (log of an empty sum).
* ``lse`` is the natural-log log-sum-exp of each row's final scores, bias
  included ("FlashAttention 常用接口简单介绍", §3.1 return values).

Inputs may be any float dtype (float16/bfloat16 tensors are upcast exactly);
all arithmetic is float64.

The backward (``attention_backward``) is the gradient of that same definition
with respect to q, k and v, written out step by step on the materialised score
rows.  The pages name the method's backward only through its two properties:
the attention weights are recomputed instead of stored (xhh.club tag page, the
summaries on tiling and recomputation; the skill page's overview), and a
deterministic mode exists (update notes, v2.4; "FlashAttention 常用接口简单介绍",
§5.3).  Neither changes the mathematical gradient, which is what this computes.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor: go through float32, exact for fp16/bf16
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def resolve_scale(softmax_scale, head_dim: int) -> float:
    """Default scale 1/sqrt(head_dim) ("FlashAttention 常用接口简单介绍", §3.1)."""
    if softmax_scale is None:
        return 1.0 / math.sqrt(head_dim)
    return float(softmax_scale)


def allowed_mask(rows, Sq: int, Sk: int, causal: bool, window=(-1, -1)) -> np.ndarray:
    """Boolean [len(rows), Sk]: may query row i attend key j?

    Bottom-right alignment (update notes, causal-mask change): the aligned
    position of row i is i' = i + Sk - Sq.  Causal forbids j > i'.  A window
    (left, right) keeps i' - left <= j <= i' + right, -1 meaning no bound on
    that side (§3.1 window_size of "FlashAttention 常用接口简单介绍").  When both
    are given the two masks intersect.
    """
    rows = np.asarray(rows, dtype=np.int64)
    ip = rows[:, None] + (Sk - Sq)          # aligned position i'
    j = np.arange(Sk, dtype=np.int64)[None, :]
    ok = np.ones((rows.size, Sk), dtype=bool)
    if causal:
        ok &= j <= ip
    left, right = int(window[0]), int(window[1])
    if left >= 0:
        ok &= j >= ip - left
    if right >= 0:
        ok &= j <= ip + right
    return ok


def _head_scores(qb, kb, rows, Sq, Sk, scale, softcap, slope, causal, window):
    """Final score rows [len(rows), Sk] of one (batch, query head), -inf where masked.

    Order: scale, then softcap on the scaled score, then the ALiBi bias, then the
    mask (plainest reading of the update notes v2.4/v2.6 and §5 of
    "FlashAttention 常用接口简单介绍").
    """
    s = scale * (qb @ kb.T)                                   # step 1: Q Kᵀ · scale
    if softcap > 0.0:                                         # step 2: softcap
        s = softcap * np.tanh(s / softcap)
    if slope is not None:                                     # step 3: ALiBi
        ip = np.asarray(rows, dtype=np.float64)[:, None] + (Sk - Sq)
        j = np.arange(Sk, dtype=np.float64)[None, :]
        s = s - slope * np.abs(ip - j)
    ok = allowed_mask(rows, Sq, Sk, causal, window)           # step 4: mask
    return np.where(ok, s, NEG_INF)


def _softmax_rows(s, vb):
    """Plain softmax of each materialised score row, times V; returns (out, lse).

    A row whose scores are all -inf has no allowed key: out 0, lse -inf.
    """
    n = s.shape[0]
    out = np.zeros((n, vb.shape[1]), dtype=np.float64)
    lse = np.full((n,), NEG_INF, dtype=np.float64)
    live = np.isfinite(s).any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)                     # row max (for a safe exp)
        e = np.exp(sl - m)                                    # masked entries give exp(-inf) = 0
        l = e.sum(axis=1, keepdims=True)
        out[live] = (e / l) @ vb
        lse[live] = (m + np.log(l))[:, 0]
    return out, lse


def attention(q, k, v, softmax_scale=None, causal=False, window=(-1, -1), softcap=0.0,
              alibi_slopes=None, rows=None, heads=None):
    """Dense attention forward on [B, S, H, D] tensors.

    q: [B, Sq, Hq, D]; k, v: [B, Sk, Hkv, D] with Hkv dividing Hq.
    rows: optional iterable of query rows to evaluate (each still sees its full
    score row); heads: optional iterable of query heads.
    Returns out [B, len(rows), Hq, D] (zeros for heads not evaluated) and
    lse [B, Hq, len(rows)] (NaN for heads not evaluated), both float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    scale = resolve_scale(softmax_scale, D)
    rows = np.arange(Sq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    slopes = None if alibi_slopes is None else _f64(alibi_slopes).reshape(-1)
    out = np.zeros((B, rows.size, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, rows.size), np.nan, dtype=np.float64)
    for b in range(B):
        for h in heads:
            hk = h // group                                   # GQA: consecutive query heads share a kv head
            s = _head_scores(q[b, rows, h, :], k[b, :, hk, :], rows, Sq, Sk, scale,
                             float(softcap), None if slopes is None else slopes[h], causal, window)
            o, ls = _softmax_rows(s, v[b, :, hk, :])
            out[b, :, h, :] = o
            lse[b, h, :] = ls
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, rows=None, **opts):
    """Packed variable-length attention ("FlashAttention 常用接口简单介绍", §3.2).

    q: [total_q, Hq, D]; k, v: [total_k, Hkv, D]; cu_seqlens_*: [B+1] prefix sums.
    Sequence b owns q rows [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]), and
    is attended on its own with its own Sq_b, Sk_b (so alignment is per sequence).
    rows: optional packed row indices to evaluate.
    Returns out [total_q, Hq, D] and lse [Hq, total_q] (NaN/0 where not evaluated).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    total_q, Hq, D = q.shape
    want = None if rows is None else set(int(r) for r in rows)
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    lse = np.full((Hq, total_q), np.nan, dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        local = [r - q0 for r in range(q0, q1) if want is None or r in want]
        if not local:
            continue
        o, ls = attention(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], rows=local, **opts)
        idx = np.asarray(local) + q0
        out[idx] = o[0]
        lse[:, idx] = ls[0]
    return out, lse


def gather_pages(pool, block_table_row, n_tokens: int, page_size: int) -> np.ndarray:
    """Dense [n_tokens, Hkv, D] copy of one sequence's cache from a page pool.

    Paged KV cache (update notes, v2.5): token t of the sequence lives in
    physical page block_table_row[t // page_size], at row t % page_size.
    pool: [num_pages, page_size, Hkv, D].
    """
    pool = _f64(pool)
    bt = np.asarray(block_table_row).reshape(-1)
    out = np.empty((n_tokens,) + pool.shape[2:], dtype=np.float64)
    for t in range(n_tokens):
        out[t] = pool[int(bt[t // page_size]), t % page_size]
    return out


def kvcache_append(k_cache, v_cache, k_new, v_new, cache_seqlens, block_table=None, page_size=None):
    """Caches after writing new tokens ("FlashAttention 常用接口简单介绍", §3.3: k and v,
    the optional new keys and values that update the cache).

    Reading: cache_seqlens counts the tokens already cached, so token t of
    sequence b's new block goes to cache position cache_seqlens[b] + t; with a
    block table that position lives in page block_table[b, pos // page_size], row
    pos % page_size (update notes, v2.5).  k_new/v_new: [B, S_new, Hkv, D].
    A position outside the cache (past Smax, past the block-table row, or a page
    number outside the pool) is not written: the library documents the same.
    Returns float64 copies; the inputs are not modified.
    """
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    kn = _f64(k_new)
    vn = _f64(v_new)
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    for b in range(kn.shape[0]):
        for t in range(kn.shape[1]):
            pos = lens[b] + t
            if pos < 0:
                continue
            if block_table is None:
                if pos >= kc.shape[1]:
                    continue
                kc[b, pos] = kn[b, t]
                vc[b, pos] = vn[b, t]
            else:
                row = np.asarray(block_table)[b]
                if pos // page_size >= row.shape[0]:
                    continue
                page = int(row[pos // page_size])
                if page < 0 or page >= kc.shape[0]:
                    continue
                kc[page, pos % page_size] = kn[b, t]
                vc[page, pos % page_size] = vn[b, t]
    return kc, vc


def attention_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, page_size=None,
                      heads=None, **opts):
    """Attention of new queries against a KV cache ("FlashAttention 常用接口简单介绍", §3.3).

    q: [B, Sq, Hq, D].  Without block_table, k_cache/v_cache are dense
    [B, Smax, Hkv, D]; with it, they are page pools [P, page_size, Hkv, D] and
    block_table is [B, max_pages] (update notes, v2.5).  Sequence b attends its
    first cache_seqlens[b] keys, bottom-right aligned against its Sq queries.
    Returns out [B, Sq, Hq, D] and lse [B, Hq, Sq].
    """
    q = _f64(q)
    B, Sq, Hq, D = q.shape
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    out = np.zeros((B, Sq, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, Sq), np.nan, dtype=np.float64)
    kc = _f64(k_cache)
    vc = _f64(v_cache)
    for b in range(B):
        n = lens[b]
        if block_table is None:
            kb, vb = kc[b, :n], vc[b, :n]
        else:
            bt = np.asarray(block_table)[b]
            kb = gather_pages(kc, bt, n, page_size)
            vb = gather_pages(vc, bt, n, page_size)
        o, ls = attention(q[b:b + 1], kb[None], vb[None], heads=heads, **opts)
        out[b] = o[0]
        lse[b] = ls[0]
    return out, lse


def combine(out_partial, lse_partial):
    """Merge attention results computed over disjoint key subsets.

    Split-KV decoding (update notes, v2.2) attends each key chunk separately and
    merges the chunks in a final reduction; "FlashAttention 常用接口简单介绍", §3.4
    gives the shapes: out_partial [B, S, H, D, n], lse_partial [B, S, H, n].  The
    formula is not printed; since every chunk's out is its own softmax average and
    lse its log normaliser, the only consistent merge is
    lse = log Σ_s exp(lse_s) and out = Σ_s exp(lse_s - lse) · out_s.
    A position whose chunks are all -inf (no allowed key anywhere) gives 0 / -inf.
    Returns out [B, S, H, D] and lse [B, S, H].
    """
    op = _f64(out_partial)
    lp = _f64(lse_partial)
    m = lp.max(axis=-1)                                       # [B,S,H]
    live = np.isfinite(m)
    msafe = np.where(live, m, 0.0)
    w = np.exp(lp - msafe[..., None])                         # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=-1)
    lse = np.where(live, msafe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    wn = np.where(live[..., None], w / np.where(live, tot, 1.0)[..., None], 0.0)
    out = (op * wn[..., None, :]).sum(axis=-1)
    return out, lse


def _head_backward(qb, kb, vb, gb, s, scale, softcap):
    """Steps 2-6 of ``attention_backward`` for one (batch, query head).

    s: the final score rows [Sq, Sk] (-inf where masked); gb: dout rows.
    Returns (dq [Sq, D], dk [Sk, D], dv [Sk, D]) of this query head.
    """
    P = np.zeros_like(s)                                                      # step 2
    live = np.isfinite(s).any(axis=1)
    if live.any():
        sl = s[live]
        e = np.exp(sl - sl.max(axis=1, keepdims=True))
        P[live] = e / e.sum(axis=1, keepdims=True)
    dv = P.T @ gb                                                             # step 3
    dP = gb @ vb.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))                       # step 4
    dU = dS                                                                   # step 5
    if softcap > 0.0:
        t = np.tanh(scale * (qb @ kb.T) / softcap)
        dU = dU * (1.0 - t * t)
    dU = dU * scale
    return dU @ kb, dU.T @ qb, dv                                             # step 6


def attention_backward(q, k, v, dout, softmax_scale=None, causal=False, window=(-1, -1), softcap=0.0,
                       alibi_slopes=None):
    """Gradients (dq, dk, dv) of the loss sum(out * dout) for the dense forward.

    Shapes as in ``attention``: q, dout [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D].
    Per (batch, query head), on the full score rows:
      1. raw u = scale · Q Kᵀ, then the forward's score s (softcap, ALiBi, mask);
      2. P = softmax of each row of s (rows with no allowed key: P = 0);
      3. dV += Pᵀ dO and dP = dO Vᵀ;
      4. dS = P ∘ (dP − rowsum(P ∘ dP)), the Jacobian of a softmax row applied
         to dP (masked entries have P = 0 and get no gradient);
      5. back through the score transform: ALiBi adds a constant (slope ·
         distance), so it passes dS unchanged; softcap s = c·tanh(u / c) has
         derivative 1 − tanh²(u / c); the scale gives a factor scale;
      6. dQ = dU K and dK += dUᵀ Q, with dU the gradient at the raw product.
    GQA: a kv head collects dk and dv from all query heads that read it.
    Returns float64 dq [B, Sq, Hq, D], dk and dv [B, Sk, Hkv, D].
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if dout.shape != q.shape or k.shape != (B, Sk, Hkv, D) or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    scale = resolve_scale(softmax_scale, D)
    slopes = None if alibi_slopes is None else _f64(alibi_slopes).reshape(-1)
    rows = np.arange(Sq)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            qb, kb, vb, gb = q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :], dout[b, :, h, :]
            s = _head_scores(qb, kb, rows, Sq, Sk, scale, float(softcap),
                             None if slopes is None else slopes[h], causal, window)     # step 1
            dqh, dkh, dvh = _head_backward(qb, kb, vb, gb, s, scale, float(softcap))
            dq[b, :, h, :] = dqh
            dk[b, :, hk, :] += dkh
            dv[b, :, hk, :] += dvh
    return dq, dk, dv


def flops(Sq: int, Sk: int, D: int, causal=False, window=(-1, -1)) -> int:
    """Algorithmic FLOPs of one (batch, head): 4·D per allowed (query, key) pair.

    Two contractions (Q Kᵀ and P V) of 2·D FLOPs each per pair; masked pairs
    are not counted.
    """
    ok = allowed_mask(np.arange(Sq), Sq, Sk, causal, window)
    return int(4 * D * int(ok.sum()))
