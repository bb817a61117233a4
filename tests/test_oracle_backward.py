"""Pins of the oracle's backward (ref.attention_backward) against things other than
its own formula (no GPU).

* central finite differences of the oracle's forward, which is itself pinned by
  the brute force, the fixtures and the closed forms in test_oracle.py: the
  gradient of sum(out * dout) with respect to every element of q, k and v, on
  tiny shapes with every option;
* closed forms: a single key, values that are the same for every key, and
  all-zero queries (uniform weights);
* GQA as repeated heads whose key/value gradients are summed;
* planted mistakes in the oracle (dropped softmax-Jacobian term, dropped
  softcap derivative, dropped scale) each fail the finite-difference pin.
"""

import zlib

import numpy as np
import pytest

from oracle import ref

OPTIONS = [
    dict(),
    dict(causal=True),
    dict(window=(2, 1)),
    dict(window=(1, 0), causal=True),
    dict(softcap=0.8),
    dict(alibi=True),
    dict(alibi=True, causal=True, softcap=1.5),
    dict(window=(0, 2), softmax_scale=0.6, softcap=2.0),
]
# (B, Sq, Sk, Hq, Hkv, D): Sq > Sk with causal leaves rows with no allowed key
SHAPES = [(1, 4, 6, 2, 1, 3), (1, 6, 3, 2, 2, 2), (2, 3, 3, 2, 1, 2)]


def _case(shape, opts, seed):
    B, Sq, Sk, Hq, Hkv, D = shape
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    g = rng.standard_normal((B, Sq, Hq, D))
    kw = dict(causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
              softcap=opts.get("softcap", 0.0), softmax_scale=opts.get("softmax_scale"),
              alibi_slopes=rng.uniform(0.1, 1.0, Hq) if opts.get("alibi") else None)
    return q, k, v, g, kw


def _finite_differences(q, k, v, g, kw, h=1e-5):
    """Central differences of L = sum(out * g) through the oracle's forward."""
    def loss(q_, k_, v_):
        out, _ = ref.attention(q_, k_, v_, **kw)
        return float((out * g).sum())
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        d = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(*args)
            x[idx] = x0 - h
            lm = loss(*args)
            x[idx] = x0
            d[idx] = (lp - lm) / (2 * h)
        grads.append(d)
    return grads


def _agrees_with_fd(shape, opts, seed, backward=None):
    q, k, v, g, kw = _case(shape, opts, seed)
    got = (backward or ref.attention_backward)(q, k, v, g, **kw)
    want = _finite_differences(q, k, v, g, kw)
    return all(np.max(np.abs(a - b)) <= 1e-6 for a, b in zip(got, want))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("opts", OPTIONS, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()) or "plain")
def test_backward_equals_finite_differences(shape, opts):
    assert _agrees_with_fd(shape, opts, seed=zlib.crc32(repr((shape, opts)).encode()) % 1000)


def test_single_key_gives_no_query_or_key_gradient():
    # one key: every weight is 1 whatever q and k are, so out = v and
    # dq = dk = 0, dv = the sum of dout over every query row and head of the group
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 5, 4, 3))
    k = rng.standard_normal((2, 1, 2, 3))
    v = rng.standard_normal((2, 1, 2, 3))
    g = rng.standard_normal((2, 5, 4, 3))
    dq, dk, dv = ref.attention_backward(q, k, v, g, softcap=1.3)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    want = g.reshape(2, 5, 2, 2, 3).sum(axis=(1, 3))            # heads 2hk, 2hk+1 -> kv head hk
    np.testing.assert_allclose(dv[:, 0], want, rtol=0, atol=1e-13)


def test_same_value_for_every_key_gives_no_query_or_key_gradient():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4, 2, 3))
    k = rng.standard_normal((1, 6, 2, 3))
    v = np.broadcast_to(rng.standard_normal((1, 1, 2, 3)), (1, 6, 2, 3)).copy()
    g = rng.standard_normal((1, 4, 2, 3))
    dq, dk, dv = ref.attention_backward(q, k, v, g, causal=True)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.abs(dv).max() > 0.1


def test_zero_queries_closed_form():
    # q = 0: every allowed weight is 1/Sk, so dv_j = (1/Sk) sum_i g_i,
    # dq_i = (scale/Sk) sum_j (g_i . (v_j - mean v)) k_j, and dk = 0
    rng = np.random.default_rng(5)
    Sq, Sk, D = 3, 5, 4
    q = np.zeros((1, Sq, 1, D))
    k = rng.standard_normal((1, Sk, 1, D))
    v = rng.standard_normal((1, Sk, 1, D))
    g = rng.standard_normal((1, Sq, 1, D))
    scale = 0.7
    dq, dk, dv = ref.attention_backward(q, k, v, g, softmax_scale=scale)
    kk, vv, gg = k[0, :, 0], v[0, :, 0], g[0, :, 0]
    want_dv = np.repeat(gg.sum(axis=0, keepdims=True) / Sk, Sk, axis=0)
    want_dq = scale / Sk * ((gg @ (vv - vv.mean(axis=0)).T) @ kk)
    np.testing.assert_allclose(dv[0, :, 0], want_dv, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq[0, :, 0], want_dq, rtol=0, atol=1e-13)
    assert np.abs(dk).max() < 1e-14


def test_gqa_equals_repeated_heads_with_summed_kv_gradients():
    rng = np.random.default_rng(6)
    B, Sq, Sk, Hq, Hkv, D = 2, 5, 7, 6, 2, 3
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    g = rng.standard_normal((B, Sq, Hq, D))
    sl = rng.uniform(0.1, 1.0, Hq)
    kw = dict(causal=True, softcap=1.1, alibi_slopes=sl)
    dq, dk, dv = ref.attention_backward(q, k, v, g, **kw)
    G = Hq // Hkv
    dq2, dk2, dv2 = ref.attention_backward(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), g, **kw)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, Sk, Hkv, G, D).sum(axis=3), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, Sk, Hkv, G, D).sum(axis=3), rtol=0, atol=1e-13)


def test_finite_difference_pin_catches_planted_mistakes(monkeypatch):
    shape, opts = (1, 4, 5, 2, 1, 3), dict(causal=True, softcap=1.2, alibi=True)
    assert _agrees_with_fd(shape, opts, 11)
    good = ref._head_backward

    # 1. softmax Jacobian without its rowsum term: dS = P * dP
    def no_rowsum(qb, kb, vb, gb, s, scale, softcap):
        dq, dk, dv = good(qb, kb, vb, gb, s, scale, softcap)
        P = np.zeros_like(s)
        live = np.isfinite(s).any(axis=1)
        e = np.exp(s[live] - s[live].max(axis=1, keepdims=True))
        P[live] = e / e.sum(axis=1, keepdims=True)
        dU = P * (gb @ vb.T) * scale
        if softcap > 0:
            dU = dU * (1 - np.tanh(scale * (qb @ kb.T) / softcap) ** 2)
        return dU @ kb, dU.T @ qb, dv
    monkeypatch.setattr(ref, "_head_backward", no_rowsum)
    assert not _agrees_with_fd(shape, opts, 11)

    # 2. the chain through tanh dropped
    monkeypatch.setattr(ref, "_head_backward",
                        lambda qb, kb, vb, gb, s, scale, softcap: good(qb, kb, vb, gb, s, scale, 0.0))
    assert not _agrees_with_fd(shape, opts, 11)

    # 3. the softmax scale dropped from the gradient
    def no_scale(qb, kb, vb, gb, s, scale, softcap):
        dq, dk, dv = good(qb, kb, vb, gb, s, scale, softcap)
        return dq / scale, dk / scale, dv
    monkeypatch.setattr(ref, "_head_backward", no_scale)
    assert not _agrees_with_fd(shape, opts, 11)

    monkeypatch.setattr(ref, "_head_backward", good)
    assert _agrees_with_fd(shape, opts, 11)
