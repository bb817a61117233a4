"""Pins of the CPU oracle against things other than itself (no GPU).

* hand-written mask fixtures from the pages' alignment and window rules
  (tests/golden/*.txt, each citing its page and section);
* an independent scalar brute force (oracle.brute) on tiny shapes with every option;
* torch's CPU scaled_dot_product_attention in float64 with an explicit mask
  (a library routine the oracle does not use);
* closed forms and invariants: identical keys, decode alignment, global
  window, softcap bounds and limits, the ALiBi shift identity, GQA as repeated
  heads, varlen as per-sequence dense, paged gather, the LSE combine.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def read_mask_cases(fname):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                kv = dict(t.split("=") for t in line.split()[1:])
                cur = dict(Sq=int(kv["Sq"]), Sk=int(kv["Sk"]), causal=bool(int(kv["causal"])),
                           window=(int(kv["left"]), int(kv["right"])), rows=[])
                cases.append(cur)
            else:
                cur["rows"].append([c == "1" for c in line])
    return cases


MASK_CASES = read_mask_cases("causal_bottom_right.txt") + read_mask_cases("window_masks.txt")


@pytest.mark.parametrize("c", MASK_CASES, ids=lambda c: f"{c['Sq']}x{c['Sk']}c{int(c['causal'])}w{c['window']}")
def test_ref_mask_matches_golden(c):
    got = ref.allowed_mask(np.arange(c["Sq"]), c["Sq"], c["Sk"], c["causal"], c["window"])
    assert got.tolist() == c["rows"]


@pytest.mark.parametrize("c", MASK_CASES, ids=lambda c: f"{c['Sq']}x{c['Sk']}c{int(c['causal'])}w{c['window']}")
def test_mask_through_attention_outputs(c):
    # q = 0 gives equal weights on every allowed key; with v_j = e_j (one-hot),
    # out[i] is 1/count on the allowed keys and 0 elsewhere.  Exercises the mask as
    # the full oracle and the brute force apply it.
    Sq, Sk = c["Sq"], c["Sk"]
    q = np.zeros((1, Sq, 1, Sk))
    k = RNG.standard_normal((1, Sk, 1, Sk))
    v = np.eye(Sk).reshape(1, Sk, 1, Sk)
    want = np.array(c["rows"], dtype=bool)
    o, lse = ref.attention(q, k, v, causal=c["causal"], window=c["window"])
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal=c["causal"], window=c["window"])
    for i in range(Sq):
        n = want[i].sum()
        exp_row = np.where(want[i], 1.0 / n, 0.0) if n else np.zeros(Sk)
        assert np.allclose(o[0, i, 0], exp_row, atol=1e-15)
        assert np.allclose(ob[0][i][0], exp_row, atol=1e-15)
        if n == 0:
            assert lse[0, 0, i] == -np.inf and lseb[0][0][i] == -math.inf
        else:
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)


def _rand_case(rng, B, Sq, Sk, Hq, Hkv, D):
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    return q, k, v


OPTION_GRID = [
    dict(),
    dict(causal=True),
    dict(window=(2, 1)),
    dict(window=(3, 0), causal=True),
    dict(window=(0, -1)),
    dict(softcap=0.7),
    dict(alibi=True),
    dict(alibi=True, causal=True, softcap=2.0),
    dict(alibi=True, window=(2, 2), softmax_scale=0.37),
    dict(causal=True, softmax_scale=1.9, softcap=1.5),
]
SHAPES = [(1, 5, 5, 2, 2, 4), (2, 3, 7, 4, 2, 3), (1, 7, 3, 3, 1, 5), (1, 1, 6, 2, 1, 8), (2, 6, 6, 4, 4, 2)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("opts", OPTION_GRID, ids=lambda o: ",".join(f"{k}={v}" for k, v in o.items()) or "plain")
def test_ref_equals_brute_force(shape, opts):
    B, Sq, Sk, Hq, Hkv, D = shape
    rng = np.random.default_rng(hash((shape, tuple(sorted(opts)))) % (2**32))
    q, k, v = _rand_case(rng, B, Sq, Sk, Hq, Hkv, D)
    slopes = rng.uniform(0.05, 1.0, Hq) if opts.get("alibi") else None
    kw = dict(causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
              softcap=opts.get("softcap", 0.0))
    o, lse = ref.attention(q, k, v, softmax_scale=opts.get("softmax_scale"), alibi_slopes=slopes, **kw)
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale=opts.get("softmax_scale"),
                               slopes=None if slopes is None else slopes.tolist(), **kw)
    ob, lseb = np.array(ob), np.array(lseb)
    assert np.max(np.abs(o - ob)) <= 1e-12
    fin = np.isfinite(lseb)
    assert (np.isfinite(lse) == fin).all()
    assert np.max(np.abs(lse[fin] - lseb[fin]), initial=0.0) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("alibi", [False, True])
def test_ref_equals_torch_sdpa_float64(causal, alibi):
    # torch.nn.functional.scaled_dot_product_attention on the CPU in float64 with an
    # explicit additive mask (its own is_causal is top-left aligned, so the
    # bottom-right mask is passed in); Sq != Sk to exercise the alignment.
    rng = np.random.default_rng(7 + causal + 2 * alibi)
    B, Sq, Sk, H, D = 2, 9, 13, 3, 16
    q, k, v = _rand_case(rng, B, Sq, Sk, H, H, D)
    slopes = rng.uniform(0.1, 0.9, H) if alibi else None
    o, _ = ref.attention(q, k, v, causal=causal, alibi_slopes=slopes)
    ok = np.ones((Sq, Sk), bool)
    if causal:
        for i in range(Sq):
            ok[i, i + Sk - Sq + 1:] = False
    bias = np.where(ok, 0.0, -np.inf)[None].repeat(H, 0)
    if alibi:
        dist = np.abs((np.arange(Sq)[:, None] + Sk - Sq) - np.arange(Sk)[None, :])
        bias = bias - slopes[:, None, None] * dist[None]  # [H, Sq, Sk]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    want = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(bias)[None].expand(B, -1, -1, -1))
    want = want.numpy().transpose(0, 2, 1, 3)
    assert np.max(np.abs(o - want)) <= 1e-12


def test_closed_form_two_keys():
    # One query, two keys, scale 1: scores (1, 0) -> weights e/(e+1), 1/(e+1).
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 2.0], [3.0, 4.0]]).reshape(1, 2, 1, 2)
    o, lse = ref.attention(q, k, v, softmax_scale=1.0)
    e = math.e
    assert o[0, 0, 0].tolist() == pytest.approx([(e + 3) / (e + 1), (2 * e + 4) / (e + 1)], abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(e + 1), abs=1e-15)


def test_default_scale_is_inverse_sqrt_head_dim():
    rng = np.random.default_rng(3)
    q, k, v = _rand_case(rng, 1, 4, 6, 2, 2, 16)
    a, la = ref.attention(q, k, v)
    b, lb = ref.attention(q, k, v, softmax_scale=0.25)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_identical_keys_give_mean_of_allowed_values():
    rng = np.random.default_rng(4)
    Sq, Sk, D = 6, 9, 8
    q = rng.standard_normal((1, Sq, 1, D))
    k = np.repeat(rng.standard_normal((1, 1, 1, D)), Sk, axis=1)
    v = rng.standard_normal((1, Sk, 1, D))
    o, _ = ref.attention(q, k, v, causal=True)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        assert np.allclose(o[0, i, 0], v[0, :n, 0].mean(axis=0), atol=1e-14)
    o, _ = ref.attention(q, k, v)
    assert np.allclose(o[0, :, 0], v[0, :, 0].mean(axis=0)[None], atol=1e-14)


def test_decode_causal_attends_every_key():
    # One new query against N+1 keys sees all of them under bottom-right causal.
    rng = np.random.default_rng(5)
    q, k, v = _rand_case(rng, 2, 1, 17, 2, 2, 8)
    a = ref.attention(q, k, v, causal=True)
    b = ref.attention(q, k, v, causal=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_first_row_and_overhang_rows():
    rng = np.random.default_rng(6)
    q, k, v = _rand_case(rng, 1, 5, 5, 1, 1, 4)
    o, lse = ref.attention(q, k, v, causal=True, softmax_scale=0.5)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert lse[0, 0, 0] == pytest.approx(0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-15)
    q, k, v = _rand_case(rng, 1, 7, 4, 1, 1, 4)          # Sq > Sk: 3 rows see nothing
    o, lse = ref.attention(q, k, v, causal=True)
    assert (o[0, :3] == 0).all() and (lse[0, 0, :3] == -np.inf).all()
    assert np.isfinite(lse[0, 0, 3:]).all()


def test_window_special_cases():
    rng = np.random.default_rng(8)
    q, k, v = _rand_case(rng, 1, 6, 8, 2, 2, 4)
    full = ref.attention(q, k, v)
    for w in [(-1, -1), (8, 8), (100, -1), (-1, 100)]:
        got = ref.attention(q, k, v, window=w)
        assert np.array_equal(got[0], full[0]) and np.array_equal(got[1], full[1])
    o, _ = ref.attention(q, k, v, window=(0, 0))
    for i in range(6):
        assert np.allclose(o[0, i], v[0, i + 2], atol=0)
    a = ref.attention(q, k, v, causal=True, window=(3, 5))
    b = ref.attention(q, k, v, causal=False, window=(3, 0))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_softcap_bounds_limit_and_symmetry():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((12, 16)) * 6.0
    kk = rng.standard_normal((10, 16)) * 6.0
    rows = np.arange(12)
    for c in (0.5, 3.0, 50.0):
        s = ref._head_scores(q, kk, rows, 12, 10, 1.0, c, None, False, (-1, -1))
        assert np.abs(s).max() <= c
        s_neg = ref._head_scores(-q, kk, rows, 12, 10, 1.0, c, None, False, (-1, -1))
        assert np.allclose(s_neg, -s, atol=1e-15)
    plain = ref._head_scores(q, kk, rows, 12, 10, 0.1, 0.0, None, False, (-1, -1))
    capped = ref._head_scores(q, kk, rows, 12, 10, 0.1, 1e6, None, False, (-1, -1))
    # c·tanh(s/c) = s - s^3/(3c^2) + ...: the gap is bounded by |s|^3 / (3 c^2)
    assert (np.abs(plain - capped) <= np.abs(plain) ** 3 / (3 * 1e12) * 1.01 + 1e-13).all()
    q4, k4, v4 = _rand_case(rng, 1, 5, 5, 1, 1, 4)
    a = ref.attention(q4, k4, v4, softcap=1e7)
    b = ref.attention(q4, k4, v4)
    assert np.max(np.abs(a[0] - b[0])) <= 1e-9


def test_alibi_zero_slope_is_no_bias():
    rng = np.random.default_rng(10)
    q, k, v = _rand_case(rng, 1, 5, 7, 2, 2, 4)
    a = ref.attention(q, k, v, alibi_slopes=np.zeros(2))
    b = ref.attention(q, k, v)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_alibi_causal_shift_identity():
    # Under causal masking -slope*|i'-j| = -slope*i' + slope*j.  The row constant
    # -slope*i' does not change out but shifts lse; the +slope*j part can be had
    # without ALiBi by appending one coordinate to q (slope/scale) and k (j).
    rng = np.random.default_rng(11)
    Sq, Sk, D, scale, slope = 6, 9, 4, 0.3, 0.45
    q, k, v = _rand_case(rng, 1, Sq, Sk, 1, 1, D)
    o, lse = ref.attention(q, k, v, causal=True, softmax_scale=scale, alibi_slopes=np.array([slope]))
    qa = np.concatenate([q, np.full((1, Sq, 1, 1), slope / scale)], axis=-1)
    ka = np.concatenate([k, np.arange(Sk, dtype=float).reshape(1, Sk, 1, 1)], axis=-1)
    va = np.concatenate([v, np.zeros((1, Sk, 1, 1))], axis=-1)
    oa, lsea = ref.attention(qa, ka, va, causal=True, softmax_scale=scale)
    assert np.max(np.abs(o - oa[..., :D])) <= 1e-13
    ip = np.arange(Sq) + Sk - Sq
    assert np.max(np.abs(lse[0, 0] - (lsea[0, 0] - slope * ip))) <= 1e-12


def test_convexity_and_key_permutation():
    rng = np.random.default_rng(12)
    q, k, v = _rand_case(rng, 1, 5, 11, 2, 2, 6)
    o, lse = ref.attention(q, k, v, window=(3, 2))
    ok = ref.allowed_mask(np.arange(5), 5, 11, False, (3, 2))
    for h in range(2):
        for i in range(5):
            vs = v[0, ok[i], h]
            assert (o[0, i, h] >= vs.min(axis=0) - 1e-14).all() and (o[0, i, h] <= vs.max(axis=0) + 1e-14).all()
    perm = rng.permutation(11)
    a = ref.attention(q, k, v)
    b = ref.attention(q, k[:, perm], v[:, perm])
    assert np.max(np.abs(a[0] - b[0])) <= 1e-14 and np.max(np.abs(a[1] - b[1])) <= 1e-13


def test_gqa_equals_repeated_heads():
    rng = np.random.default_rng(13)
    for hkv in (1, 2):
        q, k, v = _rand_case(rng, 2, 5, 7, 4, hkv, 4)
        a = ref.attention(q, k, v, causal=True)
        rep = 4 // hkv
        b = ref.attention(q, np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2), causal=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_varlen_equals_per_sequence_dense():
    from exact_attention_forward_fa_amd import inputs
    lens = [5, 1, 9, 4]
    q, k, v, cq, ck = inputs.varlen_pack(lens, [7, 3, 9, 2], 4, 2, 8, torch.float16, seed=77)
    for opts in (dict(causal=True), dict(window=(2, 1)), dict()):
        o, lse = ref.attention_varlen(q, k, v, cq, ck, **opts)
        for b in range(4):
            q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
            od, ld = ref.attention(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], **opts)
            assert np.array_equal(o[q0:q1], od[0])
            assert np.array_equal(lse[:, q0:q1], ld[0])
    # sampled rows agree with the full evaluation
    o2, l2 = ref.attention_varlen(q, k, v, cq, ck, rows=[0, 6, 14], causal=True)
    o, lse = ref.attention_varlen(q, k, v, cq, ck, causal=True)
    # (same values up to BLAS summation order: the matmul shapes differ)
    assert np.max(np.abs(o2[[0, 6, 14]] - o[[0, 6, 14]])) <= 1e-14
    assert np.max(np.abs(l2[:, [0, 6, 14]] - lse[:, [0, 6, 14]])) <= 1e-14


def test_paged_gather_equals_dense_cache():
    from exact_attention_forward_fa_amd import inputs
    pc = inputs.paged_cache(3, 1, 4, 2, 8, torch.bfloat16, seed=5, page_size=4, lengths=[9, 4, 1], max_pages=4)
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    for b, n in enumerate([9, 4, 1]):
        g = ref.gather_pages(pc.k_pool, pc.block_table[b], n, 4)
        assert np.array_equal(g, kd[b, :n].float().numpy())
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    a = ref.attention_kvcache(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 4)
    b = ref.attention_kvcache(pc.q, kd, vd, pc.cache_seqlens)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # and the per-sequence result is plain attention over the first len tokens
    for bb, n in enumerate([9, 4, 1]):
        o, l = ref.attention(pc.q[bb:bb + 1], kd[bb:bb + 1, :n], vd[bb:bb + 1, :n])
        assert np.array_equal(a[0][bb], o[0]) and np.array_equal(a[1][bb], l[0])


def _append_pins_hold(append):
    """Pins of a cache-append function: (1) gathering the appended cache gives the
    old prefix followed by the new tokens, (2) every other cache row is left as
    it was, (3) attention against the appended cache equals plain attention over
    the concatenated keys and values."""
    from exact_attention_forward_fa_amd import inputs
    final = [11, 5, 8]
    S = 3
    pc = inputs.paged_cache(3, 2, 4, 2, 8, torch.float16, seed=21, page_size=4, lengths=final, max_pages=4)
    lens = pc.cache_seqlens - S                      # tokens cached before the append
    g = torch.Generator().manual_seed(22)
    kn = torch.randn(3, S, 2, 8, generator=g).to(torch.float16)
    vn = torch.randn(3, S, 2, 8, generator=g).to(torch.float16)
    kd = inputs.dense_cache_from_pool(pc.k_pool, pc.block_table, pc.cache_seqlens)
    vd = inputs.dense_cache_from_pool(pc.v_pool, pc.block_table, pc.cache_seqlens)
    ok = True
    for paged in (True, False):
        kc, vc = (pc.k_pool, pc.v_pool) if paged else (kd, vd)
        bt, page = (pc.block_table, 4) if paged else (None, None)
        k2, v2 = append(kc, vc, kn, vn, lens, bt, page)
        touched = np.zeros(k2.shape[:2], dtype=bool)
        for b, n in enumerate(final):
            n0 = n - S
            if paged:
                got = ref.gather_pages(k2, pc.block_table[b], n, 4)
                for t in range(n0, n):
                    touched[int(pc.block_table[b, t // 4]), t % 4] = True
            else:
                got = k2[b, :n]
                touched[b, n0:n] = True
            want = np.concatenate([np.asarray(kc[b, :n0].float()) if not paged
                                   else ref.gather_pages(kc, pc.block_table[b], n0, 4),
                                   kn[b].double().numpy()])
            ok &= np.array_equal(got, want)
        ok &= np.array_equal(k2[~touched], np.asarray(kc.double())[~touched])
        ok &= np.array_equal(v2[~touched], np.asarray(vc.double())[~touched])
        o, l = ref.attention_kvcache(pc.q, k2, v2, pc.cache_seqlens, bt, page, causal=True)
        for b, n in enumerate(final):
            n0 = n - S
            kk = np.concatenate([np.asarray(kd[b, :n0].double()), kn[b].double().numpy()])[None]
            vv = np.concatenate([np.asarray(vd[b, :n0].double()), vn[b].double().numpy()])[None]
            oo, ll = ref.attention(pc.q[b:b + 1], kk, vv, causal=True)
            ok &= np.array_equal(o[b], oo[0]) and np.array_equal(l[b], ll[0])
    return ok


def test_kvcache_append_pins_and_planted_offsets():
    assert _append_pins_hold(ref.kvcache_append)
    # planted mistakes: new tokens one position late, or one early
    late = lambda kc, vc, kn, vn, lens, bt, page: ref.kvcache_append(kc, vc, kn, vn, lens + 1, bt, page)
    early = lambda kc, vc, kn, vn, lens, bt, page: ref.kvcache_append(kc, vc, kn, vn, lens - 1, bt, page)
    assert not _append_pins_hold(late)
    assert not _append_pins_hold(early)


def test_combine_of_key_chunks_equals_whole():
    rng = np.random.default_rng(14)
    B, S, H, D, Sk = 2, 3, 2, 5, 23
    q, k, v = _rand_case(rng, B, S, Sk, H, H, D)
    whole_o, whole_l = ref.attention(q, k, v, alibi_slopes=np.array([0.3, 0.1]), softcap=2.0)
    for bounds in ([0, 23], [0, 7, 14, 23], [0, 1, 2, 20, 23], [0, 0, 10, 10, 23]):
        n = len(bounds) - 1
        op = np.zeros((B, S, H, D, n))
        lp = np.zeros((B, S, H, n))
        for s in range(n):
            a, e = bounds[s], bounds[s + 1]
            if a == e:
                lp[..., s] = -np.inf
                continue
            # chunk keys sit at positions a..e-1; ALiBi distances stay those of the
            # full problem, so the chunk is the full problem with other keys masked
            mask_o, mask_l = _attention_on_key_range(q, k, v, a, e)
            op[..., s] = mask_o
            lp[..., s] = mask_l
        o, l = ref.combine(op, lp)
        assert np.max(np.abs(o - whole_o)) <= 1e-12
        assert np.max(np.abs(l - whole_l.transpose(0, 2, 1))) <= 1e-12


def _attention_on_key_range(q, k, v, a, e):
    # keys [a, e) only, with ALiBi distances measured in the full sequence:
    # Sq queries aligned to Sk keys; the chunk is evaluated as a non-causal problem
    # whose distance term is reproduced by shifting the query position.
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    out = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, Sq, H))
    slopes = np.array([0.3, 0.1])
    for b in range(B):
        for h in range(H):
            s = ref._head_scores(q[b, :, h], k[b, :, h], np.arange(Sq), Sq, Sk, 1 / math.sqrt(D), 2.0,
                                 slopes[h], False, (-1, -1))
            s[:, :a] = -np.inf
            s[:, e:] = -np.inf
            o, l = ref._softmax_rows(s, v[b, :, h])
            out[b, :, h] = o
            lse[b, :, h] = l
    return out, lse


def test_combine_of_key_slices_equals_whole():
    rng = np.random.default_rng(16)
    q, k, v = _rand_case(rng, 2, 4, 30, 2, 1, 8)
    whole_o, whole_l = ref.attention(q, k, v, softcap=3.0)
    bounds = [0, 4, 11, 29, 30]
    op = np.stack([ref.attention(q, k[:, a:e], v[:, a:e], softcap=3.0, softmax_scale=1 / math.sqrt(8))[0]
                   for a, e in zip(bounds[:-1], bounds[1:])], axis=-1)
    lp = np.stack([ref.attention(q, k[:, a:e], v[:, a:e], softcap=3.0)[1].transpose(0, 2, 1)
                   for a, e in zip(bounds[:-1], bounds[1:])], axis=-1)
    o, l = ref.combine(op, lp)
    assert np.max(np.abs(o - whole_o)) <= 1e-12
    assert np.max(np.abs(l - whole_l.transpose(0, 2, 1))) <= 1e-12


def test_combine_identity_and_empty():
    rng = np.random.default_rng(15)
    op = rng.standard_normal((1, 2, 3, 4, 1))
    lp = rng.standard_normal((1, 2, 3, 1))
    o, l = ref.combine(op, lp)
    assert np.array_equal(o, op[..., 0]) and np.array_equal(l, lp[..., 0])
    lp2 = np.full((1, 2, 3, 4), -np.inf)
    o, l = ref.combine(rng.standard_normal((1, 2, 3, 5, 4)), lp2)
    assert (o == 0).all() and (l == -np.inf).all()


def test_alibi_slope_recipes_match_golden():
    from exact_attention_forward_fa_amd import inputs
    with open(os.path.join(GOLDEN, "alibi_slopes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            H = int(parts[0].split("=")[1])
            want = [2.0 ** float(e) for e in parts[1:]]
            assert len(want) == H
            got = inputs.alibi_slopes(H).tolist()
            assert got == pytest.approx(want, rel=1e-6)
    # the closed form 2^(-8(i+1)/H) is the page's recipe for power-of-two H
    for H in (8, 32):
        assert inputs.alibi_slopes_closed_form(H).tolist() == pytest.approx(inputs.alibi_slopes(H).tolist(), rel=1e-6)


def test_flop_count_closed_forms():
    D = 64
    assert ref.flops(128, 128, D) == 4 * D * 128 * 128
    assert ref.flops(128, 128, D, causal=True) == 4 * D * 128 * 129 // 2
    assert ref.flops(1, 128, D, causal=True) == 4 * D * 128
    # window (w, 0) causal on S: row i sees min(i, w) + 1 keys
    S, w = 300, 37
    assert ref.flops(S, S, D, causal=True, window=(w, 0)) == 4 * D * sum(min(i, w) + 1 for i in range(S))


def _brute_agrees(opts, shape=(1, 5, 7, 4, 2, 3), seed=99):
    B, Sq, Sk, Hq, Hkv, D = shape
    rng = np.random.default_rng(seed)
    q, k, v = _rand_case(rng, B, Sq, Sk, Hq, Hkv, D)
    slopes = rng.uniform(0.05, 1.0, Hq) if opts.get("alibi") else None
    kw = dict(causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
              softcap=opts.get("softcap", 0.0))
    o, lse = ref.attention(q, k, v, alibi_slopes=slopes, **kw)
    ob, lseb = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                               slopes=None if slopes is None else slopes.tolist(), **kw)
    ob, lseb = np.array(ob), np.array(lseb)
    fin = np.isfinite(lseb)
    return (np.max(np.abs(o - ob)) <= 1e-12 and (np.isfinite(lse) == fin).all()
            and np.max(np.abs(lse[fin] - lseb[fin]), initial=0.0) <= 1e-12)


def test_pins_catch_planted_mistakes(monkeypatch):
    # Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.
    assert _brute_agrees(dict(causal=True, alibi=True, softcap=1.0))
    good_mask, good_scores, good_soft = ref.allowed_mask, ref._head_scores, ref._softmax_rows

    # 1. top-left causal alignment instead of bottom-right
    def top_left(rows, Sq, Sk, causal, window=(-1, -1)):
        return good_mask(rows, Sk, Sk, causal, window)
    monkeypatch.setattr(ref, "allowed_mask", top_left)
    c = [c for c in MASK_CASES if c["Sq"] != c["Sk"] and c["causal"]][0]
    assert ref.allowed_mask(np.arange(c["Sq"]), c["Sq"], c["Sk"], True).tolist() != c["rows"]
    assert not _brute_agrees(dict(causal=True))
    monkeypatch.setattr(ref, "allowed_mask", good_mask)

    # 2. ALiBi bias with the wrong sign
    def plus_bias(qb, kb, rows, Sq, Sk, scale, softcap, slope, causal, window):
        return good_scores(qb, kb, rows, Sq, Sk, scale, softcap, None if slope is None else -slope, causal, window)
    monkeypatch.setattr(ref, "_head_scores", plus_bias)
    assert not _brute_agrees(dict(alibi=True))
    # 3. softcap dropped
    def no_cap(qb, kb, rows, Sq, Sk, scale, softcap, slope, causal, window):
        return good_scores(qb, kb, rows, Sq, Sk, scale, 0.0, slope, causal, window)
    monkeypatch.setattr(ref, "_head_scores", no_cap)
    assert not _brute_agrees(dict(softcap=1.0))
    monkeypatch.setattr(ref, "_head_scores", good_scores)

    # 4. lse in base 2, 5. lse without the row max
    def lse_log2(s, vb):
        o, l = good_soft(s, vb)
        return o, l / math.log(2.0)
    monkeypatch.setattr(ref, "_softmax_rows", lse_log2)
    assert not _brute_agrees(dict())
    def lse_no_max(s, vb):
        o, l = good_soft(s, vb)
        return o, l - np.where(np.isfinite(s).any(axis=1), s.max(axis=1), 0.0)
    monkeypatch.setattr(ref, "_softmax_rows", lse_no_max)
    assert not _brute_agrees(dict())
    monkeypatch.setattr(ref, "_softmax_rows", good_soft)
    assert _brute_agrees(dict(causal=True, alibi=True, softcap=1.0))


def test_fp8_e4m3_decoding_matches_the_format_definition():
    """The oracle reads fp8 inputs through torch's float8_e4m3fn decoding; pin it to
    the OCP e4m3 definition: 1 sign, 4 exponent (bias 7) and 3 mantissa bits,
    subnormals at exponent 0, and S.1111.111 the only NaN (no infinities)."""
    codes = torch.arange(256, dtype=torch.uint8)
    got = ref._f64(codes.view(torch.float8_e4m3fn))
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(got[c]), c
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert got[c] == (-mag if s else mag), (c, got[c], mag)
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_oracle_pool_equals_oracle():
    """The parallel driver of the full-size parity tests returns what the oracle
    returns when called on the whole tensors, up to the rounding order of the
    library matmul on a row block (1e-12), including GQA, softcap, ALiBi and a
    window, over more rows than one block."""
    import oracle_pool
    from exact_attention_forward_fa_amd import inputs
    q, k, v = inputs.dense_qkv(2, 1100, 1030, 4, 2, 16, torch.float16, seed=77)
    slopes = inputs.alibi_slopes(4)
    kw = dict(causal=True, window=(300, 0), softcap=5.0, alibi_slopes=slopes, softmax_scale=0.3)
    po, pl = oracle_pool.dense_full(q, k, v, **kw)
    ro, rl = ref.attention(q, k, v, **kw)
    assert np.abs(po - ro).max() <= 1e-12
    assert (np.isneginf(pl) == np.isneginf(rl)).all()
    fin = np.isfinite(rl)
    assert np.abs(pl[fin] - rl[fin]).max() <= 1e-12
