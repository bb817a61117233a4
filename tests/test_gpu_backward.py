"""GPU parity of the backward (fa_bwd through the C ABI) against the oracle's
float64 gradients.

Tolerance.  The kernels take the fp16/bf16 inputs exactly, compute every
product in fp32, and round three things to the input dtype (unit roundoff u:
2^-11 for fp16, 2^-8 for bf16): P before dV += Pᵀ dO, dS before dK += dSᵀ Q and
dQ += dS K, and the three outputs.  Each rounding is a relative error of at most
u on one factor of a sum, so the error of a gradient element is at most
u·Σ|terms| plus u·|result|; the forward's out (rounded to the dtype) enters
through delta = dout·out with one more relative u.  The bar below is that
bound in a norm-wise form: per tensor, max |got - ref| <= 4u · max |ref| and
||got - ref||_F <= 2u · ||ref||_F.  A reference that is exactly zero (a single
key, where dP - delta cancels in exact arithmetic but not in fp32) is measured
against the largest reference gradient of the same call instead.
"""

import numpy as np
import pytest
import torch

import exact_attention_forward_fa_amd as fa
from exact_attention_forward_fa_amd import inputs
from oracle import ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def check_grads(got, want, dtype, what):
    u = U[dtype]
    floor = max(float(np.abs(w).max(initial=0.0)) for w in want)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        g = g.detach().cpu().double().numpy()
        assert g.shape == w.shape, (name, g.shape, w.shape)
        assert np.isfinite(g).all(), f"{what} {name}: non-finite values"
        if g.size == 0:
            continue
        scale = np.abs(w).max()
        err = np.abs(g - w).max()
        fro = np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300)
        print(f"  {what} {name}: max err {err:.3e} (max |ref| {scale:.3e}, ratio {err / max(scale, 1e-300):.2e}), "
              f"frobenius ratio {fro:.2e}", flush=True)
        if scale == 0:
            assert err <= 4 * u * floor, f"{what} {name}: want zeros, max |got| {err:.3e} > 4u·{floor:.3e}"
            continue
        assert err <= 4 * u * scale, f"{what} {name}: max err {err:.3e} > 4u·max|ref| = {4 * u * scale:.3e}"
        assert fro <= 2 * u, f"{what} {name}: frobenius ratio {fro:.3e} > 2u = {2 * u:.3e}"


def run(q, k, v, g, opts):
    """Forward then backward on the GPU; returns (dq, dk, dv) on the CPU."""
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    sl = opts.get("alibi_slopes")
    kw = dict(softmax_scale=opts.get("softmax_scale"), causal=opts.get("causal", False),
              window_size=opts.get("window", (-1, -1)), softcap=opts.get("softcap", 0.0),
              alibi_slopes=None if sl is None else sl.to(DEV))
    out, lse = fa.fwd(qd, kd, vd, **kw)
    dq, dk, dv = fa.bwd(gd, qd, kd, vd, out, lse, **kw)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def oracle(q, k, v, g, opts):
    return ref.attention_backward(q, k, v, g, softmax_scale=opts.get("softmax_scale"),
                                  causal=opts.get("causal", False), window=opts.get("window", (-1, -1)),
                                  softcap=opts.get("softcap", 0.0), alibi_slopes=opts.get("alibi_slopes"))


def make(B, Sq, Sk, Hq, Hkv, D, dt, seed, scale=1.0):
    q, k, v = inputs.dense_qkv(B, Sq, Sk, Hq, Hkv, D, dt, seed, scale=scale)
    gen = torch.Generator().manual_seed(seed + 7)
    g = inputs.randn(gen, (B, Sq, Hq, D), dt)
    return q, k, v, g


SLOPES = "slopes"
CASES = [
    # (B, Sq, Sk, Hq, Hkv, D, dtype, options)
    (2, 200, 200, 4, 4, 64, torch.float16, dict()),
    (1, 300, 300, 4, 2, 128, torch.bfloat16, dict(causal=True)),
    (2, 130, 257, 4, 1, 64, torch.float16, dict(causal=True)),                  # Sq < Sk, MQA
    (1, 257, 130, 2, 2, 128, torch.float16, dict(causal=True)),                 # rows with no allowed key
    (1, 333, 333, 2, 2, 64, torch.bfloat16, dict(causal=True, window=(32, 0))),
    (1, 200, 300, 4, 2, 64, torch.float16, dict(window=(20, 40))),
    (1, 256, 256, 4, 2, 128, torch.bfloat16, dict(causal=True, softcap=2.0)),
    (1, 190, 190, 4, 4, 64, torch.float16, dict(causal=True, alibi_slopes=SLOPES)),
    (1, 160, 224, 4, 2, 128, torch.bfloat16, dict(softcap=3.0, window=(50, 10), softmax_scale=0.2,
                                                  alibi_slopes=SLOPES)),
    (1, 1, 1, 2, 2, 64, torch.float16, dict()),
    (1, 1, 70, 2, 1, 128, torch.float16, dict(causal=True)),                   # one query row, decode-like
    (3, 65, 65, 2, 1, 64, torch.bfloat16, dict(causal=True, window=(0, 0))),   # each row sees one key
    (2, 200, 230, 4, 2, 32, torch.float16, dict(causal=True)),
    (1, 170, 170, 4, 4, 32, torch.bfloat16, dict(softcap=3.0, alibi_slopes=SLOPES)),
    (2, 150, 300, 4, 2, 96, torch.bfloat16, dict(causal=True)),
    (1, 257, 130, 2, 1, 96, torch.float16, dict(causal=True, window=(40, 0), softcap=4.0)),
    (1, 300, 300, 2, 1, 256, torch.bfloat16, dict(causal=True)),
    (2, 150, 270, 4, 2, 256, torch.float16, dict(window=(40, 20), softcap=3.0)),
    (1, 257, 130, 2, 2, 256, torch.float16, dict(causal=True, alibi_slopes=SLOPES)),   # rows with no allowed key
    (1, 1, 70, 2, 1, 256, torch.bfloat16, dict()),
]


def _ids(c):
    B, Sq, Sk, Hq, Hkv, D, dt, o = c
    opt = ",".join(k if v is True else f"{k}={v}" for k, v in o.items()) or "plain"
    return f"B{B}-{Sq}x{Sk}-h{Hq}/{Hkv}-d{D}-{str(dt)[6:]}-{opt}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_small(case):
    B, Sq, Sk, Hq, Hkv, D, dt, o = case
    print("case", _ids(case), flush=True)
    q, k, v, g = make(B, Sq, Sk, Hq, Hkv, D, dt, seed=4000 + Sq + 7 * Sk + D)
    opts = dict(o)
    if opts.get("alibi_slopes") == SLOPES:
        opts["alibi_slopes"] = inputs.alibi_slopes(Hq)
    got = run(q, k, v, g, opts)
    want = oracle(q, k, v, g, opts)
    check_grads(got, want, dt, _ids(case))


def test_backward_is_deterministic_and_matches_autograd_wrapper():
    print("case determinism", flush=True)
    q, k, v, g = make(2, 300, 300, 8, 2, 128, torch.bfloat16, seed=4100)
    opts = dict(causal=True, softcap=4.0)
    a = run(q, k, v, g, opts)
    b = run(q, k, v, g, opts)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    out = fa.attention(qd, kd, vd, causal=True, softcap=4.0)
    out.backward(g.to(DEV))
    torch.cuda.synchronize()
    for x, t in zip(a, (qd, kd, vd)):
        assert torch.equal(x, t.grad.cpu())


def test_backward_empty_sides():
    print("case empty sides", flush=True)
    # no keys: out = 0, lse = -inf (what the forward defines for such rows), dq = 0
    q, k, v, g = make(1, 5, 0, 2, 2, 64, torch.float16, seed=4200)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    out = torch.zeros_like(qd)
    lse = torch.full((1, 2, 5), float("-inf"), dtype=torch.float32, device=DEV)
    dq = torch.full_like(qd, float("nan"))
    fa.bwd(gd, qd, kd, vd, out, lse, dq=dq)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq) == 0
    # no queries: dk = dv = 0
    q, k, v, g = make(1, 0, 9, 2, 2, 128, torch.bfloat16, seed=4201)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    out = torch.empty_like(qd)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    fa.bwd(gd, qd, kd, vd, out, lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_backward_keys_no_query_sees_get_zero():
    # window (0, 0) with Sq < Sk: keys before the first aligned row get no gradient
    print("case unseen keys", flush=True)
    q, k, v, g = make(1, 40, 200, 2, 2, 64, torch.float16, seed=4300)
    opts = dict(causal=True, window=(3, 0))
    got = run(q, k, v, g, opts)
    want = oracle(q, k, v, g, opts)
    assert torch.count_nonzero(got[1][:, :150]) == 0 and torch.count_nonzero(got[2][:, :150]) == 0
    check_grads(got, want, torch.float16, "unseen keys")


# ---------------------------------------------------------------- packed sequences

VARLEN = [
    # (lengths_q, lengths_k, Hq, Hkv, D, dtype, options)
    ([130, 0, 257, 64], [130, 0, 257, 64], 4, 2, 64, torch.float16, dict(causal=True)),
    ([40, 300, 1], [200, 100, 77], 2, 2, 128, torch.bfloat16, dict(causal=True, softcap=3.0)),
    ([96, 33], [96, 0], 4, 1, 64, torch.bfloat16, dict(window=(16, 8), alibi_slopes=SLOPES)),
    ([70, 200], [70, 200], 2, 2, 32, torch.float16, dict(causal=True)),
    ([129, 64], [150, 64], 4, 2, 96, torch.bfloat16, dict(causal=True, softcap=2.0)),
    ([150, 0, 40], [150, 30, 170], 2, 1, 256, torch.float16, dict(causal=True, window=(60, 0))),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"q{c[0]}-k{c[1]}-d{c[4]}")
def test_backward_varlen_equals_per_sequence_dense(case):
    """Each packed sequence gets the float64 oracle's gradients within the bar,
    and exactly the bits fa_bwd gives that sequence on its own."""
    lq, lk, Hq, Hkv, D, dt, o = case
    print("case varlen", case[:6], flush=True)
    q, k, v, cq, ck = inputs.varlen_pack(lq, lk, Hq, Hkv, D, dt, seed=4500 + sum(lq))
    g = inputs.randn(torch.Generator().manual_seed(4501), q.shape, dt)
    opts = dict(o)
    if opts.get("alibi_slopes") == SLOPES:
        opts["alibi_slopes"] = inputs.alibi_slopes(Hq)
    sl = opts.get("alibi_slopes")
    kw = dict(softmax_scale=opts.get("softmax_scale"), causal=opts.get("causal", False),
              window_size=opts.get("window", (-1, -1)), softcap=opts.get("softcap", 0.0),
              alibi_slopes=None if sl is None else sl.to(DEV))
    qd, kd, vd, gd, cqd, ckd = (t.to(DEV) for t in (q, k, v, g, cq, ck))
    out, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lk), **kw)
    dq, dk, dv = fa.bwd_varlen(gd, qd, kd, vd, out, lse, cqd, ckd, max(lq), max(lk), **kw)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for b in range(len(lq)):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if q1 == q0 and k1 == k0:
            continue
        if k1 > k0 and q1 > q0:
            want = oracle(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], g[None, q0:q1], opts)
            check_grads((dq[None, q0:q1], dk[None, k0:k1], dv[None, k0:k1]), want, dt, f"varlen seq {b}")
            # the same sequence alone through the dense call
            sd = [t.to(DEV).contiguous() for t in (q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], g[None, q0:q1])]
            o1, l1 = fa.fwd(sd[0], sd[1], sd[2], **kw)
            a = fa.bwd(sd[3], sd[0], sd[1], sd[2], o1, l1, **kw)
            torch.cuda.synchronize()
            assert torch.equal(a[0].cpu()[0], dq[q0:q1]) and torch.equal(a[1].cpu()[0], dk[k0:k1]) \
                and torch.equal(a[2].cpu()[0], dv[k0:k1]), f"sequence {b} differs from its dense backward"
        else:
            # one side empty: the other side's gradients are zero
            assert torch.count_nonzero(dq[q0:q1]) == 0 and torch.count_nonzero(dk[k0:k1]) == 0 \
                and torch.count_nonzero(dv[k0:k1]) == 0


def test_backward_varlen_autograd_wrapper_matches_bwd_varlen():
    print("case varlen autograd", flush=True)
    lq = [70, 129, 1]
    q, k, v, cq, ck = inputs.varlen_pack(lq, lq, 4, 2, 128, torch.float16, seed=4600)
    g = inputs.randn(torch.Generator().manual_seed(4601), q.shape, q.dtype)
    qd, kd, vd, gd, cqd, ckd = (t.to(DEV) for t in (q, k, v, g, cq, ck))
    out, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, max(lq), max(lq), causal=True)
    want = fa.bwd_varlen(gd, qd, kd, vd, out, lse, cqd, ckd, max(lq), max(lq), causal=True)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (qd, kd, vd))
    o2 = fa.attention_varlen(qa, ka, va, cqd, ckd, max(lq), max(lq), causal=True)
    o2.backward(gd)
    torch.cuda.synchronize()
    assert torch.equal(o2.detach(), out)
    for a, t in zip(want, (qa, ka, va)):
        assert torch.equal(a, t.grad)


def test_backward_strided_views_equal_contiguous():
    """q, k, v as views into one packed [B, S, 3, H, D] tensor and dout as a
    transposed view: the strided call gives the bits of the contiguous call."""
    print("case strided views", flush=True)
    B, S, H, D = 2, 150, 4, 64
    gen = torch.Generator().manual_seed(4700)
    qkv = inputs.randn(gen, (B, S, 3, H, D), torch.bfloat16).to(DEV)
    gT = inputs.randn(gen, (B, H, S, D), torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    dout = gT.transpose(1, 2)                                  # [B, S, H, D], strides (H*S*D, D, S*D, 1)
    assert not q.is_contiguous() and not dout.is_contiguous()
    out, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(dout, q, k, v, out, lse, causal=True)
    qc, kc, vc, dc = (t.contiguous() for t in (q, k, v, dout))
    out2, lse2 = fa.fwd(qc, kc, vc, causal=True)
    b = fa.bwd(dc, qc, kc, vc, out2, lse2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_huge_sequence_stride_equals_contiguous():
    """q, k, v and dout with a sequence stride of 2^23 + 256 elements: a 128-row
    tile then spans more than 2 GiB, so the forward and both backward kernels
    take their row-by-row address path on every tile instead of the 32-bit
    per-lane offsets; the bits equal those of contiguous copies."""
    print("case huge sequence stride", flush=True)
    B, S, H, D = 1, 130, 2, 64
    ss = (1 << 23) + 256
    gen = torch.Generator().manual_seed(4750)
    small = [inputs.randn(gen, (B, S, H, D), torch.float16) for _ in range(4)]
    views = []
    for t in small:
        store = torch.zeros(B * S * ss, dtype=torch.float16, device=DEV)
        v = store.as_strided((B, S, H, D), (S * ss, ss, D, 1))
        v.copy_(t.to(DEV))
        views.append(v)
    q, k, v, dout = views
    assert q.stride(1) == ss
    out, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(dout, q, k, v, out, lse, causal=True)
    qc, kc, vc, dc = (t.to(DEV) for t in small)
    out2, lse2 = fa.fwd(qc, kc, vc, causal=True)
    b = fa.bwd(dc, qc, kc, vc, out2, lse2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- full sizes, sampled heads

@pytest.mark.parametrize("name,heads", [("c3_causal", [(1, 7), (3, 30)]), ("c4_gqa", [(1, 5)])])
def test_backward_full_size_sampled_heads(name, heads):
    """The workloads the prefill benchmarks time, with a seeded dout; the oracle
    computes the gradients of a few (batch, kv head) groups in full."""
    print("case", name, flush=True)
    c = inputs.case(name)
    q, k, v = c["q"], c["k"], c["v"]
    dt = q.dtype
    gen = torch.Generator().manual_seed(4400)
    g = inputs.randn(gen, q.shape, dt)
    opts = dict(softmax_scale=c.get("softmax_scale"), causal=c.get("causal", False),
                window=c.get("window", (-1, -1)), softcap=c.get("softcap", 0.0),
                alibi_slopes=c.get("alibi_slopes"))
    dq, dk, dv = run(q, k, v, g, opts)
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    for b, hk in heads:
        hs = slice(hk * G, (hk + 1) * G)
        sub = dict(opts)
        if sub["alibi_slopes"] is not None:
            sub["alibi_slopes"] = sub["alibi_slopes"][hs]
        want = oracle(q[b:b + 1, :, hs], k[b:b + 1, :, hk:hk + 1], v[b:b + 1, :, hk:hk + 1],
                      g[b:b + 1, :, hs], sub)
        got = (dq[b:b + 1, :, hs], dk[b:b + 1, :, hk:hk + 1], dv[b:b + 1, :, hk:hk + 1])
        check_grads(got, want, dt, f"{name} b{b} hk{hk}")


def test_backward_huge_window_equals_unbounded():
    print("case backward huge window", flush=True)
    big = 2 ** 31 - 1
    q, k, v, g = make(1, 200, 260, 4, 2, 128, torch.bfloat16, seed=4950)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    out, lse = fa.fwd(qd, kd, vd, causal=True)
    a = fa.bwd(gd, qd, kd, vd, out, lse, causal=True, window_size=(big, big))
    b = fa.bwd(gd, qd, kd, vd, out, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
