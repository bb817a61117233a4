"""Benchmark of the exact attention forward on one MI355X.

One step = one pass of the whole hot path on resident inputs:
  * prefill: causal attention, B=4, Sq=Sk=4096, Hq=Hkv=32, D=64, fp16
    (one fa_fwd launch of the MFMA prefill kernel);
  * decode: paged split-KV decode, B=64, Sq=1, Hq=32, Hkv=8, D=128, bf16,
    per-sequence cache length uniform in [1024, 16384], 256-token pages with a
    permuted block table, 16 splits + the LSE combine (one fa_fwd_kvcache call).

Prints ONE JSON line.  value = prefill TFLOP/s over algorithmic FLOPs
(4·D per allowed (query, key) pair, masked area excluded) divided by the
prefill kernel's mean duration from HIP events on the launch stream; the
decode figure (GB/s of algorithmic K/V/q/out/block-table bytes over the
decode + combine time) rides along in "decode".  "decode_append" times the
same decode call with a one-token KV append per sequence (fwd_kvcache with
k=, v=), "prefill_fp8" the prefill on the same inputs converted to fp8
e4m3, and "backward" the gradients of that prefill (fa_bwd with a seeded
dout, TFLOP/s at 10·D per allowed pair: the five products S, dP, dV, dK, dQ),
all after the timed steps.  "cpu_baseline" times the float64 CPU oracle
on a bounded sample of the prefill workload.  "prefill_configs" times the
other prefill workloads of the configurations (B1 S128 H2; B2 S1024 H8 causal,
non-causal and packed; config 3's two windows; the B2 S8192 GQA bf16 case with
softcap and ALiBi), each as TFLOP/s over its own allowed pairs and its fraction
of the dense fp16/bf16 MFMA peak, from a HIP graph of back-to-back calls (the
small configurations' kernels take less time than a Python call); the best of
three replays.  By default 10 untimed warm-up steps precede 100 timed ones,
and every leg reports the mean (and the main legs the median and minimum).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def causal_pairs(Sq: int, Sk: int) -> int:
    """Allowed (query, key) pairs of one head under bottom-right causal masking."""
    shift = Sk - Sq
    # row i sees keys 0..min(Sk-1, i+shift): count = clamp(i + shift + 1, 0, Sk)
    total = 0
    lo = max(0, -shift)                      # first row with at least one key
    full_from = max(lo, Sk - 1 - shift)      # rows from here on see all Sk keys
    if full_from > lo:
        a, b = lo + shift + 1, full_from - 1 + shift + 1
        total += (a + b) * (full_from - lo) // 2
    total += max(0, Sq - full_from) * Sk
    return total


def allowed_pairs(Sq: int, Sk: int, causal: bool = False, window=(-1, -1)) -> int:
    """Allowed (query, key) pairs of one head: bottom-right aligned causal mask and
    inclusive window [i' - left, i' + right], i' = i + Sk - Sq (-1 = unbounded)."""
    import numpy as np
    ip = np.arange(Sq, dtype=np.int64) + (Sk - Sq)
    lo = np.zeros(Sq, dtype=np.int64)
    hi = np.full(Sq, Sk - 1, dtype=np.int64)
    if window[0] >= 0:
        lo = np.maximum(lo, ip - window[0])
    if causal:
        hi = np.minimum(hi, ip)
    if window[1] >= 0:
        hi = np.minimum(hi, ip + window[1])
    return int(np.maximum(hi - lo + 1, 0).sum())


def kernel_source_hash(which: str = "prefill") -> str:
    """Short hash of the sources a kernel is built from; stored traffic figures
    are used only while it matches."""
    files = {"prefill": ("prefill.hip", "fa_device.hpp", "fa_kernels.hpp"),
             "decode": ("decode.hip", "combine.hip", "fa_device.hpp", "fa_kernels.hpp"),
             "backward": ("backward.hip", "fa_device.hpp", "fa_kernels.hpp")}[which]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_attention_forward_fa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- CPU oracle leg

def _oracle_head(args):
    q, k, v = args
    from oracle import ref
    t = time.perf_counter()
    ref.attention(q[None, :, None], k[None, :, None], v[None, :, None], causal=True)
    return time.perf_counter() - t


def cpu_baseline(case, n_heads: int, workers: int, affinity: int):
    """Time the float64 oracle on n_heads (batch, head) pairs of the prefill workload."""
    import numpy as np
    q, k, v = case["q"], case["k"], case["v"]
    B, S, H, D = q.shape
    pairs = [(i // H, i % H) for i in range(min(n_heads, B * H))]
    jobs = [(q[b, :, h].float().numpy().astype(np.float64), k[b, :, h].float().numpy().astype(np.float64),
             v[b, :, h].float().numpy().astype(np.float64)) for b, h in pairs]
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_head, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    flops = 4 * D * causal_pairs(S, S) * len(pairs)
    return dict(value=flops / wall / 1e12, unit="TFLOP/s", cores=workers, kind="oracle",
                sample=f"float64 oracle, causal, {len(pairs)} of {B * H} (batch, head) pairs of the "
                       f"B{B} S{S} H{H} D{D} prefill, all {S} rows each, {workers} single-threaded "
                       f"worker processes on {workers} of the {affinity} cores in this process's CPU "
                       f"affinity (at most 16, the host share of one GPU), {wall:.1f} s wall; FLOPs "
                       f"counted as 4·D per allowed pair; CPU {cpu_model()}, numpy {np.__version__}",
                seconds=wall)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


# ---------------------------------------------------------------- GPU legs

def decode_bytes(c) -> int:
    lens = c["cache_seqlens"].long()
    Hkv, D = c["k_pool"].shape[2], c["k_pool"].shape[3]
    es = c["k_pool"].element_size()
    kv = int(lens.sum()) * Hkv * D * 2 * es
    page = c["page_size"]
    bt = int(((lens + page - 1) // page).sum()) * 4
    q = c["q"].numel() * c["q"].element_size()
    return kv + 2 * q + bt + 4 * lens.numel()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)    # timed steps (10 warm-up + 100 timed by default)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other configurations' prefill legs")
    ap.add_argument("--cpu-heads", type=int, default=128)
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run one leg only (for profiling); the JSON line is still printed")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_forward_fa_amd as fa
    from exact_attention_forward_fa_amd import inputs

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    # inputs (CPU, seeded), then resident on the GPU
    run_p = args.only in (None, "prefill")
    run_d = args.only in (None, "decode")
    t = time.perf_counter()
    pc = inputs.case("c3_causal")
    dc = inputs.case("c5_paged") if run_d else None
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")

    cpu = None
    if not args.no_cpu_baseline:
        affinity = len(os.sched_getaffinity(0))
        workers = max(1, min(16, affinity))      # the host share of one GPU is 16 cores
        cpu = cpu_baseline(pc, args.cpu_heads, workers, affinity)
        log(f"cpu baseline: {cpu['value']:.4f} TFLOP/s in {cpu['seconds']:.1f} s on {workers} cores")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (pc[n].to(dev) for n in ("q", "k", "v"))
    B, S, H, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if run_d:
        dq = dc["q"].to(dev)
        kp, vp = dc["k_pool"].to(dev), dc["v_pool"].to(dev)
        bt, lens = dc["block_table"].to(dev), dc["cache_seqlens"].to(dev)
        ns = dc["num_splits"]
        dB, _, dH, dD = dc["q"].shape
        ws = torch.empty(fa.kvcache_workspace_size(dB, 1, dH, dD, ns), dtype=torch.uint8, device=dev)
        dout = torch.empty_like(dq)
        dlse = torch.empty((dB, dH, 1), dtype=torch.float32, device=dev)

    def step(ev=None):
        if run_p:
            if ev: ev[0].record()
            fa.fwd(q, k, v, causal=True, out=out, lse=lse)
            if ev: ev[1].record()
        if run_d:
            if ev: ev[2].record()
            fa.fwd_kvcache(dq, kp, vp, lens, block_table=bt, num_splits=ns, workspace=ws, out=dout, lse=dlse)
            if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = [e[0].elapsed_time(e[1]) for e in evs] if run_p else [float("nan")]
    d_ms = [e[2].elapsed_time(e[3]) for e in evs] if run_d else [float("nan")]
    p_mean = sum(p_ms) / len(p_ms)
    d_mean = sum(d_ms) / len(d_ms)
    p_flops = 4 * D * causal_pairs(S, S) * B * H
    tflops = p_flops / (p_mean * 1e-3) / 1e12
    d_bytes = decode_bytes(dc) if run_d else 0
    gbs = d_bytes / (d_mean * 1e-3) / 1e9

    # the same prefill with q, k, v converted to fp8 e4m3 (descales 1)
    f8_mean = None
    if run_p:
        q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
        out8 = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup):
            fa.fwd(q8, k8, v8, causal=True, out=out8, lse=lse)
        torch.cuda.synchronize()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            fev[i][0].record()
            fa.fwd(q8, k8, v8, causal=True, out=out8, lse=lse)
            fev[i][1].record()
        torch.cuda.synchronize()
        f8_ms = [e[0].elapsed_time(e[1]) for e in fev]
        f8_mean = sum(f8_ms) / len(f8_ms)
        del q8, k8, v8, out8

    # backward of the timed prefill (out and lse recomputed: the fp8 leg wrote lse), seeded dout
    b_mean = None
    if run_p:
        fa.fwd(q, k, v, causal=True, out=out, lse=lse)
        gout = inputs.randn(torch.Generator().manual_seed(4400), q.shape, q.dtype).to(dev)
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(fa.bwd_workspace_size(B, S, H), dtype=torch.uint8, device=dev)

        def bwd_step():
            fa.bwd(gout, q, k, v, out, lse, causal=True, dq=gq, dk=gk, dv=gv, workspace=bws)
        for _ in range(args.warmup):
            bwd_step()
        torch.cuda.synchronize()
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            bev[i][0].record()
            bwd_step()
            bev[i][1].record()
        torch.cuda.synchronize()
        b_ms = [e[0].elapsed_time(e[1]) for e in bev]
        b_mean = sum(b_ms) / len(b_ms)
        del gout, gq, gk, gv, bws
    b_flops = 10 * D * causal_pairs(S, S) * B * H

    # decode with a one-token KV append (fwd_kvcache with k=, v=): every
    # sequence's last cached token is written again from k_new/v_new (its own
    # values, so the cache is unchanged) and then attended with the rest
    a_mean = a_bytes = None
    if run_d:
        page = dc["page_size"]
        last = dc["cache_seqlens"].long() - 1
        pages = dc["block_table"][torch.arange(dB), last // page].long()
        kn = dc["k_pool"][pages, last % page].unsqueeze(1).contiguous().to(dev)
        vn = dc["v_pool"][pages, last % page].unsqueeze(1).contiguous().to(dev)
        lens_before = lens - 1

        def append_step():
            fa.fwd_kvcache(dq, kp, vp, lens_before, block_table=bt, num_splits=ns, workspace=ws, out=dout,
                           lse=dlse, k=kn, v=vn)
        for _ in range(args.warmup):
            append_step()
        torch.cuda.synchronize()
        aev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            aev[i][0].record()
            append_step()
            aev[i][1].record()
        torch.cuda.synchronize()
        a_ms = [e[0].elapsed_time(e[1]) for e in aev]
        a_mean = sum(a_ms) / len(a_ms)
        a_bytes = d_bytes + 2 * 2 * kn.numel() * kn.element_size()   # new K/V read + cache rows written

    # the other prefill workloads of the pages' configurations, timed the same way
    legs = {}
    if run_p and not args.no_extra:
        def time_call(fn):
            """Mean GPU time per call: args.steps calls are captured back to back in
            one HIP graph, which is replayed between two events, so host launch
            costs (tens of microseconds per Python call, more than the small
            configurations' kernels take) stay out of the figure.  Falls back to
            direct calls if capture fails."""
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            n = args.steps
            run = None
            try:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(n):
                        fn()
                torch.cuda.synchronize()
                run = g.replay
            except Exception as e:            # pragma: no cover - depends on the runtime
                log(f"graph capture failed ({e}); timing direct calls")

                def run():
                    for _ in range(n):
                        fn()
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / n
                best = t if best is None else min(best, t)
            return best

        for name in ("c1_noncausal", "c1_causal", "c1_decode", "c2_causal", "c2_noncausal", "c2_varlen",
                     "c3_win256_0", "c3_win256_256", "c4_gqa"):
            c = pc if name.startswith("c3") else inputs.case(name)
            win = {"c3_win256_0": (256, 0), "c3_win256_256": (256, 256)}.get(name, c.get("window", (-1, -1)))
            causal = {"c3_win256_0": True, "c3_win256_256": False}.get(name, c.get("causal", False))
            xq, xk, xv = (c[n].to(dev) for n in ("q", "k", "v"))
            slopes = c.get("alibi_slopes")
            slopes = None if slopes is None else slopes.to(dev)
            kw = dict(softmax_scale=c.get("softmax_scale"), causal=causal, window_size=win,
                      softcap=c.get("softcap", 0.0), alibi_slopes=slopes)
            if c["kind"] == "varlen":
                cq, ck = c["cu_seqlens_q"].to(dev), c["cu_seqlens_k"].to(dev)
                lens = (c["cu_seqlens_q"][1:] - c["cu_seqlens_q"][:-1]).tolist()
                fl = 4 * xq.shape[-1] * xq.shape[1] * sum(allowed_pairs(n, n, causal, win) for n in lens)
                ms = time_call(lambda: fa.fwd_varlen(xq, xk, xv, cq, ck, c["max_seqlen_q"], c["max_seqlen_k"], **kw))
                shape = f"varlen lengths {lens} H{xq.shape[1]} D{xq.shape[2]}"
            else:
                Bq, Sq, Hq, Dq = xq.shape
                fl = 4 * Dq * Hq * Bq * allowed_pairs(Sq, xk.shape[1], causal, win)
                ms = time_call(lambda: fa.fwd(xq, xk, xv, **kw))
                shape = f"B{Bq} Sq{Sq} Sk{xk.shape[1]} Hq{Hq} Hkv{xk.shape[2]} D{Dq}"
            tf = fl / (ms * 1e-3) / 1e12
            legs[name] = {"tflops": round(tf, 2), "frac": round(tf / PEAK_MFMA_F16_TFLOPS, 4), "ms_mean": round(ms, 5),
                          "flops": fl, "dtype": str(xq.dtype).replace("torch.", ""),
                          "shape": shape + (f", causal={causal}, window={win}" +
                                            (f", softcap={kw['softcap']}" if kw["softcap"] else "") +
                                            (", ALiBi" if slopes is not None else ""))}
            log(f"{name}: {tf:.1f} TFLOP/s ({ms * 1e3:.1f} us)")
            del xq, xk, xv

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read + {n} bytes written")

    # HBM bytes per launch from the committed counter runs (FETCH_SIZE + WRITE_SIZE,
    # scaled by a device copy), only while the kernel sources are unchanged
    traffic = d_traffic = b_traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("prefill_source_sha") == kernel_source_hash("prefill"):
            traffic = tr["prefill_bytes_per_launch"]
        if tr.get("decode_source_sha") == kernel_source_hash("decode"):
            d_traffic = tr["decode_bytes_per_call"]
        if tr.get("backward_source_sha") == kernel_source_hash("backward"):
            b_traffic = tr.get("backward_bytes_per_call")
    except (OSError, ValueError, KeyError):
        traffic = d_traffic = b_traffic = None

    line = {
        "metric": "attn fwd TFLOP/s (causal, B4 S4096 H32 D64 fp16) + paged decode HBM GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill B=4 Sq=Sk=4096 Hq=Hkv=32 D=64 fp16 (N(0,1), seed 1003) + paged "
                        "split-KV decode B=64 Sq=1 Hq=32 Hkv=8 D=128 bf16, len~U[1024,16384], 256-token "
                        "pages, permuted block table, 16 splits + LSE combine (seed 1005)",
            "global_batch": B, "seq_len": S, "parallelism": "single GPU",
        },
        "prefill": {"ms_mean": round(p_mean, 5), "ms_median": round(median(p_ms), 5), "ms_min": round(min(p_ms), 5),
                    "flops": p_flops, "tflops": round(tflops, 2),
                    "exps": B * H * causal_pairs(S, S),
                    "exps_per_s": round(B * H * causal_pairs(S, S) / (p_mean * 1e-3), 1)},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", "ms_mean": round(d_mean, 5),
                   "ms_median": round(median(d_ms), 5), "ms_min": round(min(d_ms), 5), "bytes": d_bytes,
                   "dtype": "bf16",
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": d_traffic}},
        "prefill_fp8": None if f8_mean is None else {
            "value": round(p_flops / (f8_mean * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_mean": round(f8_mean, 5),
            "dtype": "fp8 e4m3 in (Q K^T on fp8 MFMA), bf16 P V and out"},
        "backward": None if b_mean is None else {
            "value": round(b_flops / (b_mean * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_mean": round(b_mean, 5),
            "flops": b_flops, "dtype": "fp16",
            "roofline": {"bound": "mfma", "achieved": round(b_flops / (b_mean * 1e-3) / 1e12, 2),
                         "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(b_flops / (b_mean * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
                         "traffic": b_traffic}},
        "decode_append": None if a_mean is None else {
            "value": round(a_bytes / (a_mean * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_mean": round(a_mean, 5),
            "bytes": a_bytes, "new_tokens_per_sequence": 1,
            "extra_us_over_decode": round((a_mean - d_mean) * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None if cpu is None else {kk: cpu[kk] for kk in ("value", "unit", "cores", "kind", "sample")},
        "prefill_configs": legs or None,
    }
    if cpu is not None:
        line["cpu_baseline"]["value"] = round(cpu["value"], 6)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
