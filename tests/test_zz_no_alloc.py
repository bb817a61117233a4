"""The KV-cache entry point that allocates nothing (fa_fwd_kvcache_noalloc: the
decode workspace is the library's static device array) against fa_fwd_kvcache
with a caller-given workspace.  Two calls in a row, the second on a smaller
input, so the second runs on the array the first one left behind; each output
must equal the workspace call bit for bit and meet the oracle bars."""

import pytest
import torch

import exact_attention_forward_fa_amd as fa
from exact_attention_forward_fa_amd import inputs
from oracle import ref

from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(q, kp, vp, lens, bt, ns, page, dt, **kw):
    B, Sq, Hq, D = q.shape
    g = [t.to(DEV) for t in (q, kp, vp, lens, bt)]
    out = torch.full_like(g[0], float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_kvcache_noalloc(g[0], g[1], g[2], g[3], out, lse, block_table=g[4], num_splits=ns, **kw)
    want = fa.fwd_kvcache(g[0], g[1], g[2], g[3], block_table=g[4], num_splits=ns, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, want[0]) and torch.equal(lse, want[1])
    ro, rl = ref.attention_kvcache(q, kp, vp, lens, bt, page, causal=kw.get("causal", False),
                                   window=kw.get("window_size", (-1, -1)), softcap=kw.get("softcap", 0.0))
    check(out.cpu(), lse.cpu(), ro, rl, dt, f"noalloc B{B} Sq{Sq} Hq{Hq} D{D} splits {ns}")


def test_noalloc_equals_workspace_call_twice_second_smaller():
    print("case noalloc config 5 then a smaller decode", flush=True)
    c = inputs.case("c5_paged")            # 64 x 32 rows x 16 splits: about 17 MB of partials
    need = fa.kvcache_workspace_size(64, 1, 32, 128, 16)
    assert need <= fa.kvcache_noalloc_max_bytes()
    _both(c["q"], c["k_pool"], c["v_pool"], c["cache_seqlens"], c["block_table"], 16, 256, torch.bfloat16)
    pc = inputs.paged_cache(3, 2, 8, 2, 64, torch.float16, seed=4321, page_size=16, lengths=[50, 7, 300],
                            tail_fill="nan")
    _both(pc.q, pc.k_pool, pc.v_pool, pc.cache_seqlens, pc.block_table, 3, 16, torch.float16, causal=True,
          softcap=6.0)
