"""hs_decode_select_attn_static (no workspace: a fixed per-GPU scratch array
inside the library) against hs_decode_select_attn with a workspace, through
the C ABI: two calls in a row, the second on a smaller input, both bit for
bit equal to the entry point with a workspace (the same kernels run)."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from parity import dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _token_case(B, C, kb, R, lens, seed_layer=0):
    """fp8 token-mode decode inputs, the full layer and the selection (existing
    entry points); returns what one sparse layer call needs."""
    cfg = gen.config(5, B=B, T=C, Hq=8, Hkv=2, d=128, kb=kb, n_recent=R, N=seed_layer + 1,
                     L_lo=1, L_hi=C)
    inp = gen.make_decode(cfg)
    inp.lens = np.asarray(lens, np.int32)
    kc = np.empty((B, cfg.Hkv, C, cfg.d), np.uint8)
    vc = np.empty((B, cfg.Hkv, C, cfg.d), np.uint8)
    gen.fill_decode_cache(inp, kc, vc, v_block_major=False)
    k, v = dev(kc), dev(vc)
    scale = dev(inp.kv_scale)
    lens_d = torch.from_numpy(inp.lens).cuda()
    q = dev(inp.q)
    o = torch.empty((B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, cfg.Hq), device="cuda")
    raw = torch.empty((B, cfg.Hq, C), device="cuda")
    hb.decode_full_attn_scores(q, k, v, lens_d, o, lse, raw, block=1, kv_scale=scale)
    idx = torch.empty((B, cfg.Hkv, kb + R), dtype=torch.int32, device="cuda")
    hb.decode_block_topk(q, k, lens_d, raw, lse, kb, idx, block=1, n_recent=R, kv_scale=scale)
    return dict(q=dev(inp.layers[seed_layer]["q"]), k=k, v=v, lens=lens_d, idx=idx, n=kb + R, scale=scale,
                shape=(B, cfg.Hq, cfg.d))


def _both(c):
    o_ws = torch.full(c["shape"], float("nan"), dtype=torch.bfloat16, device="cuda")
    o_st = torch.full(c["shape"], float("nan"), dtype=torch.bfloat16, device="cuda")
    hb.decode_select_attn(c["q"], c["k"], c["v"], c["lens"], c["idx"], c["n"], None, None, 0, None, o_ws,
                          block=1, kv_scale=c["scale"])
    hb.decode_select_attn_static(c["q"], c["k"], c["v"], c["lens"], c["idx"], c["n"], None, None, 0, None,
                                 o_st, block=1, kv_scale=c["scale"])
    torch.cuda.synchronize()
    return host(o_ws), host(o_st)


def test_static_scratch_matches_workspace_two_calls():
    # first call: 25 tiles of 64 tokens per row -> 4 work groups per (sequence, kv head)
    say("[static scratch] call 1: B=4 C=16384 top-1500 + 100 recent")
    big = _token_case(4, 16384, 1500, 100, [3, 900, 7777, 16384])
    a, b = _both(big)
    say(f"  max|d|={np.abs(a - b).max():.3g}")
    assert not np.isnan(b).any() and np.array_equal(a, b)
    # second call, smaller: 17 tiles -> 3 work groups per (sequence, kv head);
    # the scratch still holds the first call's partials
    say("[static scratch] call 2: B=3 C=8192 top-1000 + 64 recent")
    small = _token_case(3, 8192, 1000, 64, [70, 5000, 8192], seed_layer=1)
    a, b = _both(small)
    say(f"  max|d|={np.abs(a - b).max():.3g}")
    assert not np.isnan(b).any() and np.array_equal(a, b)


def test_static_scratch_block_mode():
    """Block mode needs no scratch: the static entry point runs the same kernel."""
    say("[static scratch] block mode")
    cfg = gen.config(4, B=3, T=2048, Hq=8, Hkv=2, d=128, kb=5, W=100, N=1, L_lo=1, L_hi=2048)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([64, 1000, 2048], np.int32)
    kc = np.empty((cfg.B, cfg.Hkv, cfg.T, cfg.d), np.uint16)
    vc = np.empty((cfg.B, cfg.Hkv, cfg.T // 64, cfg.d, 64), np.uint16)
    gen.fill_decode_cache(inp, kc, vc)
    k, v = dev(kc), dev(vc)
    lens = torch.from_numpy(inp.lens).cuda()
    q = dev(inp.q)
    o = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.B, cfg.Hq), device="cuda")
    raw = torch.empty((cfg.B, cfg.Hq, cfg.T // 64), device="cuda")
    hb.decode_full_attn_scores(q, k, v, lens, o, lse, raw)
    idx = torch.empty((cfg.B, cfg.Hkv, cfg.kb), dtype=torch.int32, device="cuda")
    hb.decode_block_topk(q, k, lens, raw, lse, cfg.kb, idx)
    lay = inp.layers[0]
    args = (dev(lay["q"]), k, v, lens, idx, cfg.kb, dev(lay["k_ring"]), dev(gen.block_major(lay["v_ring"])),
            cfg.W, dev(lay["gates"]))
    o1 = torch.full_like(o, float("nan"))
    o2 = torch.full_like(o, float("nan"))
    hb.decode_select_attn(*args, o1)
    hb.decode_select_attn_static(*args, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and not torch.isnan(o2).any()


def test_static_scratch_largest_split():
    """The split is capped at one work group per compute unit, so on a 256-CU
    device the largest partial state (16 heads per group, head_dim 128, 256
    groups: 2.1 MB) fits the 8 MiB static scratch.  Such a case runs through
    the static entry point and equals the workspace entry point."""
    B, Hq, Hkv, C, d, n = 16, 64, 4, 8192, 128, 4096
    say(f"[static scratch] largest split: B={B} Hq={Hq} Hkv={Hkv} C={C} n={n}")
    g = torch.Generator(device="cuda").manual_seed(7)
    k = torch.randint(0, 120, (B, Hkv, C, d), dtype=torch.uint8, device="cuda", generator=g)
    v = torch.randint(0, 120, (B, Hkv, C, d), dtype=torch.uint8, device="cuda", generator=g)
    idx = torch.stack([torch.randperm(C, device="cuda", generator=g)[:n].sort().values
                       for _ in range(B * Hkv)]).view(B, Hkv, n).to(torch.int32).contiguous()
    c = dict(q=torch.randn((B, Hq, d), device="cuda", generator=g).to(torch.bfloat16), k=k, v=v,
             lens=torch.full((B,), C, dtype=torch.int32, device="cuda"), idx=idx, n=n,
             scale=torch.full((2, Hkv), 0.03, device="cuda"), shape=(B, Hq, d))
    a, b = _both(c)
    say(f"  max|d|={np.abs(a - b).max():.3g}")
    assert not np.isnan(b).any() and np.array_equal(a, b)
