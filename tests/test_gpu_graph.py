"""HIP graph capture of whole hybrid blocks through the C ABI: the library
allocates nothing and records no memory-set nodes, so a prefill block and a
decode step (block mode with window, gates and sinks; token mode with split
work groups, selected in two calls or in the fused call) can be captured once
and replayed.  Every replay must reproduce
the eager results bit for bit, with eager work and synchronisations between
replays and the outputs poisoned before each one."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from parity import dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _replay_matches(step, outs, n=3):
    """Run `step` eagerly, capture it, and check n replays against the eager
    outputs (each replay after poisoning the outputs and some eager work)."""
    step()
    torch.cuda.synchronize()
    want = [x.clone() for x in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(n):
        for x in outs:
            x.fill_(float("nan") if x.is_floating_point() else -3)
        junk.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, w) in enumerate(zip(outs, want)):
            same = torch.equal(torch.nan_to_num(x.float(), 7.0), torch.nan_to_num(w.float(), 7.0))
            assert same, f"replay {r}: output {i} differs from the eager run"
    say(f"  {n} replays bit-identical to the eager run ({len(outs)} outputs)")


def test_prefill_block_graph():
    say("[graph] prefill block T=700 Hq=8 Hkv=2 d=128 bf16, 2 sparse layers with sinks")
    cfg = gen.config(1, T=700, Hq=8, Hkv=2, d=128, dtype="bf16", kb=4, W=100, N=2)
    inp = gen.make_prefill(cfg)
    B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d
    q, k, vb = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(gen.block_major(inp.v), "bf16")
    o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    raw = torch.zeros((B, Hq, T, cfg.nblk), device="cuda")
    idx = torch.empty((B, Hkv, T, cfg.kb), dtype=torch.int32, device="cuda")
    layers = [dict(q=dev(l["q"], "bf16"), k=dev(l["k"], "bf16"), v=dev(gen.block_major(l["v"]), "bf16"),
                   g=dev(l["gates"]), s=dev(gen.make_sinks(cfg, i)),
                   o=torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda"))
              for i, l in enumerate(inp.layers)]

    def step():
        hb.full_attn_fwd_scores(q, k, vb, o, lse, raw)
        hb.block_topk((B, T, Hq, Hkv, d, hb.HS_BF16), raw, lse, cfg.kb, idx)
        for l in layers:
            hb.sparse_attn_fwd(l["q"], k, vb, idx, cfg.kb, l["k"], l["v"], cfg.W, l["g"], l["o"],
                               sinks=l["s"])

    # raw entries above the causal diagonal are never written: keep them out
    _replay_matches(step, [o, lse, idx] + [l["o"] for l in layers])


@pytest.mark.parametrize("mode", ["block", "token", "token_fused"])
def test_decode_step_graph(mode):
    say(f"[graph] decode step, {mode}")
    token = mode != "block"
    if token:
        cfg = gen.config(5, B=3, T=8192, Hq=8, Hkv=2, d=128, kb=600, n_recent=32, N=2,
                         L_lo=100, L_hi=8192)
    else:
        cfg = gen.config(4, B=5, T=4096, Hq=8, Hkv=2, d=128, kb=6, W=100, N=2,
                         L_lo=1, L_hi=4096)
    inp = gen.make_decode(cfg)
    B, Hq, Hkv, C, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
    if token:
        kc = np.empty((B, Hkv, C, d), np.uint8)
        vc = np.empty((B, Hkv, C, d), np.uint8)
        gen.fill_decode_cache(inp, kc, vc, v_block_major=False)
        scale = dev(inp.kv_scale)
        blk, nsel = 1, cfg.kb + cfg.n_recent
    else:
        kc = np.empty((B, Hkv, C, d), np.uint16)
        vc = np.empty((B, Hkv, C // 64, d, 64), np.uint16)
        gen.fill_decode_cache(inp, kc, vc)
        scale = None
        blk, nsel = 64, cfg.kb
    k, v = dev(kc), dev(vc)
    lens = torch.from_numpy(inp.lens.astype(np.int32)).cuda()
    q = dev(inp.q)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    raw = torch.zeros((B, Hq, C // blk), device="cuda")
    idx = torch.empty((B, Hkv, nsel), dtype=torch.int32, device="cuda")
    shape = hb.decode_shape(q, k, lens, scale)
    ws_full = torch.empty(max(16, hb.workspace_size(hb.HS_FN_FULL_ATTN, shape, blk)),
                          dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(max(16, hb.workspace_size(hb.HS_FN_DECODE_SELECT, shape, blk)),
                         dtype=torch.uint8, device="cuda")
    ws_tsel = None
    if mode == "token_fused":
        ws_tsel = torch.empty(hb.workspace_size(hb.HS_FN_DECODE_TOKEN_SELECT, shape, 1, cfg.kb),
                              dtype=torch.uint8, device="cuda")
    layers = []
    for i, lay in enumerate(inp.layers):
        ent = dict(q=dev(lay["q"]), s=dev(gen.make_sinks(cfg, i)), o=torch.empty_like(o))
        if not token:
            ent.update(kr=dev(lay["k_ring"]), vr=dev(gen.block_major(lay["v_ring"])),
                       g=dev(lay["gates"]))
        layers.append(ent)

    def step():
        if mode == "token_fused":
            # full layer and token selection in one call (bounds, rescoring)
            hb.decode_token_select(q, k, v, lens, o, lse, cfg.kb, cfg.n_recent, idx, scale, ws=ws_tsel)
        else:
            hb.decode_full_attn_scores(q, k, v, lens, o, lse, raw, block=blk, ws=ws_full, kv_scale=scale)
            hb.decode_block_topk(q, k, lens, raw, lse, cfg.kb, idx, block=blk, n_recent=cfg.n_recent,
                                 kv_scale=scale)
        for l in layers:
            if token:
                hb.decode_select_attn(l["q"], k, v, lens, idx, nsel, None, None, 0, None, l["o"],
                                      block=1, kv_scale=scale, ws=ws_sel, sinks=l["s"])
            else:
                hb.decode_select_attn(l["q"], k, v, lens, idx, nsel, l["kr"], l["vr"], cfg.W, l["g"],
                                      l["o"], ws=ws_sel, sinks=l["s"])

    _replay_matches(step, [o, lse, idx] + [l["o"] for l in layers])
