"""GPU parity of the backward pass (bf16 inputs, fp32 gradients) against the
fp64 backward oracle (pinned by torch autograd and finite differences),
through the C ABI: the full layer, a sparse layer (both branches, gates,
sinks; its share of the shared K/V gradient added to the full layer's), and
the training forward's branch outputs.

Tolerance: gradients have no fixed scale (dK and dV sum over every query that
attends a key), so each gradient tensor is compared at 2e-2 max-abs relative
to its own largest reference entry, max(1, max|ref|) -- the bf16 output bound
applied to the tensor's scale (P and dS enter the matrix products in bf16)."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from oracle import hs_oracle as ora
from parity import dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close(name, got, want, rel=2e-2):
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got - want).max())
    say(f"  {name}: max|d|={err:.3g} (scale {scale:.3g})")
    assert err <= rel * scale, name


def bf16_dout(cfg, seed, shape):
    r = np.random.default_rng(seed)
    return gen.f32_to_bf16_bits(r.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("T,Hq,Hkv,d", [(1, 4, 1, 64), (65, 4, 4, 128), (200, 8, 2, 128), (333, 16, 2, 64),
                                        (257, 8, 1, 128)])
def test_full_layer_backward(T, Hq, Hkv, d):
    say(f"[bwd full] T={T} Hq={Hq} Hkv={Hkv} d={d}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", kb=2, W=0, N=0)
    inp = gen.make_prefill(cfg, n_layers=0)
    B = 1
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    raw = torch.empty((B, Hq, T, cfg.nblk), device="cuda")
    hb.full_attn_fwd_scores(q, k, vb, o, lse, raw)
    do_bits = bf16_dout(cfg, 5, (B, T, Hq, d))
    dq = torch.full((B, T, Hq, d), float("nan"), device="cuda")
    dk = torch.full((B, Hkv, T, d), float("nan"), device="cuda")
    dv = torch.full((B, Hkv, T, d), float("nan"), device="cuda")
    hb.full_attn_bwd(q, k, vb, o, lse, dev(do_bits), dq, dk, dv)
    torch.cuda.synchronize()
    f = lambda n: inp.f64(n)[0]
    do64 = gen.bf16_bits_to_f32(do_bits[0]).astype(np.float64)
    rq, rk, rv = ora.full_attention_bwd(f("q"), f("k"), f("v"), do64)
    close("dq", host(dq)[0], rq)
    close("dk", host(dk)[0], rk)
    close("dv", host(dv)[0], rv)


def _sparse_setup(T, Hq, Hkv, d, kb, W, gates=True, sinks=True, seed_do=7):
    """Full layer, selection (top-max(kb, 1)) and the training forward of one
    sparse layer with top-kb (kb = 0: no selected block)."""
    kb_sel = max(kb, 1)
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", kb=kb_sel, W=W, N=1)
    inp = gen.make_prefill(cfg)
    B = 1
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    raw = torch.empty((B, Hq, T, cfg.nblk), device="cuda")
    hb.full_attn_fwd_scores(q, k, vb, o, lse, raw)
    idx = torch.empty((B, Hkv, T, kb_sel), dtype=torch.int32, device="cuda")
    hb.block_topk((B, T, Hq, Hkv, d, hb.HS_BF16), raw, lse, kb_sel, idx)
    lay = inp.layers[0]
    sk = gen.make_sinks(cfg, 0) if sinks else None
    g = dev(lay["gates"]) if gates else None
    qs = dev(lay["q"])
    ks = dev(lay["k"]) if W else None
    vs = dev(gen.block_major(lay["v"])) if W else None
    os_ = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    ob = torch.full((2, B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lb = torch.full((2, B, Hq, T), float("nan"), device="cuda")
    hb.sparse_attn_fwd_train(qs, k, vb, idx, kb, ks, vs, W, g, os_, ob, lb,
                             sinks=None if sk is None else dev(sk))
    return cfg, inp, dict(q=q, k=k, vb=vb, o=o, lse=lse, idx=idx, qs=qs, ks=ks, vs=vs, g=g, os=os_, ob=ob, lb=lb,
                          sk=sk)


@pytest.mark.parametrize("T,Hq,Hkv,d,kb,W,gates,sinks", [
    (200, 8, 2, 128, 2, 50, True, True),
    (333, 4, 1, 64, 3, 100, True, False),
    (300, 16, 1, 128, 2, 64, False, True),
    (257, 8, 8, 64, 2, 0, True, False),      # no window
    (130, 8, 2, 128, 0, 40, True, True),     # no selection (window only)
])
def test_sparse_layer_backward(T, Hq, Hkv, d, kb, W, gates, sinks):
    say(f"[bwd sparse] T={T} Hq={Hq} Hkv={Hkv} d={d} kb={kb} W={W} gates={gates} sinks={sinks}")
    cfg, inp, x = _sparse_setup(T, Hq, Hkv, d, kb, W, gates, sinks)
    kb_used = kb
    B = 1
    do_bits = bf16_dout(cfg, 9, (B, T, Hq, d))
    dq = torch.full((B, T, Hq, d), float("nan"), device="cuda")
    dk = torch.zeros((B, Hkv, T, d), device="cuda")     # the layer's share is added to these
    dv = torch.zeros((B, Hkv, T, d), device="cuda")
    dks = torch.full((B, Hkv, T, d), float("nan"), device="cuda") if W else None
    dvs = torch.full((B, Hkv, T, d), float("nan"), device="cuda") if W else None
    dg = torch.full((B, T, Hq, 2), float("nan"), device="cuda") if gates else None
    dsk = torch.full((2, Hq), float("nan"), device="cuda") if sinks else None
    hb.sparse_attn_bwd(x["qs"], x["k"], x["vb"], x["idx"], kb_used, x["ks"], x["vs"], W, x["g"],
                       None if x["sk"] is None else dev(x["sk"]), x["ob"], x["lb"], dev(do_bits), dq, dk, dv,
                       dks, dvs, dg, dsk)
    torch.cuda.synchronize()
    f = lambda n, l=None: inp.f64(n, l)[0]
    idx = host(x["idx"])[0].astype(np.int64)
    if kb_used == 0:
        idx = np.full((Hkv, T, 1), -1, np.int64)
    do64 = gen.bf16_bits_to_f32(do_bits[0]).astype(np.float64)
    ref = ora.sparse_layer_bwd(f("q", 0), f("k"), f("v"), idx, f("k", 0), f("v", 0), W,
                               f("gates", 0) if gates else None, do64,
                               sinks=None if x["sk"] is None else x["sk"].astype(np.float64))
    # the training forward's branch outputs and LSEs
    pos = np.arange(T)
    sk = None if x["sk"] is None else x["sk"].astype(np.float64)
    o_sp = ora.sparse_branch_rows(f("q", 0), pos, f("k"), f("v"), idx, sink=None if sk is None else sk[0])
    o_sw = ora.window_branch_rows(f("q", 0), pos, f("k", 0), f("v", 0), W, sink=None if sk is None else sk[1])
    ob = host(x["ob"])
    close("o_branch sparse", ob[0, 0], o_sp)
    close("o_branch window", ob[1, 0], o_sw)
    close("dq", host(dq)[0], ref["dq"])
    if kb_used:
        close("dk (shared, this layer)", host(dk)[0], ref["dk"])
        close("dv (shared, this layer)", host(dv)[0], ref["dv"])
    if W:
        close("dk window", host(dks)[0], ref["dks"])
        close("dv window", host(dvs)[0], ref["dvs"])
    if gates:
        close("dgates", host(dg)[0], ref["dgates"])
    if sinks:
        close("dsinks", host(dsk), ref["dsinks"])


def _block_backward(inp, cfg, kb, W, seed_do=11):
    """Training forward and backward of a whole hybrid block on the GPU:
    full layer + selection + N sparse layers, then the full layer's backward
    and every sparse layer's, the latter adding into the shared dK/dV."""
    B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    raw = torch.empty((B, Hq, T, cfg.nblk), device="cuda")
    hb.full_attn_fwd_scores(q, k, vb, o, lse, raw)
    idx = torch.empty((B, Hkv, T, kb), dtype=torch.int32, device="cuda")
    hb.block_topk((B, T, Hq, Hkv, d, hb.HS_BF16), raw, lse, kb, idx)
    r = np.random.default_rng(seed_do)
    do_full = gen.f32_to_bf16_bits(r.standard_normal((B, T, Hq, d)).astype(np.float32))
    dq = torch.empty((B, T, Hq, d), device="cuda")
    dk = torch.empty((B, Hkv, T, d), device="cuda")
    dv = torch.empty((B, Hkv, T, d), device="cuda")
    ws = hb.full_attn_bwd(q, k, vb, o, lse, dev(do_full), dq, dk, dv)
    layers = []
    for lay in inp.layers:
        qs, ks, vs, g = dev(lay["q"]), dev(lay["k"]), dev(gen.block_major(lay["v"])), dev(lay["gates"])
        os_ = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
        ob = torch.empty((2, B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
        lb = torch.empty((2, B, Hq, T), device="cuda")
        hb.sparse_attn_fwd_train(qs, k, vb, idx, kb, ks, vs, W, g, os_, ob, lb)
        do_l = gen.f32_to_bf16_bits(r.standard_normal((B, T, Hq, d)).astype(np.float32))
        dql = torch.empty((B, T, Hq, d), device="cuda")
        dks = torch.empty((B, Hkv, T, d), device="cuda")
        dvs = torch.empty((B, Hkv, T, d), device="cuda")
        dg = torch.empty((B, T, Hq, 2), device="cuda")
        ws = hb.sparse_attn_bwd(qs, k, vb, idx, kb, ks, vs, W, g, None, ob, lb, dev(do_l), dql, dk, dv, dks, dvs,
                                dg, None, ws=ws)
        layers.append(dict(do=do_l, dq=dql, dks=dks, dvs=dvs, dg=dg, ob=ob))
    torch.cuda.synchronize()
    return dict(idx=idx, do=do_full, dq=dq, dk=dk, dv=dv, o=o, layers=layers)


def test_hybrid_block_backward_accumulates():
    """T = 1024 (16 tiles), two sparse layers: the shared dK/dV equal the full
    layer's gradient plus both sparse layers' shares (oracle, all rows)."""
    say("[bwd hybrid block] T=1024 Hq=8 Hkv=2 d=128 kb=4 W=128, 2 sparse layers")
    cfg = gen.config(1, T=1024, Hq=8, Hkv=2, d=128, dtype="bf16", kb=4, W=128, N=2)
    inp = gen.make_prefill(cfg)
    res = _block_backward(inp, cfg, cfg.kb, cfg.W)
    f = lambda n, l=None: inp.f64(n, l)[0]
    up = lambda bits: gen.bf16_bits_to_f32(bits[0]).astype(np.float64)
    rq, rk, rv = ora.full_attention_bwd(f("q"), f("k"), f("v"), up(res["do"]))
    idx = host(res["idx"])[0].astype(np.int64)
    for l, lay in enumerate(res["layers"]):
        g = ora.sparse_layer_bwd(f("q", l), f("k"), f("v"), idx, f("k", l), f("v", l), cfg.W, f("gates", l),
                                 up(lay["do"]))
        rk = rk + g["dk"]
        rv = rv + g["dv"]
        close(f"layer {l} dq", host(lay["dq"])[0], g["dq"])
        close(f"layer {l} dk window", host(lay["dks"])[0], g["dks"])
        close(f"layer {l} dgates", host(lay["dg"])[0], g["dgates"])
    close("full dq", host(res["dq"])[0], rq)
    close("shared dk (full + 2 sparse)", host(res["dk"])[0], rk)
    close("shared dv (full + 2 sparse)", host(res["dv"])[0], rv)


def test_sparse_backward_split_lists():
    """A block selected by more positions than one key-side work unit takes
    (block 0 here: every position past the first block selects it, 2536 per
    kv group, so three units) is split over several work groups whose shares
    are summed afterwards, in a fixed order, into the existing gradient. Every
    key's dK and dV against the oracle, with nonzero gradients already in place."""
    T, Hq, Hkv, d, W = 2600, 8, 2, 64, 64
    say(f"[bwd sparse, split lists] T={T} Hq={Hq} Hkv={Hkv} d={d} W={W}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", kb=3, W=W, N=1)
    inp = gen.make_prefill(cfg)
    B, kb = 1, 3
    idx_np = np.full((B, Hkv, T, kb), -1, np.int32)
    for g in range(Hkv):
        for t in range(64, T):
            past = t // 64  # fully-past blocks 0 .. past-1
            sel = sorted({0, past - 1, (7 * t + 3 * g) % past})
            idx_np[0, g, t, :len(sel)] = sel
    idx = dev(idx_np)
    lay = inp.layers[0]
    k, vb = dev(inp.k), dev(gen.block_major(inp.v))
    qs, ks, vs, g = dev(lay["q"]), dev(lay["k"]), dev(gen.block_major(lay["v"])), dev(lay["gates"])
    os_ = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty((2, B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lb = torch.empty((2, B, Hq, T), device="cuda")
    hb.sparse_attn_fwd_train(qs, k, vb, idx, kb, ks, vs, W, g, os_, ob, lb)
    do_bits = bf16_dout(cfg, 11, (B, T, Hq, d))
    r = np.random.default_rng(3)
    dk0 = r.standard_normal((B, Hkv, T, d)).astype(np.float32)
    dv0 = r.standard_normal((B, Hkv, T, d)).astype(np.float32)
    dq = torch.empty((B, T, Hq, d), device="cuda")
    dk, dv = dev(dk0), dev(dv0)
    dks = torch.empty((B, Hkv, T, d), device="cuda")
    dvs = torch.empty((B, Hkv, T, d), device="cuda")
    dg = torch.empty((B, T, Hq, 2), device="cuda")
    hb.sparse_attn_bwd(qs, k, vb, idx, kb, ks, vs, W, g, None, ob, lb, dev(do_bits), dq, dk, dv, dks, dvs, dg)
    torch.cuda.synchronize()
    f = lambda n, l=None: inp.f64(n, l)[0]
    do64 = gen.bf16_bits_to_f32(do_bits[0]).astype(np.float64)
    ref = ora.sparse_layer_bwd(f("q", 0), f("k"), f("v"), idx_np[0].astype(np.int64), f("k", 0), f("v", 0), W,
                               f("gates", 0), do64)
    close("dq", host(dq)[0], ref["dq"])
    close("dk (shared, added to what was there)", host(dk)[0] - dk0[0], ref["dk"])
    close("dv (shared, added to what was there)", host(dv)[0] - dv0[0], ref["dv"])
    close("dk (window)", host(dks)[0], ref["dks"])
    close("dv (window)", host(dvs)[0], ref["dvs"])
    # a second call on the same inputs gives the same bits (sums in a fixed order)
    dq2, dk2, dv2 = torch.empty_like(dq), dev(dk0), dev(dv0)
    hb.sparse_attn_bwd(qs, k, vb, idx, kb, ks, vs, W, g, None, ob, lb, dev(do_bits), dq2, dk2, dv2, dks, dvs, dg)
    torch.cuda.synchronize()
    assert torch.equal(dk2, dk) and torch.equal(dv2, dv) and torch.equal(dq2, dq)


def test_backward_7b_shape_sampled():
    """The 7B-shaped block (T = 8192, 32/8 heads, 3 sparse layers): dQ of the
    full layer and of sparse layer 0 on sampled rows against the oracle's
    row-local backward; the shared dK/dV through two identities that hold at
    any size: for every kv group, the dV rows sum to the gated dO summed over
    the queries that reach a key ((sum_i p_ti) = 1 per branch with keys),
    and the dK rows sum to zero (sum_i dS_ti = 0 per row)."""
    say("[bwd 7B-shaped] T=8192 Hq=32 Hkv=8 d=128, 3 sparse layers")
    cfg = gen.config(2)
    inp = gen.make_prefill(cfg)
    res = _block_backward(inp, cfg, cfg.kb, cfg.W)
    f = lambda n, l=None: inp.f64(n, l)[0]
    up = lambda bits: gen.bf16_bits_to_f32(bits[0]).astype(np.float64)
    rows = np.array([0, 1, 63, 64, 1000, 4095, 4096, 6000, 8190, 8191])
    rq, _, _ = ora.full_attention_bwd(f("q"), f("k"), f("v"), up(res["do"]), rows=rows)
    close("full dq (sampled rows)", host(res["dq"])[0][rows], rq[rows])
    idx = host(res["idx"])[0].astype(np.int64)
    lay0 = res["layers"][0]
    g = ora.sparse_layer_bwd(f("q", 0), f("k"), f("v"), idx, f("k", 0), f("v", 0), cfg.W, f("gates", 0),
                             up(lay0["do"]), rows=rows)
    close("layer 0 dq (sampled rows)", host(lay0["dq"])[0][rows], g["dq"][rows])
    close("layer 0 dgates (sampled rows)", host(lay0["dg"])[0][rows], g["dgates"][rows])
    # identities: sum over keys of dV = sum over (t, h in g) of dO~ of every
    # branch that reaches keys of this cache; sum over keys of dK = 0
    G = cfg.G
    want = up(res["do"]).reshape(cfg.T, cfg.Hkv, G, cfg.d).sum(axis=(0, 2))      # full layer
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    for l, lay in enumerate(res["layers"]):
        s0 = sig(f("gates", l)[..., 0])[..., None]                                # [T, Hq, 1]
        has = (idx >= 0).any(axis=2).T[:, :, None].repeat(G, axis=1)              # [T, Hq, 1] any selected block
        dob = up(lay["do"]) * s0 * has
        want = want + dob.reshape(cfg.T, cfg.Hkv, G, cfg.d).sum(axis=(0, 2))
    close("sum_i dV (shared)", host(res["dv"])[0].sum(axis=1), want)
    close("sum_i dK (shared) = 0", host(res["dk"])[0].sum(axis=1), np.zeros((cfg.Hkv, cfg.d)))
