"""GPU parity of the decode path (block mode): split-K full layer with block
scores, selection, sparse layers with the window ring and gates, against the
fp64 oracle, through the C ABI.  Cache positions >= L_b hold NaN, so any read
past a sequence's length shows up in the outputs."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from oracle import hs_oracle as ora
from parity import SIDE_TOL, TOL, check_index_row, check_index_set, dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class DecodeRun:
    def __init__(self, inp, n_layers=None, gates=True, W=None, sinks=False):
        cfg = inp.cfg
        self.cfg, self.inp = cfg, inp
        B, Hq, Hkv, C, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
        self.W = cfg.W if W is None else W
        kc = np.empty((B, Hkv, C, d), np.uint16)
        vc = np.empty((B, Hkv, C // 64, d, 64), np.uint16)
        gen.fill_decode_cache(inp, kc, vc)
        self.k, self.v = dev(kc), dev(vc)
        del kc, vc
        self.lens = torch.from_numpy(inp.lens.astype(np.int32)).cuda()
        q = dev(inp.q)
        self.o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((B, Hq), float("nan"), device="cuda")
        self.raw = torch.full((B, Hq, C // 64), float("nan"), device="cuda")
        hb.decode_full_attn_scores(q, self.k, self.v, self.lens, self.o, self.lse, self.raw)
        self.idx = torch.full((B, Hkv, cfg.kb), -7, dtype=torch.int32, device="cuda")
        self.gs = torch.full((B, Hkv, C // 64), float("nan"), device="cuda")
        hb.decode_block_topk(q, self.k, self.lens, self.raw, self.lse, cfg.kb, self.idx, self.gs)
        self.outs = []
        layers = inp.layers if n_layers is None else inp.layers[:n_layers]
        self.sinks = [gen.make_sinks(cfg, l) if sinks else None for l in range(len(layers))]
        for l, lay in enumerate(layers):
            o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
            kr = dev(lay["k_ring"]) if self.W else None
            vr = dev(gen.block_major(lay["v_ring"])) if self.W else None
            g = dev(lay["gates"]) if gates else None
            sk = None if self.sinks[l] is None else dev(self.sinks[l])
            hb.decode_select_attn(dev(lay["q"]), self.k, self.v, self.lens, self.idx, cfg.kb,
                                  kr, vr, self.W, g, o, sinks=sk)
            self.outs.append(o)
        torch.cuda.synchronize()


def f64_bf16(a):
    return gen.bf16_bits_to_f32(a).astype(np.float64)


def _pool_map(fn, items):
    """Oracle checks of independent sequences on a thread pool (numpy releases
    the GIL in its matrix products and random draws); one BLAS thread each."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1), ThreadPoolExecutor(min(16, len(items))) as ex:
        return list(ex.map(fn, items))


def check_sequences(run, seqs, gates=True):
    cfg, inp = run.cfg, run.inp
    tol = TOL["bf16"]
    o_g, lse_g, raw_g = host(run.o), host(run.lse), host(run.raw)
    idx_g, gs_g = host(run.idx), host(run.gs)
    outs_g = [host(o) for o in run.outs]

    def one(b):
        w = dict(o=0.0, lse=0.0, raw=0.0, layer=0.0, ties=0)
        L = int(inp.lens[b])
        ks, vs = zip(*(inp.kv_slab_f64(b, g) for g in range(cfg.Hkv)))
        k, v = np.stack(ks), np.stack(vs)
        layers = []
        for l, lay in enumerate(inp.layers[: len(run.outs)]):
            layers.append(dict(q=f64_bf16(lay["q"][b]),
                               k_ring=f64_bf16(lay["k_ring"][b]) if run.W else None,
                               v_ring=f64_bf16(lay["v_ring"][b]) if run.W else None,
                               gates=lay["gates"][b].astype(np.float64) if gates else None,
                               sinks=None if run.sinks[l] is None else run.sinks[l].astype(np.float64)))
        ref = ora.decode_step(f64_bf16(inp.q[b]), k, v, L, [], cfg.kb, run.W)
        nb = (L - 1) // 64 + 1
        w["o"] = np.abs(o_g[b] - ref["o"]).max()
        w["lse"] = np.abs(lse_g[b] - ref["lse"]).max()
        w["raw"] = np.abs(raw_g[b][:, :nb] - ref["raw"][:, :nb]).max()
        assert np.abs(gs_g[b][:, :nb] - ref["Sg"][:, :nb]).max() <= 1e-4 * ref["Sg"][:, :nb].max(), b
        for g in range(cfg.Hkv):
            ranked = ref["ranked"][g]
            ok, tie = check_index_row(idx_g[b, g], ref["idx"][g], ranked, cfg.kb)
            if tie:
                w["ties"] += 1
                cand = np.arange((L - 1) // 64)
                ok = ok and check_index_set(idx_g[b, g], ref["Sg"][g], cand, cfg.kb, ranked)
            assert ok, (b, g, idx_g[b, g], ref["idx"][g])
        for l, lay in enumerate(layers):
            want = ora.decode_sparse_layer(lay, k, v, L, idx_g[b].astype(np.int64), run.W)
            w["layer"] = max(w["layer"], np.abs(outs_g[l][b] - want).max())
        return w

    res = _pool_map(one, list(seqs))
    worst = {key: max(r[key] for r in res) for key in ("o", "lse", "raw", "layer")}
    ties = sum(r["ties"] for r in res)
    say(f"  {len(res)} seqs max|dO|={worst['o']:.3g} max|dLSE|={worst['lse']:.3g} "
        f"max|draw|={worst['raw']:.3g} sparse max|dO|={worst['layer']:.3g} near-tie={ties}")
    assert worst["o"] <= tol and worst["layer"] <= tol
    assert worst["lse"] <= SIDE_TOL and worst["raw"] <= SIDE_TOL
    # NaN poison beyond L must never leak into the outputs
    assert not np.isnan(o_g).any() and all(not np.isnan(x).any() for x in outs_g)


@pytest.mark.parametrize("W,gates,sinks", [(100, True, False), (64, False, False), (0, True, False),
                                           (300, True, False), (100, True, True), (0, False, True)])
def test_small_ragged(W, gates, sinks):
    say(f"[decode small] W={W} gates={gates} sinks={sinks}")
    cfg = gen.config(4, B=6, T=1024, Hq=8, Hkv=2, d=128, kb=3, W=W, N=2, L_lo=1, L_hi=1024)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([1, 63, 64, 65, 700, 1024], np.int32)
    run = DecodeRun(inp, gates=gates, sinks=sinks)
    check_sequences(run, range(6), gates=gates)


def test_many_sequences_unit_numbering():
    """More than 128 sequences: the full layer numbers its live split-K units
    with a prefix over the lengths taken 64 sequences at a time, so ids past
    the first 64 and 128 sequences go through the carried part of the scan."""
    say("[decode many sequences] B=150 C=2048 Hq=4 Hkv=2 d=64")
    cfg = gen.config(4, B=150, T=2048, Hq=4, Hkv=2, d=64, kb=4, W=64, N=1, L_lo=1, L_hi=2048)
    inp = gen.make_decode(cfg)
    lens = np.random.default_rng(11).integers(1, 2049, size=150).astype(np.int32)
    lens[[0, 63, 64, 127, 128, 149]] = [2048, 1, 1025, 64, 2047, 1024]
    inp.lens = lens
    run = DecodeRun(inp)
    check_sequences(run, [0, 1, 62, 63, 64, 65, 100, 127, 128, 129, 140, 148, 149])


def test_large_logits():
    """Queries scaled by 24: logits reach the hundreds, so the split-K
    partial states of one row carry maxima far apart and the merge must
    rescale them exactly; sparse layers with sinks and the window."""
    say("[decode large logits] q x 24")
    cfg = gen.config(4, B=3, T=2048, Hq=8, Hkv=2, d=128, kb=4, W=100, N=1, L_lo=1, L_hi=2048)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([70, 1500, 2048], np.int32)
    up = lambda a: gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(a) * 24.0)
    inp.q = up(inp.q)
    inp.layers[0]["q"] = up(inp.layers[0]["q"])
    run = DecodeRun(inp, sinks=True)
    check_sequences(run, range(3))


def test_long_capacity_chunks():
    """Capacity above 128K: the full layer's split-K chunks are 32 tiles long."""
    say("[decode capacity 196608] B=2 Hq=8 Hkv=2 d=128")
    cfg = gen.config(4, B=2, T=196608, Hq=8, Hkv=2, d=128, kb=8, W=128, N=1, L_lo=1, L_hi=196608)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([150001, 196608], np.int32)
    run = DecodeRun(inp)
    check_sequences(run, range(2))


def test_max_capacity_block_mode():
    """Block mode at the largest capacity the selection takes (262144 slots,
    4096 blocks per row), one sequence at the full length."""
    say("[decode capacity 262144] B=2 Hq=4 Hkv=1 d=128")
    cfg = gen.config(4, B=2, T=262144, Hq=4, Hkv=1, d=128, kb=16, W=128, N=1, L_lo=1, L_hi=262144)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([100003, 262144], np.int32)
    run = DecodeRun(inp)
    check_sequences(run, range(2))


def test_group_of_16_and_d64():
    say("[decode G=16 d=64]")
    cfg = gen.config(4, B=3, T=2048, Hq=16, Hkv=1, d=64, kb=5, W=128, N=1, L_lo=300, L_hi=2048)
    inp = gen.make_decode(cfg)
    run = DecodeRun(inp)
    check_sequences(run, range(3))


def test_config4_full_size_all_sequences():
    say("[config 4] 64 seqs, capacity 65536, L ~ U[32768, 65536], kb=32, W=128 (layers 0-1 of 11), "
        "every sequence")
    inp = gen.make_decode(gen.config(4), n_layers=2)
    run = DecodeRun(inp)
    check_sequences(run, range(64))


def _messy_rows(clean, n_out, bad, seed):
    """Index rows [B, Hkv, n_out] holding the same sets as `clean` (ids >= 0)
    but shuffled, with some ids repeated and invalid ids (`bad(b)`: negative
    or out of range) mixed in anywhere."""
    rng = np.random.default_rng(seed)
    B, Hkv, _ = clean.shape
    out = np.empty((B, Hkv, n_out), np.int32)
    for b in range(B):
        for g in range(Hkv):
            live = clean[b, g][clean[b, g] >= 0]
            extra = [int(x) for x in rng.choice(live, size=min(3, live.size))] if live.size else []
            row = list(live) + extra + list(bad(b))
            row += [-1] * (n_out - len(row))
            assert len(row) == n_out
            out[b, g] = rng.permutation(np.array(row, np.int32))
    return out


def test_index_rows_are_sets_block_mode():
    """The block-mode sparse layer reads each idx row as a set: a shuffled
    row with repeated ids, -1 and out-of-range ids anywhere gives bit-for-bit
    the output of the clean ascending row, and matches the oracle given the
    messy row directly."""
    say("[decode idx as a set] block mode")
    cfg = gen.config(4, B=4, T=2048, Hq=8, Hkv=2, d=128, kb=6, W=100, N=1, L_lo=1, L_hi=2048)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([40, 200, 1500, 2048], np.int32)
    run = DecodeRun(inp)
    clean = host(run.idx).astype(np.int32)
    C = cfg.T
    bad = lambda b: [-1, -5, (int(inp.lens[b]) + 63) // 64, C // 64 + 7, 1 << 30]
    n_out = cfg.kb + 3 + 5 + 4
    messy = _messy_rows(clean, n_out, bad, seed=3)
    lay = inp.layers[0]
    o2 = torch.full_like(run.outs[0], float("nan"))
    hb.decode_select_attn(dev(lay["q"]), run.k, run.v, run.lens, dev(messy), n_out,
                          dev(lay["k_ring"]), dev(gen.block_major(lay["v_ring"])), cfg.W,
                          dev(lay["gates"]), o2)
    torch.cuda.synchronize()
    a, b2 = host(run.outs[0]), host(o2)
    say(f"  messy vs clean rows: max|dO|={np.abs(a - b2).max():.3g}")
    assert np.array_equal(a, b2)
    for b in range(cfg.B):
        L = int(inp.lens[b])
        ks, vs = zip(*(inp.kv_slab_f64(b, g) for g in range(cfg.Hkv)))
        want = ora.decode_sparse_layer(dict(q=f64_bf16(lay["q"][b]), k_ring=f64_bf16(lay["k_ring"][b]),
                                            v_ring=f64_bf16(lay["v_ring"][b]),
                                            gates=lay["gates"][b].astype(np.float64)),
                                       np.stack(ks), np.stack(vs), L, messy[b].astype(np.int64), cfg.W)
        assert np.abs(b2[b] - want).max() <= TOL["bf16"], b


@pytest.mark.parametrize("W", [0, 100])
def test_empty_selection_block_mode(W):
    """n_sel = 0 with no index list at all: the sparse branch is empty, so
    the layer output is the gated window branch (0 without a window)."""
    say(f"[decode empty selection] W={W}")
    cfg = gen.config(4, B=3, T=1024, Hq=8, Hkv=2, d=128, kb=4, W=W, N=1, L_lo=1, L_hi=1024)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([1, 300, 1024], np.int32)
    kc = np.empty((cfg.B, cfg.Hkv, cfg.T, cfg.d), np.uint16)
    vc = np.empty((cfg.B, cfg.Hkv, cfg.T // 64, cfg.d, 64), np.uint16)
    gen.fill_decode_cache(inp, kc, vc)
    k, v = dev(kc), dev(vc)
    lens = torch.from_numpy(inp.lens).cuda()
    lay = inp.layers[0]
    o = torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    kr = dev(lay["k_ring"]) if W else None
    vr = dev(gen.block_major(lay["v_ring"])) if W else None
    hb.decode_select_attn(dev(lay["q"]), k, v, lens, None, 0, kr, vr, W, dev(lay["gates"]), o)
    torch.cuda.synchronize()
    got = host(o)
    for b in range(cfg.B):
        L = int(inp.lens[b])
        want = ora.decode_sparse_layer(
            dict(q=f64_bf16(lay["q"][b]), gates=lay["gates"][b].astype(np.float64),
                 k_ring=f64_bf16(lay["k_ring"][b]) if W else None,
                 v_ring=f64_bf16(lay["v_ring"][b]) if W else None),
            np.zeros((cfg.Hkv, L, cfg.d)), np.zeros((cfg.Hkv, L, cfg.d)), L,
            np.full((cfg.Hkv, 0), -1, np.int64), W)
        assert np.abs(got[b] - want).max() <= TOL["bf16"], b
    if W == 0:
        assert np.all(got == 0)


# --------------------------------------------------------------- token level
class TokenRun:
    """Token-level decode (fp8 e4m3 caches, position-major): full layer with
    per-token logits, top-k tokens + the newest n_recent, sparse layers."""

    def __init__(self, inp, n_layers=None, sinks=False, ws=None):
        cfg = inp.cfg
        self.cfg, self.inp = cfg, inp
        B, Hq, Hkv, C, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
        R, kb = cfg.n_recent, cfg.kb
        kc = np.empty((B, Hkv, C, d), np.uint8)
        vc = np.empty((B, Hkv, C, d), np.uint8)
        gen.fill_decode_cache(inp, kc, vc, v_block_major=False)
        self.k, self.v = dev(kc), dev(vc)
        del kc, vc
        self.scale = dev(inp.kv_scale)
        self.lens = torch.from_numpy(inp.lens.astype(np.int32)).cuda()
        q = dev(inp.q)
        self.o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((B, Hq), float("nan"), device="cuda")
        self.raw = torch.full((B, Hq, C), float("nan"), device="cuda")
        hb.decode_full_attn_scores(q, self.k, self.v, self.lens, self.o, self.lse, self.raw,
                                   block=1, kv_scale=self.scale)
        self.idx = torch.full((B, Hkv, kb + R), -7, dtype=torch.int32, device="cuda")
        self.gs = torch.full((B, Hkv, C), float("nan"), device="cuda")
        hb.decode_block_topk(q, self.k, self.lens, self.raw, self.lse, kb, self.idx, self.gs,
                             block=1, n_recent=R, kv_scale=self.scale)
        self.outs = []
        layers = inp.layers if n_layers is None else inp.layers[:n_layers]
        self.sinks = [gen.make_sinks(cfg, l) if sinks else None for l in range(len(layers))]
        for l, lay in enumerate(layers):
            o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
            sk = None if self.sinks[l] is None else dev(self.sinks[l])
            hb.decode_select_attn(dev(lay["q"]), self.k, self.v, self.lens, self.idx, kb + R,
                                  None, None, 0, None, o, block=1, kv_scale=self.scale,
                                  sinks=sk, ws=ws)
            self.outs.append(o)
        torch.cuda.synchronize()


def token_idx_row_ok(row, ref, g, L, kb, R, rel, where):
    """One (sequence, kv group) row of a token selection against the oracle:
    ascending, -1 padded, the newest tokens last; equal to the oracle's row
    unless its k-th and (k+1)-th scores are within rel (then every token
    clearly above the k-th is in and none clearly below).  Returns 1 for a
    near-tie row."""
    ncand = max(0, L - R)
    want = ref["idx"][g]
    n_out = min(kb, ncand) + min(R, L)
    assert np.all(row[n_out:] == -1) and np.all(np.diff(row[:n_out]) > 0), where
    assert np.array_equal(row[n_out - min(R, L):n_out], np.arange(L - min(R, L), L)), where
    ranked = ref["ranked"][g]
    if ncand > kb:
        sk, sk1 = ranked[kb - 1], ranked[kb]
        if (sk - sk1) / sk < rel:
            got = row[: n_out - min(R, L)]
            Sg = ref["Sg"][g]
            cand = np.arange(ncand)
            must = cand[Sg[cand] > sk * (1 + rel)]
            banned = cand[Sg[cand] < sk * (1 - rel)]
            assert np.all(np.isin(must, got)) and not np.any(np.isin(banned, got)), where
            return 1
    assert np.array_equal(row[:n_out], want[:n_out]), where
    return 0


def check_token_sequences(run, seqs, rel=1e-4):
    cfg, inp = run.cfg, run.inp
    R, kb = cfg.n_recent, cfg.kb
    o_g, lse_g, raw_g = host(run.o), host(run.lse), host(run.raw)
    idx_g, gs_g = host(run.idx), host(run.gs)
    outs_g = [host(o) for o in run.outs]
    scale = inp.kv_scale.astype(np.float64)

    def one(b):
        w = dict(o=0.0, lse=0.0, raw=0.0, layer=0.0, gs=0.0, ties=0)
        L = int(inp.lens[b])
        ks, vs = zip(*(inp.kv_slab(b, g) for g in range(cfg.Hkv)))
        k, v = ora.dequantize_kv(np.stack(ks), np.stack(vs), scale, L)
        ref = ora.decode_step(f64_bf16(inp.q[b]), k, v, L, [], kb, 0, block=1, n_recent=R)
        w["o"] = np.abs(o_g[b] - ref["o"]).max()
        w["lse"] = np.abs(lse_g[b] - ref["lse"]).max()
        w["raw"] = np.abs(raw_g[b][:, :L] - ref["raw"][:, :L]).max()
        w["gs"] = (np.abs(gs_g[b][:, :L] - ref["Sg"][:, :L]) / ref["Sg"][:, :L].max()).max()
        for g in range(cfg.Hkv):
            w["ties"] += token_idx_row_ok(idx_g[b, g], ref, g, L, kb, R, rel, (b, g))
        for l in range(len(run.outs)):
            lay = dict(q=f64_bf16(inp.layers[l]["q"][b]),
                       sinks=None if run.sinks[l] is None else run.sinks[l].astype(np.float64))
            want = ora.decode_sparse_layer(lay, k, v, L, idx_g[b].astype(np.int64), 0, block=1)
            w["layer"] = max(w["layer"], np.abs(outs_g[l][b] - want).max())
        return w

    res = _pool_map(one, list(seqs))
    worst = {key: max(r[key] for r in res) for key in ("o", "lse", "raw", "layer", "gs")}
    ties = sum(r["ties"] for r in res)
    say(f"  {len(res)} seqs max|dO|={worst['o']:.3g} max|dLSE|={worst['lse']:.3g} "
        f"max|draw|={worst['raw']:.3g} rel|dSg|={worst['gs']:.3g} "
        f"sparse max|dO|={worst['layer']:.3g} near-tie={ties}")
    tol = TOL["fp8"]
    assert worst["o"] <= tol and worst["layer"] <= tol
    assert worst["lse"] <= SIDE_TOL and worst["raw"] <= SIDE_TOL and worst["gs"] < 1e-4
    assert not np.isnan(o_g).any() and all(not np.isnan(x).any() for x in outs_g)


def test_token_small_ragged():
    say("[token small] fp8, C=4096, top-256 + 16 recent")
    cfg = gen.config(5, B=4, T=4096, Hq=8, Hkv=2, d=128, kb=256, n_recent=16, N=2,
                     L_lo=1, L_hi=4096)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([1, 200, 300, 4096], np.int32)
    run = TokenRun(inp)
    check_token_sequences(run, range(4))


@pytest.mark.parametrize("split", [True, False])
def test_token_sinks(split):
    """Sink logits in the token-mode sparse layer, added by the merge kernel
    (split work groups) or by the one group per (sequence, kv head)."""
    say(f"[token sinks] split={split}")
    cfg = gen.config(5, B=4, T=8192, Hq=8, Hkv=2, d=128, kb=700, n_recent=64, N=2,
                     L_lo=1, L_hi=8192)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([5, 1000, 6000, 8192], np.int32)
    ws = None if split else torch.empty(16, dtype=torch.uint8, device="cuda")
    run = TokenRun(inp, sinks=True, ws=ws)
    check_token_sequences(run, range(4))


def test_token_d64_group16():
    say("[token d=64 G=16]")
    cfg = gen.config(5, B=2, T=8192, Hq=16, Hkv=1, d=64, kb=100, n_recent=128, N=1,
                     L_lo=5000, L_hi=8192)
    inp = gen.make_decode(cfg)
    run = TokenRun(inp)
    check_token_sequences(run, range(2))


# ------------------------------------- token level, selection from bounds
class TokenSelectRun:
    """hs_decode_token_select (the full layer and the token selection in one
    call, the selection from bounds and exact rescoring) beside the two-call
    path on the same inputs."""

    def __init__(self, inp):
        cfg = inp.cfg
        self.cfg, self.inp = cfg, inp
        self.base = TokenRun(inp, n_layers=0)
        B, Hq, Hkv, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.d
        self.o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((B, Hq), float("nan"), device="cuda")
        self.idx = torch.full((B, Hkv, cfg.kb + cfg.n_recent), -7, dtype=torch.int32, device="cuda")
        hb.decode_token_select(dev(inp.q), self.base.k, self.base.v, self.base.lens, self.o, self.lse, cfg.kb,
                               cfg.n_recent, self.idx, self.base.scale)
        torch.cuda.synchronize()


def check_token_select(run, seqs, rel=1e-4):
    cfg, inp = run.cfg, run.inp
    R, kb = cfg.n_recent, cfg.kb
    # the full layer's arithmetic is the same: o and lse bit for bit
    assert torch.equal(run.o, run.base.o) and torch.equal(run.lse, run.base.lse)
    idx_g = host(run.idx)
    scale = inp.kv_scale.astype(np.float64)

    def one(b):
        L = int(inp.lens[b])
        ks, vs = zip(*(inp.kv_slab(b, g) for g in range(cfg.Hkv)))
        k, v = ora.dequantize_kv(np.stack(ks), np.stack(vs), scale, L)
        ref = ora.decode_step(f64_bf16(inp.q[b]), k, v, L, [], kb, 0, block=1, n_recent=R)
        return sum(token_idx_row_ok(idx_g[b, g], ref, g, L, kb, R, rel, (b, g)) for g in range(cfg.Hkv))

    ties = sum(_pool_map(one, list(seqs)))
    say(f"  {len(list(seqs))} seqs: selection from bounds matches the oracle (near-tie rows {ties})")


def test_token_select_small_ragged():
    say("[token select] fp8, C=4096, top-256 + 16 recent, lengths 1 .. 4096")
    cfg = gen.config(5, B=4, T=4096, Hq=8, Hkv=2, d=128, kb=256, n_recent=16, N=0, L_lo=1, L_hi=4096)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([1, 200, 300, 4096], np.int32)
    check_token_select(TokenSelectRun(inp), range(4))


def test_token_select_d64_group16():
    say("[token select] d=64, G=16")
    cfg = gen.config(5, B=2, T=8192, Hq=16, Hkv=1, d=64, kb=100, n_recent=128, N=0, L_lo=5000, L_hi=8192)
    check_token_select(TokenSelectRun(gen.make_decode(cfg)), range(2))


def test_token_select_all_tied_takes_the_whole_row():
    """All logits of one sequence equal (q = 0): every old token is a
    candidate, far past the candidate store, so the scores of the whole row
    are computed exactly and selected there; ties go to the smaller id."""
    say("[token select ties] fp8, C=16384, top-2048 + 128 recent, one sequence with q = 0")
    cfg = gen.config(5, B=2, T=16384, Hq=8, Hkv=2, d=128, kb=2048, n_recent=128, N=0,
                     L_lo=16384, L_hi=16384)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([16384, 12000], np.int32)
    inp.q[0] = 0
    run = TokenSelectRun(inp)
    idx = host(run.idx)
    for g in range(cfg.Hkv):
        want = np.concatenate([np.arange(2048), np.arange(16384 - 128, 16384)])
        assert np.array_equal(idx[0, g], want), g
    check_token_select(run, range(2))


def test_token_select_peaked_scores_open_bin():
    """One sequence's queries scaled by 40: its scores spread over hundreds of
    log2 units, so fewer than k lower bounds lie within 32 of zero.  The k-th
    bound falls in the open bottom bin, every old token is a candidate (more
    than the candidate store holds), and the pick takes exact scores of the
    whole row.  The second sequence is unscaled."""
    say("[token select peaked] fp8, C=16384, top-2048 + 128 recent, one sequence with q x 40")
    cfg = gen.config(5, B=2, T=16384, Hq=8, Hkv=2, d=128, kb=2048, n_recent=128, N=0,
                     L_lo=16384, L_hi=16384)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([16384, 9000], np.int32)
    inp.q[0] = gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(inp.q[0]) * 40.0)
    check_token_select(TokenSelectRun(inp), range(2))


def test_token_select_config5_full_size_all_sequences():
    say("[token select, config 5] 16 seqs x 262144 fp8 tokens, top-2048 + 128 recent, every sequence")
    inp = gen.make_decode(gen.config(5), n_layers=0)
    check_token_select(TokenSelectRun(inp), range(16))


def test_config5_token_level_full_size_all_sequences():
    say("[config 5] 16 seqs x 262144 fp8 tokens, top-2048 + 128 recent (layers 0-1 of 11), "
        "every sequence")
    inp = gen.make_decode(gen.config(5), n_layers=2)
    run = TokenRun(inp)
    check_token_sequences(run, range(16))


def test_token_many_tied_candidates():
    """Every logit of one sequence equal (its query is zero): all old tokens
    tie, far more than the 8192 candidates the threshold pass keeps, so the
    pick takes the radix select over the whole row.  Ties go to the smaller
    token id: the selection is tokens 0 .. k-1 plus the newest ones."""
    say("[token ties] fp8, C=16384, top-2048 + 128 recent, one sequence with q = 0")
    cfg = gen.config(5, B=2, T=16384, Hq=8, Hkv=2, d=128, kb=2048, n_recent=128, N=1,
                     L_lo=16384, L_hi=16384)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([16384, 12000], np.int32)
    inp.q[0] = 0
    run = TokenRun(inp)
    idx = host(run.idx)
    for g in range(cfg.Hkv):
        want = np.concatenate([np.arange(2048), np.arange(16384 - 128, 16384)])
        assert np.array_equal(idx[0, g], want), g
    check_token_sequences(run, range(2))


@pytest.mark.parametrize("split", [True, False])
def test_index_rows_are_sets_token_mode(split):
    """Token mode reads each idx row as a set too: shuffled, repeated,
    negative and out-of-range (>= L) token ids give bit-for-bit the output
    of the clean row, and match the oracle given the messy row."""
    say(f"[decode idx as a set] token mode split={split}")
    cfg = gen.config(5, B=3, T=8192, Hq=8, Hkv=2, d=128, kb=700, n_recent=64, N=1,
                     L_lo=1, L_hi=8192)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([50, 3000, 8192], np.int32)
    ws = None if split else torch.empty(16, dtype=torch.uint8, device="cuda")
    run = TokenRun(inp, ws=ws)
    clean = host(run.idx).astype(np.int32)
    bad = lambda b: [-1, -9, int(inp.lens[b]), int(inp.lens[b]) + 5, cfg.T + 100, 1 << 30]
    n_out = cfg.kb + cfg.n_recent + 3 + 6 + 20
    messy = _messy_rows(clean, n_out, bad, seed=4)
    lay = inp.layers[0]
    o2 = torch.full_like(run.outs[0], float("nan"))
    hb.decode_select_attn(dev(lay["q"]), run.k, run.v, run.lens, dev(messy), n_out, None, None, 0,
                          None, o2, block=1, kv_scale=run.scale, ws=ws)
    torch.cuda.synchronize()
    a, b2 = host(run.outs[0]), host(o2)
    say(f"  messy vs clean rows: max|dO|={np.abs(a - b2).max():.3g}")
    if split:
        # the split over work groups follows the list length: equal to rounding
        assert np.abs(a - b2).max() <= 1e-2
    else:
        assert np.array_equal(a, b2)
    for b in range(cfg.B):
        L = int(inp.lens[b])
        ks, vs = zip(*(inp.kv_slab(b, g) for g in range(cfg.Hkv)))
        want = ora.decode_sparse_layer(dict(q=f64_bf16(lay["q"][b])), np.stack(ks), np.stack(vs), L,
                                       messy[b].astype(np.int64), 0, block=1,
                                       kv_scale=inp.kv_scale.astype(np.float64))
        assert np.abs(b2[b] - want).max() <= TOL["fp8"], b


def test_token_split_work_groups():
    """Token-mode sparse layer spread over several work groups per (sequence,
    group) (workspace given) against the oracle and against the one-group
    path (no workspace), on ragged lengths with many empty tail tiles."""
    say("[token split] fp8, C=16384, top-1500 + 100 recent, lens 1..16384")
    cfg = gen.config(5, B=4, T=16384, Hq=8, Hkv=2, d=128, kb=1500, n_recent=100, N=1,
                     L_lo=1, L_hi=16384)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([3, 900, 7777, 16384], np.int32)
    run = TokenRun(inp)
    check_token_sequences(run, range(4))
    lay = inp.layers[0]
    B, Hq, d = cfg.B, cfg.Hq, cfg.d
    o1 = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    tiny = torch.empty(16, dtype=torch.uint8, device="cuda")  # too small: one group per (b, g)
    hb.decode_select_attn(dev(lay["q"]), run.k, run.v, run.lens, run.idx, cfg.kb + cfg.n_recent,
                          None, None, 0, None, o1, block=1, kv_scale=run.scale, ws=tiny)
    torch.cuda.synchronize()
    a, b = host(run.outs[0]), host(o1)
    say(f"  split vs one group max|dO|={np.abs(a - b).max():.3g}")
    assert not np.isnan(b).any() and np.abs(a - b).max() <= 2e-2
