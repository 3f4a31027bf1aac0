"""GPU parity of the fp8 prefill path (reading R15: e4m3 codes with one scale
per head; the kernels use the fp8 matrix units) against the fp64 oracle on the
dequantised values, through the C ABI.  Outputs within the fp8 tolerance
(6e-2); LSE, block scores and group scores within the fp32 side tolerance
(the logits are exact); indices under the near-tie rule."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from oracle import hs_oracle as ora
from parity import SIDE_TOL, TOL, compare_indices, dev, host, sample_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class RunF8:
    def __init__(self, inp, score=hb.HS_SCORE_MAX, include_diag=False, sparse=True, sinks=False):
        cfg = inp.cfg
        self.cfg, self.inp = cfg, inp
        B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d
        self.kb, self.W = cfg.kb, cfg.W
        q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
        qs, kvs = dev(inp.q_scale), dev(inp.kv_scale)
        self.o = torch.full((B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((B, Hq, T), float("nan"), device="cuda")
        self.raw = torch.full((B, Hq, T, cfg.nblk), float("nan"), device="cuda")
        hb.full_attn_fwd_scores(q, k, vb, self.o, self.lse, self.raw, score=score, q_scale=qs, kv_scale=kvs)
        self.idx = torch.full((B, Hkv, T, self.kb), -7, dtype=torch.int32, device="cuda")
        self.gs = torch.full((B, Hkv, T, cfg.nblk), float("nan"), device="cuda")
        hb.block_topk((B, T, Hq, Hkv, d, hb.HS_FP8_E4M3), self.raw, self.lse, self.kb, self.idx, self.gs,
                      include_diag=include_diag)
        self.outs = []
        self.sinks = [gen.make_sinks(cfg, l) if sinks else None for l in range(len(inp.layers))]
        if sparse:
            for l, lay in enumerate(inp.layers):
                o = torch.full((B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
                sk = None if self.sinks[l] is None else dev(self.sinks[l])
                hb.sparse_attn_fwd(dev(lay["q"]), k, vb, self.idx, self.kb, dev(lay["k"]) if self.W else None,
                                   dev(gen.block_major(lay["v"])) if self.W else None, self.W, dev(lay["gates"]),
                                   o, sinks=sk, q_scale=dev(lay["q_scale"]), kv_scale=kvs,
                                   swa_scale=dev(lay["swa_scale"]))
                self.outs.append(o)
        torch.cuda.synchronize()


def f64_inputs(inp, b=0):
    """The oracle's float64 values of the stored fp8 codes (code * scale)."""
    q = ora.dequantize_e4m3(inp.q[b], inp.q_scale, head_axis=1)
    k = ora.dequantize_e4m3(inp.k[b], inp.kv_scale[0], head_axis=0)
    v = ora.dequantize_e4m3(inp.v[b], inp.kv_scale[1], head_axis=0)
    layers = []
    for lay in inp.layers:
        layers.append(dict(q=ora.dequantize_e4m3(lay["q"][b], lay["q_scale"], head_axis=1),
                           k=ora.dequantize_e4m3(lay["k"][b], lay["swa_scale"][0], head_axis=0),
                           v=ora.dequantize_e4m3(lay["v"][b], lay["swa_scale"][1], head_axis=0),
                           gates=lay["gates"][b].astype(np.float64)))
    return q, k, v, layers


def check_f8(run, pos, score="max", include_diag=False, b=0):
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    q64, k64, v64, lays = f64_inputs(run.inp, b)
    pos = np.asarray(pos)

    def one(p):
        ref = ora.hybrid_block_rows(q64, k64, v64, [], p, run.kb, run.W, include_diag=include_diag, score=score)
        dpos = torch.from_numpy(p.astype(np.int64)).cuda()
        e = {"o": np.abs(host(run.o[b][dpos]) - ref["o"]).max(),
             "lse": np.abs(host(run.lse[b][:, dpos]) - ref["lse"]).max()}
        nb = ref["raw"].shape[-1]
        raw = host(run.raw[b][:, dpos])[..., :nb]
        valid = ~np.isnan(ref["raw"])
        e["raw"] = np.abs(raw[valid] - ref["raw"][valid]).max()
        gs = host(run.gs[b][:, dpos])[..., :nb]
        vg = ~np.isnan(ref["Sg"])
        e["gs"] = np.abs(gs[vg] - ref["Sg"][vg]).max() / np.abs(ref["Sg"][vg]).max()
        gidx = host(run.idx[b][:, dpos])
        n, ties, fails = compare_indices(gidx, ref, p, run.kb, include_diag)
        assert not fails, fails[:3]
        e["ties"] = ties
        for l, o in enumerate(run.outs):
            lay = lays[l]
            sk = None if run.sinks[l] is None else run.sinks[l].astype(np.float64)
            want = ora.sparse_layer_rows(lay["q"][p], p, k64, v64, gidx, lay["k"], lay["v"], run.W,
                                         lay["gates"][p], sinks=sk)
            e[f"l{l}"] = np.abs(host(o[b][dpos]) - want).max()
        return e

    chunks = [c for c in np.array_split(pos, max(1, min(32, len(pos) // 16))) if len(c)]
    with threadpool_limits(limits=1), ThreadPoolExecutor(min(16, len(chunks))) as ex:
        res = list(ex.map(one, chunks))
    err = {key: max(r[key] for r in res) for key in res[0] if key != "ties"}
    say("  " + " ".join(f"{k}={v:.3g}" for k, v in err.items()) + f" near-tie={sum(r['ties'] for r in res)}")
    assert err["o"] <= TOL["fp8"]
    assert err["lse"] <= SIDE_TOL and err["raw"] <= SIDE_TOL and err["gs"] < 1e-4
    for key in err:
        if key.startswith("l"):
            assert err[key] <= TOL["fp8"], key


SMALL = [
    # T, Hq, Hkv, kb, W
    (1, 4, 1, 2, 16),
    (200, 8, 2, 2, 7),
    (333, 8, 2, 4, 100),
    (130, 16, 1, 3, 200),
    (257, 2, 2, 2, 64),
    (640, 4, 1, 8, 128),
    (2113, 8, 2, 4, 300),
]


@pytest.mark.parametrize("T,Hq,Hkv,kb,W", SMALL)
def test_f8_small_shapes_all_rows(T, Hq, Hkv, kb, W):
    say(f"[fp8 small] T={T} Hq={Hq} Hkv={Hkv} kb={kb} W={W}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=128, dtype="fp8", kb=kb, W=W, N=2)
    run = RunF8(gen.make_prefill(cfg))
    check_f8(run, np.arange(T))


@pytest.mark.parametrize("score", ["max", "lse"])
@pytest.mark.parametrize("include_diag", [False, True])
def test_f8_score_modes(score, include_diag):
    say(f"[fp8 modes] score={score} include_diag={include_diag}")
    cfg = gen.config(1, T=300, Hq=8, Hkv=2, d=128, dtype="fp8", kb=3, W=50, N=1)
    run = RunF8(gen.make_prefill(cfg), score=hb.HS_SCORE_LSE if score == "lse" else hb.HS_SCORE_MAX,
                include_diag=include_diag, sparse=False)
    check_f8(run, np.arange(300), score=score, include_diag=include_diag)


def test_f8_config2_shape_sampled():
    say("[fp8 7B-shaped] T=8192 Hq=32 Hkv=8 d=128 fp8, sampled rows")
    cfg = gen.config(2, dtype="fp8")
    run = RunF8(gen.make_prefill(cfg, n_layers=2))
    check_f8(run, sample_rows(8192, every=101))


def test_f8_config3_shape_sampled():
    """The 32K-token 1:11 shape in fp8: all rows of the first and last four
    blocks and every 61st row, sparse layers 0-1 of 11."""
    say("[fp8 32K-token] T=32768 Hq=32 Hkv=4 d=128 fp8, sampled rows")
    cfg = gen.config(3, dtype="fp8")
    run = RunF8(gen.make_prefill(cfg, n_layers=2))
    check_f8(run, sample_rows(32768, every=61, head=256, tail=256))


@pytest.mark.parametrize("T,Hq,Hkv,W", [(333, 8, 2, 100), (257, 4, 4, 0), (300, 16, 1, 64)])
def test_f8_sinks(T, Hq, Hkv, W):
    say(f"[fp8 sinks] T={T} Hq={Hq} Hkv={Hkv} W={W}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=128, dtype="fp8", kb=3, W=W, N=1)
    run = RunF8(gen.make_prefill(cfg), sinks=True)
    check_f8(run, np.arange(T))
