"""GPU parity of the prefill path (full layer + scores, selection, sparse
layers) against the fp64 oracle, called through the C ABI.

Small shapes are compared on every row; the full-size 7B-shaped (T=8192) and
80B-shaped (T=32768) workloads on sampled rows.  Sparse-layer outputs are
compared with the oracle evaluated on the GPU's own indices (a legal near-tie
swap cannot fail an output check) and the indices themselves under the
near-tie rule."""
import math
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


class Run:
    """One prefill hybrid block on the GPU, with its buffers."""

    def __init__(self, inp, score=hb.HS_SCORE_MAX, include_diag=False, kb=None, W=None,
                 gates=True, sinks=False):
        cfg = inp.cfg
        self.cfg, self.inp = cfg, inp
        B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d
        self.kb = cfg.kb if kb is None else kb
        self.W = cfg.W if W is None else W
        nblk = cfg.nblk
        tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        q, k = dev(inp.q, cfg.dtype), dev(inp.k, cfg.dtype)
        vb = dev(gen.block_major(inp.v), cfg.dtype)
        self.o = torch.full((B, T, Hq, d), float("nan"), dtype=tdt, device="cuda")
        self.lse = torch.full((B, Hq, T), float("nan"), device="cuda")
        self.raw = torch.full((B, Hq, T, nblk), float("nan"), device="cuda")
        hb.full_attn_fwd_scores(q, k, vb, self.o, self.lse, self.raw, score=score)
        self.idx = torch.full((B, Hkv, T, self.kb), -7, dtype=torch.int32, device="cuda")
        self.gs = torch.full((B, Hkv, T, nblk), float("nan"), device="cuda")
        dt = hb.HS_F32 if cfg.dtype == "f32" else hb.HS_BF16
        hb.block_topk((B, T, Hq, Hkv, d, dt), self.raw, self.lse, self.kb, self.idx, self.gs,
                      include_diag=include_diag)
        self.outs = []
        self.sinks = [gen.make_sinks(cfg, l) if sinks else None for l in range(len(inp.layers))]
        for l, lay in enumerate(inp.layers):
            qs, ks = dev(lay["q"], cfg.dtype), dev(lay["k"], cfg.dtype)
            vsb = dev(gen.block_major(lay["v"]), cfg.dtype)
            g = dev(lay["gates"]) if gates else None
            o = torch.full((B, T, Hq, d), float("nan"), dtype=tdt, device="cuda")
            sk = None if self.sinks[l] is None else dev(self.sinks[l])
            hb.sparse_attn_fwd(qs, k, vb, self.idx, self.kb, ks if self.W else None,
                               vsb if self.W else None, self.W, g, o, sinks=sk)
            self.outs.append(o)
        torch.cuda.synchronize()


def _f64_inputs(inp, gates=True, b=0):
    """float64 copies of one sequence's stored inputs (made once per check)."""
    layers = [dict(q=inp.f64("q", l)[b], k=inp.f64("k", l)[b], v=inp.f64("v", l)[b],
                   gates=inp.f64("gates", l)[b] if gates else None)
              for l in range(len(inp.layers))]
    return inp.f64("q")[b], inp.f64("k")[b], inp.f64("v")[b], layers


def oracle_rows(inp, pos, kb, W, score="max", include_diag=False, gates=True, b=0):
    q, k, v, layers = _f64_inputs(inp, gates, b)
    return ora.hybrid_block_rows(q, k, v, layers, pos, kb, W, include_diag=include_diag, score=score)


def _check_chunk(run, x64, pos, score, include_diag, layers, b):
    """Errors of the rows `pos` against the oracle; asserts the index rule."""
    cfg = run.cfg
    q64, k64, v64, lays = x64
    ref = ora.hybrid_block_rows(q64, k64, v64, [], pos, run.kb, run.W, include_diag=include_diag,
                                score=score)
    dpos = torch.from_numpy(np.asarray(pos, np.int64)).cuda()  # rows picked on the device
    e = {}
    e["o"] = np.abs(host(run.o[b][dpos]) - ref["o"]).max()
    e["lse"] = np.abs(host(run.lse[b][:, dpos]) - ref["lse"]).max()
    nb = ref["raw"].shape[-1]  # blocks up to the chunk's last row
    raw = host(run.raw[b][:, dpos])[..., :nb]
    valid = ~np.isnan(ref["raw"])
    e["raw"] = np.abs(raw[valid] - ref["raw"][valid]).max()
    gs = host(run.gs[b][:, dpos])[..., :nb]
    vg = ~np.isnan(ref["Sg"])
    e["gs"] = np.abs(gs[vg] - ref["Sg"][vg]).max() / np.abs(ref["Sg"][vg]).max()
    gidx = host(run.idx[b][:, dpos])
    n, ties, fails = compare_indices(gidx, ref, pos, run.kb, include_diag)
    assert not fails, fails[:5]
    e["rows"], e["ties"] = n, ties
    for l in range(len(run.inp.layers)) if layers is None else layers:
        lay = lays[l]
        gl = None if lay["gates"] is None else lay["gates"][pos]
        sk = None if run.sinks[l] is None else run.sinks[l].astype(np.float64)
        want = ora.sparse_layer_rows(lay["q"][pos], pos, k64, v64, gidx, lay["k"], lay["v"], run.W, gl,
                                     sinks=sk)
        e[f"l{l}"] = np.abs(host(run.outs[l][b][dpos]) - want).max()
    return e


def check_run(run, pos, score="max", include_diag=False, gates=True, layers=None, b=0):
    """Compare the rows `pos` of sequence b with the oracle.  Large row sets
    are split into chunks checked on a thread pool (numpy releases the GIL in
    its matrix products); the oracle is row-local, so chunks are independent."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    cfg = run.cfg
    tol = TOL[cfg.dtype]
    x64 = _f64_inputs(run.inp, gates, b)
    pos = np.asarray(pos)
    nch = max(1, min(32, len(pos) // 16))
    chunks = [c for c in np.array_split(pos, nch) if len(c)]
    with threadpool_limits(limits=1), ThreadPoolExecutor(min(16, len(chunks))) as ex:
        res = list(ex.map(lambda c: _check_chunk(run, x64, c, score, include_diag, layers, b), chunks))
    err = {key: max(r[key] for r in res) for key in res[0] if key not in ("rows", "ties")}
    say(f"  full layer: max|dO|={err['o']:.3g} max|dLSE|={err['lse']:.3g} max|draw|={err['raw']:.3g}")
    say(f"  selection: rows={sum(r['rows'] for r in res)} near-tie={sum(r['ties'] for r in res)} "
        f"rel|dSg|={err['gs']:.3g}")
    assert err["o"] <= tol and err["lse"] <= SIDE_TOL and err["raw"] <= SIDE_TOL
    assert err["gs"] < 1e-4
    for key in sorted(k for k in err if k.startswith("l")):
        say(f"  sparse layer {key[1:]}: max|dO|={err[key]:.3g}")
        assert err[key] <= tol


SMALL = [
    # T, Hq, Hkv, d, dtype, kb, W
    (1, 4, 1, 64, "f32", 4, 128),
    (63, 8, 2, 64, "bf16", 2, 16),
    (65, 4, 4, 128, "f32", 1, 1),
    (200, 8, 1, 128, "bf16", 2, 7),
    (130, 16, 2, 64, "bf16", 3, 200),
    (257, 2, 2, 64, "f32", 2, 64),
    (333, 32, 4, 128, "bf16", 4, 100),
    (640, 4, 1, 64, "f32", 8, 128),
    # more than one run of staged block scores, ragged last run (34 blocks:
    # rows not 16-byte aligned; 35 blocks with head_dim 64: runs of 16)
    (2113, 8, 2, 128, "bf16", 4, 300),
    (2200, 4, 1, 64, "bf16", 3, 100),
    # 331 selection rows (8*41 + 3): the top-k kernel's last work group has a
    # wave with one row of its two and two waves with none
    (331, 4, 1, 64, "bf16", 3, 64),
]


@pytest.mark.parametrize("T,Hq,Hkv,d,dtype,kb,W", SMALL)
def test_small_shapes_all_rows(T, Hq, Hkv, d, dtype, kb, W):
    say(f"[small] T={T} Hq={Hq} Hkv={Hkv} d={d} {dtype} kb={kb} W={W}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, kb=kb, W=W, N=2)
    inp = gen.make_prefill(cfg)
    run = Run(inp)
    check_run(run, np.arange(T))


@pytest.mark.parametrize("T,Hq,Hkv,d,dtype,kb,W", [
    (333, 8, 2, 128, "bf16", 4, 100),   # two groups per CU
    (257, 4, 2, 64, "f32", 2, 64),
    (200, 8, 2, 128, "f32", 2, 50),     # fp32 head_dim 128: 8-wave one-column-tile kernel
])
def test_sinks_all_rows(T, Hq, Hkv, d, dtype, kb, W):
    """Per-head sink logits in both branches (paper 4.1)."""
    say(f"[sinks] T={T} Hq={Hq} Hkv={Hkv} d={d} {dtype} kb={kb} W={W}")
    cfg = gen.config(1, T=T, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, kb=kb, W=W, N=2)
    run = Run(gen.make_prefill(cfg), sinks=True)
    check_run(run, np.arange(T))


def test_large_logits():
    """Queries scaled by 24 (fp32 inputs): logits reach the hundreds and the
    running maximum jumps by far more than the rescale slack between tiles;
    every row of the full layer, the selection and the sparse layers (with
    sinks) must still match."""
    say("[large logits] T=400 Hq=4 Hkv=2 d=64 fp32, q x 24")
    cfg = gen.config(1, T=400, Hq=4, Hkv=2, d=64, dtype="f32", kb=3, W=70, N=1)
    inp = gen.make_prefill(cfg)
    inp.q = (inp.q * 24.0).astype(np.float32)
    inp.layers[0]["q"] = (inp.layers[0]["q"] * 24.0).astype(np.float32)
    run = Run(inp, sinks=True)
    check_run(run, np.arange(cfg.T))


def test_window_shares_full_kv():
    """Ablation of the paper's study 2: the window branch reads the full layer's
    own K/V instead of a K'/V' of its own (no new kernel: the shared tensors go
    in as the window cache)."""
    say("[window shares the full layer's K/V]")
    cfg = gen.config(1, T=300, Hq=8, Hkv=2, d=128, dtype="bf16", kb=3, W=90, N=1)
    inp = gen.make_prefill(cfg)
    inp.layers[0]["k"] = inp.k
    inp.layers[0]["v"] = inp.v
    check_run(Run(inp), np.arange(cfg.T))


@pytest.mark.parametrize("score", ["max", "lse"])
@pytest.mark.parametrize("include_diag", [False, True])
@pytest.mark.parametrize("Hq,Hkv,d,dtype", [
    (8, 2, 64, "f32"),
    (8, 2, 128, "bf16"),      # the default bf16 full-layer kernel (groups of <= 16 heads)
    (32, 1, 128, "bf16"),     # a group of 32 heads: the four-wave full-layer kernel
])
def test_score_modes_and_candidates(score, include_diag, Hq, Hkv, d, dtype):
    say(f"[modes] score={score} include_diag={include_diag} Hq={Hq} Hkv={Hkv} d={d} {dtype}")
    cfg = gen.config(1, T=300, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, kb=3, W=50, N=1 if Hq // Hkv <= 16 else 0)
    inp = gen.make_prefill(cfg, n_layers=cfg.N)
    run = Run(inp, score=hb.HS_SCORE_LSE if score == "lse" else hb.HS_SCORE_MAX,
              include_diag=include_diag)
    check_run(run, np.arange(300), score=score, include_diag=include_diag)


def test_ungated_and_no_window():
    say("[variants] gates=None, W=0")
    cfg = gen.config(1, T=260, Hq=4, Hkv=1, d=128, dtype="bf16", kb=2, W=0, N=1)
    inp = gen.make_prefill(cfg)
    run = Run(inp, gates=False)
    check_run(run, np.arange(260), gates=False)


def test_dense_reduction_on_gpu():
    """Every block selected (diagonal included), no window, no gate: each sparse
    layer equals dense causal attention of its own queries over the shared K/V."""
    say("[dense reduction]")
    T = 256
    cfg = gen.config(1, T=T, Hq=4, Hkv=2, d=64, dtype="f32", kb=4, W=0, N=1)
    inp = gen.make_prefill(cfg)
    run = Run(inp, include_diag=True, gates=False)
    assert np.array_equal(host(run.idx)[0][:, 255], np.tile(np.arange(4), (2, 1)))
    qs = inp.f64("q", 0)[0]
    o, _, _ = ora.full_attention_rows(qs, np.arange(T), inp.f64("k")[0], inp.f64("v")[0])
    got = host(run.outs[0])[0]
    # rows t < 192 have fewer than 4 candidate blocks, so all of theirs are selected too
    assert np.abs(got - o).max() < 1e-4


def _golden_inputs(T):
    """The hand-worked examples padded to d=64: q = 8 e (tau*q.k = k component)."""
    d = 64
    q = np.zeros((1, T, 2, d), np.float32)
    q[0, :, 0, 0] = 8.0
    q[0, :, 1, 1] = 8.0
    k = np.zeros((1, 1, T, d), np.float32)
    k[0, 0, 5, 0] = math.log(3.0)
    k[0, 0, :64, 1] = math.log(2.0)
    k[0, 0, 100, 1] = k[0, 0, 101, 1] = math.log(4.0)
    v = np.zeros((1, 1, T, d), np.float32)
    v[0, 0, 5, 0] = 1.0
    v[0, 0, 100, 1] = v[0, 0, 101, 1] = 1.0
    return q, k, v


def test_hand_worked_examples_on_gpu():
    from test_oracle_pins import _read_golden

    say("[golden E1/E2]")
    g1 = _read_golden("e1_two_blocks.txt")
    q, k, v = _golden_inputs(128)
    cfg = gen.config(1, T=128, Hq=2, Hkv=1, d=64, kb=1, W=0, N=0)
    inp = gen.PrefillInputs(cfg, q, k, v, [], [])
    run = Run(inp, include_diag=True)
    S = np.exp(host(run.raw)[0][:, 127] - host(run.lse)[0][:, 127:128])
    assert np.abs(S[0] - g1["S_A"]).max() < 1e-6 and np.abs(S[1] - g1["S_B"]).max() < 1e-6
    assert np.abs(host(run.gs)[0][0, 127, :2] - g1["S_g"]).max() < 1e-6
    assert host(run.idx)[0][0, 127, 0] == 0
    o = host(run.o)[0][127]
    assert np.abs(o[0, :2] - g1["o_A"]).max() < 1e-6 and np.abs(o[1, :2] - g1["o_B"]).max() < 1e-6
    run = Run(inp, score=hb.HS_SCORE_LSE, include_diag=True)
    assert np.abs(host(run.gs)[0][0, 127, :2] - g1["S_g_lse_mode"]).max() < 1e-6

    g2 = _read_golden("e2_three_blocks_gated.txt")
    T = 192
    q, k, v = _golden_inputs(T)
    vs = np.zeros((1, 1, T, 64), np.float32)
    vs[0, 0, :, 0] = np.arange(T)
    vs[0, 0, :, 1] = -np.arange(T)
    gates = np.zeros((1, T, 2, 2), np.float32)
    gates[..., 1] = math.log(3.0)
    lay = dict(q=q, k=np.zeros((1, 1, T, 64), np.float32), v=vs, gates=gates)
    cfg = gen.config(1, T=T, Hq=2, Hkv=1, d=64, kb=1, W=2, N=1)
    inp = gen.PrefillInputs(cfg, q, k, v, [lay], [])
    run = Run(inp)
    assert np.abs(host(run.gs)[0][0, 191, :2] - g2["S_g"]).max() < 1e-6
    assert host(run.idx)[0][0, 191, 0] == 0
    o = host(run.outs[0])[0][191]
    # fp32 inputs: every term of the example is exact in fp32
    assert np.abs(o[0, :2] - g2["o_A"]).max() < 1e-4
    assert np.abs(o[1, :2] - g2["o_B"]).max() < 1e-4


def test_config1_tiny_block_all_rows():
    say("[config 1] T=1024 Hq=4 Hkv=1 d=64 fp32, 3 sparse layers")
    inp = gen.make_prefill(gen.config(1))
    run = Run(inp)
    check_run(run, np.arange(1024))


def test_config2_7b_shaped_sampled():
    say("[config 2] T=8192 Hq=32 Hkv=8 d=128 bf16, 3 sparse layers, sampled rows")
    inp = gen.make_prefill(gen.config(2))
    run = Run(inp)
    pos = sample_rows(8192, every=101)
    check_run(run, pos)


def test_config3_80b_shaped_sampled():
    """All rows of the first and last four blocks and every 61st row."""
    say("[config 3] T=32768 Hq=32 Hkv=4 d=128 bf16, sampled rows, layers 0-1 of 11")
    inp = gen.make_prefill(gen.config(3), n_layers=2)
    run = Run(inp)
    pos = sample_rows(32768, every=61, head=256, tail=256)
    check_run(run, pos)


def test_longest_sequence_group4():
    """T = 239616, the longest sequence the sparse layer takes with four heads
    per kv group (its selection bitsets fill the 48 KiB allowed): every
    kernel at its largest shape, sampled rows."""
    say("[longest] T=239616 Hq=4 Hkv=1 d=64 bf16, sampled rows")
    cfg = gen.config(1, T=239616, Hq=4, Hkv=1, d=64, dtype="bf16", kb=8, W=64, N=1)
    inp = gen.make_prefill(cfg)
    run = Run(inp, sinks=True)
    pos = sample_rows(239616, every=4999, head=8, tail=8)
    check_run(run, pos)


@pytest.mark.parametrize("sinks", [False, True])
def test_long_sequence_wide_bitsets(sinks):
    """T = 53312 with one head per kv group: the selection bitsets of a
    four-wave group would pass 16 KiB of LDS, so the sparse layer takes the
    8-wave kernel with three tile buffers."""
    say(f"[long] T=53312 Hq=2 Hkv=2 d=64 bf16, sampled rows, sinks={sinks}")
    cfg = gen.config(1, T=53312, Hq=2, Hkv=2, d=64, dtype="bf16", kb=8, W=64, N=1)
    inp = gen.make_prefill(cfg)
    run = Run(inp, sinks=sinks)
    pos = sample_rows(53312, every=997, head=64, tail=64)
    check_run(run, pos)


def test_repeat_runs_are_bitwise_identical():
    say("[determinism]")
    inp = gen.make_prefill(gen.config(1, T=500, Hq=8, Hkv=2, d=128, dtype="bf16", N=1))
    a, b = Run(inp), Run(inp)
    for x, y in ((a.o, b.o), (a.raw, b.raw), (a.idx, b.idx), (a.outs[0], b.outs[0])):
        assert torch.equal(torch.nan_to_num(x.float(), 123.0), torch.nan_to_num(y.float(), 123.0))


def test_batch2_group16_both_sequences():
    """Two sequences, 16 query heads per kv head (the widest group of the
    sparse layers): every row of both sequences."""
    say("[batch 2, G=16] T=200 Hq=16 Hkv=1 d=64 bf16")
    cfg = gen.config(1, B=2, T=200, Hq=16, Hkv=1, d=64, dtype="bf16", kb=2, W=40, N=2)
    inp = gen.make_prefill(cfg)
    run = Run(inp)
    for b in range(2):
        check_run(run, np.arange(cfg.T), b=b)


def test_group32_full_layer_and_selection():
    """G = 32 (full layer and selection only; the sparse layers take G <= 16)."""
    say("[G=32] T=150 Hq=32 Hkv=1 d=128 bf16, full layer + top-k")
    cfg = gen.config(1, T=150, Hq=32, Hkv=1, d=128, dtype="bf16", kb=1, W=0, N=0)
    inp = gen.make_prefill(cfg, n_layers=0)
    run = Run(inp)
    check_run(run, np.arange(cfg.T))
