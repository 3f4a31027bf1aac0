"""Benchmark of the hybrid-block prefill hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 2] [--no-cpu]
                    [--decode [4] [5]]

One step = one whole hybrid block over one batch of synthetic input: the full
causal GQA layer with block scores, the top-k selection, then the N sparse
layers (block-sparse branch over the shared K/V + sliding window + gates), all
through the C ABI on the current torch stream.  Inputs are resident in HBM
before the timed region starts.  Prints one JSON line.

Workload (default, --config 2): the 7B-shaped 1:3 hybrid block, B=1, T=8192,
Hq=32, Hkv=8, d=128, bf16, top-16 blocks of 64, window 512, 3 sparse layers.

Algorithmic work (counted, never the work actually issued): 4*d FLOP per
(query head, key) pair, over the causal pairs of the full layer plus, per
sparse layer and query, min(kb, floor(t/64))*64 selected keys and
min(t+1, W) window keys.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0  # TFLOP/s, MI355X dense bf16 MFMA
PEAK_F32 = 157.3    # TFLOP/s, MI355X fp32 matrix
PEAK_HBM = 8000.0   # GB/s
METRIC = "hybrid-block prefill tokens/s + % MFMA peak; sparse decode GB/s + % HBM peak"


def full_flops(cfg) -> float:
    T = cfg.T
    return 4.0 * cfg.d * cfg.Hq * cfg.B * T * (T + 1) / 2


def sparse_flops_per_layer(cfg, kb=None, W=None) -> float:
    kb = cfg.kb if kb is None else kb
    W = cfg.W if W is None else W
    t = np.arange(cfg.T, dtype=np.float64)
    keys = np.minimum(kb, np.floor(t / 64)) * 64 + np.minimum(t + 1, W)
    return 4.0 * cfg.d * cfg.Hq * cfg.B * keys.sum()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_sparse_attention_causal_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/sparse_prefill_7b_hbm_traffic.txt: FETCH_SIZE and WRITE_SIZE per
    dispatch, scaled by a plain-copy calibration), if it was taken on the
    current kernel sources and the same workload; else None."""
    path = os.path.join(ROOT, "profiles", "sparse_prefill_7b_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    ent = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, _, val = line.partition(":")
            ent[key.strip()] = val.strip()
    if ent.get("kernel") != kernel or ent.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(ent["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, budget_s: float = 12.0):
    """Time the fp64 oracle (as it stands, one BLAS thread) on a bounded sample of
    query rows of the same workload and scale it by the algorithmic work."""
    from threadpoolctl import threadpool_limits

    from oracle import hs_oracle as ora

    cfg = inp.cfg
    T = cfg.T
    rng = np.random.default_rng(12345)
    order = rng.permutation(T)
    f = lambda n, l=None: inp.f64(n, l)[0]
    q, k, v = f("q"), f("k"), f("v")
    layers = [dict(q=f("q", l), k=f("k", l), v=f("v", l), gates=f("gates", l))
              for l in range(len(inp.layers))]

    def row_work(t):
        sel = min(cfg.kb, t // 64) * 64 + min(t + 1, cfg.W)
        return 4.0 * cfg.d * cfg.Hq * ((t + 1) + len(layers) * sel)

    total = sum(row_work(t) for t in range(T))
    done_w, n_rows = 0.0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for i in range(0, T, 8):
            rows = np.sort(order[i:i + 8])
            ora.hybrid_block_rows(q, k, v, layers, rows, cfg.kb, cfg.W)
            done_w += sum(row_work(int(t)) for t in rows)
            n_rows += len(rows)
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
    block_s = el * total / done_w
    return {"value": cfg.B * T / block_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_rows} random query rows of {T} (all heads, full layer, selection and "
                      f"{len(layers)} sparse layers) in {el:.1f} s, scaled by algorithmic FLOPs "
                      f"({done_w / total * 100:.2f}% of the block)"}


def decode_bytes(inp) -> float:
    """Algorithmic HBM bytes of one decode step: the full layer reads every
    cached key and value once; each sparse layer reads its selected blocks (or
    tokens) of the shared cache and its own window ring; plus queries, outputs,
    gates and indices.  Score intermediates and workspace are not counted."""
    cfg = inp.cfg
    e = 1 if cfg.dtype == "fp8" else 2
    L = inp.lens.astype(np.float64)
    d, Hq, Hkv, N = cfg.d, cfg.Hq, cfg.Hkv, cfg.N
    full = (L.sum() * Hkv * d * 2 * e) + cfg.B * Hq * d * 2 * 2
    if cfg.kind == "decode_token":
        ncand = np.maximum(0, L - cfg.n_recent)
        nsel = np.minimum(cfg.kb, ncand) + np.minimum(cfg.n_recent, L)
        per_layer = (nsel.sum() * Hkv * d * 2 * e + cfg.B * Hq * d * 2 * 2
                     + cfg.B * Hkv * (cfg.kb + cfg.n_recent) * 4)
    else:
        nsel = np.minimum(cfg.kb, np.floor((L - 1) / 64))
        ring = np.minimum(L, cfg.W)
        per_layer = ((nsel.sum() * 64 + ring.sum()) * Hkv * d * 2 * e + cfg.B * Hq * d * 2 * 2
                     + cfg.B * Hq * 2 * 4 + cfg.B * Hkv * cfg.kb * 4)
    return float(full + N * per_layer)


def bench_decode(cid: int, steps: int, sinks: bool = False):
    """Time full decode steps of the 1:11 decode workload (block or token mode)
    on a cold cache; returns a dict for the JSON line."""
    import torch

    from hybrid_sparse_attention_causal_amd import binding as hb
    from hybrid_sparse_attention_causal_amd import inputs as gen

    cfg = gen.config(cid)
    inp = gen.make_decode(cfg)
    B, Hq, Hkv, C, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d
    token = cfg.kind == "decode_token"

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if token:
        kc = np.empty((B, Hkv, C, d), np.uint8)
        vc = np.empty((B, Hkv, C, d), np.uint8)
        gen.fill_decode_cache(inp, kc, vc, v_block_major=False)
    else:
        kc = np.empty((B, Hkv, C, d), np.uint16)
        vc = np.empty((B, Hkv, C // 64, d, 64), np.uint16)
        gen.fill_decode_cache(inp, kc, vc)
    k, v = dev(kc), dev(vc)
    del kc, vc
    scale = dev(inp.kv_scale) if token else None
    lens = torch.from_numpy(inp.lens.astype(np.int32)).cuda()
    q = dev(inp.q)
    blk = 1 if token else 64
    nsel = cfg.kb + cfg.n_recent if token else cfg.kb
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    raw = torch.empty((B, Hq, C // blk), device="cuda")
    idx = torch.empty((B, Hkv, nsel), dtype=torch.int32, device="cuda")
    shape = hb.decode_shape(q, k, lens, scale)
    ws_full = torch.empty(max(16, hb.workspace_size(hb.HS_FN_FULL_ATTN, shape, blk)),
                          dtype=torch.uint8, device="cuda")
    layers = []
    for li, lay in enumerate(inp.layers):
        ent = dict(q=dev(lay["q"]), o=torch.empty_like(o),
                   s=dev(gen.make_sinks(cfg, li)) if sinks else None)
        if not token:
            ent.update(kr=dev(lay["k_ring"]), vr=dev(gen.block_major(lay["v_ring"])),
                       g=dev(lay["gates"]))
        layers.append(ent)
    stream = torch.cuda.current_stream()
    nsel_ws = hb.workspace_size(hb.HS_FN_DECODE_SELECT, shape, blk)
    ws_sel = torch.empty(max(16, nsel_ws), dtype=torch.uint8, device="cuda")

    def step():
        hb.decode_full_attn_scores(q, k, v, lens, o, lse, raw, block=blk, ws=ws_full,
                                   kv_scale=scale, stream=stream)
        hb.decode_block_topk(q, k, lens, raw, lse, cfg.kb, idx, block=blk, n_recent=cfg.n_recent,
                             kv_scale=scale, stream=stream)
        for l in layers:
            if token:
                hb.decode_select_attn(l["q"], k, v, lens, idx, nsel, None, None, 0, None, l["o"],
                                      block=1, kv_scale=scale, stream=stream, ws=ws_sel, sinks=l["s"])
            else:
                hb.decode_select_attn(l["q"], k, v, lens, idx, nsel, l["kr"], l["vr"], cfg.W, l["g"],
                                      l["o"], stream=stream, sinks=l["s"])

    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        scrub.fill_(1)  # evicts L2 and the MALL; outside the timed events
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    warm0, warm1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm0.record(stream)
    for _ in range(steps):
        step()
    warm1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median(times))
    nbytes = decode_bytes(inp)
    return {"workload": {4: "1:11 hybrid block decode, 64 seqs, L~U[32768,65536], top-32 blocks, W=128",
                         5: "token-level decode, 16 seqs x 262144, fp8 KV, top-2048 + 128 recent"}[cid],
            "ms_per_step_cold": ms, "ms_per_step_warm": warm0.elapsed_time(warm1) / steps,
            "algorithmic_bytes": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM, "sinks": bool(sinks)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first; the GPU clock takes some 30 ms of load to settle")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode", type=int, nargs="*", default=[4], choices=[4, 5],
                    help="decode workloads also measured (default: 4); pass none to skip")
    ap.add_argument("--sinks", action="store_true",
                    help="give every sparse layer per-head sink logits (not part of the workloads)")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_ref:
        import torch

        n = args.copy_ref << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_ref_bytes": n, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: "
              "the library has no multi-GPU path (prefill would shard by kv group with no "
              "exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    from hybrid_sparse_attention_causal_amd import binding as hb
    from hybrid_sparse_attention_causal_amd import inputs as gen

    hb.load()
    cfg = gen.config(args.config)
    inp = gen.make_prefill(cfg)
    B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt = hb.HS_BF16 if cfg.dtype == "bf16" else hb.HS_F32
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    layers = [dict(q=dev(l["q"]), k=dev(l["k"]), v=dev(gen.block_major(l["v"])),
                   g=dev(l["gates"]), o=torch.empty((B, T, Hq, d), dtype=tdt, device="cuda"),
                   s=dev(gen.make_sinks(cfg, i)) if args.sinks else None)
              for i, l in enumerate(inp.layers)]
    o = torch.empty((B, T, Hq, d), dtype=tdt, device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    raw = torch.empty((B, Hq, T, cfg.nblk), device="cuda")
    idx = torch.empty((B, Hkv, T, cfg.kb), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    names = ["full_attn", "block_topk"] + [f"sparse_{i}" for i in range(len(layers))]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        hb.full_attn_fwd_scores(q, k, vb, o, lse, raw, stream=stream)
        mark(1)
        hb.block_topk((B, T, Hq, Hkv, d, dt), raw, lse, cfg.kb, idx, stream=stream)
        mark(2)
        for i, l in enumerate(layers):
            hb.sparse_attn_fwd(l["q"], k, vb, idx, cfg.kb, l["k"], l["v"], cfg.W, l["g"], l["o"],
                               stream=stream, sinks=l["s"])
            mark(3 + i)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}

    ff = full_flops(cfg)
    fs = sparse_flops_per_layer(cfg)
    total_flops = ff + len(layers) * fs
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_F32
    sparse_ms = float(np.mean([per[n] for n in names[2:]]))
    # dominant kernel by time per step
    if per["full_attn"] >= sparse_ms * len(layers):
        dom, dom_ms, dom_flops, dom_kernel = "full_attn", per["full_attn"], ff, "full_prefill_kernel"
    else:
        dom, dom_ms, dom_flops, dom_kernel = "sparse_layer", sparse_ms, fs, "sparse_prefill_kernel"
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(dom_kernel) if cfg.cid == 2 else None
    out = {
        "metric": METRIC,
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator, planted salient keys)",
        "config": {"workload": {2: "7B-shaped 1:3 hybrid block prefill",
                                3: "80B-MoE-shaped 1:11 hybrid block prefill",
                                1: "tiny 1:3 hybrid block prefill"}[cfg.cid],
                   "batch": B, "seq_len": T, "hq": Hq, "hkv": Hkv, "head_dim": d,
                   "block": 64, "topk_blocks": cfg.kb, "window": cfg.W,
                   "sparse_layers": len(layers), "sinks": bool(args.sinks),
                   "parallelism": "single GPU"},
        "block_tflops": total_flops / (ms_step * 1e-3) / 1e12,
        "block_mfma_frac": total_flops / (ms_step * 1e-3) / 1e12 / peak,
        "kernel_ms": per,
        "roofline": {"kernel": dom_kernel, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic},
    }
    if args.decode:
        del layers, q, k, vb, o, lse, raw, idx
        torch.cuda.empty_cache()
        out["decode"] = [bench_decode(c, max(3, min(args.steps, 10)), args.sinks) for c in args.decode]
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
