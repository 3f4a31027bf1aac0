"""Benchmark of the hybrid-block attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 30] [--config 3] [--extra 2]
                    [--decode [4] [5]] [--no-cpu] [--sinks]

One step = one whole hybrid block over one batch of synthetic input: the full
causal GQA layer with block scores, the top-k selection, then the N sparse
layers (block-sparse branch over the shared K/V + sliding window + gates), all
through the C ABI on the current torch stream.  Inputs are resident in HBM
before the timed region starts.  Prints one JSON line.

Workload (default, --config 3): the 80B-MoE-shaped 1:11 hybrid block, B=1,
T=32768, Hq=32, Hkv=4, d=128, bf16, top-32 blocks of 64, window 128, 11
sparse layers.  --extra 2 also times the 7B-shaped 1:3 block (T=8192) and
reports it under "prefill_extra"; --decode 4 5 times one decode step of the
64-sequence block-mode workload and of the 16 x 262144 fp8 token-level
workload under "decode".

Progress lines go to stderr, one per finished part; stdout carries only the
JSON line.  The CPU oracle baseline runs first, in a child process of its own
(cpu_baseline_isolated), before this process touches the GPU.

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
PEAK_FP8 = 5000.0   # TFLOP/s, MI355X dense fp8 MFMA
PEAK_F32 = 157.3    # TFLOP/s, MI355X fp32 matrix
PEAK_HBM = 8000.0   # GB/s
METRIC = "hybrid-block prefill tokens/s + % MFMA peak; sparse decode GB/s + % HBM peak"


_T0 = time.perf_counter()


def progress(msg: str) -> None:
    """One line per finished part on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.perf_counter() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def full_flops(cfg) -> float:
    T = cfg.T
    return 4.0 * cfg.d * cfg.Hq * cfg.B * T * (T + 1) / 2


def sparse_flops_per_layer(cfg, kb=None, W=None) -> float:
    kb = cfg.kb if kb is None else kb
    W = cfg.W if W is None else W
    t = np.arange(cfg.T, dtype=np.float64)
    keys = np.minimum(kb, np.floor(t / 64)) * 64 + np.minimum(t + 1, W)
    return 4.0 * cfg.d * cfg.Hq * cfg.B * keys.sum()


# the sources the prefill kernels are built from (their argument structs are
# declared next to the kernels' other interfaces, which change more often)
PREFILL_SOURCES = ("hs_prefill.hip", "hs_device.h")
TRAFFIC_FILES = {2: "sparse_prefill_7b_hbm_traffic.txt", 3: "sparse_prefill_32k_hbm_traffic.txt"}


def kernel_source_hash(names=PREFILL_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_sparse_attention_causal_amd", "csrc")
    for n in sorted(names):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def sparse_kernel_name(cfg) -> str:
    """The kernel hs_sparse_attn_fwd launches for this shape (the library's
    dispatch: two four-wave work groups per CU while their selection bitsets
    fit 16 KiB of LDS, else the eight-wave ping-pong kernel; fp32 with
    head_dim 128 takes the one-column-tile kernel)."""
    if cfg.dtype == "fp8":
        return "sparse_prefill_f8_kernel"
    if cfg.dtype == "f32" and cfg.d == 128:
        return "sparse_prefill_kernel"
    pwg = 4 * (32 // cfg.G)
    nw32 = (cfg.nblk + 31) // 32
    lds = ((1 + 4 + pwg) * nw32 + cfg.nblk + 1) * 4
    return "sparse_prefill_dual_kernel" if lds <= 16 * 1024 else "sparse_prefill_pp_kernel"


def full_kernel_name(cfg) -> str:
    """The kernel hs_full_attn_fwd_scores launches in prefill."""
    if cfg.dtype == "fp8":
        return "full_prefill_f8_kernel"
    if cfg.G <= 16 and not (cfg.dtype == "f32" and cfg.d == 128):
        return "full_prefill_pp_kernel"
    return "full_prefill_kernel"


def measured_traffic(cid: int, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    workload `cid` (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a
    plain-copy calibration), if it was taken on the current prefill kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILES.get(cid, "-"))
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


_POOL_DATA = {}


def _oracle_rows_worker(rows):
    """One process-pool task: the oracle's whole hybrid block at `rows`.  The
    stored inputs come from the parent (forked); float64 copies are made only
    of the rows this task reads (np.zeros pages never written cost no memory)."""
    from threadpoolctl import threadpool_limits

    from hybrid_sparse_attention_causal_amd import inputs as gen
    from oracle import hs_oracle as ora

    inp, k64, v64 = _POOL_DATA["inp"], _POOL_DATA["k"], _POOL_DATA["v"]
    cfg = inp.cfg
    conv = lambda a: gen.to_f32(a, cfg.dtype).astype(np.float64)  # noqa: E731
    rows = np.asarray(rows)
    win = np.unique(np.concatenate([np.arange(max(0, t - cfg.W + 1), t + 1) for t in rows]))
    with threadpool_limits(limits=1):
        q = np.zeros((cfg.T, cfg.Hq, cfg.d))
        q[rows] = conv(inp.q[0][rows])
        layers = []
        for lay in inp.layers:
            ent = dict(q=np.zeros((cfg.T, cfg.Hq, cfg.d)), k=np.zeros((cfg.Hkv, cfg.T, cfg.d)),
                       v=np.zeros((cfg.Hkv, cfg.T, cfg.d)), gates=np.zeros((cfg.T, cfg.Hq, 2)))
            ent["q"][rows] = conv(lay["q"][0][rows])
            ent["gates"][rows] = lay["gates"][0][rows]
            ent["k"][:, win] = conv(lay["k"][0][:, win])
            ent["v"][:, win] = conv(lay["v"][0][:, win])
            layers.append(ent)
        ora.hybrid_block_rows(q, k64, v64, layers, rows, cfg.kb, cfg.W)
    return len(rows)


def host_cores() -> int:
    """Cores the baseline may use: this process's affinity set, capped at the
    16-core CPU share of one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(inp, budget_s: float = 12.0):
    """Time the fp64 oracle (as it stands) on a bounded random sample of query
    rows of the same workload, on a process pool over the host cores (one BLAS
    thread per process), and scale the wall time by the algorithmic work.
    Call it in a process that has not touched the GPU: the pool is forked."""
    import multiprocessing as mp

    from hybrid_sparse_attention_causal_amd import inputs as gen

    cfg = inp.cfg
    T = cfg.T
    nl = len(inp.layers)
    order = np.random.default_rng(12345).permutation(T)
    chunks = [np.sort(order[i:i + 8]) for i in range(0, T, 8)]

    def row_work(t):
        sel = min(cfg.kb, t // 64) * 64 + min(t + 1, cfg.W)
        return 4.0 * cfg.d * cfg.Hq * ((t + 1) + nl * sel)

    total = sum(row_work(t) for t in range(T))
    cores = host_cores()
    conv = lambda a: gen.to_f32(a, cfg.dtype).astype(np.float64)  # noqa: E731
    _POOL_DATA.update(inp=inp, k=conv(inp.k[0]), v=conv(inp.v[0]))
    done_w, n_rows = 0.0, 0
    stalled = False
    with mp.get_context("fork").Pool(cores) as pool:
        t0 = time.perf_counter()
        it = pool.imap(_oracle_rows_worker, chunks, chunksize=1)
        for i in range(len(chunks)):
            try:
                # a worker that does not finish a few rows in this long is
                # stuck (a forked process can inherit a held lock): the
                # baseline then stops with what was done, not the benchmark
                n = it.next(timeout=budget_s + 60.0)
            except mp.TimeoutError:
                stalled = True
                break
            done_w += sum(row_work(int(t)) for t in chunks[i])
            n_rows += n
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
        pool.terminate()
    _POOL_DATA.clear()
    if done_w == 0.0:
        return None
    block_s = el * total / done_w
    return {"value": cfg.B * T / block_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_rows} random query rows of {T} (all heads, full layer, selection and "
                      f"{nl} sparse layers) in {el:.1f} s wall on a pool of {cores} processes, "
                      f"scaled by algorithmic FLOPs ({done_w / total * 100:.2f}% of the block)"
                      + (", stopped early: a worker stalled" if stalled else "")}


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
    ws_tsel = None
    if token:
        ws_tsel = torch.empty(max(16, hb.workspace_size(hb.HS_FN_DECODE_TOKEN_SELECT, shape, 1, cfg.kb)),
                              dtype=torch.uint8, device="cuda")

    def step(two_call=False):
        if token and not two_call:
            # full layer + token selection in one call (bounds, exact rescoring)
            hb.decode_token_select(q, k, v, lens, o, lse, cfg.kb, cfg.n_recent, idx, scale, ws=ws_tsel,
                                   stream=stream)
        else:
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
        if token:
            step(True)
    torch.cuda.synchronize()

    def cold(two_call=False):
        times = []
        for _ in range(steps):
            scrub.fill_(1)  # evicts L2 and the MALL; outside the timed events
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(two_call)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    ms = cold()
    ms_two = cold(True) if token else None
    warm0, warm1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm0.record(stream)
    for _ in range(steps):
        step()
    warm1.record(stream)
    torch.cuda.synchronize()
    nbytes = decode_bytes(inp)
    res = {"workload": {4: "1:11 hybrid block decode, 64 seqs, L~U[32768,65536], top-32 blocks, W=128",
                        5: "token-level decode, 16 seqs x 262144, fp8 KV, top-2048 + 128 recent"}[cid],
           "ms_per_step_cold": ms, "ms_per_step_warm": warm0.elapsed_time(warm1) / steps,
           "algorithmic_bytes": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM, "sinks": bool(sinks)}
    if token:
        # the step through hs_decode_token_select; the two-call step (per-token
        # logits written and read back) for comparison
        res["selection"] = "hs_decode_token_select (bounds + exact rescoring)"
        res["ms_per_step_cold_two_call"] = ms_two
    return res


PEAK_PCIE = 64.0  # GB/s, PCIe 5.0 x16 host link, one direction


def bench_decode_offload(cid: int, steps: int, chunk: int = 8):
    """One decode step of the block-mode workload with the full layer's cache
    held in pinned host memory: the offload pipeline (chunked prefetch over
    PCIe overlapped with the full layer, selection and gather of the previous
    chunk) plus the N sparse layers on the compact cache of the selected
    blocks.  Also times a plain host-to-device copy of the same live bytes."""
    import torch

    from hybrid_sparse_attention_causal_amd import binding as hb
    from hybrid_sparse_attention_causal_amd import inputs as gen

    cfg = gen.config(cid)
    inp = gen.make_decode(cfg)
    B, Hq, Hkv, C, d, kb = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d, cfg.kb

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    kt = torch.empty((B, Hkv, C, d), dtype=torch.int16, pin_memory=True)
    vt = torch.empty((B, Hkv, C // 64, d, 64), dtype=torch.int16, pin_memory=True)
    gen.fill_decode_cache(inp, kt.numpy().view(np.uint16), vt.numpy().view(np.uint16))
    kt, vt = kt.view(torch.bfloat16), vt.view(torch.bfloat16)
    lens_h = torch.from_numpy(inp.lens.astype(np.int32))
    lens = lens_h.cuda()
    q = dev(inp.q)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    raw = torch.empty((B, Hq, C // 64), device="cuda")
    idx = torch.empty((B, Hkv, kb), dtype=torch.int32, device="cuda")
    k_sel = torch.empty((B, Hkv, kb * 64, d), dtype=torch.bfloat16, device="cuda")
    v_sel = torch.empty((B, Hkv, kb, d, 64), dtype=torch.bfloat16, device="cuda")
    idx_sel = torch.empty((B, Hkv, kb), dtype=torch.int32, device="cuda")
    ws = torch.empty(hb.offload_workspace_size(q, kt, lens, chunk), dtype=torch.uint8, device="cuda")
    layers = [dict(q=dev(l["q"]), kr=dev(l["k_ring"]), vr=dev(gen.block_major(l["v_ring"])), g=dev(l["gates"]),
                   o=torch.empty_like(o)) for l in inp.layers]
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()

    def step():
        hb.offload_full_select(q, kt, vt, lens, lens_h, o, lse, raw, kb, idx, k_sel, v_sel, idx_sel, chunk, ws,
                               stream=stream, copy_stream=copy_stream)
        for l in layers:
            hb.decode_select_attn(l["q"], k_sel, v_sel, lens, idx_sel, kb, l["kr"], l["vr"], cfg.W, l["g"], l["o"],
                                  stream=stream)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    L = inp.lens.astype(np.float64)
    live = float((L * d * 2 + np.ceil(L / 64) * 64 * d * 2).sum() * Hkv)  # live K rows + V blocks
    # a plain copy of the same number of bytes, pinned host -> device
    nbytes = int(live)
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    dst.copy_(src, non_blocking=True)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1)
    resident = (k_sel.numel() + v_sel.numel()) * 2 + idx_sel.numel() * 4
    return {"workload": "1:11 hybrid block decode, 64 seqs, L~U[32768,65536], top-32 blocks, W=128, "
                        "full-layer cache in pinned host memory",
            "chunk_seqs": chunk, "ms_per_step": ms, "pcie_bytes_per_step": live,
            "pcie_GB_per_s": live / (ms * 1e-3) / 1e9, "pcie_frac": live / (ms * 1e-3) / 1e9 / PEAK_PCIE,
            "plain_copy_GB_per_s": live / (copy_ms * 1e-3) / 1e9,
            "gpu_bytes_selected_blocks": resident, "gpu_bytes_staging": ws.numel(),
            "gpu_bytes_full_cache_if_resident": (kt.numel() + vt.numel()) * 2}


def bench_training(cid: int, steps: int, warmup: int):
    """One training step of a prefill hybrid block (bf16): the forward (full
    layer, selection, N sparse layers writing their branch outputs) and the
    backward (full layer, then every sparse layer adding its share into the
    shared dK/dV).  Algorithmic FLOPs: the forward's count, plus 2.5 times it
    for the backward (per attended pair: S, dP, dV, dK, dQ at 2d each)."""
    import torch

    from hybrid_sparse_attention_causal_amd import binding as hb
    from hybrid_sparse_attention_causal_amd import inputs as gen

    cfg = gen.config(cid)
    inp = gen.make_prefill(cfg)
    B, T, Hq, Hkv, d, kb, W = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d, cfg.kb, cfg.W

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    o = torch.empty((B, T, Hq, d), **bf)
    lse = torch.empty((B, Hq, T), **f32)
    raw = torch.empty((B, Hq, T, cfg.nblk), **f32)
    idx = torch.empty((B, Hkv, T, kb), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(77)
    mk_do = lambda: dev(gen.f32_to_bf16_bits(rng.standard_normal((B, T, Hq, d)).astype(np.float32)))
    do_full = mk_do()
    dq = torch.empty((B, T, Hq, d), **f32)
    dk = torch.empty((B, Hkv, T, d), **f32)
    dv = torch.empty((B, Hkv, T, d), **f32)
    layers = [dict(q=dev(l["q"]), k=dev(l["k"]), v=dev(gen.block_major(l["v"])), g=dev(l["gates"]),
                   o=torch.empty((B, T, Hq, d), **bf), ob=torch.empty((2, B, T, Hq, d), **bf),
                   lb=torch.empty((2, B, Hq, T), **f32), do=mk_do(), dq=torch.empty((B, T, Hq, d), **f32),
                   dks=torch.empty((B, Hkv, T, d), **f32), dvs=torch.empty((B, Hkv, T, d), **f32),
                   dg=torch.empty((B, T, Hq, 2), **f32)) for l in inp.layers]
    ws = [None]
    stream = torch.cuda.current_stream()
    names = ["fwd_full", "fwd_topk"] + [f"fwd_sparse_{i}" for i in range(len(layers))] + ["bwd_full"] + \
            [f"bwd_sparse_{i}" for i in range(len(layers))]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        hb.full_attn_fwd_scores(q, k, vb, o, lse, raw, stream=stream)
        mark(1)
        hb.block_topk((B, T, Hq, Hkv, d, hb.HS_BF16), raw, lse, kb, idx, stream=stream)
        mark(2)
        for i, l in enumerate(layers):
            hb.sparse_attn_fwd_train(l["q"], k, vb, idx, kb, l["k"], l["v"], W, l["g"], l["o"], l["ob"], l["lb"],
                                     stream=stream)
            mark(3 + i)
        n0 = 3 + len(layers)
        ws[0] = hb.full_attn_bwd(q, k, vb, o, lse, do_full, dq, dk, dv, ws=ws[0], stream=stream)
        mark(n0)
        for i, l in enumerate(layers):
            ws[0] = hb.sparse_attn_bwd(l["q"], k, vb, idx, kb, l["k"], l["v"], W, l["g"], None, l["ob"], l["lb"],
                                       l["do"], l["dq"], dk, dv, l["dks"], l["dvs"], l["dg"], None, ws=ws[0],
                                       stream=stream)
            mark(n0 + 1 + i)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for st in range(steps):
        step(evs[st])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    per = {n: float(np.mean([evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(steps)]))
           for i, n in enumerate(names)}
    fwd = full_flops(cfg) + len(layers) * sparse_flops_per_layer(cfg)
    total = 3.5 * fwd
    bwd_full_flops = 2.5 * full_flops(cfg)
    return {"workload": WORKLOAD_NAMES[cid] + ", training step (forward + backward)",
            "ms_per_step": ms_step, "tokens_per_s": B * T / (ms_step * 1e-3),
            "algorithmic_tflop": total / 1e12, "tflops": total / (ms_step * 1e-3) / 1e12,
            "mfma_frac": total / (ms_step * 1e-3) / 1e12 / PEAK_BF16,
            "bwd_full_tflops": bwd_full_flops / (per["bwd_full"] * 1e-3) / 1e12,
            "kernel_ms": per}


WORKLOAD_NAMES = {1: "tiny 1:3 hybrid block prefill", 2: "7B-shaped 1:3 hybrid block prefill",
                  3: "80B-MoE-shaped 1:11 hybrid block prefill"}


def bench_prefill(inp, steps: int, warmup: int, sinks: bool = False):
    """Time whole prefill hybrid blocks of `inp` (inputs resident in HBM);
    per-kernel HIP events on the launch stream inside the timed region."""
    import torch

    from hybrid_sparse_attention_causal_amd import binding as hb
    from hybrid_sparse_attention_causal_amd import inputs as gen

    cfg = inp.cfg
    B, T, Hq, Hkv, d = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    f8 = cfg.dtype == "fp8"
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    dt = {"bf16": hb.HS_BF16, "f32": hb.HS_F32, "fp8": hb.HS_FP8_E4M3}[cfg.dtype]
    q, k, vb = dev(inp.q), dev(inp.k), dev(gen.block_major(inp.v))
    qsc = dev(inp.q_scale) if f8 else None
    kvsc = dev(inp.kv_scale) if f8 else None
    layers = [dict(q=dev(l["q"]), k=dev(l["k"]), v=dev(gen.block_major(l["v"])),
                   g=dev(l["gates"]), o=torch.empty((B, T, Hq, d), dtype=tdt, device="cuda"),
                   s=dev(gen.make_sinks(cfg, i)) if sinks else None,
                   qs=dev(l["q_scale"]) if f8 else None, ss=dev(l["swa_scale"]) if f8 else None)
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
        hb.full_attn_fwd_scores(q, k, vb, o, lse, raw, stream=stream, q_scale=qsc, kv_scale=kvsc)
        mark(1)
        hb.block_topk((B, T, Hq, Hkv, d, dt), raw, lse, cfg.kb, idx, stream=stream)
        mark(2)
        for i, l in enumerate(layers):
            hb.sparse_attn_fwd(l["q"], k, vb, idx, cfg.kb, l["k"], l["v"], cfg.W, l["g"], l["o"],
                               stream=stream, sinks=l["s"], q_scale=l["qs"], kv_scale=kvsc, swa_scale=l["ss"])
            mark(3 + i)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(steps):
        step(evs[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    per = {n: float(np.mean([evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(steps)]))
           for i, n in enumerate(names)}
    del layers, q, k, vb, o, lse, raw, idx
    torch.cuda.empty_cache()

    ff = full_flops(cfg)
    fs = sparse_flops_per_layer(cfg)
    nl = len(inp.layers)
    total_flops = ff + nl * fs
    peak = {"bf16": PEAK_BF16, "f32": PEAK_F32, "fp8": PEAK_FP8}[cfg.dtype]
    sparse_ms = float(np.mean([per[n] for n in names[2:]])) if nl else 0.0
    # dominant kernel: the one taking most of the step
    if per["full_attn"] >= sparse_ms * nl:
        dom_ms, dom_flops, dom_kernel = per["full_attn"], ff, full_kernel_name(cfg)
    else:
        dom_ms, dom_flops, dom_kernel = sparse_ms, fs, sparse_kernel_name(cfg)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    return {
        "ms_per_step": ms_step,
        "tokens_per_s": B * T / (ms_step * 1e-3),
        "dtype": cfg.dtype,
        "config": {"workload": WORKLOAD_NAMES[cfg.cid] + (", fp8 e4m3 Q/K/V with per-head scales" if f8 else ""),
                   "batch": B, "seq_len": T, "hq": Hq, "hkv": Hkv, "head_dim": d,
                   "block": 64, "topk_blocks": cfg.kb, "window": cfg.W,
                   "sparse_layers": nl, "sinks": bool(sinks), "parallelism": "single GPU"},
        "block_tflops": total_flops / (ms_step * 1e-3) / 1e12,
        "block_mfma_frac": total_flops / (ms_step * 1e-3) / 1e12 / peak,
        "mfma_peak_tflops": peak,
        "kernel_ms": per,
        "roofline": {"kernel": dom_kernel, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(cfg.cid, dom_kernel),
                     "work_per_launch": dom_flops, "avg_launch_ms": dom_ms},
    }


def cpu_baseline_isolated(cid: int, timeout_s: float = 180.0):
    """cpu_baseline of workload `cid` in a child process of its own session
    (it builds its own inputs and forks its own pool), so that a stuck pool
    can neither hang nor outlive the benchmark: past `timeout_s` the whole
    process group is killed and the baseline is reported as missing."""
    import signal
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", str(cid)]
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                            start_new_session=True)
    try:
        out, err = proc.communicate(timeout=timeout_s)
    except subprocess.TimeoutExpired:
        os.killpg(proc.pid, signal.SIGKILL)
        proc.communicate()
        progress(f"CPU oracle baseline: no result within {timeout_s:.0f} s, process group killed")
        return None
    lines = [l for l in out.splitlines() if l.startswith("{")]
    if proc.returncode != 0 or not lines:
        progress(f"CPU oracle baseline failed (exit {proc.returncode}): {err.strip()[-300:]}")
        return None
    return json.loads(lines[-1])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first; the GPU clock takes some 30 ms of load to settle")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3])
    ap.add_argument("--extra", type=int, nargs="*", default=[2], choices=[1, 2, 3],
                    help="prefill workloads also timed and reported under prefill_extra")
    ap.add_argument("--fp8", type=int, nargs="*", default=[3], choices=[2, 3],
                    help="prefill workloads also timed with fp8 e4m3 Q/K/V (fp8 matrix products)")
    ap.add_argument("--train", type=int, nargs="*", default=[2], choices=[1, 2, 3],
                    help="prefill workloads also timed as a training step (forward + backward)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode", type=int, nargs="*", default=[4, 5], choices=[4, 5],
                    help="decode workloads also measured (default: 4 5); pass none to skip")
    ap.add_argument("--offload", type=int, nargs="*", default=[4], choices=[4],
                    help="decode workloads also timed with the full-layer cache in host memory")
    ap.add_argument("--sinks", action="store_true",
                    help="give every sparse layer per-head sink logits (not part of the workloads)")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--cpu-baseline-only", type=int, default=0, metavar="CONFIG",
                    help=argparse.SUPPRESS)  # the child process of cpu_baseline_isolated
    args = ap.parse_args()
    if args.cpu_baseline_only:
        from hybrid_sparse_attention_causal_amd import inputs as gen

        print(json.dumps(cpu_baseline(gen.make_prefill(gen.config(args.cpu_baseline_only)))), flush=True)
        return
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

    from hybrid_sparse_attention_causal_amd import inputs as gen

    # the oracle baseline runs first, in a child process, so that the GPU
    # work does not share the host cores with it
    cpu = None if args.no_cpu else cpu_baseline_isolated(args.config)
    if cpu is not None:
        progress("CPU oracle baseline done")
    progress(f"prefill workload {args.config}: preparing inputs")
    inp = gen.make_prefill(gen.config(args.config))
    progress(f"inputs of workload {args.config} ready")

    from hybrid_sparse_attention_causal_amd import binding as hb

    hb.load()
    res = bench_prefill(inp, args.steps, args.warmup, args.sinks)
    progress(f"prefill workload {args.config}: {res['ms_per_step']:.3f} ms per block")
    del inp
    cfg = gen.config(args.config)
    out = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator, planted salient keys)",
        "config": res["config"],
        "block_tflops": res["block_tflops"],
        "block_mfma_frac": res["block_mfma_frac"],
        "kernel_ms": res["kernel_ms"],
        "roofline": res["roofline"],
    }
    extra = [c for c in args.extra if c != args.config]
    if extra:
        out["prefill_extra"] = []
        for c in extra:
            progress(f"prefill workload {c}: preparing inputs")
            r = bench_prefill(gen.make_prefill(gen.config(c)), args.steps, args.warmup, args.sinks)
            out["prefill_extra"].append(r)
            progress(f"prefill workload {c}: {r['ms_per_step']:.3f} ms per block")
    if args.fp8:
        out["prefill_fp8"] = []
        for c in args.fp8:
            progress(f"fp8 prefill workload {c}: preparing inputs")
            out["prefill_fp8"].append(bench_prefill(gen.make_prefill(gen.config(c, dtype="fp8")), args.steps,
                                                    args.warmup, args.sinks))
            progress(f"fp8 prefill workload {c} done")
    if args.train:
        out["training"] = []
        for c in args.train:
            progress(f"training step of workload {c}: preparing inputs")
            out["training"].append(bench_training(c, max(3, min(args.steps, 10)), 3))
            progress(f"training step of workload {c} done")
    if args.decode:
        out["decode"] = []
        for c in args.decode:
            progress(f"decode workload {c}: preparing inputs")
            out["decode"].append(bench_decode(c, max(3, min(args.steps, 10)), args.sinks))
            progress(f"decode workload {c} done")
    if args.offload:
        out["decode_offload"] = []
        for c in args.offload:
            progress(f"offloaded decode workload {c}: preparing inputs")
            out["decode_offload"].append(bench_decode_offload(c, 3))
            progress(f"offloaded decode workload {c} done")
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
