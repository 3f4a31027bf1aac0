"""GPU parity of the KV-offload path (paper section 5, "Potential of HySparse
for Efficient KV Cache Offloading"): the gather of the selected blocks
against the oracle's K~, V~, and the pipelined decode step over a host-held
full-layer cache (prefetch + full layer + selection + gather) against the
device-resident calls, bit for bit; the sparse layers then run on the compact
cache of the selected blocks and must equal the resident sparse layers."""
import sys

import numpy as np
import pytest
import torch

from hybrid_sparse_attention_causal_amd import binding as hb
from hybrid_sparse_attention_causal_amd import inputs as gen
from oracle import hs_oracle as ora
from parity import TOL, dev, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64_bf16(a):
    return gen.bf16_bits_to_f32(a).astype(np.float64)


def _pinned_caches(inp):
    """Block-mode caches written straight into pinned host memory (NaN past L)."""
    cfg = inp.cfg
    B, Hkv, C, d = cfg.B, cfg.Hkv, cfg.T, cfg.d
    kt = torch.empty((B, Hkv, C, d), dtype=torch.int16, pin_memory=True)
    vt = torch.empty((B, Hkv, C // 64, d, 64), dtype=torch.int16, pin_memory=True)
    gen.fill_decode_cache(inp, kt.numpy().view(np.uint16), vt.numpy().view(np.uint16))
    return kt.view(torch.bfloat16), vt.view(torch.bfloat16)


def test_gather_matches_oracle():
    """Messy index rows (shuffled, repeats, -1, the diagonal block, ids past
    the sequence or the cache): the compact cache holds the fully-past live
    blocks in ascending order, idx_sel numbers them, later slots are left
    alone."""
    say("[gather] B=3 C=2048 Hkv=2 d=128")
    cfg = gen.config(4, B=3, T=2048, Hq=4, Hkv=2, d=128, kb=12, W=0, N=0, L_lo=1, L_hi=2048)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([100, 1000, 2048], np.int32)
    kt, vt = _pinned_caches(inp)
    k, v = kt.cuda(), vt.cuda()
    lens = torch.from_numpy(inp.lens).cuda()
    rng = np.random.default_rng(9)
    n = cfg.kb
    idx = np.full((cfg.B, cfg.Hkv, n), -1, np.int32)
    for b in range(cfg.B):
        L = int(inp.lens[b])
        last = (L - 1) // 64                      # the diagonal block
        for g in range(cfg.Hkv):
            live = rng.choice(max(last, 1), size=min(last, 5), replace=False) if last else []
            row = list(live) + list(live[:2]) + [-1, last, 10 ** 6, 2048 // 64]
            row += [-1] * (n - len(row))
            idx[b, g] = rng.permutation(np.array(row[:n], np.int32))
    sentinel = 0x3F80  # bf16 1.0
    k_sel = torch.full((cfg.B, cfg.Hkv, n * 64, cfg.d), sentinel, dtype=torch.int16, device="cuda")
    v_sel = torch.full((cfg.B, cfg.Hkv, n, cfg.d, 64), sentinel, dtype=torch.int16, device="cuda")
    idx_sel = torch.full((cfg.B, cfg.Hkv, n), -7, dtype=torch.int32, device="cuda")
    hb.gather_blocks(k, v, lens, dev(idx), n, k_sel.view(torch.bfloat16), v_sel.view(torch.bfloat16), idx_sel)
    torch.cuda.synchronize()
    ks, vs, isel = (host(k_sel.view(torch.bfloat16)), host(v_sel.view(torch.bfloat16)), host(idx_sel))
    for b in range(cfg.B):
        L = int(inp.lens[b])
        kk, vv = zip(*(inp.kv_slab_f64(b, g) for g in range(cfg.Hkv)))
        want_k, want_v, want_i = ora.gather_blocks(np.stack(kk), np.stack(vv), idx[b].astype(np.int64), L)
        for g in range(cfg.Hkv):
            nl = int((want_i[g] >= 0).sum())
            assert np.array_equal(isel[b, g], want_i[g]), (b, g)
            assert np.array_equal(ks[b, g, : 64 * nl], want_k[g, : 64 * nl]), (b, g)
            vb = gen.block_major(want_v[g, : 64 * nl]) if nl else np.zeros((0, cfg.d, 64))
            assert np.array_equal(vs[b, g, :nl], vb), (b, g)
            assert np.all(ks[b, g, 64 * nl:] == 1.0) and np.all(vs[b, g, nl:] == 1.0), (b, g)


class OffloadRun:
    """The same decode step twice: device-resident caches, and host-held
    caches through the offload pipeline + sparse layers on the compact cache."""

    def __init__(self, inp, chunk, n_layers):
        cfg = inp.cfg
        B, Hq, Hkv, C, d, kb = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d, cfg.kb
        kt, vt = _pinned_caches(inp)
        k, v = kt.cuda(), vt.cuda()
        lens_h = torch.from_numpy(inp.lens.astype(np.int32))
        lens = lens_h.cuda()
        q = dev(inp.q)

        def outs():
            return (torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda"),
                    torch.full((B, Hq), float("nan"), device="cuda"),
                    torch.full((B, Hq, C // 64), float("nan"), device="cuda"),
                    torch.full((B, Hkv, kb), -7, dtype=torch.int32, device="cuda"))

        self.res = outs()
        o, lse, raw, idx = self.res
        hb.decode_full_attn_scores(q, k, v, lens, o, lse, raw)
        hb.decode_block_topk(q, k, lens, raw, lse, kb, idx)
        self.off = outs()
        o2, lse2, raw2, idx2 = self.off
        self.k_sel = torch.empty((B, Hkv, kb * 64, d), dtype=torch.bfloat16, device="cuda")
        self.v_sel = torch.empty((B, Hkv, kb, d, 64), dtype=torch.bfloat16, device="cuda")
        self.idx_sel = torch.empty((B, Hkv, kb), dtype=torch.int32, device="cuda")
        ws = torch.empty(hb.offload_workspace_size(q, kt, lens, chunk), dtype=torch.uint8, device="cuda")
        copy_stream = torch.cuda.Stream()
        hb.offload_full_select(q, kt, vt, lens, lens_h, o2, lse2, raw2, kb, idx2, self.k_sel, self.v_sel,
                               self.idx_sel, chunk, ws, copy_stream=copy_stream)
        self.lay_res, self.lay_off = [], []
        for lay in inp.layers[:n_layers]:
            qs, kr, vr, gt = dev(lay["q"]), dev(lay["k_ring"]), dev(gen.block_major(lay["v_ring"])), dev(lay["gates"])
            a = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
            hb.decode_select_attn(qs, k, v, lens, idx, kb, kr, vr, cfg.W, gt, a)
            b2 = torch.full_like(a, float("nan"))
            hb.decode_select_attn(qs, self.k_sel, self.v_sel, lens, self.idx_sel, kb, kr, vr, cfg.W, gt, b2)
            self.lay_res.append(a)
            self.lay_off.append(b2)
        torch.cuda.synchronize()
        self.cfg, self.inp = cfg, inp

    def check(self, oracle_seqs=()):
        for name, x, y in zip(("o", "lse", "raw", "idx"), self.res, self.off):
            assert torch.equal(torch.nan_to_num(x.float(), 7.0), torch.nan_to_num(y.float(), 7.0)), name
        for l, (x, y) in enumerate(zip(self.lay_res, self.lay_off)):
            assert not torch.isnan(y).any() and torch.equal(x, y), l
        cfg, inp = self.cfg, self.inp
        idx = host(self.off[3])
        isel = host(self.idx_sel)
        for b in range(cfg.B):
            L = int(inp.lens[b])
            nl = (idx[b] >= 0).sum(axis=1)
            for g in range(cfg.Hkv):
                assert np.array_equal(isel[b, g], np.where(np.arange(cfg.kb) < nl[g], np.arange(cfg.kb), -1))
        o, lay = host(self.off[0]), [host(x) for x in self.lay_off]
        for b in oracle_seqs:
            L = int(inp.lens[b])
            kk, vv = zip(*(inp.kv_slab_f64(b, g) for g in range(cfg.Hkv)))
            k64, v64 = np.stack(kk), np.stack(vv)
            ref = ora.decode_step(f64_bf16(inp.q[b]), k64, v64, L, [], cfg.kb, cfg.W)
            assert np.abs(o[b] - ref["o"]).max() <= TOL["bf16"]
            ks, vs, _ = ora.gather_blocks(k64, v64, idx[b].astype(np.int64), L)
            ksel = host(self.k_sel[b])
            for g in range(cfg.Hkv):
                n = int((idx[b, g] >= 0).sum())
                assert np.array_equal(ksel[g, : 64 * n], ks[g, : 64 * n]), (b, g)
            src = inp.layers[0]
            want = ora.decode_sparse_layer(dict(q=f64_bf16(src["q"][b]), k_ring=f64_bf16(src["k_ring"][b]),
                                                v_ring=f64_bf16(src["v_ring"][b]),
                                                gates=src["gates"][b].astype(np.float64)),
                                           k64, v64, L, idx[b].astype(np.int64), cfg.W)
            assert np.abs(lay[0][b] - want).max() <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [1, 2, 7])
def test_offload_small_ragged(chunk):
    say(f"[offload] B=7 C=4096 Hq=8 Hkv=2 kb=5 W=100 chunk={chunk}")
    cfg = gen.config(4, B=7, T=4096, Hq=8, Hkv=2, d=128, kb=5, W=100, N=2, L_lo=1, L_hi=4096)
    inp = gen.make_decode(cfg)
    inp.lens = np.array([1, 63, 64, 65, 130, 4000, 4096], np.int32)
    run = OffloadRun(inp, chunk, n_layers=2)
    run.check(oracle_seqs=[3, 5, 6])


def test_offload_config4_full_size():
    say("[offload config 4] 64 seqs, capacity 65536, chunks of 8 sequences, layers 0-1 of 11")
    inp = gen.make_decode(gen.config(4), n_layers=2)
    run = OffloadRun(inp, 8, n_layers=2)
    run.check(oracle_seqs=[0, 63])


def test_offload_concurrent_host_threads():
    """Two host threads run the offload pipeline at the same time, each on its
    own compute and copy streams with its own workspace and outputs: the
    library enqueues each call under a lock (its events are shared per
    device), and every result equals the device-resident step bit for bit."""
    import threading

    say("[offload, two host threads] B=7 C=4096 Hq=8 Hkv=2 kb=5 chunk=2, 4 calls each")
    cfg = gen.config(4, B=7, T=4096, Hq=8, Hkv=2, d=128, kb=5, W=100, N=0, L_lo=1, L_hi=4096)
    inp = gen.make_decode(cfg, n_layers=0)
    inp.lens = np.array([1, 63, 64, 65, 130, 4000, 4096], np.int32)
    B, Hq, Hkv, C, d, kb = cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d, cfg.kb
    kt, vt = _pinned_caches(inp)
    k, v = kt.cuda(), vt.cuda()
    lens_h = torch.from_numpy(inp.lens.astype(np.int32))
    lens = lens_h.cuda()
    q = dev(inp.q)

    def outs():
        return (torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda"),
                torch.full((B, Hq), float("nan"), device="cuda"),
                torch.full((B, Hq, C // 64), float("nan"), device="cuda"),
                torch.full((B, Hkv, kb), -7, dtype=torch.int32, device="cuda"))

    want = outs()
    hb.decode_full_attn_scores(q, k, v, lens, *want[:3])
    hb.decode_block_topk(q, k, lens, want[2], want[1], kb, want[3])
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            s, cs = torch.cuda.Stream(), torch.cuda.Stream()
            got = outs()
            k_sel = torch.empty((B, Hkv, kb * 64, d), dtype=torch.bfloat16, device="cuda")
            v_sel = torch.empty((B, Hkv, kb, d, 64), dtype=torch.bfloat16, device="cuda")
            idx_sel = torch.empty((B, Hkv, kb), dtype=torch.int32, device="cuda")
            ws = torch.empty(hb.offload_workspace_size(q, kt, lens, 2), dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            for _ in range(4):
                hb.offload_full_select(q, kt, vt, lens, lens_h, *got[:3], kb, got[3], k_sel, v_sel, idx_sel, 2, ws,
                                       stream=s, copy_stream=cs)
            s.synchronize()
            results[i] = got
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for i in range(2):
        for name, x, y in zip(("o", "lse", "raw", "idx"), want, results[i]):
            assert torch.equal(torch.nan_to_num(x.float(), 7.0), torch.nan_to_num(y.float(), 7.0)), (i, name)
