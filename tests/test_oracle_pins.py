"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

* hand-worked examples E1/E2 (tests/golden/, exact rationals from the pages'
  equations),
* library routines: torch's scaled_dot_product_attention in float64 (dense
  causal and banded attention), scipy's expit/logsumexp, torch's float8_e4m3fn
  and bfloat16 conversions,
* closed forms (a single salient key), invariants (probability rows sum to 1,
  the top block score equals exp(max logit - LSE), block masses sum to 1),
* brute force over a materialised attention matrix for T <= 256.

Each pin is also run against deliberately broken copies of oracle functions
(the mutations at the end): a pin set is only useful if a plausible mistake
fails it.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import hs_oracle as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            vals[key] = [float(sum(Fraction(p) for p in tok.split("+"))) for tok in rhs.split()]
    return vals


def _e_inputs(T):
    s2 = math.sqrt(2.0)
    q = np.zeros((T, 2, 2))
    q[:, 0, 0] = s2
    q[:, 1, 1] = s2
    k = np.zeros((1, T, 2))
    k[0, 5, 0] = math.log(3.0)
    k[0, :64, 1] = math.log(2.0)
    k[0, 100, 1] = k[0, 101, 1] = math.log(4.0)
    v = np.zeros((1, T, 2))
    v[0, 5] = (1.0, 0.0)
    v[0, 100] = v[0, 101] = (0.0, 1.0)
    return q, k, v


# ------------------------------------------------------------------ pins
def pin_e1(o):
    g = _read_golden("e1_two_blocks.txt")
    q, k, v = _e_inputs(128)
    pos = np.array([127])
    lay = dict(q=q, k=np.zeros_like(k), v=np.zeros_like(v), gates=None)
    r = o.hybrid_block_rows(q, k, v, [lay], pos, kb=1, W=0, include_diag=True)
    errs = []
    errs.append(abs(np.exp(r["lse"][0, 0]) - g["Z_A"][0]))
    errs.append(abs(np.exp(r["lse"][1, 0]) - g["Z_B"][0]))
    S = o.block_scores(r["raw"], r["lse"])
    errs += list(np.abs(S[0, 0] - g["S_A"]))
    errs += list(np.abs(S[1, 0] - g["S_B"]))
    errs += list(np.abs(r["Sg"][0, 0] - g["S_g"]))
    errs += list(np.abs(r["o"][0, 0] - g["o_A"]))
    errs += list(np.abs(r["o"][0, 1] - g["o_B"]))
    # the only sparse layer's window is empty (W=0) and it is ungated
    errs += list(np.abs(r["layer_out"][0][0, 0] - g["sparse_o_A"]))
    errs += list(np.abs(r["layer_out"][0][0, 1] - g["sparse_o_B"]))
    ok = max(errs) < 1e-12 and list(r["idx"][0, 0]) == [int(g["idx"][0])]
    # block log-sum-exp scores
    _, lse2, raw2 = o.full_attention_rows(q[pos], pos, k, v, score="lse")
    Sg2 = o.group_max(o.block_scores(raw2, lse2), 1)
    ok = ok and np.max(np.abs(Sg2[0, 0] - g["S_g_lse_mode"])) < 1e-12
    return ok


def pin_e2(o):
    g = _read_golden("e2_three_blocks_gated.txt")
    T = 192
    q, k, v = _e_inputs(T)
    pos = np.array([191])
    vs = np.zeros((1, T, 2))
    vs[0, :, 0] = np.arange(T)
    vs[0, :, 1] = -np.arange(T)
    gates = np.zeros((T, 2, 2))
    gates[..., 1] = math.log(3.0)
    lay = dict(q=q, k=np.zeros((1, T, 2)), v=vs, gates=gates)
    r = o.hybrid_block_rows(q, k, v, [lay], pos, kb=1, W=2, include_diag=False)
    errs = [abs(np.exp(r["lse"][0, 0]) - g["Z_A"][0]), abs(np.exp(r["lse"][1, 0]) - g["Z_B"][0])]
    errs += list(np.abs(r["Sg"][0, 0, :2] - g["S_g"]))
    ow = o.window_branch_rows(q[pos], pos, lay["k"], vs, 2)
    errs += list(np.abs(ow[0, 0] - g["window_o"]))
    osp = o.sparse_branch_rows(q[pos], pos, k, v, r["idx"])
    errs += list(np.abs(osp[0, 0] - g["sparse_o_A"]))
    errs += list(np.abs(osp[0, 1] - g["sparse_o_B"]))
    errs += list(np.abs(r["layer_out"][0][0, 0] - g["o_A"]))
    errs += list(np.abs(r["layer_out"][0][0, 1] - g["o_B"]))
    return max(errs) < 1e-11 and list(r["idx"][0, 0]) == [int(g["idx"][0])]


def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in float64: q [T,Hq,d], k/v [Hkv,T,d] -> [T,Hq,d]."""
    Hq, Hkv = q.shape[1], k.shape[0]
    G = Hq // Hkv
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = torch.from_numpy(k).repeat_interleave(G, 0)[None]
    V = torch.from_numpy(v).repeat_interleave(G, 0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal)
    return out[0].permute(1, 0, 2).numpy()


def _rand(T=200, Hq=4, Hkv=2, d=16, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, Hq, d)), r.standard_normal((Hkv, T, d)),
            r.standard_normal((Hkv, T, d)))


def pin_dense_reduction(o):
    """Check (a): full layer == dense causal attention, and the sparse branch
    with every block selected (diagonal included), no window and no gate == the
    same dense attention."""
    q, k, v = _rand()
    T = q.shape[0]
    pos = np.arange(T)
    ref = _sdpa(q, k, v, causal=True)
    of, _, _ = o.full_attention_rows(q, pos, k, v)
    nblk = (T + 63) // 64
    idx = np.broadcast_to(np.arange(nblk), (k.shape[0], T, nblk)).copy()
    lay = dict(q=q, k=k, v=v, gates=None)
    osp = o.sparse_layer_rows(q, pos, k, v, idx, k, v, 0, None)
    return max(np.abs(of - ref).max(), np.abs(osp - ref).max()) < 1e-12 and lay is not None


def pin_window(o):
    """Window branch == banded SDPA (keys t-W+1..t), and == causal SDPA for W >= T."""
    q, k, v = _rand(T=150, seed=1)
    T = q.shape[0]
    pos = np.arange(T)
    ok = True
    for W in (1, 7, 64, 100):
        i = np.arange(T)
        band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
        ref = _sdpa(q, k, v, mask=band)
        ok = ok and np.abs(o.window_branch_rows(q, pos, k, v, W) - ref).max() < 1e-12
    ref = _sdpa(q, k, v, causal=True)
    ok = ok and np.abs(o.window_branch_rows(q, pos, k, v, T + 5) - ref).max() < 1e-12
    ok = ok and np.abs(o.window_branch_rows(q, pos, k, v, 0)).max() == 0.0
    return ok


def pin_sinks(o):
    """Sink biases (reading R14) against the gpt-oss form built from torch's
    float64 SDPA: one extra key with zero key and value vectors whose logit
    is the sink, added through SDPA's additive mask; both branches (the
    sparse one with every block selected), a -inf sink changing nothing, an
    empty selection staying 0, and with all logits 0 and equal values
    o = n v / (n + e^b)."""
    q, k, v = _rand(T=90, seed=7)
    T, Hq, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    pos = np.arange(T)
    sink = np.random.default_rng(3).normal(1.0, 1.5, size=Hq)
    i = np.arange(T)

    def sdpa_sink(allowed):
        Q = torch.from_numpy(q).permute(1, 0, 2)[None]
        K = torch.from_numpy(np.concatenate([k, np.zeros((Hkv, 1, d))], 1)).repeat_interleave(G, 0)[None]
        V = torch.from_numpy(np.concatenate([v, np.zeros((Hkv, 1, d))], 1)).repeat_interleave(G, 0)[None]
        bias = np.broadcast_to(np.where(allowed, 0.0, -np.inf), (Hq, T, T))
        col = np.broadcast_to(sink[:, None, None], (Hq, T, 1))
        mask = torch.from_numpy(np.ascontiguousarray(np.concatenate([bias, col], 2)))[None]
        out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        return out[0].permute(1, 0, 2).numpy()

    ok = True
    for W in (1, 20, T + 5):
        band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
        got = o.window_branch_rows(q, pos, k, v, W, sink=sink)
        ok = ok and np.abs(got - sdpa_sink(band)).max() < 1e-12
    nblk = (T + 63) // 64
    idx = np.broadcast_to(np.arange(nblk), (Hkv, T, nblk))
    got = o.sparse_branch_rows(q, pos, k, v, idx, sink=sink)
    ok = ok and np.abs(got - sdpa_sink(i[None, :] <= i[:, None])).max() < 1e-12
    off = np.full(Hq, -np.inf)
    ok = ok and np.array_equal(o.window_branch_rows(q, pos, k, v, 20, sink=off),
                               o.window_branch_rows(q, pos, k, v, 20))
    none = np.full((Hkv, T, 2), -1)
    ok = ok and np.abs(o.sparse_branch_rows(q, pos, k, v, none, sink=sink)).max() == 0.0
    vconst = np.broadcast_to(np.arange(1.0, d + 1.0), (Hkv, T, d)).copy()
    got = o.window_branch_rows(np.zeros_like(q[10:]), pos[10:], k, vconst, 5, sink=sink)
    want = (5.0 / (5.0 + np.exp(sink)))[:, None] * np.arange(1.0, d + 1.0)[None, :]
    ok = ok and np.abs(got - want[None]).max() < 1e-12
    return ok


def pin_invariants(o):
    """Check (b): softmax rows sum to 1; max_j S = exp(max logit - LSE); LSE
    matches scipy's logsumexp; block masses (score='lse') sum to 1."""
    from scipy.special import logsumexp

    q, k, v = _rand(T=300, Hq=4, Hkv=1, d=8, seed=2)
    T = q.shape[0]
    pos = np.arange(T)
    _, lse, raw = o.full_attention_rows(q, pos, k, v)
    _, lse2, raw2 = o.full_attention_rows(q, pos, k, v, score="lse")
    tau = 1.0 / math.sqrt(q.shape[2])
    ok = True
    for h in range(4):
        logits = tau * q[:, h] @ k[0].T
        logits[np.triu_indices(T, 1)] = -np.inf
        ref_lse = logsumexp(logits, axis=1)
        ok = ok and np.abs(lse[h] - ref_lse).max() < 1e-12
        p = np.exp(logits - lse[h][:, None])
        ok = ok and np.abs(p.sum(axis=1) - 1).max() < 1e-12
        S = o.block_scores(raw[h:h + 1], lse[h:h + 1])[0]
        ok = ok and np.abs(np.nanmax(S, axis=1) - np.exp(logits.max(axis=1) - lse[h])).max() < 1e-12
        S2 = o.block_scores(raw2[h:h + 1], lse2[h:h + 1])[0]
        ok = ok and np.abs(np.nansum(S2, axis=1) - 1).max() < 1e-12
    return ok


def pin_bruteforce(o, include_diag=False):
    """Check (c): T <= 256, materialise the whole probability matrix with torch,
    take block maxima by reshaping, group max, rank every row with a full sort."""
    T, Hq, Hkv, d, kb = 256, 4, 2, 8, 2
    q, k, v = _rand(T, Hq, Hkv, d, seed=3)
    pos = np.arange(T)
    r = o.hybrid_block_rows(q, k, v, [], pos, kb=kb, W=0, include_diag=include_diag)
    Q = torch.from_numpy(q).permute(1, 0, 2)
    K = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 0)
    logits = Q @ K.transpose(1, 2) / math.sqrt(d)
    logits = logits.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    P = torch.softmax(logits, dim=-1)                              # [Hq, T, T]
    Sb = P.reshape(Hq, T, T // 64, 64).amax(-1)                    # [Hq, T, nblk]
    Sg = Sb.reshape(Hkv, Hq // Hkv, T, T // 64).amax(1).numpy()
    ok = True
    for g in range(Hkv):
        for t in range(T):
            last = t // 64 + (1 if include_diag else 0)
            sc = Sg[g, t, :last]
            order = sorted(range(last), key=lambda j: (-sc[j], j))[:kb]
            want = sorted(order) + [-1] * (kb - len(order))
            ok = ok and list(r["idx"][g, t]) == want
            ok = ok and np.allclose(r["Sg"][g, t, : t // 64 + 1], Sg[g, t, : t // 64 + 1],
                                    rtol=1e-12, atol=0)
    return ok


def pin_single_salient(o):
    """Closed form: all logits 0 except one key at logit a -> row t has
    Z = e^a + t, S(block of the key) = e^a/Z, every other block 1/Z."""
    T, d, a, istar = 4096, 64, 2.5, 777
    q = np.zeros((T, 2, d))
    q[:, :, 0] = math.sqrt(d)
    k = np.zeros((1, T, d))
    k[0, istar, 0] = a
    v = np.zeros((1, T, d))
    pos = np.array([776, 777, 1000, 2047, 4095])
    _, lse, raw = o.full_attention_rows(q[pos], pos, k, v)
    S = o.block_scores(raw, lse)
    ok = True
    for r, t in enumerate(pos):
        has = t >= istar
        Z = (math.exp(a) + t) if has else (t + 1)
        ok = ok and abs(np.exp(lse[0, r]) - Z) < 1e-9 * Z
        nb = t // 64 + 1
        want = np.full(nb, 1.0 / Z)
        if has:
            want[istar // 64] = math.exp(a) / Z
        ok = ok and np.abs(S[0, r, :nb] - want).max() < 1e-14
    return ok


def pin_topk_ties(o):
    """Ties go to the lower index; fewer candidates than k pad with -1; an empty
    candidate set gives no blocks and a zero sparse branch."""
    s = np.array([0.5, 0.7, 0.7, 0.1, 0.7, 0.2])
    idx, srt = o.topk_select(s, np.arange(6), 2)
    ok = list(idx) == [1, 2] and list(srt[:3]) == [0.7, 0.7, 0.7]
    idx, _ = o.topk_select(s, np.arange(3), 5)
    ok = ok and list(idx) == [0, 1, 2, -1, -1]
    idx, _ = o.topk_select(s, np.arange(0), 3)
    ok = ok and list(idx) == [-1, -1, -1]
    q, k, v = _rand(T=100, Hq=2, Hkv=1, d=4, seed=4)
    pos = np.array([10, 63])
    e = o.sparse_branch_rows(q[pos], pos, k, v, np.full((1, 2, 3), -1))
    return ok and np.abs(e).max() == 0.0


def pin_gates():
    from scipy.special import expit

    x = np.linspace(-30, 30, 101)
    a = np.ones((1, 1, 3))
    b = 2 * np.ones((1, 1, 3))
    ok = np.abs(ora.sigmoid(x) - expit(x)).max() < 1e-15
    out = ora.gated_fusion(a, b, np.array([[[40.0, -40.0]]]))
    ok = ok and np.abs(out - a).max() < 1e-15
    out = ora.gated_fusion(a, b, np.array([[[0.0, math.log(3.0)]]]))
    return ok and np.abs(out - (0.5 + 1.5)).max() < 1e-15


def pin_fp8(o):
    """All 256 e4m3fn codes against torch.float8_e4m3fn."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = o.decode_e4m3fn(codes)
    nan_ok = np.array_equal(np.isnan(ref), np.isnan(mine))
    fin = ~np.isnan(ref)
    return nan_ok and np.array_equal(ref[fin], mine[fin]) and int(np.isnan(mine).sum()) == 2


def pin_fp8_scales(o):
    """fp8 caches with one scale per (K|V, kv head): token-mode decode with
    k >= L - n_recent selects every token, so the full layer and the sparse
    layer both equal dense attention over the dequantised cache.  The
    reference dequantises through torch's float8_e4m3fn and multiplies by the
    scale itself; every K/V scale and every head's scale differs, so a
    swapped scale row or a head slip changes the result."""
    rng = np.random.default_rng(17)
    L, Hq, Hkv, d, R = 300, 4, 2, 16, 16
    kv_scale = np.array([[0.02, 0.5], [3.0, 0.07]])          # [K|V, kv head]
    xk = rng.standard_normal((Hkv, L, d)) * 40.0
    xv = rng.standard_normal((Hkv, L, d)) * 40.0
    f8 = lambda x: torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    kc = np.stack([f8(xk[g]).view(torch.uint8).numpy() for g in range(Hkv)])
    vc = np.stack([f8(xv[g]).view(torch.uint8).numpy() for g in range(Hkv)])
    deq = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    kref = np.stack([deq(kc[g], kv_scale[0, g]) for g in range(Hkv)])
    vref = np.stack([deq(vc[g], kv_scale[1, g]) for g in range(Hkv)])
    q = rng.standard_normal((L, Hq, d))
    qs = rng.standard_normal((L, Hq, d))
    dec = o.decode_step(q[L - 1], kc, vc, L, [dict(q=qs[L - 1])], kb=L, W=0, block=1,
                        n_recent=R, kv_scale=kv_scale)
    ok = np.array_equal(dec["idx"][0], np.arange(L))
    ok = ok and np.abs(dec["o"] - _sdpa(q, kref, vref, causal=True)[L - 1]).max() < 1e-12
    ok = ok and np.abs(dec["layer_out"][0] - _sdpa(qs, kref, vref, causal=True)[L - 1]).max() < 1e-12
    # the sparse layer on its own, over a hand-made subset of tokens
    sel = np.array([[3, 7, 250, 299], [0, 1, 2, 299]])
    got = o.decode_sparse_layer(dict(q=qs[L - 1]), kc, vc, L, sel, 0, block=1, kv_scale=kv_scale)
    for g in range(Hkv):
        heads = slice(g * 2, g * 2 + 2)
        want = _sdpa(qs[L - 1:L, heads], kref[g:g + 1, sel[g]], vref[g:g + 1, sel[g]])[0]
        ok = ok and np.abs(got[heads] - want).max() < 1e-12
    return bool(ok)


def pin_gather(o):
    """The gathered cache of the selected blocks (eq. K~,V~) is what the
    sparse branch attends: a decode sparse layer over (k_sel, v_sel, idx_sel)
    equals the layer over the whole cache with the fully-past ids of a messy
    list (shuffled, a repeat, -1, the diagonal block and out-of-range ids).
    Also checked: each live block lands whole in its slot, and the slots after
    the live ones stay 0."""
    rng = np.random.default_rng(23)
    Hkv, Hq, d, L, n = 2, 4, 8, 700, 9
    k = rng.standard_normal((Hkv, L, d))
    v = rng.standard_normal((Hkv, L, d))
    idx = np.array([[7, 2, -1, 7, 10, 0, 3, 11, 5], [1, 4, 4, 4, -1, -1, 9, 200, 6]])
    k_sel, v_sel, idx_sel = o.gather_blocks(k, v, idx, L)
    lay = dict(q=rng.standard_normal((Hq, d)))
    past = np.where(idx < (L - 1) // 64, idx, -1)     # block 10 holds the query: not fully past
    a = ora.decode_sparse_layer(lay, k, v, L, past, 0)
    b = ora.decode_sparse_layer(lay, k_sel, v_sel, L, idx_sel, 0)
    ok = np.abs(a - b).max() < 1e-13
    live = [[0, 2, 3, 5, 7], [1, 4, 6, 9]]            # ids with j < 10, each once
    for g in range(Hkv):
        ok = ok and list(idx_sel[g]) == list(range(len(live[g]))) + [-1] * (n - len(live[g]))
        for p, j in enumerate(live[g]):
            ok = ok and np.array_equal(k_sel[g, 64 * p: 64 * p + 64], k[g, 64 * j: 64 * j + 64])
            ok = ok and np.array_equal(v_sel[g, 64 * p: 64 * p + 64], v[g, 64 * j: 64 * j + 64])
        ok = ok and not k_sel[g, 64 * len(live[g]):].any()
    return bool(ok)


def pin_fp8_prefill(o):
    """fp8 prefill (reading R15): a full layer and a sparse layer over e4m3
    codes with one scale per query head and per kv head equal torch SDPA on
    the values torch's float8_e4m3fn decode gives, times the scales."""
    rng = np.random.default_rng(29)
    T, Hq, Hkv, d = 200, 4, 2, 16
    f8 = lambda x: torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    deq = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    qs = np.array([0.01, 0.05, 0.2, 1.5])            # per query head
    ks = np.array([0.03, 0.4])                        # per kv head
    vs = np.array([2.0, 0.09])
    qc = f8(rng.standard_normal((T, Hq, d)) * 30).view(torch.uint8).numpy()
    kc = f8(rng.standard_normal((Hkv, T, d)) * 30).view(torch.uint8).numpy()
    vc = f8(rng.standard_normal((Hkv, T, d)) * 30).view(torch.uint8).numpy()
    qref = deq(qc) * qs[None, :, None]
    kref = deq(kc) * ks[:, None, None]
    vref = deq(vc) * vs[:, None, None]
    q = o.dequantize_e4m3(qc, qs, head_axis=1)
    k = o.dequantize_e4m3(kc, ks, head_axis=0)
    v = o.dequantize_e4m3(vc, vs, head_axis=0)
    pos = np.arange(T)
    out, _, _ = o.full_attention_rows(q[pos], pos, k, v)
    ok = np.abs(out - _sdpa(qref, kref, vref, causal=True)).max() < 1e-12
    idx = np.tile(np.arange(4), (Hkv, T, 1))          # every block, diagonal included
    sp = o.sparse_branch_rows(q[pos], pos, k, v, idx)
    return bool(ok and np.abs(sp - _sdpa(qref, kref, vref, causal=True)).max() < 1e-12)


def pin_bwd_full(o):
    """Backward of the full layer equals torch autograd through float64 SDPA
    (causal, GQA by repeated kv heads)."""
    rng = np.random.default_rng(31)
    T, Hq, Hkv, d = 90, 4, 2, 8
    q, k, v, do = (rng.standard_normal((T, Hq, d)), rng.standard_normal((Hkv, T, d)),
                   rng.standard_normal((Hkv, T, d)), rng.standard_normal((T, Hq, d)))
    dq, dk, dv = o.full_attention_bwd(q, k, v, do)
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        Q.permute(1, 0, 2)[None], K.repeat_interleave(Hq // Hkv, 0)[None], V.repeat_interleave(Hq // Hkv, 0)[None],
        is_causal=True)[0].permute(1, 0, 2)
    (out * torch.from_numpy(do)).sum().backward()
    return max(np.abs(dq - Q.grad.numpy()).max(), np.abs(dk - K.grad.numpy()).max(),
               np.abs(dv - V.grad.numpy()).max()) < 1e-12


def _sparse_case(seed=37):
    rng = np.random.default_rng(seed)
    T, Hq, Hkv, d, W = 150, 4, 2, 4, 20
    x = dict(qs=rng.standard_normal((T, Hq, d)), k=rng.standard_normal((Hkv, T, d)),
             v=rng.standard_normal((Hkv, T, d)), ks=rng.standard_normal((Hkv, T, d)),
             vs=rng.standard_normal((Hkv, T, d)), gates=rng.standard_normal((T, Hq, 2)),
             sinks=rng.standard_normal((2, Hq)))
    idx = np.stack([np.stack([rng.choice(max(t // 64, 1), size=2) - (t < 64) for t in range(T)])
                    for _ in range(Hkv)])                  # repeats and -1 included
    return x, idx, W, rng.standard_normal((T, Hq, d))


def pin_bwd_sparse(o):
    """Backward of a sparse layer (both branches, gates, sinks) against central
    finite differences of the forward oracle, along one random direction per
    input: (L(x + e u) - L(x - e u)) / 2e = <dL/dx, u> with L = sum(dO * o)."""
    x, idx, W, do = _sparse_case()
    T = do.shape[0]
    pos = np.arange(T)

    def loss(y):
        out = ora.sparse_layer_rows(y["qs"], pos, y["k"], y["v"], idx, y["ks"], y["vs"], W, y["gates"],
                                    sinks=y["sinks"])
        return float((out * do).sum())

    g = o.sparse_layer_bwd(x["qs"], x["k"], x["v"], idx, x["ks"], x["vs"], W, x["gates"], do, sinks=x["sinks"])
    names = dict(qs="dq", k="dk", v="dv", ks="dks", vs="dvs", gates="dgates", sinks="dsinks")
    rng = np.random.default_rng(41)
    eps = 1e-5
    ok = True
    for name, gname in names.items():
        u = rng.standard_normal(x[name].shape)
        yp = dict(x, **{name: x[name] + eps * u})
        ym = dict(x, **{name: x[name] - eps * u})
        fd = (loss(yp) - loss(ym)) / (2 * eps)
        an = float((g[gname] * u).sum())
        ok = ok and abs(fd - an) <= 1e-6 * max(1.0, abs(an))
    return ok


def pin_bwd_sparse_dense(o):
    """Every block selected (diagonal included), no window, no gate, no sink:
    the sparse layer is dense causal attention over the shared K/V, so its
    gradients equal the full layer's (torch autograd is behind that one)."""
    rng = np.random.default_rng(43)
    T, Hq, Hkv, d = 130, 4, 2, 8
    qs, k, v, do = (rng.standard_normal((T, Hq, d)), rng.standard_normal((Hkv, T, d)),
                    rng.standard_normal((Hkv, T, d)), rng.standard_normal((T, Hq, d)))
    idx = np.tile(np.arange(3), (Hkv, T, 1))
    g = o.sparse_layer_bwd(qs, k, v, idx, k, v, 0, None, do)
    dq, dk, dv = o.full_attention_bwd(qs, k, v, do)
    return max(np.abs(g["dq"] - dq).max(), np.abs(g["dk"] - dk).max(), np.abs(g["dv"] - dv).max()) < 1e-12


# ------------------------------------------------------------- the tests
def test_e1_two_blocks():
    assert pin_e1(ora)


def test_e2_three_blocks_gated():
    assert pin_e2(ora)


def test_dense_reduction_matches_sdpa():
    assert pin_dense_reduction(ora)


def test_window_matches_banded_sdpa():
    assert pin_window(ora)


def test_invariants():
    assert pin_invariants(ora)


@pytest.mark.parametrize("include_diag", [False, True])
def test_bruteforce_block_ranking(include_diag):
    assert pin_bruteforce(ora, include_diag)


def test_single_salient_closed_form():
    assert pin_single_salient(ora)


def test_topk_ties_and_padding():
    assert pin_topk_ties(ora)


def test_sinks():
    assert pin_sinks(ora)


def test_gates():
    assert pin_gates()


def test_fp8_table():
    assert pin_fp8(ora)


def test_fp8_scales():
    assert pin_fp8_scales(ora)


def test_fp8_prefill():
    assert pin_fp8_prefill(ora)


def test_bwd_full():
    assert pin_bwd_full(ora)


def test_bwd_sparse_finite_differences():
    assert pin_bwd_sparse(ora)


def test_bwd_sparse_dense_case():
    assert pin_bwd_sparse_dense(ora)


def test_gather():
    assert pin_gather(ora)


def test_index_order_does_not_matter():
    q, k, v = _rand(T=256, Hq=4, Hkv=2, d=8, seed=5)
    pos = np.array([130, 200, 255])
    idx = np.array([[[0, 2, 1]] * 3, [[1, 0, -1]] * 3])
    perm = idx[:, :, ::-1].copy()
    a = ora.sparse_branch_rows(q[pos], pos, k, v, idx)
    b = ora.sparse_branch_rows(q[pos], pos, k, v, perm)
    assert np.abs(a - b).max() < 1e-14
    # the list is a set: repeated ids and -1 anywhere in it change nothing
    dup = np.array([[[2, -1, 0, 2, 1, 0]] * 3, [[-1, 1, 1, 0, -1, -1]] * 3])
    c = ora.sparse_branch_rows(q[pos], pos, k, v, dup)
    assert np.abs(a - c).max() < 1e-14


def test_decode_equals_last_prefill_row():
    """Decode at an L-token context equals row L-1 of the prefill block on the
    same data, with the window read from a ring (slot = pos mod W)."""
    rng = np.random.default_rng(6)
    T, Hq, Hkv, d, W, kb = 700, 4, 2, 8, 96, 3
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((Hkv, T, d))
    v = rng.standard_normal((Hkv, T, d))
    lay = dict(q=rng.standard_normal((T, Hq, d)), k=rng.standard_normal((Hkv, T, d)),
               v=rng.standard_normal((Hkv, T, d)), gates=rng.standard_normal((T, Hq, 2)))
    for L in (1, 64, 65, 129, 700):
        pre = ora.hybrid_block_rows(q, k, v, [lay], np.array([L - 1]), kb, W)
        ring_k = np.zeros((Hkv, W, d))
        ring_v = np.zeros((Hkv, W, d))
        for p in range(max(0, L - W), L):
            ring_k[:, p % W] = lay["k"][:, p]
            ring_v[:, p % W] = lay["v"][:, p]
        dl = dict(q=lay["q"][L - 1], k_ring=ring_k, v_ring=ring_v, gates=lay["gates"][L - 1])
        dec = ora.decode_step(q[L - 1], k, v, L, [dl], kb, W)
        assert np.abs(dec["o"] - pre["o"][0]).max() < 1e-13
        assert np.array_equal(dec["idx"], pre["idx"][:, 0])
        assert np.abs(dec["layer_out"][0] - pre["layer_out"][0][0]).max() < 1e-13


def test_token_mode_covering_everything_is_dense():
    """Token mode with k >= L - n_recent selects every token: the sparse layer
    is then dense attention over the whole context (torch SDPA, last row)."""
    rng = np.random.default_rng(7)
    L, Hq, Hkv, d = 300, 4, 1, 16
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((Hkv, L, d))
    v = rng.standard_normal((Hkv, L, d))
    qs = rng.standard_normal((L, Hq, d))
    dec = ora.decode_step(q, k, v, L, [dict(q=qs[L - 1])], kb=L, W=0, block=1, n_recent=16)
    assert np.array_equal(dec["idx"][0], np.arange(L))
    ref = _sdpa(qs, k, v, causal=True)[L - 1]
    assert np.abs(dec["layer_out"][0] - ref).max() < 1e-12


def test_token_mode_recent_is_forced_and_free():
    Sg = np.array([9.0, 8.0, 7.0, 6.0, 0.0, 0.0, 0.0])
    sel, _ = ora.select_with_recent(Sg, t=6, k=2, n_recent=3)
    assert list(sel) == [0, 1, 4, 5, 6]
    sel, _ = ora.select_with_recent(Sg, t=1, k=2, n_recent=3)
    assert list(sel) == [0, 1]


# ------------------------------------------------------------ mutations
class _Mutant:
    """The oracle module with one function replaced by a broken copy."""

    def __init__(self, **repl):
        self.__dict__.update({k: getattr(ora, k) for k in dir(ora) if not k.startswith("__")})
        self._repl = repl

    def __enter__(self):
        self._saved = {k: getattr(ora, k) for k in self._repl}
        for k, f in self._repl.items():
            setattr(ora, k, f)
        return ora

    def __exit__(self, *a):
        for k, f in self._saved.items():
            setattr(ora, k, f)


def _unnormalised_scores(raw, lse):          # forgets the -LSE of the rescale
    return np.exp(raw)


def _window_off_by_one(qs, pos, ks, vs, W, scale=None, sink=None):
    return _orig_window(qs, pos, ks, vs, W + 1, scale, sink)


def _gates_swapped(o_sparse, o_window, g):
    return _orig_fusion(o_window, o_sparse, g)


def _causal_leak(q_rows, pos, k, v, scale=None, block=64, score="max"):
    n = k.shape[1]
    return _orig_full(q_rows, np.minimum(pos + 1, n - 1), k, v, scale, block, score)


def _ties_high(scores_row, cand, k):        # breaks ties towards the higher index
    sc = scores_row[cand]
    order = np.lexsort((-cand, -sc))
    take = cand[order[: min(k, cand.size)]]
    idx = np.full(k, -1, np.int64)
    idx[: take.size] = np.sort(take)
    return idx, sc[order]


def _fp8_bias8(codes):
    return _orig_fp8(codes) / 2.0


def _sink_ignored(logits, values, sink=None):
    return _orig_attend(logits, values)


def _sink_negated(logits, values, sink=None):
    return _orig_attend(logits, values, None if sink is None else -np.asarray(sink))


def _no_diag_clip(qs_rows, pos, k, v, idx, block=64, scale=None, sink=None):
    return _orig_sparse(qs_rows, np.full_like(pos, k.shape[1] - 1), k, v, idx, block, scale, sink)


def _kv_scale_rows_swapped(k, v, kv_scale, L=None):
    return _orig_deq_kv(k, v, np.asarray(kv_scale)[::-1], L)


def _scale_heads_reversed(codes, scale, head_axis=0):
    return _orig_deq(codes, np.asarray(scale)[::-1], head_axis)


def _gather_keeps_repeats(k, v, idx, L, block=64):
    # a repeated id gets a slot of its own (the list taken as a sequence, not a set)
    Hkv, _, d = k.shape
    n = idx.shape[1]
    k_sel = np.zeros((Hkv, n * block, d))
    v_sel = np.zeros((Hkv, n * block, d))
    idx_sel = np.full((Hkv, n), -1, np.int64)
    for g in range(Hkv):
        live = np.sort(idx[g][(idx[g] >= 0) & (idx[g] < (L - 1) // block)])
        for p, j in enumerate(live):
            k_sel[g, p * block: (p + 1) * block] = k[g, j * block: (j + 1) * block]
            v_sel[g, p * block: (p + 1) * block] = v[g, j * block: (j + 1) * block]
        idx_sel[g, : live.size] = np.arange(live.size)
    return k_sel, v_sel, idx_sel


def _gather_shifted(k, v, idx, L, block=64):
    return _orig_gather(k, v, np.where(idx >= 0, idx + 1, idx), L, block)


def _bwd_no_delta(s_, values, keys, q, do, tau, sink=None):
    # forgets the -do.o term of ds = p (dp - do.o)
    dq, dk, dv, dsk = _orig_attend_bwd(s_, values, keys, q, do, tau, sink)
    n = values.shape[0]
    if n == 0:
        return dq, dk, dv, dsk
    m = s_.max() if sink is None else max(s_.max(), sink)
    e = np.exp(s_ - m)
    z = e.sum() + (np.exp(sink - m) if sink is not None else 0.0)
    p = e / z
    ds = p * (values @ do)
    return tau * (ds @ keys), tau * np.outer(ds, q), dv, dsk


def _bwd_sparse_gate_sigma(qs, k, v, idx, ks, vs, W, gates, do, block=64, scale=None, sinks=None):
    # gate derivative taken as sigma instead of sigma (1 - sigma)
    out = _orig_sparse_bwd(qs, k, v, idx, ks, vs, W, gates, do, block, scale, sinks)
    if gates is not None:
        sg = 1.0 / (1.0 + np.exp(-gates))
        out["dgates"] = out["dgates"] / (1.0 - sg)
    return out


_orig_attend = ora._attend
_orig_window = ora.window_branch_rows
_orig_fusion = ora.gated_fusion
_orig_full = ora.full_attention_rows
_orig_topk = ora.topk_select
_orig_fp8 = ora.decode_e4m3fn
_orig_sparse = ora.sparse_branch_rows
_orig_deq_kv = ora.dequantize_kv
_orig_deq = ora.dequantize_e4m3
_orig_gather = ora.gather_blocks
_orig_attend_bwd = ora._attend_bwd
_orig_sparse_bwd = ora.sparse_layer_bwd


@pytest.mark.parametrize("name,repl,pins", [
    ("unnormalised group max", dict(block_scores=_unnormalised_scores), [pin_e1]),
    ("window off by one", dict(window_branch_rows=_window_off_by_one), [pin_window, pin_e2]),
    ("gates swapped", dict(gated_fusion=_gates_swapped), [pin_e2]),
    ("causal leak", dict(full_attention_rows=_causal_leak), [pin_dense_reduction]),
    ("ties to the higher index", dict(topk_select=_ties_high), [pin_topk_ties]),
    ("fp8 exponent bias", dict(decode_e4m3fn=_fp8_bias8), [pin_fp8]),
    ("diagonal block not clipped", dict(sparse_branch_rows=_no_diag_clip), [pin_dense_reduction]),
    ("sink ignored", dict(_attend=_sink_ignored), [pin_sinks]),
    ("sink sign flipped", dict(_attend=_sink_negated), [pin_sinks]),
    ("fp8 K and V scale rows swapped", dict(dequantize_kv=_kv_scale_rows_swapped), [pin_fp8_scales]),
    ("fp8 scale taken from the wrong head", dict(dequantize_e4m3=_scale_heads_reversed),
     [pin_fp8_scales, pin_fp8_prefill]),
    ("gather keeps a repeated block twice", dict(gather_blocks=_gather_keeps_repeats), [pin_gather]),
    ("gather one block off", dict(gather_blocks=_gather_shifted), [pin_gather]),
    ("backward without the -do.o term", dict(_attend_bwd=_bwd_no_delta), [pin_bwd_full, pin_bwd_sparse]),
    ("gate derivative without (1 - sigma)", dict(sparse_layer_bwd=_bwd_sparse_gate_sigma), [pin_bwd_sparse]),
])
def test_planted_mistakes_fail_their_pins(name, repl, pins):
    with _Mutant(**repl) as m:
        for pin in pins:
            assert not pin(m), f"pin {pin.__name__} did not catch: {name}"
