"""fp64 CPU oracle of the HySparse hybrid-block attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP path (it imports numpy and nothing from the product package); inputs
arrive as float64 arrays holding the exact stored values (fp8 codes are
decoded here, by `decode_e4m3fn`).

Every function is the plain definition from the pages, in float64, computed
row by row (a query row only needs keys up to its own position), so sampled
rows of a full-size workload cost seconds.  Nothing is blocked, fused or
reordered beyond what the definitions state.

Sources (cited by page title and section):
  [X]  "HySparse: A Hybrid Sparse Attention Architecture with Oracle Token
       Selection and KV Cache Sharing" -- explainer page (paper-graph-ui),
       sections 3.4.1-3.4.3.
  [P]  The same paper's own text (paperpeel page), sections 3.1-3.3.
  [H2] HySparse2 explainer page (deep-reads), "Precise retrieval without a
       separate indexer" and the decode_one_token pseudocode.

Readings where the pages leave a step open:
  R1  The block score is the post-softmax maximum (eq. S_t^i of [X] 3.4.1);
      the printed rescale of [X] "Modified FlashAttention Kernel" is read as
      exp(S - m)/l, i.e. exp(raw - LSE), which is the only form that makes the
      stored value equal eq. S_t^i.  An alternative block log-sum-exp score
      (block probability mass) is offered as score='lse'.
  R2  Candidate blocks: by default only fully-past blocks j < floor(t/B);
      include_diag=True adds the (causally clipped) diagonal block, which is
      the literal reading of B_i = {(i-1)B+1 .. min(iB, t)}.
  R3  Fewer candidates than k: all are selected, the rest is padded with -1;
      an empty selection gives a zero sparse-branch output.
  R4  Ties: order by score descending, then block index ascending; the index
      list is emitted in ascending order.
  R5  Gates are per (token, head) logits; gates=None means both gates are 1.
  R6  The window holds the min(t+1, W) keys [t-W+1, t], the query's own
      position included.
  R7  Query head h belongs to kv group floor(h / G) (contiguous grouping).
  R8  Decode: the new token is already in the cache, so the query sits at
      position L-1 of an L-token context.  The window ring keeps position p in
      slot p mod W.
  R9  Token-level selection ([H2]): block size 1, candidates are the tokens
      older than the newest n_recent, which are always added and do not use
      the k budget; no window branch and no gate.  The group score is the
      same group-wise maximum of post-softmax weights.
  R15 fp8 prefill: the queries, keys and values of the full layer, and each
      sparse layer's queries and window K'/V', may be stored as e4m3 codes
      with one fp32 scale per head (queries per query head, keys and values
      per kv head).  The path computes the same definitions on the values
      code * scale (dequantize_e4m3); rounding the probabilities to fp8 for
      the value product is the kernels' approximation, covered by the fp8
      tolerance, not part of the definition.
  R16 Backward ([P] 4.1 trains the architecture end to end; [X] 3.4 shares
      the full layer's K/V with every sparse layer): the selection is a
      discrete choice of the forward pass, so indices and block scores get no
      gradient; each branch is a softmax attention with its own LSE; with
      o = s0 o~ + s1 o' (s = sigmoid of the gate logits), do~ = s0 do,
      do' = s1 do and dG_b = s_b (1 - s_b) do.o_b; the sparse branch's dK/dV
      is this layer's share of the shared K/V's gradient.
  R17 Offloaded cache ([P] 5, KV offloading): the compact cache holds whole
      fully-past selected blocks (the decode candidates of R2), each once,
      ascending (gather_blocks).
  R18 Index rows are sets: any order, duplicates once, -1 and out-of-range
      ids ignored anywhere in a row (K~, V~ of [X] 3.4.3 is a union).
  R14 Sink biases ([P] 4.1, "Experiments Setup": per-head learnable sink
      biases in the sparse and the window branch, following gpt-oss): each
      branch's softmax takes one extra logit b_h, in the units of tau q.k,
      that carries no value, o = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{b_h}).
      Sinks are optional ([2, Hq]: [0] sparse branch, [1] window branch;
      token mode uses [0]); without them nothing changes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------- helpers
def softmax_scale(d: int) -> float:
    """tau = 1/sqrt(d) ([X] 3.4.1, "Standard Attention Formulation")."""
    return 1.0 / np.sqrt(d)


def _attend(logits: np.ndarray, values: np.ndarray, sink=None):
    """Softmax over the last axis of `logits` ([..., n]) applied to values [n, d].

    Returns (o [..., d], lse [...]).  An empty key set (n == 0, or every logit
    -inf) gives o = 0 and lse = -inf (reading R3).  `sink` (broadcast to the
    leading shape, or None) is one more logit per row with no value (reading
    R14): it joins the maximum and the denominator, and the lse then
    includes it.
    """
    lead = logits.shape[:-1]
    d = values.shape[-1]
    b = None if sink is None else np.broadcast_to(np.asarray(sink, np.float64), lead)[..., None]
    if logits.shape[-1] == 0:
        m = np.full((*lead, 1), -np.inf)
    else:
        m = logits.max(axis=-1, keepdims=True)
    if b is not None:
        m = np.maximum(m, b)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(logits - m_safe)
    l = e.sum(axis=-1, keepdims=True)
    if b is not None:
        l = l + np.exp(b - m_safe)
    l_safe = np.where(l > 0, l, 1.0)
    o = (e @ values) / l_safe if logits.shape[-1] else np.zeros((*lead, d))
    lse = np.where(finite & (l > 0), m_safe + np.log(l_safe), -np.inf)[..., 0]
    o = np.where(finite & (l > 0), o, 0.0)
    return o, lse


def group_of(h: int, G: int) -> int:
    """Reading R7: query head h uses kv head floor(h/G)."""
    return h // G


# ------------------------------------------------------- full attention layer
def full_attention_rows(q_rows: np.ndarray, pos: np.ndarray, k: np.ndarray,
                        v: np.ndarray, scale: float | None = None,
                        block: int = BLOCK, score: str = "max"):
    """Causal GQA attention of the full layer plus its block scores, for a set of rows.

    q_rows [R, Hq, d]: the queries at positions `pos` [R]; k, v [Hkv, >=max(pos)+1, d].
    o_t = sum_{i<=t} softmax_i(tau q_t.k_i) v_i   ([X] 3.4.1 eq. o_t; [P] 3.2)
    LSE_t = log sum_{i<=t} exp(tau q_t.k_i)
    raw[h, r, j] = max_{i in B_j, i<=t} tau q.k_i  (score='max'), i.e. the
        pre-softmax block maximum that the modified FlashAttention pass stores
        ([X] "Modified FlashAttention Kernel", first pass), or the block
        log-sum-exp (score='lse').  Only j <= t//block is defined; later
        entries are NaN.
    Returns o [R, Hq, d], lse [Hq, R], raw [Hq, R, nblk] with nblk = ceil((max(pos)+1)/block).
    """
    R, Hq, d = q_rows.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    tau = softmax_scale(d) if scale is None else scale
    n = int(pos.max()) + 1
    nblk = (n + block - 1) // block
    o = np.zeros((R, Hq, d))
    lse = np.zeros((Hq, R))
    raw = np.full((Hq, R, nblk), np.nan)
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        for r in range(R):
            t = int(pos[r])
            s = tau * (q_rows[r, heads] @ k[g, : t + 1].T)          # [G, t+1]
            o[r, heads], lse[heads, r] = _attend(s, v[g, : t + 1])
            nb = t // block + 1
            padded = np.full((G, nb * block), -np.inf)
            padded[:, : t + 1] = s
            blocks = padded.reshape(G, nb, block)
            if score == "max":
                raw[heads, r, :nb] = blocks.max(axis=-1)
            elif score == "lse":
                mb = blocks.max(axis=-1, keepdims=True)
                raw[heads, r, :nb] = mb[..., 0] + np.log(np.exp(blocks - mb).sum(axis=-1))
            else:
                raise ValueError(score)
    return o, lse, raw


def block_scores(raw: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """Post-softmax block scores S_{h,t,j} = exp(raw - LSE_t)  (reading R1).

    With score='max' this is eq. S_t^i of [X] 3.4.1: the largest attention
    weight that query t gives to any key of block j.  raw [Hq, R, nblk],
    lse [Hq, R]; NaN entries (future blocks) stay NaN.
    """
    return np.exp(raw - lse[..., None])


def group_max(S: np.ndarray, Hkv: int) -> np.ndarray:
    """S_g = max over the heads h of group g of S_h  ([X] "Grouped-Query
    Attention (GQA) Aggregation", eq. S_g; [P] 3.2).  S [Hq, ...] -> [Hkv, ...]."""
    Hq = S.shape[0]
    G = Hq // Hkv
    return S.reshape(Hkv, G, *S.shape[1:]).max(axis=1)


def candidates(t: int, block: int = BLOCK, include_diag: bool = False,
               n_recent: int = 0) -> np.ndarray:
    """Candidate key blocks (or tokens when block == 1) of query position t.

    Block mode (reading R2): j < floor(t/block), plus j = floor(t/block) when
    include_diag.  Token mode (reading R9): tokens i < t+1-n_recent.
    """
    if block == 1 and n_recent:
        return np.arange(max(0, t + 1 - n_recent))
    last = t // block
    return np.arange(last + 1 if include_diag else last)


def topk_select(scores_row: np.ndarray, cand: np.ndarray, k: int):
    """TopK of [X] 3.4.2 / [P] 3.2 over one row: the k candidates with the
    highest score, ties to the lower index (R4); returned ascending and padded
    with -1 to length k (R3).  Also returns the candidates' scores sorted
    descending (used for the near-tie rule of the parity tests)."""
    s = scores_row[cand]
    order = np.lexsort((cand, -s))
    take = cand[order[: min(k, cand.size)]]
    idx = np.full(k, -1, np.int64)
    idx[: take.size] = np.sort(take)
    return idx, s[order]


def select_with_recent(scores_row: np.ndarray, t: int, k: int, n_recent: int):
    """Token-level selection of [H2]: top-k of the old tokens united with the
    n_recent newest visible tokens (which do not use the k budget), ascending.
    Returns the selected token ids (length min(k, #old) + min(n_recent, t+1))
    and the sorted scores of the old candidates."""
    old = candidates(t, 1, n_recent=n_recent)
    top, sorted_s = topk_select(scores_row, old, k)
    top = top[top >= 0]
    recent = np.arange(max(0, t + 1 - n_recent), t + 1)
    return np.sort(np.concatenate([top, recent])), sorted_s


# --------------------------------------------------------------- sparse layer
def sparse_branch_rows(qs_rows: np.ndarray, pos: np.ndarray, k: np.ndarray,
                       v: np.ndarray, idx: np.ndarray, block: int = BLOCK,
                       scale: float | None = None, sink=None) -> np.ndarray:
    """Block-sparse attention branch over the full layer's own K/V.

    K~, V~ = concat of the selected blocks (eq. K~,V~ of [X] 3.4.3, "Branch 1");
    o~_t = softmax(tau q'_t . K~) V~ (eq. o~_t).  Keys after t inside a selected
    diagonal block are excluded (causality).  idx [Hkv, R, n_sel] holds block
    ids (or token ids with block=1), -1 = unused; the order of the list does
    not matter.  sink [Hq] or None: the branch's sink logits (R14).
    Returns o~ [R, Hq, d].
    """
    R, Hq, d = qs_rows.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    tau = softmax_scale(d) if scale is None else scale
    out = np.zeros((R, Hq, d))
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        for r in range(R):
            t = int(pos[r])
            sel = idx[g, r]
            sel = np.unique(sel[sel >= 0])
            keys = (sel[:, None] * block + np.arange(block)[None, :]).reshape(-1)
            keys = keys[keys <= t]
            s = tau * (qs_rows[r, heads] @ k[g, keys].T)
            out[r, heads], _ = _attend(s, v[g, keys], None if sink is None else sink[heads])
    return out


def window_branch_rows(qs_rows: np.ndarray, pos: np.ndarray, ks: np.ndarray,
                       vs: np.ndarray, W: int, scale: float | None = None,
                       sink=None) -> np.ndarray:
    """Sliding-window branch with the layer's own K'/V' ([X] 3.4.3 "Branch 2",
    eq. o'_t): keys [t-W+1, t] (reading R6).  W = 0 gives 0.
    ks, vs [Hkv, >=max(pos)+1, d]; sink [Hq] or None (R14).
    Returns o' [R, Hq, d]."""
    R, Hq, d = qs_rows.shape
    Hkv = ks.shape[0]
    G = Hq // Hkv
    tau = softmax_scale(d) if scale is None else scale
    out = np.zeros((R, Hq, d))
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        for r in range(R):
            t = int(pos[r])
            lo = max(0, t - W + 1)
            keys = np.arange(lo, t + 1) if W > 0 else np.arange(0)
            s = tau * (qs_rows[r, heads] @ ks[g, keys].T)
            out[r, heads], _ = _attend(s, vs[g, keys], None if sink is None else sink[heads])
    return out


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def gated_fusion(o_sparse: np.ndarray, o_window: np.ndarray,
                 gate_logits: np.ndarray | None) -> np.ndarray:
    """o_t = sigma(g~) o~_t + sigma(g') o'_t  ([X] 3.4.3 "Gated Fusion"; [P] 3.1).
    Two independent sigmoids per (token, head) (R5); gate_logits [R, Hq, 2]
    with [..., 0] for the sparse and [..., 1] for the window branch."""
    if gate_logits is None:
        return o_sparse + o_window
    g = sigmoid(gate_logits)
    return g[..., 0:1] * o_sparse + g[..., 1:2] * o_window


# ------------------------------------------------------------- hybrid block
def select_rows(raw: np.ndarray, lse: np.ndarray, pos: np.ndarray, Hkv: int, kb: int,
                block: int = BLOCK, include_diag: bool = False):
    """Finalise, group-aggregate and select for each row: returns
    idx [Hkv, R, kb], S_g [Hkv, R, nblk] and the sorted candidate scores
    (list over (g, r))."""
    Sg = group_max(block_scores(raw, lse), Hkv)
    R = pos.size
    idx = np.full((Hkv, R, kb), -1, np.int64)
    ranked = {}
    for g in range(Hkv):
        for r in range(R):
            t = int(pos[r])
            cand = candidates(t, block, include_diag)
            idx[g, r], ranked[g, r] = topk_select(Sg[g, r], cand, kb)
    return idx, Sg, ranked


def sparse_layer_rows(qs_rows, pos, k, v, idx, ks, vs, W, gates_rows,
                      block: int = BLOCK, scale: float | None = None, sinks=None):
    """One sparse layer ([X] 3.4.3, [P] 3.1/3.3): block-sparse branch over the
    shared K/V at the inherited indices, window branch over its own K'/V',
    merged by the sigmoid gates.  sinks [2, Hq] or None (R14)."""
    o_sp = sparse_branch_rows(qs_rows, pos, k, v, idx, block, scale,
                              None if sinks is None else sinks[0])
    o_sw = window_branch_rows(qs_rows, pos, ks, vs, W, scale,
                              None if sinks is None else sinks[1])
    return gated_fusion(o_sp, o_sw, gates_rows)


def hybrid_block_rows(q, k, v, layers, pos, kb, W, block=BLOCK,
                      include_diag=False, score="max", scale=None):
    """The whole prefill hybrid block [Full, Sparse x N] for one sequence, at the
    query positions `pos` ([X] 3.2 information flow; [P] 3.1).

    q [T, Hq, d]; k, v [Hkv, T, d]; layers: list of dicts with q [T,Hq,d],
    k, v [Hkv,T,d] (the layer's own window K'/V') and gates [T,Hq,2] or None.
    Returns dict(o, lse, raw, Sg, idx, ranked, layer_out=[...]).
    """
    Hkv = k.shape[0]
    o, lse, raw = full_attention_rows(q[pos], pos, k, v, scale, block, score)
    idx, Sg, ranked = select_rows(raw, lse, pos, Hkv, kb, block, include_diag)
    outs = []
    for lay in layers:
        gates = None if lay.get("gates") is None else lay["gates"][pos]
        outs.append(sparse_layer_rows(lay["q"][pos], pos, k, v, idx, lay["k"], lay["v"],
                                      W, gates, block, scale, lay.get("sinks")))
    return dict(o=o, lse=lse, raw=raw, Sg=Sg, idx=idx, ranked=ranked, layer_out=outs)


# -------------------------------------------------------------------- decode
def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 e4m3fn code -> value (float64), from the bit fields: sign, 4-bit
    exponent with bias 7, 3-bit mantissa; exponent 0 is subnormal
    (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return s * val


def dequantize_e4m3(codes: np.ndarray, scale, head_axis: int = 0) -> np.ndarray:
    """Stored fp8 tensor -> values: decode_e4m3fn(code) * scale[h], with one
    fp32 scale per head along `head_axis` (reading R10: "per-head fp32
    scale")."""
    c = np.asarray(codes)
    s = np.asarray(scale, np.float64)
    shape = [1] * c.ndim
    shape[head_axis] = s.size
    return decode_e4m3fn(c) * s.reshape(shape)


def dequantize_kv(k: np.ndarray, v: np.ndarray, kv_scale, L: int | None = None):
    """fp8 key and value caches [Hkv, C, d] -> values of the first L positions:
    row 0 of kv_scale [2, Hkv] scales the keys, row 1 the values (R10)."""
    kv_scale = np.asarray(kv_scale, np.float64)
    return (dequantize_e4m3(k[:, :L], kv_scale[0], 0),
            dequantize_e4m3(v[:, :L], kv_scale[1], 0))


def window_from_ring(k_ring: np.ndarray, v_ring: np.ndarray, L: int, W: int):
    """Keys/values of the last min(L, W) positions, read from a W-slot ring
    where position p sits in slot p mod W (reading R8).  Returns them in
    position order, [Hkv, n, d] each."""
    p = np.arange(max(0, L - W), L)
    return k_ring[:, p % W], v_ring[:, p % W]


def decode_step(q, k, v, L, layers, kb, W, block=BLOCK, n_recent=0,
                kv_scale=None, scale=None):
    """One decode step of a hybrid block for one sequence ([H2] decode_one_token:
    exact scores of the full layer, selection, then the sparse followers).

    q [Hq, d]; k, v [Hkv, >=L, d] float64 values, or fp8 codes when kv_scale
    [2, Hkv] is given (value = decode_e4m3fn(code) * scale[K|V, g]).
    layers: dicts with q [Hq,d], optional k_ring/v_ring [Hkv,W,d], gates [Hq,2].
    block=64: block mode (top-kb blocks of the fully-past candidates, window
    branch, gates).  block=1: token mode of [H2] (top-kb old tokens + n_recent
    newest, no window, no gate).
    """
    Hkv = k.shape[0]
    if kv_scale is not None:
        k, v = dequantize_kv(k, v, kv_scale, L)
    pos = np.array([L - 1])
    o, lse, raw = full_attention_rows(q[None], pos, k, v, scale, block)
    Sg = group_max(block_scores(raw, lse), Hkv)          # [Hkv, 1, nblk]
    if block == 1:
        sel = []
        ranked = []
        for g in range(Hkv):
            s, rk = select_with_recent(Sg[g, 0], L - 1, kb, n_recent)
            sel.append(s)
            ranked.append(rk)
        n = max(len(s) for s in sel)
        idx = np.full((Hkv, 1, n), -1, np.int64)
        for g in range(Hkv):
            idx[g, 0, : len(sel[g])] = sel[g]
    else:
        idx, Sg, ranked_d = select_rows(raw, lse, pos, Hkv, kb, block, False)
        ranked = [ranked_d[g, 0] for g in range(Hkv)]
    outs = [decode_sparse_layer(lay, k, v, L, idx[:, 0], W, block, scale=scale) for lay in layers]
    return dict(o=o[0], lse=lse[:, 0], raw=raw[:, 0], Sg=Sg[:, 0], idx=idx[:, 0],
                ranked=ranked, layer_out=outs)


def decode_sparse_layer(lay, k, v, L, idx, W, block=BLOCK, kv_scale=None, scale=None):
    """One sparse layer at decode time for one sequence: the sparse branch over
    the selected blocks (block=64) or tokens (block=1) of the full layer's
    cache, the window branch over the layer's own ring, the sigmoid gates
    ([X] 3.4.3; [H2] decode_one_token).  idx [Hkv, n] (-1 = unused).
    Token mode has no window and no gate (reading R9).  lay["sinks"] [2, Hq]
    (optional, R14).  Returns o [Hq, d]."""
    if kv_scale is not None:
        k, v = dequantize_kv(k, v, kv_scale, L)
    pos = np.array([L - 1])
    qs = lay["q"][None]
    sinks = lay.get("sinks")
    o_sp = sparse_branch_rows(qs, pos, k, v, idx[:, None, :], block, scale,
                              None if sinks is None else sinks[0])
    if block == 1:
        return o_sp[0]
    if W == 0 or lay.get("k_ring") is None:
        o_sw = np.zeros_like(o_sp)
    else:
        kw, vw = window_from_ring(lay["k_ring"], lay["v_ring"], L, W)
        # window keys re-indexed 0..n-1 with the query at n-1
        o_sw = window_branch_rows(qs, np.array([kw.shape[1] - 1]), kw, vw, W, scale,
                                  None if sinks is None else sinks[1])
    gates = lay.get("gates")
    return gated_fusion(o_sp, o_sw, None if gates is None else gates[None])[0]


# --------------------------------------------------------------- KV offload
def gather_blocks(k: np.ndarray, v: np.ndarray, idx: np.ndarray, L: int, block: int = BLOCK):
    """K~, V~ of [X] 3.4.3 ("Branch 1", eq. K~,V~) as a stored cache: the
    selected blocks' keys and values concatenated, for one sequence.  This is
    what stays on the GPU when the full layer's cache is offloaded ([P] 5,
    "Potential of HySparse for Efficient KV Cache Offloading").

    k, v [Hkv, >=L, d]; idx [Hkv, n] block ids, read as a set of fully-past
    blocks, the decode candidates of reading R2 (ids 0 <= j < floor((L-1)/block),
    each once, ascending; a gathered block is whole, so the partly visible
    diagonal block is not kept).  Returns k_sel, v_sel [Hkv, n*block, d] (rows
    past the live blocks are zero) and idx_sel [Hkv, n]: p for the p-th live
    block, then -1.  A sparse branch over (k_sel, v_sel, idx_sel) at the query
    position L-1 attends exactly the keys it attends over (k, v, idx).
    """
    Hkv, _, d = k.shape
    n = idx.shape[1]
    k_sel = np.zeros((Hkv, n * block, d))
    v_sel = np.zeros((Hkv, n * block, d))
    idx_sel = np.full((Hkv, n), -1, np.int64)
    for g in range(Hkv):
        live = np.unique(idx[g][(idx[g] >= 0) & (idx[g] < (L - 1) // block)])
        for p, j in enumerate(live):
            k_sel[g, p * block: (p + 1) * block] = k[g, j * block: (j + 1) * block]
            v_sel[g, p * block: (p + 1) * block] = v[g, j * block: (j + 1) * block]
        idx_sel[g, : live.size] = np.arange(live.size)
    return k_sel, v_sel, idx_sel


# ----------------------------------------------------------------- backward
# Training backward of the hybrid block ([P] 4.1 "Experiments Setup": the
# models are pretrained with this architecture; [X] 3.4 "Training Pipeline":
# the sparse layers' gradients reach W_k, W_v through the shared K/V).  The
# selection is a discrete choice taken in the forward pass: indices are
# inputs here and get no gradient, nor do the block scores.  Each function
# is the chain rule of the forward definitions above, for one query row at a
# time; dO is the gradient of the loss with respect to a layer's output.
def _attend_bwd(s, values, keys, q, do, tau, sink=None):
    """Gradients of o = softmax([s, sink]) . values for one query row (s = tau
    q.keys^T over n keys, sink an extra logit with no value).  Returns dq
    [d], dkeys [n, d], dvalues [n, d], dsink (0 without a sink).  With
    p = softmax and o = p values: dvalues = p^T do, dp = values do,
    ds = p (dp - do.o), dq = tau ds keys, dkeys = tau ds^T q, and the sink's
    logit gets -p_sink do.o."""
    n, d = values.shape
    if n == 0 and sink is None:
        return np.zeros(q.shape[-1]), np.zeros((0, keys.shape[-1] if keys.ndim == 2 else 0)), np.zeros((0, d)), 0.0
    m = s.max() if n else -np.inf
    if sink is not None:
        m = max(m, sink)
    e = np.exp(s - m)
    z = e.sum() + (np.exp(sink - m) if sink is not None else 0.0)
    p = e / z
    o = p @ values if n else np.zeros(d)
    delta = float(do @ o)
    dvalues = np.outer(p, do)
    dp = values @ do
    ds = p * (dp - delta)
    dq = tau * (ds @ keys) if n else np.zeros(q.shape[-1])
    dkeys = tau * np.outer(ds, q)
    dsink = -float(np.exp(sink - m) / z) * delta if sink is not None else 0.0
    return dq, dkeys, dvalues, dsink


def full_attention_bwd(q, k, v, do, scale=None, rows=None):
    """Backward of the full causal layer (eq. o_t of [X] 3.4.1).
    q, do [T, Hq, d]; k, v [Hkv, T, d].  Returns dq [T, Hq, d], dk, dv [Hkv, T, d].
    rows: query positions to take (default all); dq is then exact at those
    rows, and dk, dv hold only those rows' contributions."""
    T, Hq, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    tau = softmax_scale(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for t in (range(T) if rows is None else rows):
        for h in range(Hq):
            g = h // G
            s = tau * (k[g, : t + 1] @ q[t, h])
            a, b_, c, _ = _attend_bwd(s, v[g, : t + 1], k[g, : t + 1], q[t, h], do[t, h], tau)
            dq[t, h] = a
            dk[g, : t + 1] += b_
            dv[g, : t + 1] += c
    return dq, dk, dv


def sparse_layer_bwd(qs, k, v, idx, ks, vs, W, gates, do, block=BLOCK, scale=None, sinks=None, rows=None):
    """Backward of one sparse layer ([X] 3.4.3: block-sparse branch over the
    shared K/V at the inherited indices, window branch over the layer's own
    K'/V', sigmoid gates; reading R14 sinks).
    qs, do [T, Hq, d]; k, v, ks, vs [Hkv, T, d]; idx [Hkv, T, n] (read as a
    set, as in the forward); gates [T, Hq, 2] or None; sinks [2, Hq] or None.
    Returns dict(dq [T,Hq,d], dk, dv [Hkv,T,d] (the shared K/V's share from
    this layer), dks, dvs [Hkv,T,d], dgates [T,Hq,2] or None, dsinks [2,Hq]
    or None).  With o = s0 o~ + s1 o' (s = sigmoid of the gate logits):
    do~ = s0 do, do' = s1 do, dG0 = s0 (1 - s0) do.o~, dG1 likewise.
    rows: as in full_attention_bwd."""
    T, Hq, d = qs.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    tau = softmax_scale(d) if scale is None else scale
    out = dict(dq=np.zeros_like(qs), dk=np.zeros_like(k), dv=np.zeros_like(v), dks=np.zeros_like(ks),
               dvs=np.zeros_like(vs), dgates=None if gates is None else np.zeros_like(gates),
               dsinks=None if sinks is None else np.zeros_like(sinks))
    for t in (range(T) if rows is None else rows):
        for h in range(Hq):
            g = h // G
            sel = idx[g, t]
            sel = np.unique(sel[sel >= 0])
            keys = (sel[:, None] * block + np.arange(block)[None, :]).reshape(-1)
            keys = keys[keys <= t]
            win = np.arange(max(0, t - W + 1), t + 1) if W > 0 else np.arange(0)
            b0 = None if sinks is None else sinks[0, h]
            b1 = None if sinks is None else sinks[1, h]
            o_sp, _ = _attend(tau * (qs[t, h] @ k[g, keys].T), v[g, keys], b0)
            o_sw, _ = _attend(tau * (qs[t, h] @ ks[g, win].T), vs[g, win], b1)
            s0, s1 = (1.0, 1.0) if gates is None else (sigmoid(gates[t, h, 0]), sigmoid(gates[t, h, 1]))
            if gates is not None:
                out["dgates"][t, h, 0] = s0 * (1 - s0) * float(do[t, h] @ o_sp)
                out["dgates"][t, h, 1] = s1 * (1 - s1) * float(do[t, h] @ o_sw)
            for (kk, vv, idxs, dkey, dval, gsc, sk, br) in (
                    (k, v, keys, "dk", "dv", s0, b0, 0), (ks, vs, win, "dks", "dvs", s1, b1, 1)):
                if idxs.size == 0 and sk is None:
                    continue
                sc = tau * (kk[g, idxs] @ qs[t, h])
                a, b_, c, dsk = _attend_bwd(sc, vv[g, idxs], kk[g, idxs], qs[t, h], gsc * do[t, h], tau, sk)
                out["dq"][t, h] += a
                np.add.at(out[dkey][g], idxs, b_)
                np.add.at(out[dval][g], idxs, c)
                if sinks is not None:
                    out["dsinks"][br, h] += dsk
    return out
