"""Seeded synthetic inputs for the hybrid-block attention path.

This module is shared by the fp64 oracle tests and by the GPU path (tests, bench).
It only draws random numbers, plants the salient keys, rounds to the storage
format and rearranges memory layouts; it contains none of the attention
arithmetic. It imports numpy only (torch is used lazily for the fp8 encoder).

Workloads (the five seeded configurations of this repository):
  1  tiny 1:3 prefill      B=1  T=1024  Hq=4  Hkv=1 d=64  fp32  kb=4  W=128 N=3  f=2%
  2  7B-shaped 1:3 prefill B=1  T=8192  Hq=32 Hkv=8 d=128 bf16  kb=16 W=512 N=3  f=1%
  3  80B-shaped 1:11       B=1  T=32768 Hq=32 Hkv=4 d=128 bf16  kb=32 W=128 N=11 f=0.5%
  4  1:11 decode           B=64 L~U[32768,65536] Hq=32 Hkv=4 d=128 bf16 kb=32 W=128 N=11
  5  token-level decode    B=16 L=262144 Hq=32 Hkv=4 d=128 fp8-e4m3 KV, top-2048 + 128 recent, N=11

Value recipe (HySparse explainer, "3.4.1 Full Attention Layer" for the GQA
shapes; the salient-key structure stands in for the salient tokens of the
paper's section 2.3):
  * Q, K, V ~ N(0,1)/d^(1/4); one random unit vector c_g per kv head.
  * round(f*L) salient key positions per sequence (shared by all kv heads):
    K[g, i] += 3 c_g.  Every query row of group g (full and sparse layers) gets
    += 1.5 c_g.
  * Sliding-window K', V' ~ N(0,1); gate logits ~ N(0,1) per token and head.
  * Decode configuration 5: K, V ~ N(0,1) rounded to bf16, planted, then
    quantised to OCP fp8 e4m3 with one fp32 scale per (K or V, kv head)
    = amax/448 over that head's whole tensor.
  * fp8 prefill (dtype 'fp8' on a prefill configuration): every tensor is
    drawn and planted as for bf16, rounded to bf16, then quantised to e4m3
    with one scale per head = amax/448 over that head's values: queries per
    query head (q_scale [Hq]), K and V per kv head (kv_scale [2, Hkv]), each
    layer's queries and window K'/V' likewise (q_scale, swa_scale).

Storage formats: 'f32' -> float32 arrays, 'bf16' -> uint16 bit patterns (RNE),
'fp8' -> uint8 e4m3fn codes plus float32 scales.

Random streams: numpy default_rng([seed, stream, *slab]) where seed is the
configuration number, so any slab (one sequence, one kv head) can be
regenerated on its own; stream ids: 0 Q, 1 K, 2 V, 3 c, 4 salient positions,
5 sequence lengths, 10+l Q'_l, 30+l K'_l, 50+l V'_l, 70+l gates_l,
90+l sinks_l.

Sink logits (optional, not part of the five workloads): per layer, [2][Hq]
float32 ~ N(2, 1.5^2), row 0 for the sparse and row 1 for the window branch,
so that they sit near the typical largest logit and matter.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BLOCK = 64


@dataclass(frozen=True)
class Config:
    cid: int
    kind: str          # 'prefill' | 'decode_block' | 'decode_token'
    B: int
    T: int             # prefill length, or cache capacity (decode)
    Hq: int
    Hkv: int
    d: int
    dtype: str         # storage dtype of Q/K/V: 'f32' | 'bf16' | 'fp8' (KV only)
    N: int             # sparse layers per hybrid block
    frac: float        # planted salient fraction
    kb: int            # top-k in blocks (block mode) or tokens (token mode)
    W: int             # sliding window (0 = none)
    L_lo: int = 0      # decode: ragged length range (inclusive)
    L_hi: int = 0
    n_recent: int = 0  # token mode: newest tokens forced into the selection
    include_diag: bool = False
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nblk(self) -> int:
        return (self.T + BLOCK - 1) // BLOCK


CONFIGS = {
    1: Config(1, "prefill", 1, 1024, 4, 1, 64, "f32", 3, 0.02, 4, 128, seed=1),
    2: Config(2, "prefill", 1, 8192, 32, 8, 128, "bf16", 3, 0.01, 16, 512, seed=2),
    3: Config(3, "prefill", 1, 32768, 32, 4, 128, "bf16", 11, 0.005, 32, 128, seed=3),
    4: Config(4, "decode_block", 64, 65536, 32, 4, 128, "bf16", 11, 0.005, 32, 128,
              L_lo=32768, L_hi=65536, seed=4),
    5: Config(5, "decode_token", 16, 262144, 32, 4, 128, "fp8", 11, 0.001, 2048, 0,
              L_lo=262144, L_hi=262144, n_recent=128, seed=5),
}


def config(cid: int, **overrides) -> Config:
    c = CONFIGS[cid]
    return replace(c, **overrides) if overrides else c


# --------------------------------------------------------------------------- rng
def _rng(cfg: Config, stream: int, *slab: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, stream, *slab])


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    return out


_CHUNK = 1 << 22  # elements per independently seeded chunk


def _normal_big(cfg: "Config", stream: int, shape) -> np.ndarray:
    """N(0,1) float32 array drawn in fixed 4M-element chunks, chunk i from
    default_rng([seed, stream, 1000 + i]); filled by a thread pool, the result
    does not depend on the thread count."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1)
    n = flat.size
    nch = (n + _CHUNK - 1) // _CHUNK

    def one(i):
        seg = flat[i * _CHUNK: min(n, (i + 1) * _CHUNK)]
        _rng(cfg, stream, 1000 + i).standard_normal(out=seg, dtype=np.float32)

    if nch <= 1:
        one(0) if n else None
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nch)))
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ------------------------------------------------------------------ encodings
def _bf16_chunk(u: np.ndarray, out: np.ndarray) -> None:
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    out[...] = r


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 (or float64, first rounded to float32) to bf16, RNE.
    Works in 1M-element chunks on a thread pool (numpy releases the GIL)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    uf, of = u.reshape(-1), out.reshape(-1)
    n, ch = uf.size, 1 << 20
    if n <= ch:
        _bf16_chunk(uf, of)
        return out
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda i: _bf16_chunk(uf[i:i + ch], of[i:i + ch]), range(0, n, ch)))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP fp8 e4m3fn codes, round-to-nearest-even, saturating at 448."""
    import torch

    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float32 (exact for f32/bf16)."""
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(dtype)


def block_major(v: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """[..., T, d] -> [..., ceil(T/block), d, block] (each block stored d-major).

    This is the value-cache layout the HIP kernels read; the tail of the last
    block is zero-filled.  Pure data movement.
    """
    *lead, T, d = v.shape
    nb = (T + block - 1) // block
    pad = nb * block - T
    if pad:
        v = np.concatenate([v, np.zeros((*lead, pad, d), v.dtype)], axis=-2)
    v = v.reshape(*lead, nb, block, d)
    return np.ascontiguousarray(np.swapaxes(v, -1, -2))


# --------------------------------------------------------------------- prefill
@dataclass
class PrefillInputs:
    cfg: Config
    q: np.ndarray                 # [B,T,Hq,d] stored
    k: np.ndarray                 # [B,Hkv,T,d] stored
    v: np.ndarray                 # [B,Hkv,T,d] stored
    layers: list = field(default_factory=list)  # per sparse layer dict q,k,v,gates
                                                 # (+ q_scale, swa_scale for fp8)
    salient: list = field(default_factory=list)  # per batch index arrays
    q_scale: np.ndarray | None = None   # fp8: [Hq] float32
    kv_scale: np.ndarray | None = None  # fp8: [2, Hkv] float32

    def f64(self, name: str, layer: int | None = None) -> np.ndarray:
        """Stored values as float64 (f32/bf16 storage; gates).  fp8 codes are
        decoded by the oracle, with the scales, not here."""
        src = self.layers[layer][name] if layer is not None else getattr(self, name)
        if name == "gates":
            return src.astype(np.float64)
        return to_f32(src, self.cfg.dtype).astype(np.float64)


def _fp8_per_head(x: np.ndarray, head_axis: int):
    """Round float32 values to bf16, then quantise to e4m3 codes with one
    scale per index of `head_axis` = amax/448 of that head's values."""
    x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    axes = tuple(i for i in range(x.ndim) if i != head_axis)
    amax = np.abs(x).max(axis=axes).astype(np.float64)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    return encode_e4m3(x / scale.reshape(shape)), scale


def _unit_vectors(cfg: Config) -> np.ndarray:
    z = _rng(cfg, 3).standard_normal((cfg.Hkv, cfg.d))
    return z / np.linalg.norm(z, axis=1, keepdims=True)


def _salient(cfg: Config, L: int, b: int) -> np.ndarray:
    n = int(round(cfg.frac * L))
    return np.sort(_rng(cfg, 4, b).choice(L, size=n, replace=False))


def _queries(cfg: Config, stream: int, c: np.ndarray, lead) -> np.ndarray:
    """Q ~ N(0,1)/d^(1/4) + 1.5 c_g, shape [*lead, Hq, d] (float32)."""
    x = _normal_big(cfg, stream, (*lead, cfg.Hq, cfg.d))
    x *= np.float32(cfg.d ** -0.25)
    x += (1.5 * np.repeat(c, cfg.G, axis=0)).astype(np.float32)
    return x


def make_prefill(cfg: Config, n_layers: int | None = None) -> PrefillInputs:
    """All inputs of one prefill hybrid block (full layer + n_layers sparse)."""
    assert cfg.kind == "prefill"
    B, T, Hkv, d = cfg.B, cfg.T, cfg.Hkv, cfg.d
    nl = cfg.N if n_layers is None else n_layers
    c = _unit_vectors(cfg)
    s = np.float32(d ** -0.25)
    q = _queries(cfg, 0, c, (B, T))
    k = _normal_big(cfg, 1, (B, Hkv, T, d)) * s
    v = _normal_big(cfg, 2, (B, Hkv, T, d)) * s
    sal = []
    for b in range(B):
        pos = _salient(cfg, T, b)
        sal.append(pos)
        k[b][:, pos, :] += (3.0 * c[:, None, :]).astype(np.float32)
    layers = []
    for l in range(nl):
        ql = _queries(cfg, 10 + l, c, (B, T))
        kl = _normal_big(cfg, 30 + l, (B, Hkv, T, d))
        vl = _normal_big(cfg, 50 + l, (B, Hkv, T, d))
        gl = _normal_big(cfg, 70 + l, (B, T, cfg.Hq, 2))
        if cfg.dtype == "fp8":
            qc, qs = _fp8_per_head(ql, 2)
            kc, ks = _fp8_per_head(kl, 1)
            vc, vs = _fp8_per_head(vl, 1)
            layers.append(dict(q=qc, k=kc, v=vc, gates=gl, q_scale=qs, swa_scale=np.stack([ks, vs])))
        else:
            layers.append(dict(q=store(ql, cfg.dtype), k=store(kl, cfg.dtype),
                               v=store(vl, cfg.dtype), gates=gl))
    if cfg.dtype == "fp8":
        qc, qs = _fp8_per_head(q, 2)
        kc, ks = _fp8_per_head(k, 1)
        vc, vs = _fp8_per_head(v, 1)
        return PrefillInputs(cfg, qc, kc, vc, layers, sal, qs, np.stack([ks, vs]))
    return PrefillInputs(cfg, store(q, cfg.dtype), store(k, cfg.dtype),
                         store(v, cfg.dtype), layers, sal)


# ---------------------------------------------------------------------- decode
@dataclass
class DecodeInputs:
    cfg: Config
    lens: np.ndarray              # [B] int32 context lengths (query at L-1)
    q: np.ndarray                 # [B,Hq,d] stored (bf16 for fp8 configs)
    layers: list                  # per layer dict q [B,Hq,d], k_ring/v_ring [B,Hkv,W,d], gates [B,Hq,2]
    c: np.ndarray                 # [Hkv,d] planted directions
    kv_scale: np.ndarray | None   # [2,Hkv] fp32 (fp8 only)
    qdtype: str

    def kv_slab(self, b: int, g: int):
        """Stored K, V of one (sequence, kv head): [L_b, d] each."""
        return _decode_kv_slab(self.cfg, self.c, int(self.lens[b]), b, g, self.kv_scale)

    def kv_slab_f64(self, b: int, g: int):
        k, v = self.kv_slab(b, g)
        if self.cfg.dtype == "fp8":
            return k, v  # codes; the oracle decodes them itself
        return (to_f32(k, self.cfg.dtype).astype(np.float64),
                to_f32(v, self.cfg.dtype).astype(np.float64))


def _decode_lens(cfg: Config) -> np.ndarray:
    if cfg.L_lo == cfg.L_hi:
        return np.full(cfg.B, cfg.L_hi, np.int32)
    return _rng(cfg, 5).integers(cfg.L_lo, cfg.L_hi, size=cfg.B, endpoint=True).astype(np.int32)


def _kv_raw(cfg: Config, c: np.ndarray, L: int, b: int, g: int):
    """float32 K, V of one slab before storage rounding (planted)."""
    scale = np.float32(1.0) if cfg.dtype == "fp8" else np.float32(cfg.d ** -0.25)
    k = _normal(_rng(cfg, 1, b, g), (L, cfg.d)) * scale
    v = _normal(_rng(cfg, 2, b, g), (L, cfg.d)) * scale
    if cfg.dtype == "fp8":
        k = bf16_bits_to_f32(f32_to_bf16_bits(k))
        v = bf16_bits_to_f32(f32_to_bf16_bits(v))
    pos = _salient(cfg, L, b)
    k[pos] += (3.0 * c[g]).astype(np.float32)
    if cfg.dtype == "fp8":
        k = bf16_bits_to_f32(f32_to_bf16_bits(k))
    return k, v


def _decode_kv_slab(cfg, c, L, b, g, kv_scale):
    k, v = _kv_raw(cfg, c, L, b, g)
    if cfg.dtype == "fp8":
        return encode_e4m3(k / kv_scale[0, g]), encode_e4m3(v / kv_scale[1, g])
    return store(k, cfg.dtype), store(v, cfg.dtype)


def _fp8_scales(cfg: Config, c: np.ndarray, lens: np.ndarray) -> np.ndarray:
    amax = np.zeros((2, cfg.Hkv), np.float64)

    def one(bg):
        b, g = bg
        k, v = _kv_raw(cfg, c, int(lens[b]), b, g)
        return b, g, float(np.abs(k).max()), float(np.abs(v).max())

    jobs = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        for b, g, ka, va in ex.map(one, jobs):
            amax[0, g] = max(amax[0, g], ka)
            amax[1, g] = max(amax[1, g], va)
    return (amax / 448.0).astype(np.float32)


def make_sinks(cfg: Config, layer: int = 0) -> np.ndarray:
    """Sink logits [2, Hq] float32 of sparse layer `layer` (stream 90+layer)."""
    r = _rng(cfg, 90 + layer)
    return (2.0 + 1.5 * r.standard_normal((2, cfg.Hq))).astype(np.float32)


def make_decode(cfg: Config, n_layers: int | None = None) -> DecodeInputs:
    assert cfg.kind.startswith("decode")
    B, Hkv, d = cfg.B, cfg.Hkv, cfg.d
    nl = cfg.N if n_layers is None else n_layers
    c = _unit_vectors(cfg)
    lens = _decode_lens(cfg)
    qd = "bf16" if cfg.dtype == "fp8" else cfg.dtype
    q = store(_queries(cfg, 0, c, (B,)), qd)
    layers = []
    for l in range(nl):
        lay = dict(q=store(_queries(cfg, 10 + l, c, (B,)), qd))
        if cfg.W > 0:
            lay["k_ring"] = store(_normal(_rng(cfg, 30 + l), (B, Hkv, cfg.W, d)), qd)
            lay["v_ring"] = store(_normal(_rng(cfg, 50 + l), (B, Hkv, cfg.W, d)), qd)
        if cfg.kind == "decode_block":
            lay["gates"] = _normal(_rng(cfg, 70 + l), (B, cfg.Hq, 2))
        layers.append(lay)
    scale = _fp8_scales(cfg, c, lens) if cfg.dtype == "fp8" else None
    return DecodeInputs(cfg, lens, q, layers, c, scale, qd)


def fill_decode_cache(inp: DecodeInputs, k_out: np.ndarray, v_out: np.ndarray,
                      v_block_major: bool = True, poison: bool = True) -> None:
    """Write every (sequence, kv head) slab into caller-provided cache arrays.

    k_out: [B,Hkv,T,d]; v_out: [B,Hkv,T/64,d,64] (block-major) or [B,Hkv,T,d].
    Positions >= L_b are poisoned with NaN (bf16/f32) or the fp8 NaN code 0x7F.
    """
    cfg = inp.cfg
    nan = {"bf16": np.uint16(0x7FC0), "f32": np.float32(np.nan), "fp8": np.uint8(0x7F)}[cfg.dtype]

    def one(bg):
        b, g = bg
        L = int(inp.lens[b])
        k, v = inp.kv_slab(b, g)
        k_out[b, g, :L] = k
        if poison:
            k_out[b, g, L:] = nan
        if v_block_major:
            nb = (L + BLOCK - 1) // BLOCK
            vb = block_major(v)
            v_out[b, g, :nb] = vb
            if poison:
                if L % BLOCK:
                    v_out[b, g, nb - 1, :, L % BLOCK:] = nan
                v_out[b, g, nb:] = nan
        else:
            v_out[b, g, :L] = v
            if poison:
                v_out[b, g, L:] = nan

    jobs = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, jobs))


def ring_slot_positions(L: int, W: int) -> np.ndarray:
    """Position held by each slot of a W-slot ring after L tokens (slot = pos mod W);
    -1 for slots never written (L < W)."""
    pos = np.full(W, -1, np.int64)
    for p in range(max(0, L - W), L):
        pos[p % W] = p
    return pos


def stored_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[dtype]
