"""Thin ctypes binding of libhysparse.so (include/hysparse.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  A missing library raises immediately: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhysparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_WORKSPACE, HS_ERR_LAUNCH = range(5)
HS_F32, HS_BF16, HS_FP8_E4M3 = 0, 1, 2
HS_SCORE_MAX, HS_SCORE_LSE = 0, 1
HS_SEL_FULLY_PAST, HS_SEL_INCLUDE_DIAG = 0, 2
HS_FN_FULL_ATTN, HS_FN_BLOCK_TOPK, HS_FN_SPARSE_ATTN, HS_FN_DECODE_SELECT = range(4)
HS_FN_FULL_ATTN_BWD, HS_FN_SPARSE_ATTN_BWD = 4, 5
HS_FN_DECODE_TOKEN_SELECT = 6

EXPORTS = ("hs_full_attn_fwd_scores", "hs_block_topk", "hs_sparse_attn_fwd",
           "hs_decode_select_attn", "hs_decode_select_attn_static", "hs_gather_blocks",
           "hs_offload_full_select", "hs_offload_workspace_size", "hs_sparse_attn_fwd_train",
           "hs_full_attn_bwd", "hs_sparse_attn_bwd", "hs_decode_token_select", "hs_workspace_size",
           "hs_last_error", "hs_version")
HS_STATIC_SCRATCH_BYTES = 8 << 20


class HsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hysparse status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("batch", ctypes.c_int), ("q_len", ctypes.c_int), ("kv_len", ctypes.c_int),
        ("hq", ctypes.c_int), ("hkv", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("kv_lens", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p), ("swa_scale", ctypes.c_void_p),
    ]


def make_shape(batch, q_len, kv_len, hq, hkv, head_dim, dtype, kv_dtype=None, scale=0.0,
               kv_lens=None, kv_scale=None, q_scale=None, swa_scale=None) -> Shape:
    s = Shape()
    s.struct_size = ctypes.sizeof(Shape)
    s.batch, s.q_len, s.kv_len = batch, q_len, kv_len
    s.hq, s.hkv, s.head_dim = hq, hkv, head_dim
    s.dtype = dtype
    s.kv_dtype = dtype if kv_dtype is None else kv_dtype
    s.scale = scale
    s.kv_lens = _ptr(kv_lens)
    s.kv_scale = _ptr(kv_scale)
    s.q_scale = _ptr(q_scale)
    s.swa_scale = _ptr(swa_scale)
    return s


_lib = None


def load() -> ctypes.CDLL:
    """Load libhysparse.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m hybrid_sparse_attention_causal_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    SP = ctypes.POINTER(Shape)
    lib.hs_full_attn_fwd_scores.argtypes = [SP, P, P, P, P, P, P, I, I, P, Z, P]
    lib.hs_block_topk.argtypes = [SP, P, P, I, I, I, I, P, P, P, Z, P]
    lib.hs_sparse_attn_fwd.argtypes = [SP, P, P, P, P, I, P, P, I, P, P, P, P]
    lib.hs_decode_select_attn.argtypes = [SP, P, P, P, P, I, I, P, P, I, P, P, P, P, Z, P]
    lib.hs_decode_select_attn_static.argtypes = [SP, P, P, P, P, I, I, P, P, I, P, P, P, P]
    lib.hs_gather_blocks.argtypes = [SP, P, P, P, I, P, P, P, P]
    lib.hs_offload_full_select.argtypes = [SP, P, P, P, P, P, P, P, I, P, P, P, P, I, P, Z, P, P]
    lib.hs_offload_workspace_size.argtypes = [SP, I]
    lib.hs_offload_workspace_size.restype = Z
    lib.hs_sparse_attn_fwd_train.argtypes = [SP, P, P, P, P, I, P, P, I, P, P, P, P, P, P]
    lib.hs_full_attn_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.hs_sparse_attn_bwd.argtypes = [SP, P, P, P, P, I, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.hs_decode_token_select.argtypes = [SP, P, P, P, P, P, I, I, P, P, Z, P]
    lib.hs_workspace_size.argtypes = [I, SP, I, I, I]
    lib.hs_workspace_size.restype = Z
    lib.hs_last_error.restype = ctypes.c_char_p
    lib.hs_version.restype = I
    for name in ("hs_full_attn_fwd_scores", "hs_block_topk", "hs_sparse_attn_fwd",
                 "hs_decode_select_attn", "hs_decode_select_attn_static", "hs_gather_blocks",
                 "hs_offload_full_select", "hs_sparse_attn_fwd_train", "hs_full_attn_bwd",
                 "hs_sparse_attn_bwd", "hs_decode_token_select"):
        getattr(lib, name).restype = I
    del F
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream().cuda_stream


def _check(status: int):
    if status != HS_OK:
        raise HsError(status, load().hs_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: HS_F32, torch.bfloat16: HS_BF16, torch.uint8: HS_FP8_E4M3,
            torch.float8_e4m3fn: HS_FP8_E4M3}[t.dtype]


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to hysparse must be contiguous")


def _check_f32(name, t, shape):
    """fp32 side inputs read as raw floats by the kernels (gates, sinks)."""
    if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must be a float32 tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


# ------------------------------------------------------------------ prefill
def full_attn_fwd_scores(q, k, v_blk, o, lse, blk_raw, score=HS_SCORE_MAX, scale=0.0,
                         stream=None, q_scale=None, kv_scale=None):
    """Prefill full layer.  q [B,T,Hq,d], k [B,Hkv,T,d], v_blk [B,Hkv,nblk,d,64];
    outputs o [B,T,Hq,d], lse [B,Hq,T] fp32, blk_raw [B,Hq,T,nblk] fp32.
    fp8 (uint8 e4m3 codes): q_scale [Hq] and kv_scale [2,Hkv] fp32; o is bf16."""
    _contig(q, k, v_blk, o, lse, blk_raw, q_scale, kv_scale)
    B, T, Hq, d = q.shape
    Hkv = k.shape[1]
    _check_f32("q_scale", q_scale, (Hq,))
    _check_f32("kv_scale", kv_scale, (2, Hkv))
    s = make_shape(B, T, T, Hq, Hkv, d, dtype_code(q), scale=scale, kv_scale=kv_scale, q_scale=q_scale)
    _check(load().hs_full_attn_fwd_scores(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v_blk),
                                          _ptr(o), _ptr(lse), _ptr(blk_raw), 64, score,
                                          None, 0, _stream(stream)))


def block_topk(q_shape, blk_raw, lse, topk, idx, grp_score=None, include_diag=False,
               stream=None):
    """Prefill selection.  q_shape = (B, T, Hq, Hkv, d, dtype_code);
    idx [B,Hkv,T,topk] int32, grp_score [B,Hkv,T,nblk] fp32 or None."""
    _contig(blk_raw, lse, idx, grp_score)
    B, T, Hq, Hkv, d, dt = q_shape
    s = make_shape(B, T, T, Hq, Hkv, d, dt)
    flags = HS_SEL_INCLUDE_DIAG if include_diag else HS_SEL_FULLY_PAST
    _check(load().hs_block_topk(ctypes.byref(s), _ptr(blk_raw), _ptr(lse), 64, topk, 0, flags,
                                _ptr(grp_score), _ptr(idx), None, 0, _stream(stream)))


def sparse_attn_fwd(q_sp, k, v_blk, idx, topk, k_swa, v_swa_blk, window, gate_logits, o,
                    scale=0.0, stream=None, sinks=None, q_scale=None, kv_scale=None, swa_scale=None):
    """One prefill sparse layer.  q_sp/o [B,T,Hq,d]; k [B,Hkv,T,d]; v_blk, v_swa_blk
    [B,Hkv,nblk,d,64]; idx [B,Hkv,T,topk]; k_swa [B,Hkv,T,d]; gates [B,T,Hq,2] or None;
    sinks [2,Hq] fp32 (sparse, window branch) or None.  fp8 codes: q_scale [Hq],
    kv_scale [2,Hkv] (shared K, V), swa_scale [2,Hkv] (window K', V'); o is bf16."""
    _contig(q_sp, k, v_blk, idx, k_swa, v_swa_blk, gate_logits, sinks, o, q_scale, kv_scale, swa_scale)
    B, T, Hq, d = q_sp.shape
    _check_f32("gate_logits", gate_logits, (B, T, Hq, 2))
    _check_f32("sinks", sinks, (2, Hq))
    Hkv = (k if k is not None else k_swa).shape[1]
    _check_f32("q_scale", q_scale, (Hq,))
    _check_f32("kv_scale", kv_scale, (2, Hkv))
    _check_f32("swa_scale", swa_scale, (2, Hkv))
    s = make_shape(B, T, T, Hq, Hkv, d, dtype_code(q_sp), scale=scale, kv_scale=kv_scale, q_scale=q_scale,
                   swa_scale=swa_scale)
    _check(load().hs_sparse_attn_fwd(ctypes.byref(s), _ptr(q_sp), _ptr(k), _ptr(v_blk),
                                     _ptr(idx), topk, _ptr(k_swa), _ptr(v_swa_blk), window,
                                     _ptr(gate_logits), _ptr(sinks), _ptr(o), _stream(stream)))


# ------------------------------------------------------------------- decode
def workspace_size(fn_id, shape: Shape, block=64, topk=0, window=0) -> int:
    return load().hs_workspace_size(fn_id, ctypes.byref(shape), block, topk, window)


def decode_shape(q, k, lens, kv_scale=None, scale=0.0) -> Shape:
    """q [B,Hq,d]; k [B,Hkv,C,d] (the key cache); lens [B] int32 on the device."""
    B, Hq, d = q.shape
    Hkv, C = k.shape[1], k.shape[2]
    return make_shape(B, 1, C, Hq, Hkv, d, dtype_code(q), dtype_code(k), scale, lens, kv_scale)


def decode_full_attn_scores(q, k, v, lens, o, lse, raw, block=64, ws=None, kv_scale=None,
                            scale=0.0, stream=None):
    """Decode full layer.  q/o [B,Hq,d]; k [B,Hkv,C,d]; v [B,Hkv,C/64,d,64];
    lse [B,Hq]; raw [B,Hq,C/block].  ws: uint8 device tensor (allocated here
    when None)."""
    _contig(q, k, v, lens, o, lse, raw)
    s = decode_shape(q, k, lens, kv_scale, scale)
    need = workspace_size(HS_FN_FULL_ATTN, s, block)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(load().hs_full_attn_fwd_scores(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          _ptr(lse), _ptr(raw), block, HS_SCORE_MAX, _ptr(ws),
                                          ws.numel(), _stream(stream)))
    return ws


def decode_block_topk(q, k, lens, raw, lse, topk, idx, grp_score=None, block=64, n_recent=0,
                      kv_scale=None, stream=None):
    """Decode selection; idx [B,Hkv,topk(+n_recent)] int32."""
    _contig(raw, lse, idx, grp_score)
    s = decode_shape(q, k, lens, kv_scale)
    need = workspace_size(HS_FN_BLOCK_TOPK, s, block, topk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=raw.device) if need else None
    _check(load().hs_block_topk(ctypes.byref(s), _ptr(raw), _ptr(lse), block, topk, n_recent,
                                HS_SEL_FULLY_PAST, _ptr(grp_score), _ptr(idx), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)))


def decode_token_select(q, k, v, lens, o, lse, topk, n_recent, idx, kv_scale, ws=None, stream=None):
    """Token-level decode: the full layer's o [B,Hq,d], lse [B,Hq] and the
    token selection idx [B,Hkv,topk+n_recent] in one call, without per-token
    logits (fp8 caches k, v [B,Hkv,C,d] uint8 with kv_scale [2,Hkv]).  ws:
    uint8 device workspace (allocated here when None or too small); returned."""
    _contig(q, k, v, o, lse, idx)
    s = decode_shape(q, k, lens, kv_scale)
    need = workspace_size(HS_FN_DECODE_TOKEN_SELECT, s, 1, topk)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(load().hs_decode_token_select(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), topk,
                                         n_recent, _ptr(idx), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def decode_select_attn(q_sp, k, v, lens, idx, n_sel, k_ring, v_ring, window, gate_logits, o,
                       block=64, kv_scale=None, scale=0.0, stream=None, ws=None, sinks=None):
    """One decode sparse layer.  q_sp/o [B,Hq,d]; idx [B,Hkv,n_sel];
    k_ring [B,Hkv,W,d]; v_ring [B,Hkv,ceil(W/64),d,64]; gates [B,Hq,2] or None;
    sinks [2,Hq] fp32 or None (token mode uses row 0).
    ws: uint8 device workspace (allocated here when None and one is needed)."""
    _contig(q_sp, k, v, lens, idx, k_ring, v_ring, gate_logits, sinks, o)
    _check_f32("gate_logits", gate_logits, (q_sp.shape[0], q_sp.shape[1], 2))
    _check_f32("sinks", sinks, (2, q_sp.shape[1]))
    s = decode_shape(q_sp, k, lens, kv_scale, scale)
    if ws is None:
        need = workspace_size(HS_FN_DECODE_SELECT, s, block)
        ws = torch.empty(need, dtype=torch.uint8, device=q_sp.device) if need else None
    _check(load().hs_decode_select_attn(ctypes.byref(s), _ptr(q_sp), _ptr(k), _ptr(v), _ptr(idx),
                                        n_sel, block, _ptr(k_ring), _ptr(v_ring), window,
                                        _ptr(gate_logits), _ptr(sinks), _ptr(o), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)))
    return ws


def decode_select_attn_static(q_sp, k, v, lens, idx, n_sel, k_ring, v_ring, window, gate_logits, o,
                              block=64, kv_scale=None, scale=0.0, stream=None, sinks=None):
    """hs_decode_select_attn_static: decode_select_attn with no workspace (the
    library's fixed per-GPU scratch holds the token-mode split partials)."""
    _contig(q_sp, k, v, lens, idx, k_ring, v_ring, gate_logits, sinks, o)
    _check_f32("gate_logits", gate_logits, (q_sp.shape[0], q_sp.shape[1], 2))
    _check_f32("sinks", sinks, (2, q_sp.shape[1]))
    s = decode_shape(q_sp, k, lens, kv_scale, scale)
    _check(load().hs_decode_select_attn_static(ctypes.byref(s), _ptr(q_sp), _ptr(k), _ptr(v), _ptr(idx),
                                               n_sel, block, _ptr(k_ring), _ptr(v_ring), window,
                                               _ptr(gate_logits), _ptr(sinks), _ptr(o), _stream(stream)))


# ------------------------------------------------------------- training
def sparse_attn_fwd_train(q_sp, k, v_blk, idx, topk, k_swa, v_swa_blk, window, gate_logits, o, o_branch,
                          lse_branch, scale=0.0, stream=None, sinks=None):
    """sparse_attn_fwd (bf16) that also writes each branch's output o_branch
    [2,B,T,Hq,d] bf16 and LSE lse_branch [2,B,Hq,T] fp32 for the backward."""
    _contig(q_sp, k, v_blk, idx, k_swa, v_swa_blk, gate_logits, sinks, o, o_branch, lse_branch)
    B, T, Hq, d = q_sp.shape
    _check_f32("gate_logits", gate_logits, (B, T, Hq, 2))
    _check_f32("sinks", sinks, (2, Hq))
    Hkv = (k if k is not None else k_swa).shape[1]
    s = make_shape(B, T, T, Hq, Hkv, d, dtype_code(q_sp), scale=scale)
    _check(load().hs_sparse_attn_fwd_train(ctypes.byref(s), _ptr(q_sp), _ptr(k), _ptr(v_blk), _ptr(idx), topk,
                                           _ptr(k_swa), _ptr(v_swa_blk), window, _ptr(gate_logits), _ptr(sinks),
                                           _ptr(o), _ptr(o_branch), _ptr(lse_branch), _stream(stream)))


def _bwd_ws(fn_id, s, device, ws, topk=0):
    need = load().hs_workspace_size(fn_id, ctypes.byref(s), 64, topk, 0)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws


def full_attn_bwd(q, k, v_blk, o, lse, dout, dq, dk, dv, ws=None, scale=0.0, stream=None):
    """Backward of the full layer (bf16).  dq [B,T,Hq,d], dk/dv [B,Hkv,T,d] fp32
    (overwritten).  ws: uint8 device workspace (allocated here when None or
    too small); returned for reuse."""
    _contig(q, k, v_blk, o, lse, dout, dq, dk, dv)
    B, T, Hq, d = q.shape
    s = make_shape(B, T, T, Hq, k.shape[1], d, dtype_code(q), scale=scale)
    ws = _bwd_ws(HS_FN_FULL_ATTN_BWD, s, q.device, ws)
    _check(load().hs_full_attn_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v_blk), _ptr(o), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def sparse_attn_bwd(q_sp, k, v_blk, idx, topk, k_swa, v_swa_blk, window, gate_logits, sinks, o_branch,
                    lse_branch, dout, dq, dk, dv, dk_swa, dv_swa, dgate=None, dsinks=None, ws=None, scale=0.0,
                    stream=None):
    """Backward of one sparse layer (bf16).  dq [B,T,Hq,d] fp32 (out); dk/dv
    [B,Hkv,T,d] fp32 receive this layer's share ADDED; dk_swa/dv_swa
    [B,Hkv,T,d] fp32, dgate [B,T,Hq,2], dsinks [2,Hq] (out)."""
    _contig(q_sp, k, v_blk, idx, k_swa, v_swa_blk, gate_logits, sinks, o_branch, lse_branch, dout, dq, dk, dv,
            dk_swa, dv_swa, dgate, dsinks)
    B, T, Hq, d = q_sp.shape
    Hkv = (k if k is not None else k_swa).shape[1]
    s = make_shape(B, T, T, Hq, Hkv, d, dtype_code(q_sp), scale=scale)
    ws = _bwd_ws(HS_FN_SPARSE_ATTN_BWD, s, q_sp.device, ws, topk)
    _check(load().hs_sparse_attn_bwd(ctypes.byref(s), _ptr(q_sp), _ptr(k), _ptr(v_blk), _ptr(idx), topk,
                                     _ptr(k_swa), _ptr(v_swa_blk), window, _ptr(gate_logits), _ptr(sinks),
                                     _ptr(o_branch), _ptr(lse_branch), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _ptr(dk_swa), _ptr(dv_swa), _ptr(dgate), _ptr(dsinks), _ptr(ws), ws.numel(),
                                     _stream(stream)))
    return ws


# ------------------------------------------------------------ KV offload
def gather_blocks(k, v, lens, idx, n_sel, k_sel, v_sel, idx_sel, stream=None):
    """Selected blocks of a block-mode cache into a compact cache.  k [B,Hkv,C,d],
    v [B,Hkv,C/64,d,64]; idx [B,Hkv,n_sel]; k_sel [B,Hkv,n_sel*64,d],
    v_sel [B,Hkv,n_sel,d,64], idx_sel [B,Hkv,n_sel] int32 (out)."""
    _contig(k, v, lens, idx, k_sel, v_sel, idx_sel)
    B, Hkv, C, d = k.shape
    s = make_shape(B, 1, C, Hkv, Hkv, d, HS_BF16, HS_BF16, 0.0, lens, None)
    _check(load().hs_gather_blocks(ctypes.byref(s), _ptr(k), _ptr(v), _ptr(idx), n_sel, _ptr(k_sel),
                                   _ptr(v_sel), _ptr(idx_sel), _stream(stream)))


def offload_workspace_size(q, k_host, lens, chunk) -> int:
    return load().hs_offload_workspace_size(ctypes.byref(decode_shape(q, k_host, lens)), chunk)


def offload_full_select(q, k_host, v_host, lens, lens_host, o, lse, raw, topk, idx, k_sel, v_sel, idx_sel,
                        chunk, ws, stream=None, copy_stream=None, scale=0.0):
    """Full layer + selection + gather over host-resident caches (pinned CPU
    tensors k_host [B,Hkv,C,d], v_host [B,Hkv,C/64,d,64]); lens on the device
    and lens_host (int32 CPU tensor) with the same values; ws a uint8 device
    tensor of offload_workspace_size bytes."""
    _contig(q, k_host, v_host, lens, lens_host, o, lse, raw, idx, k_sel, v_sel, idx_sel, ws)
    if lens_host.dtype != torch.int32 or lens_host.device.type != "cpu":
        raise ValueError("lens_host must be an int32 CPU tensor")
    s = decode_shape(q, k_host, lens, None, scale)
    cs = _stream(copy_stream) if copy_stream is not None else None
    _check(load().hs_offload_full_select(ctypes.byref(s), _ptr(lens_host), _ptr(q), _ptr(k_host), _ptr(v_host),
                                         _ptr(o), _ptr(lse), _ptr(raw), topk, _ptr(idx), _ptr(k_sel), _ptr(v_sel),
                                         _ptr(idx_sel), chunk, _ptr(ws), ws.numel(), _stream(stream), cs))


def version() -> int:
    return load().hs_version()
