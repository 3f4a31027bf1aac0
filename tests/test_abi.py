"""The C-ABI library: it loads, exports every symbol include/hysparse.h
declares, and rejects bad arguments before touching the GPU (so these run on a
machine without one: validation happens before any HIP call)."""
import ctypes
import os
import re

import pytest

from hybrid_sparse_attention_causal_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hysparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hb.LIB_PATH),
                                reason="libhysparse.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_0-9]+)\s*\(", src)))


def test_no_undefined_library_symbols():
    """Every symbol of the library's own code (kernel launch stubs included)
    is defined in it: an undefined one would only fail at its first launch."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", hb.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    own = [l.split()[-1] for l in out.splitlines() if "_ZN2hs" in l or l.split()[-1].startswith("hs_")]
    assert not own, own[:5]


def test_exports_every_declared_symbol():
    lib = hb.load()
    names = declared_functions()
    assert set(names) == set(hb.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert hb.version() >= 100


def _shape(**kw):
    args = dict(batch=1, q_len=128, kv_len=128, hq=8, hkv=2, head_dim=128, dtype=hb.HS_BF16)
    args.update(kw)
    return hb.make_shape(**args)


FAKE = 1 << 20  # a 16-byte aligned non-null pointer value; never dereferenced


def _full(s, block=64, flags=0, ptrs=FAKE):
    lib = hb.load()
    return lib.hs_full_attn_fwd_scores(ctypes.byref(s), ptrs, ptrs, ptrs, ptrs, ptrs, ptrs,
                                       block, flags, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=6, hkv=4), hb.HS_ERR_INVALID_ARG),
    (dict(hq=12, hkv=4), hb.HS_ERR_UNSUPPORTED),      # group of 3
    (dict(head_dim=96), hb.HS_ERR_UNSUPPORTED),
    (dict(dtype=hb.HS_FP8_E4M3, head_dim=64), hb.HS_ERR_UNSUPPORTED),   # fp8 prefill: head_dim 128
    (dict(dtype=hb.HS_FP8_E4M3, hq=64, hkv=2), hb.HS_ERR_UNSUPPORTED),  # fp8 prefill: groups <= 16
    (dict(dtype=hb.HS_FP8_E4M3), hb.HS_ERR_INVALID_ARG),                # no q_scale / kv_scale
    (dict(dtype=hb.HS_FP8_E4M3, kv_dtype=hb.HS_BF16), hb.HS_ERR_UNSUPPORTED),
    (dict(q_len=-1), hb.HS_ERR_INVALID_ARG),
    (dict(kv_len=64), hb.HS_ERR_INVALID_ARG),          # prefill needs q_len == kv_len
    (dict(scale=float("nan")), hb.HS_ERR_INVALID_ARG),
])
def test_full_attn_rejects_bad_shapes(kw, status):
    assert _full(_shape(**kw)) == status
    assert hb.load().hs_last_error().decode()


def test_full_attn_rejects_bad_args():
    s = _shape()
    assert _full(s, block=32) == hb.HS_ERR_UNSUPPORTED
    assert _full(s, flags=7) == hb.HS_ERR_INVALID_ARG
    assert _full(s, ptrs=None) == hb.HS_ERR_INVALID_ARG
    assert _full(s, ptrs=FAKE + 4) == hb.HS_ERR_INVALID_ARG   # misaligned
    bad = _shape()
    bad.struct_size = 8
    assert _full(bad) == hb.HS_ERR_INVALID_ARG
    assert hb.load().hs_full_attn_fwd_scores(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 0,
                                             None, 0, None) == hb.HS_ERR_INVALID_ARG


def test_shape_without_appended_fields():
    """A caller built against the first hs_shape (ending after kv_scale) is
    accepted: the appended fields are read as NULL."""
    s = _shape()
    s.struct_size = hb.Shape.kv_scale.offset + ctypes.sizeof(ctypes.c_void_p)
    s.q_scale = FAKE + 3          # garbage past the caller's struct is not read
    assert _full(s, ptrs=None) == hb.HS_ERR_INVALID_ARG   # fails on the null q, not the struct
    assert "q is NULL" in hb.load().hs_last_error().decode()
    s.struct_size -= 8
    assert _full(s) == hb.HS_ERR_INVALID_ARG
    assert "struct_size" in hb.load().hs_last_error().decode()


def test_empty_problem_is_a_no_op():
    assert _full(_shape(q_len=0, kv_len=0), ptrs=None) == hb.HS_OK
    assert _full(_shape(batch=0), ptrs=None) == hb.HS_OK


def test_topk_and_sparse_validation():
    lib = hb.load()
    s = _shape()
    assert lib.hs_block_topk(ctypes.byref(s), FAKE, FAKE, 64, 0, 0, 0, None, FAKE, None, 0,
                             None) == hb.HS_ERR_INVALID_ARG
    assert lib.hs_block_topk(ctypes.byref(s), FAKE, FAKE, 64, 4, 0, 5, None, FAKE, None, 0,
                             None) == hb.HS_ERR_INVALID_ARG
    assert lib.hs_block_topk(ctypes.byref(s), None, FAKE, 64, 4, 0, 0, None, FAKE, None, 0,
                             None) == hb.HS_ERR_INVALID_ARG
    assert lib.hs_sparse_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 4, None, None, 16,
                                  None, None, FAKE, None) == hb.HS_ERR_INVALID_ARG   # window w/o cache
    assert lib.hs_sparse_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, -1, None, None, 0,
                                  None, None, FAKE, None) == hb.HS_ERR_INVALID_ARG


def test_binding_rejects_bad_side_inputs():
    """Gates and sinks are read as raw fp32 by the kernels: the binding checks
    their dtype and shape before anything is launched."""
    import torch

    B, T, Hq, Hkv, d = 1, 64, 4, 2, 64
    q = torch.zeros((B, T, Hq, d), dtype=torch.bfloat16)
    k = torch.zeros((B, Hkv, T, d), dtype=torch.bfloat16)
    v = torch.zeros((B, Hkv, 1, d, 64), dtype=torch.bfloat16)
    idx = torch.zeros((B, Hkv, T, 2), dtype=torch.int32)
    o = torch.zeros_like(q)
    good_g = torch.zeros((B, T, Hq, 2))
    for g, s in ((good_g.double(), None), (torch.zeros((B, T, Hq, 3)), None),
                 (good_g, torch.zeros((2, Hq), dtype=torch.float64)), (good_g, torch.zeros((1, Hq)))):
        with pytest.raises(ValueError):
            hb.sparse_attn_fwd(q, k, v, idx, 2, None, None, 0, g, o, sinks=s)


def _dshape(**kw):
    """A decode shape whose kv_lens points at a fake (never read) address."""
    args = dict(batch=2, q_len=1, kv_len=1024, hq=8, hkv=2, head_dim=128, dtype=hb.HS_BF16,
                kv_lens=FAKE)
    args.update(kw)
    return hb.make_shape(**args)


def _dsel(s, idx=FAKE, n_sel=4, block=64, ring=FAKE, window=64, gates=None, ptrs=FAKE, ws=None, ws_bytes=0):
    lib = hb.load()
    return lib.hs_decode_select_attn(ctypes.byref(s), ptrs, ptrs, ptrs, idx, n_sel, block, ring, ring,
                                     window, gates, None, ptrs, ws, ws_bytes, None)


def test_decode_select_validation():
    """hs_decode_select_attn rejects bad arguments before any launch."""
    s = _dshape()
    assert _dsel(s, n_sel=-1) == hb.HS_ERR_INVALID_ARG
    assert _dsel(s, n_sel=8193) == hb.HS_ERR_INVALID_ARG
    assert _dsel(s, idx=None) == hb.HS_ERR_INVALID_ARG                 # n_sel > 0 needs idx
    assert _dsel(s, ring=None) == hb.HS_ERR_INVALID_ARG                # window needs the ring
    assert _dsel(s, window=-1) == hb.HS_ERR_INVALID_ARG
    assert _dsel(s, window=2048) == hb.HS_ERR_INVALID_ARG              # window > capacity
    assert _dsel(s, block=32) == hb.HS_ERR_INVALID_ARG
    assert _dsel(s, block=1) == hb.HS_ERR_UNSUPPORTED                  # token mode needs fp8 caches
    assert _dsel(s, gates=FAKE + 4) == hb.HS_ERR_INVALID_ARG           # gates misaligned
    assert _dsel(s, ptrs=FAKE + 2) == hb.HS_ERR_INVALID_ARG            # q misaligned
    assert _dsel(_dshape(kv_lens=None)) == hb.HS_ERR_INVALID_ARG       # decode needs kv_lens
    assert _dsel(_dshape(kv_len=1000)) == hb.HS_ERR_INVALID_ARG        # capacity not a multiple of 64
    assert _dsel(_dshape(q_len=2)) == hb.HS_ERR_INVALID_ARG
    assert _dsel(_dshape(hq=64, hkv=2)) == hb.HS_ERR_UNSUPPORTED       # group of 32
    f8 = _dshape(kv_dtype=hb.HS_FP8_E4M3, kv_scale=FAKE)
    assert _dsel(f8, block=1, window=64) == hb.HS_ERR_INVALID_ARG      # token mode: no window
    assert _dsel(f8, block=1, window=0, gates=FAKE) == hb.HS_ERR_INVALID_ARG  # token mode: no gate
    assert _dsel(_dshape(kv_dtype=hb.HS_FP8_E4M3), block=1, window=0) == hb.HS_ERR_INVALID_ARG  # no scale
    # nothing to do: no sequences
    assert _dsel(_dshape(batch=0), ptrs=None, idx=None, ring=None) == hb.HS_OK
    assert hb.load().hs_last_error().decode() == ""


def _tsel(s, topk=64, n_recent=8, ptrs=FAKE, idx=FAKE, ws=None, ws_bytes=0):
    lib = hb.load()
    return lib.hs_decode_token_select(ctypes.byref(s), ptrs, ptrs, ptrs, ptrs, ptrs, topk, n_recent, idx, ws,
                                      ws_bytes, None)


def test_decode_token_select_validation():
    """hs_decode_token_select rejects bad arguments before any launch, and
    sizes its workspace through hs_workspace_size."""
    f8 = _dshape(kv_dtype=hb.HS_FP8_E4M3, kv_scale=FAKE)
    need = hb.workspace_size(hb.HS_FN_DECODE_TOKEN_SELECT, f8, 1, 64)
    # split-K partials + bounds (z per token and group, offsets per tile and head, widths) + selection
    assert need >= 2 * 2 * 1024 * 4 + 2 * 2 * 16 * 4 * 4
    assert _tsel(f8) == hb.HS_ERR_WORKSPACE                                  # no workspace
    assert _tsel(f8, ws=FAKE, ws_bytes=need - 1) == hb.HS_ERR_WORKSPACE
    assert _tsel(f8, ws=FAKE + 4, ws_bytes=need) == hb.HS_ERR_INVALID_ARG    # misaligned workspace
    assert _tsel(f8, topk=0, ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG
    assert _tsel(f8, topk=4097, ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG
    assert _tsel(f8, n_recent=-1, ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG
    assert _tsel(f8, idx=None, ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG
    assert _tsel(_dshape(), ws=FAKE, ws_bytes=need) == hb.HS_ERR_UNSUPPORTED          # needs fp8 caches
    assert _tsel(_dshape(kv_dtype=hb.HS_FP8_E4M3), ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG  # no scale
    assert _tsel(_dshape(kv_dtype=hb.HS_FP8_E4M3, kv_scale=FAKE, kv_lens=None),
                 ws=FAKE, ws_bytes=need) == hb.HS_ERR_INVALID_ARG                     # decode needs kv_lens
    assert _tsel(_dshape(kv_dtype=hb.HS_FP8_E4M3, kv_scale=FAKE, batch=0), ptrs=None, idx=None) == hb.HS_OK
