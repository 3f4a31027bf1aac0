"""The seeded input generator: determinism, storage rounding, layouts."""
import numpy as np
import torch

from hybrid_sparse_attention_causal_amd import inputs as gen


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), ref)
    assert np.array_equal(gen.bf16_bits_to_f32(ref),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_fp8_encoder_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    fin = np.isfinite(vals)
    back = gen.encode_e4m3(vals[fin])
    # +0/-0 both round-trip; every finite code maps back to itself
    assert np.array_equal(back, codes[fin])
    assert gen.encode_e4m3(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def test_prefill_generator_is_deterministic_and_planted():
    cfg = gen.config(1, T=256)
    a = gen.make_prefill(cfg)
    b = gen.make_prefill(cfg)
    for name in ("q", "k", "v"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert np.array_equal(a.layers[2]["gates"], b.layers[2]["gates"])
    assert a.q.shape == (1, 256, 4, 64) and a.k.shape == (1, 1, 256, 64)
    assert len(a.salient[0]) == round(0.02 * 256)
    c = gen._unit_vectors(cfg)
    proj = a.k[0, 0] @ c[0]
    sal = a.salient[0]
    rest = np.setdiff1d(np.arange(256), sal)
    assert proj[sal].min() > proj[rest].max()


def test_block_major_layout():
    v = np.arange(2 * 130 * 3, dtype=np.float32).reshape(2, 130, 3)
    vb = gen.block_major(v)
    assert vb.shape == (2, 3, 3, 64)
    for t in range(130):
        assert np.array_equal(vb[:, t // 64, :, t % 64], v[:, t])
    assert np.all(vb[:, 2, :, 2:] == 0)


def test_decode_generator_slabs_and_poison():
    cfg = gen.config(4, B=2, T=256, L_lo=70, L_hi=200, N=1)
    inp = gen.make_decode(cfg)
    assert inp.lens.min() >= 70 and inp.lens.max() <= 200
    k = np.zeros((2, 4, 256, 128), np.uint16)
    v = np.zeros((2, 4, 4, 128, 64), np.uint16)
    gen.fill_decode_cache(inp, k, v)
    for b in range(2):
        L = int(inp.lens[b])
        ks, vs = inp.kv_slab(b, 1)
        assert np.array_equal(k[b, 1, :L], ks)
        assert np.all(k[b, 1, L:] == 0x7FC0)
        assert np.array_equal(v[b, 1, (L - 1) // 64, :, (L - 1) % 64], vs[L - 1])
        if L % 64:
            assert np.all(v[b, 1, L // 64, :, L % 64:] == 0x7FC0)


def test_ring_slots():
    assert list(gen.ring_slot_positions(5, 4)) == [4, 1, 2, 3]
    assert list(gen.ring_slot_positions(2, 4)) == [0, 1, -1, -1]
