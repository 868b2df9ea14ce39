"""The seeded input generators: determinism, chunk independence, bf16 rounding."""
import numpy as np
import pytest

import synth


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0]    # ties to even, plain values
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.bf16_round(x), want)


def test_generators_are_deterministic_and_chunked():
    wl = synth.get("attn4096").resized(rows=16, n=256, tokens=2 * synth.CHUNK + 100)
    a = synth.activations_raw(wl)
    b = synth.activations_raw(wl)
    assert a.shape == (2 * synth.CHUNK + 100, 256) and a.dtype == np.uint16
    assert np.array_equal(a, b)
    c2 = synth.activations_chunk_raw(wl, 2)
    assert np.array_equal(c2, a[2 * synth.CHUNK:])
    w = synth.weights(wl)
    assert w.shape == (16, 256) and np.array_equal(w, synth.weights(wl))


def test_outlier_channels_present():
    wl = synth.get("attn4096").resized(rows=4, n=1000, tokens=4096)
    x = synth.activations(wl)
    rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))
    big = np.sort(rms)[-10:]
    assert np.all(big > 10 * np.median(rms))          # 1% of 1000 channels scaled x20


def test_toy_is_fp32_and_shaped():
    wl = synth.get("toy256")
    x = synth.activations(wl)
    assert x.dtype == np.float32 and x.shape == (2048, 256)
    assert synth.weights(wl).shape == (256, 256)


def test_matmul_inputs_are_deterministic_and_well_formed():
    for act in (False, True):
        codes, s, z, g_idx = synth.quantized_layer(3, 20, 256, 4, 64, act_order=act)
        codes2, s2, z2, g2 = synth.quantized_layer(3, 20, 256, 4, 64, act_order=act)
        assert np.array_equal(codes, codes2) and np.array_equal(s, s2) and np.array_equal(g_idx, g2)
        assert codes.shape == (20, 256) and codes.min() >= 0 and codes.max() <= 15
        assert s.shape == z.shape == (4, 20) and s.dtype == z.dtype == np.float16
        assert np.all(s > 0) and np.array_equal(z, np.round(z))
        assert np.array_equal(np.bincount(g_idx, minlength=4), [64] * 4)
        assert act == (not np.array_equal(g_idx, np.arange(256) // 64))
    _, s, _, g_idx = synth.quantized_layer(1, 4, 256, 3, -1)
    assert s.shape == (1, 4) and not g_idx.any()
    a = synth.decode_activations_raw(5, 3, 1000)
    assert a.dtype == np.uint16 and a.shape == (3, 1000)
    assert np.array_equal(a, synth.decode_activations_raw(5, 3, 1000))
    v = a.view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(v)) and (np.abs(v) > 10).any(axis=0).sum() >= 5


def test_random_qweight():
    q = synth.random_qweight(2, 24, 256, 3)
    assert q.shape == (24, 24) and q.dtype == np.uint32
    assert np.array_equal(q, synth.random_qweight(2, 24, 256, 3))
    bits = np.unpackbits(q.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 0.02


def test_parallel_generation_is_identical():
    wl = synth.get("attn4096").resized(rows=16, n=256, tokens=2 * synth.CHUNK + 17)
    a = synth.activations_raw_parallel(wl, 0, workers=2)
    assert np.array_equal(a, synth.activations_raw(wl, 0))
    got = {}
    synth.activations_raw_parallel(wl, 0, workers=2, out=lambda t0, c: got.__setitem__(t0, c))
    assert sorted(got) == [0, synth.CHUNK, 2 * synth.CHUNK]
    assert np.array_equal(np.concatenate([got[k] for k in sorted(got)]), a)


def test_sets_with_equal_descriptions_are_independent_of_order():
    """Activation sets with the same description (the block's q/k/v-in, o-in
    and gate/up-in) each have their own seeded loadings, whatever set was
    generated first in the process."""
    import dataclasses
    base = synth.get("llama2block")
    wl = dataclasses.replace(base, name="order-check", tokens=64,
                             xsets=((96, "factor", 0, 1.0), (96, "factor", 0, 1.0)))
    synth._STATIC_CACHE.clear()
    b_first = synth.activations_chunk_raw(wl, 0, 1)
    a_after = synth.activations_chunk_raw(wl, 0, 0)
    synth._STATIC_CACHE.clear()
    a_first = synth.activations_chunk_raw(wl, 0, 0)
    b_after = synth.activations_chunk_raw(wl, 0, 1)
    assert np.array_equal(a_first, a_after) and np.array_equal(b_first, b_after)
    assert not np.array_equal(a_first, b_first)
