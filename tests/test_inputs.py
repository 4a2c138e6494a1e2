"""The seeded input generator: determinism, shapes and value distributions."""
import numpy as np
import torch

import oracle
import q4k_inputs as qi


def test_weights_are_deterministic_and_shaped():
    a = qi.weight_bytes(qi.rng(5), 7, 512)
    b = qi.weight_bytes(qi.rng(5), 7, 512)
    assert a.shape == (7, 2 * 144) and a.dtype == np.uint8
    assert np.array_equal(a, b)
    assert not np.array_equal(a, qi.weight_bytes(qi.rng(6), 7, 512))


def test_field_distributions_match_the_workload_recipe():
    W = qi.weight_bytes(qi.rng(0), 512, 2560)
    q, sc, m, d, dm = oracle.unpack_fields(W)
    dv = d.view(np.float16).astype(np.float64)
    dmv = dm.view(np.float16).astype(np.float64)
    # |N(0,1)| * 2e-3 has median 0.6745 * 2e-3 and mean 0.7979 * 2e-3
    for v in (dv, dmv):
        assert np.all(v >= 0)
        assert abs(np.median(v) / 2e-3 - 0.6745) < 0.02
        assert abs(v.mean() / 2e-3 - 0.7979) < 0.02
    for f, top in ((sc, 63), (m, 63), (q, 15)):
        counts = np.bincount(f.ravel(), minlength=top + 1)
        assert counts.size == top + 1
        expected = f.size / (top + 1)
        assert np.all(np.abs(counts - expected) < 6 * np.sqrt(expected))


def test_activations_are_bf16_of_standard_normal():
    X = qi.activations(qi.rng(1), 4, 4096)
    x = qi.bf16_bits_to_f32(X)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    z = qi.rng(1).standard_normal((4, 4096), dtype=np.float32)
    ref = torch.from_numpy(z).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(X, ref)


def test_workload_shapes():
    layer = qi.decode_layer(1, 0, 1)
    assert [(n, N, K) for n, N, K, _, _ in layer] == qi.PROJECTIONS
    for _, N, K, W, X in layer:
        assert W.shape == (N, K // 256 * 144) and X.shape == (1, K)
    total = sum(W.nbytes for _, _, _, W, _ in layer)
    assert total == 56_770_560          # 56.77 MB of Q4_K weights per layer
    name, N, K, W, X = qi.prefill_projection(2, 3, 6, 33)
    assert (name, N, K, X.shape) == ("down", 2560, 9728, (33, 9728))
