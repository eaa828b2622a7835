"""The seeded generator: bf16 rounding, determinism, workload shapes."""
import numpy as np
import torch

from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_inputs


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200_000).astype(np.float32) * 10 ** g.uniform(-30, 30, 200_000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38], np.float32)])
    x = x[np.isfinite(x)]
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    a = make_inputs([3, 0, 17], d=16, k=8, seed=5)
    b = make_inputs([3, 0, 17], d=16, k=8, seed=5)
    for f in ("H", "Wk", "Wv", "P", "offsets"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.H.shape == (20, 16) and a.P.shape == (8, 16)
    np.testing.assert_array_equal(a.offsets, [0, 3, 3, 20])
    np.testing.assert_array_equal(bf16_bits_to_f32(a.H_bits), a.H)
    c = make_inputs([3, 0, 17], d=16, k=8, seed=6)
    assert not np.array_equal(a.H, c.H)


def test_config_registry_shapes():
    c1 = make_config("c1_fp32_n4096_d64_k64")
    assert c1.dtype == "f32" and c1.H.shape == (4096, 64) and c1.k == 64
    # variance 1/d for the weights, unit variance for the history
    assert abs(c1.P.std() * 8 - 1) < 0.05 and abs(c1.H.std() - 1) < 0.02
    m = make_config("small_mask_d128_k512")
    assert m.mask is not None and m.valid_tokens() == 1000 - 100 + 1777 - 177 + 64 - 6
    assert set(CONFIGS) >= {"c2_n100k_d128_k1024", "c3_r40_ragged_d128_k1024"}
