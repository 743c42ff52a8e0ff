"""Seeded input generation: rounding matches torch's dtype casts, slices are
reproducible on their own, and the workload table is as documented (CPU only)."""
import numpy as np
import torch

import attn_inputs as A


def test_bf16_and_fp16_rounding_match_torch_casts():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 37
    x[:6] = [1.00390625, 1.005859375, -1.00390625, 3.0e38, 1e-40, 0.0]
    t = torch.from_numpy(x)
    np.testing.assert_array_equal(A.bf16_round(x), t.to(torch.bfloat16).float().numpy())
    y = x / 1000
    np.testing.assert_array_equal(A.fp16_round(y), torch.from_numpy(y).half().float().numpy())


def test_slices_are_deterministic_and_independent():
    cfg = A.get_config(2).with_(B=2, H_q=3, H_kv=3, N_q=40, N_kv=40)
    full = A.tensor_values(cfg, "k")
    s = A.slice_values(cfg.cid, "k", 1, 2, 40, cfg.d, cfg.sigma, cfg.dtype)
    np.testing.assert_array_equal(full[1, 2], s)
    assert not np.array_equal(full[1, 1], s)
    # values are exactly representable in bf16
    np.testing.assert_array_equal(A.bf16_round(full), full)


def test_sigma_scaling_is_exact():
    a = A.slice_values(3, "q", 0, 0, 64, 64, 1.0, "f32")
    b = A.slice_values(3, "q", 0, 0, 64, 64, 0.5, "f32")
    np.testing.assert_array_equal(a * np.float32(0.5), b)


def test_config_table():
    c = A.CONFIGS
    assert (c[2].B, c[2].H_q, c[2].N_q, c[2].d, c[2].dtype, c[2].causal) == (4, 32, 4096, 128, "bf16", True)
    assert (c[3].N_q, c[3].H_q, c[3].d, c[3].dtype, c[3].sigma) == (23400, 12, 64, "f16", 0.5)
    assert (c[4].H_q, c[4].H_kv, c[4].G, c[4].N_q) == (32, 4, 8, 32768)
    assert (c[5].B, c[5].N_q, c[5].N_kv, c[5].G) == (64, 1, 32768, 8)
    assert c[1].scale == np.float32(0.125)
    lens = A.ragged_lengths(c[6])
    assert lens.shape == (64,) and lens.min() >= 1 and lens.max() <= 32768
    np.testing.assert_array_equal(lens, A.ragged_lengths(c[6]))
    # multi-token decode shares config 5's caches (same seeds), 4 queries per head
    assert (c[7].cid, c[7].N_q, c[7].N_kv, c[7].causal, c[7].G) == (5, 4, 32768, True, 8)
    assert (c[8].cid, c[8].N_q, c[8].N_kv, c[8].causal) == (5, 64, 32768, True)


def test_output_gradient_has_its_own_stream():
    """dO (tensor id 4) is shaped like Q and drawn from its own seed stream."""
    cfg = A.CONFIGS[2]
    q = A.slice_values(cfg.cid, "q", 1, 3, 64, cfg.d, cfg.sigma, cfg.dtype)
    g = A.slice_values(cfg.cid, "do", 1, 3, 64, cfg.d, cfg.sigma, cfg.dtype)
    assert g.shape == q.shape and not np.array_equal(g, q)
    assert np.array_equal(g, A.slice_values(cfg.cid, "do", 1, 3, 64, cfg.d, cfg.sigma, cfg.dtype))
    assert np.array_equal(g, A.bf16_round(g))
