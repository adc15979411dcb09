"""The seeded input recipes are reproducible and have the stated shapes and ranges."""
import numpy as np

import workloads


def test_varlen_lengths_follow_the_rule():
    seed, lens = workloads.varlen_lengths_rule()
    assert seed == 17
    assert lens == workloads.VARLEN_LENGTHS
    assert sum(lens) == 129148


def test_tiny_recipe():
    d = workloads.tiny_numpy()
    assert d["q"].shape == (256, 1, 32) and d["q"].dtype == np.float32
    np.testing.assert_allclose(np.linalg.norm(d["k"], axis=-1), 1.0, rtol=1e-6)
    a = np.exp(d["log_alpha"].astype(np.float64))
    assert a.min() >= 0.9 - 1e-7 and a.max() < 1.0 + 1e-7
    assert 0.0 <= d["beta"].min() and d["beta"].max() < 1.0
    d2 = workloads.tiny_numpy()
    for k in d:
        np.testing.assert_array_equal(d[k], d2[k])


def test_torch_generator_is_seeded():
    import torch
    a = workloads.gen_forward(300, 2, 16, 8, gates="softplus", seed=5, init_std=0.1)
    b = workloads.gen_forward(300, 2, 16, 8, gates="softplus", seed=5, init_std=0.1)
    for k in ("q", "k", "v", "log_alpha", "beta", "init_state"):
        assert torch.equal(a[k], b[k])
    assert a["q"].dtype == torch.bfloat16
    assert float(a["log_alpha"].float().max()) <= 0.0
