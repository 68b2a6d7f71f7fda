"""The seeded input generator: deterministic, thread-count independent, bf16 by RNE."""
import numpy as np
import torch

import moe_workloads as W


def test_deterministic_and_thread_independent():
    s = W.shape(T=300, H=128, I=64, E=7, k=3, seed=3)
    a = W.generate(s, threads=1)
    b = W.generate(s, threads=4)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = W.generate(W.shape(T=300, H=128, I=64, E=7, k=3, seed=4))
    assert not np.array_equal(a["x"], c["x"])


def test_bf16_inputs_are_rne_of_float32_draws():
    f = (np.random.default_rng(1).standard_normal(100000) * 3).astype(np.float32)
    ours = W._f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_named_shapes_and_bias():
    assert [W.SHAPES[n].T for n in W.SHAPE_ORDER] == [256, 4096, 8192, 512, 65536]
    for n in W.SHAPE_ORDER:
        assert W.SHAPES[n].waves == 8
    z = W.expert_bias(W.SHAPES["small_m_zipf"])
    p = np.exp(z) / np.exp(z).sum()
    r = np.arange(1, 65, dtype=np.float64) ** -1.2
    np.testing.assert_allclose(p, r / r.sum(), rtol=1e-12)
    s = W.shape("tiny")
    d = W.generate(s)
    assert d["x"].shape == (256, 512) and d["w1"].shape == (8, 2048, 512) and d["w2"].shape == (8, 512, 1024)
    x = (d["x"].astype(np.uint32) << 16).view(np.float32)
    assert 0.015 < x.std() < 0.025
