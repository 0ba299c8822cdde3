"""The seeded input generators: determinism, shapes and the input recipe."""
import numpy as np
import torch

from gated_delta_rule_42_amd import workloads as wl


def test_tiny_prefill_shapes_and_recipe():
    c = wl.tiny_prefill()
    assert c.q.shape == (64, 2, 16) and c.q.dtype == torch.float32
    assert c.pool.shape == (1, 2, 16, 16) and float(c.pool.abs().max()) == 0.0
    assert c.chunk_size == 16 and c.has_init.tolist() == [0]
    n = torch.linalg.vector_norm(c.q.double(), dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    assert float(c.g.max()) < 0.0 and 0.0 < float(c.beta.min()) and float(c.beta.max()) < 1.0


def test_generators_are_deterministic():
    a, b = wl.tiny_prefill(), wl.tiny_prefill()
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta)]:
        assert torch.equal(x, y)
    c = wl.random_prefill(9, [5, 0, 7], 2, 8, 8)
    d = wl.random_prefill(9, [5, 0, 7], 2, 8, 8)
    assert torch.equal(c.q, d.q) and torch.equal(c.slots, d.slots)
    assert c.cu_seqlens.tolist() == [0, 5, 5, 12]


def test_varlen_structure():
    rng = np.random.default_rng(3)
    lens = wl.varlen_lengths(rng)
    assert len(lens) == 8 and sum(lens) <= 16384 and min(lens) >= 256 and max(lens) <= 4096


def test_long_context_calls_are_independent_of_order():
    lc = wl.long_context(T_total=64, T_call=32, H=2, d=16)
    c1 = lc.call(1)
    lc.call(0)
    assert torch.equal(c1.x, lc.call(1).x)
    assert c1.x.shape == (32, 3 * 2 * 16) and c1.gate.shape == (32, 2, 16)
    assert lc.conv_weight.shape == (96, 4) and lc.n_calls == 2
