"""The seeded input generator: determinism, recipe, and BF16 rounding against torch."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.exp2(rng.uniform(-130, 120, 100000)).astype(np.float32)])
    mine = wl.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)


def test_generator_is_deterministic_and_follows_the_recipe():
    w = wl.BY_NAME["mlp7b_up_fwd"]
    spec = w.tensor("X")
    a = wl.draw_f32(w.config_id, spec, (64, 128))
    b = wl.draw_f32(w.config_id, spec, (64, 128))
    assert np.array_equal(a, b) and a.dtype == np.float32
    base = wl.rng_for(w.config_id, spec.tensor_id).standard_normal(64 * 128, dtype=np.float32)
    changed = np.flatnonzero(a.ravel() != base)
    assert changed.size == round(1e-3 * 64 * 128)
    assert np.allclose(a.ravel()[changed], base[changed] * 20.0)
    xb = wl.draw(w.config_id, spec, (64, 128))
    assert xb.dtype == np.uint16 and np.array_equal(xb, wl.f32_to_bf16_bits(a))


def test_workload_shapes():
    assert [w.name for w in wl.WORKLOADS] == ["tiny_fwd_256", "mlp7b_up_fwd", "mlp7b_bwd_hybrid",
                                               "proj13b_fwd", "slice70b_fwd"]
    c3 = wl.BY_NAME["mlp7b_bwd_hybrid"]
    for g in c3.gemms:
        ta = c3.tensor(g.a).shape
        tb = c3.tensor(g.b).shape
        am, ak = (ta[1], ta[0]) if g.a_transposed else ta
        bn, bk = (tb[1], tb[0]) if g.b_transposed else tb
        assert (am, bn, ak) == (g.m, g.n, g.k) and ak == bk
    u = wl.step_factors(0, 16)
    assert u.shape == (16,) and (u >= 0.5).all() and (u < 2.0).all()
