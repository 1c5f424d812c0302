"""The per-layer (pyramid) budget of the synthetic workload.

PyramidInfer page ("PyramidInfer: Pyramid KV Cache Compression for
High-throughput LLM Inference"), abstract and technical-approach list: deeper
layers keep fewer keys and values.  The workload reads this as a keep-rate
factor falling linearly from 1.5 at layer 0 to 0.5 at the last layer, so the
mean keep rate over the model is that of the flat workload.  These tests check
the schedule, that it only rescales the flat draws, and that the stored rows
of the compact store follow it (counted by the oracle)."""
import numpy as np
import pytest

import oracle
import workload


@pytest.mark.parametrize("L", [2, 16, 36])
def test_schedule_shape(L):
    cfg = workload.pyramid(workload.custom(L=L))
    f = np.array([workload.layer_budget(cfg, l) for l in range(L)])
    assert f[0] == 1.5 and abs(f[-1] - 0.5) < 1e-12
    assert np.all(np.diff(f) < 0)                      # strictly falling with depth
    assert abs(f.mean() - 1.0) < 1e-12                 # same mean budget as flat
    assert np.allclose(np.diff(f), -1.0 / (L - 1))     # linear


def test_flat_and_single_layer_are_unscaled():
    flat = workload.custom(L=8)
    assert all(workload.layer_budget(flat, l) == 1.0 for l in range(8))
    assert workload.layer_budget(workload.pyramid(workload.custom(L=1)), 0) == 1.0
    with pytest.raises(ValueError):
        workload.layer_budget(workload.custom(L=4, budget="bogus"), 1)


@pytest.mark.parametrize("lo,hi", [(0.3, 0.3), (0.1, 0.9)])
def test_pyramid_rescales_the_flat_draws(lo, hi):
    flat = workload.custom(L=5, B=2, Hkv=3, T=200, S=3, keep_lo=lo, keep_hi=hi, seed=77)
    pyr = workload.pyramid(flat)
    for l in range(5):
        a, b = workload.make_layer(flat, l), workload.make_layer(pyr, l)
        f = workload.layer_budget(pyr, l)
        np.testing.assert_array_equal(b.rate.numpy(),
                                      np.minimum(a.rate.numpy() * np.float32(f), 1.0))
        # K, V and q come from the same generator after the same draws
        assert a.k.equal(b.k) and a.v.equal(b.v) and a.q.equal(b.q)


def test_named_pyramid_workloads():
    for base in ("llama_c8", "qwen_c8"):
        p = workload.CONFIGS[base + "_pyramid"]
        assert p.budget == "pyramid"
        assert p == workload.pyramid(workload.CONFIGS[base])
        assert workload.CONFIGS[base].budget == "flat"


def test_stored_rows_fall_with_depth():
    cfg = workload.pyramid(workload.custom(L=6, B=2, Hkv=4, T=3000, S=1, W=64,
                                           keep_lo=0.2, keep_hi=0.2, seed=5))
    # compact rows (the kept tokens older than the W-row window) scale with
    # the layer's factor
    comp = np.array([oracle.prefill_layout(workload.make_layer(cfg, l).keep, cfg.T, cfg.W, 0)
                     ["comp_len"].sum() for l in range(cfg.L)], dtype=float)
    f = np.array([workload.layer_budget(cfg, l) for l in range(cfg.L)])
    expect = 0.2 * f * (cfg.T - cfg.W) * cfg.B * cfg.Hkv
    sd = np.sqrt(expect)                        # binomial, rate <= 0.3
    assert np.all(np.abs(comp - expect) < 5 * sd)
    assert np.all(np.diff(comp) < 0)
