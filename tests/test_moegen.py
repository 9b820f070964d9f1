"""The seeded input generator: stream definition, distributions, recipes.

The generator holds none of the layer's arithmetic; these tests pin its
stream (SplitMix64 reference vector), its N(0,1) draws, the regenerability of
every slice, and the workload recipes' shapes and value ranges.
"""
import os

import numpy as np
import pytest
import scipy.stats

import moegen
from tests._util import from_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_vector():
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt")) as f:
        want = [int(l) for l in f if l.strip() and not l.startswith("#")]
    got = [moegen.lib().moegen_splitmix(1234567, i) for i in range(len(want))]
    assert got == want


def test_normal_draws_are_standard_normal():
    n = 2_000_000
    z = np.empty(n, np.float64)
    moegen.lib().moegen_normal_f64_host(987654321, 0, n, z.ctypes.data, moegen.threads())
    assert abs(z.mean()) < 3e-3
    assert abs(z.std() - 1.0) < 3e-3
    assert abs(scipy.stats.kurtosis(z, fisher=False) - 3.0) < 0.02
    assert scipy.stats.kstest(z[:200_000], "norm").pvalue > 1e-4


def test_slices_are_regenerable():
    L = moegen.lib()
    key = moegen.lib().moegen_stream_key(5, 2, moegen.KIND_W_GATE_UP, 17)
    full = np.empty(10_000, np.uint16)
    L.moegen_normal_bf16_host(key, 0, full.size, 0.02, full.ctypes.data, 4)
    part = np.empty(777, np.uint16)
    L.moegen_normal_bf16_host(key, 4321, part.size, 0.02, part.ctypes.data, 1)
    np.testing.assert_array_equal(part, full[4321:4321 + 777])
    # The per-expert fill uses the same key for its expert.
    cfg = moegen.custom(0, seed=5)
    ex = np.empty(3 * 10_000, np.uint16)
    L.moegen_experts_bf16_host(5, 2, moegen.KIND_W_GATE_UP, 16, 3, 10_000, 0.02, ex.ctypes.data, 4)
    np.testing.assert_array_equal(ex[10_000:20_000], full)
    assert moegen.key(cfg, 2, moegen.KIND_W_GATE_UP, 17) == key


def test_distinct_streams_differ():
    cfg = moegen.CONFIGS[0]
    keys = {moegen.key(cfg, l, kind, e) for l in range(3) for kind in range(1, 9) for e in range(4)}
    assert len(keys) == 3 * 8 * 4


@pytest.mark.parametrize("idx", [0, 1, 3])
def test_recipe_shapes_and_ranges(idx):
    cfg = moegen.CONFIGS[idx]
    x = moegen.x(cfg)
    assert x.shape == (cfg.T, cfg.d) and x.dtype == np.uint16
    xf = from_bf16(x).astype(np.float64)
    rms = np.sqrt((xf ** 2).mean(1))
    if cfg.x_rms:
        np.testing.assert_allclose(rms, 1.0, atol=2e-3)
    else:
        assert abs(rms.mean() - 1.0) < 0.05
    wr = from_bf16(moegen.router(cfg))
    assert wr.shape == (cfg.E, cfg.d) and abs(wr.std() - 0.02) < 1e-3
    b = moegen.sel_bias(cfg)
    assert b.shape == (cfg.E,) and np.all(np.abs(b) <= cfg.bias) and b.std() > cfg.bias / 3
    c = moegen.logit_bias(cfg)
    if cfg.zipf_s:
        r = moegen.zipf_ranks(cfg)
        np.testing.assert_array_equal(np.sort(r), np.arange(1, cfg.E + 1))
        np.testing.assert_allclose(c, cfg.zipf_amp * r.astype(np.float64) ** -cfg.zipf_s, rtol=1e-6)
    else:
        assert c is None


def test_expert_weights_host_shapes():
    cfg = moegen.CONFIGS[0]
    w = moegen.expert_weights_host(cfg, 0, [3])
    gu, dn = w[3]
    assert gu.shape == (2 * cfg.h, cfg.d) and dn.shape == (cfg.d, cfg.h)
    assert abs(from_bf16(gu).std() - 0.02) < 1e-3
    sgu, sdn = moegen.shared_weights_host(cfg)
    assert sgu.shape == (2 * cfg.hs, cfg.d) and sdn.shape == (cfg.d, cfg.hs)
    assert not np.array_equal(sgu, gu)


@pytest.mark.slow
def test_skew_recipe_hits_ten_times_mean_load():
    # The skewed workload asks for the busiest expert at about 10x the mean
    # load and some experts at 0-2 tokens; routing by the oracle.
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    cfg = moegen.CONFIGS[3]
    x, wr, b, c = moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg), moegen.logit_bias(cfg)
    with ThreadPoolExecutor(moegen.threads()) as pool:
        parts = pool.map(lambda idx: oracle.route(x[idx], wr, b, cfg.k, logit_bias=c)[0],
                         np.array_split(np.arange(cfg.T), 16))
        ids = np.concatenate(list(parts))
    cnt = np.bincount(ids.ravel(), minlength=cfg.E)
    mean = cfg.T * cfg.k / cfg.E
    assert 9.5 <= cnt.max() / mean <= 10.5
    assert (cnt <= 2).sum() >= 10
