"""The CPU / GPU share policy: the oracle pinned to what Eq. 1-2 of [InplaceKVCache] §5.2-5.3
fix, then the library (kvattn_share_*) against the oracle.  Host code only.

Pins that do not restate Eq. 2:
  * r(L) minimises the step time max(T_CPU, T_GPU) of Eq. 1 (brute force over a grid of r);
  * inside (0, 1) the two latencies of Eq. 1 are equal at r(L);
  * r(L) -> p = B / (A + B) for long sequences, r = p for every L when the overheads match,
    r = 1 when the CPU is free, r = 0 when the GPU is free and starts no later;
  * R(L) with R(L0) = r(L0) equals r(L) for every longer L (unclamped range);
  * a stream of routed batches keeps the cumulative CPU tokens within D/2 of r(L) L and the
    fraction of CPU batches tends to p;
  * latencies generated exactly from T = A n + C_CPU give A back exactly; a change of A is
    picked up once the window holds only new samples;
  * the line fit equals numpy.polyfit and recovers an exact line.
"""

import random

import numpy as np
import pytest

from oracle import share as osh
from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import KvattnError, ShareController, share_fit, share_optimum


def _models(seed, count):
    rng = random.Random(seed)
    out = []
    for _ in range(count):
        A = rng.uniform(0.05, 5.0)
        B = rng.uniform(0.05, 5.0)
        C_cpu = rng.uniform(0.0, 2000.0)
        C_gpu = rng.uniform(0.0, 2000.0)
        L = rng.choice([16, 100, 1000, 4096, 32768, 131072]) * rng.uniform(0.5, 2.0)
        out.append((A, B, C_cpu, C_gpu, L))
    return out


# ---------------------------------------------------------------- oracle pins


@pytest.mark.parametrize("model", _models(1, 40))
def test_optimum_minimises_eq1_step_time(model):
    A, B, C_cpu, C_gpu, L = model
    r_star = osh.optimum(A, B, C_cpu, C_gpu, L)
    grid = np.linspace(0.0, 1.0, 20001)
    t_cpu, t_gpu = osh.step_latencies(grid, L, A, B, C_cpu, C_gpu)
    r_grid = grid[int(np.argmin(np.maximum(t_cpu, t_gpu)))]
    assert abs(r_grid - r_star) <= 1.0 / 20000 + 1e-12
    best = max(osh.step_latencies(r_star, L, A, B, C_cpu, C_gpu))
    assert best <= float(np.min(np.maximum(t_cpu, t_gpu))) * (1 + 1e-12)


@pytest.mark.parametrize("model", _models(2, 40))
def test_latencies_balance_inside_the_unit_interval(model):
    A, B, C_cpu, C_gpu, L = model
    r = osh.optimum(A, B, C_cpu, C_gpu, L)
    t_cpu, t_gpu = osh.step_latencies(r, L, A, B, C_cpu, C_gpu)
    if 0.0 < r < 1.0:
        assert t_cpu == pytest.approx(t_gpu, rel=1e-12)
    elif r == 0.0:
        assert t_gpu <= t_cpu  # the whole sequence on the GPU beats the CPU's overhead alone
    else:
        assert t_cpu <= t_gpu  # the whole sequence on the CPU beats the GPU's overhead alone


def test_limits_and_special_cases():
    A, B = 3.0, 1.0
    p = osh.converged(A, B)
    assert p == 0.25
    assert osh.optimum(A, B, 0.0, 5000.0, 1e15) == pytest.approx(p, abs=1e-9)
    assert osh.optimum(A, B, 5000.0, 0.0, 1e15) == pytest.approx(p, abs=1e-9)
    for L in [1.0, 7.0, 1e3, 1e9]:
        assert osh.optimum(A, B, 40.0, 40.0, L) == p           # equal overheads
        assert osh.optimum(0.0, B, 10.0, 50.0, L) == 1.0      # CPU free, GPU overhead larger
        assert osh.optimum(A, 0.0, 10.0, 5.0, L) == 0.0       # GPU free and starts first
    assert osh.optimum(A, B, 0.0, 1e9, 10.0) == 1.0            # huge GPU overhead: all CPU
    assert osh.optimum(A, B, 1e9, 0.0, 10.0) == 0.0            # huge CPU overhead: all GPU


@pytest.mark.parametrize("seed", range(6))
def test_cumulative_share_tracks_the_optimum(seed):
    rng = random.Random(seed)
    A, B = rng.uniform(0.5, 3.0), rng.uniform(0.5, 3.0)
    C_cpu, C_gpu = rng.uniform(0, 200), rng.uniform(0, 200)
    p = osh.converged(A, B)
    L0 = 4096.0
    R0 = osh.optimum(A, B, C_cpu, C_gpu, L0)
    if not 0.0 < R0 < 1.0:
        pytest.skip("clamped at admission")
    for L in [L0, 5000.0, 1e4, 1e5, 1e7]:
        assert osh.cumulative_share(R0, L0, L, p) == pytest.approx(
            osh.optimum(A, B, C_cpu, C_gpu, L), abs=1e-12)
    assert osh.cumulative_share(R0, L0, L0, p) == pytest.approx(R0, abs=1e-15)


@pytest.mark.parametrize("seed", range(8))
def test_routing_keeps_half_a_batch_of_the_target(seed):
    rng = random.Random(100 + seed)
    A, B = rng.uniform(0.2, 4.0), rng.uniform(0.2, 4.0)
    C_cpu, C_gpu = rng.uniform(0, 3000), rng.uniform(0, 3000)
    D, bs = rng.choice([64, 128, 256]), 64
    ctl = osh.Controller(A, B, C_cpu, C_gpu, window=256)
    L0 = rng.randrange(0, 20000)
    c0 = ctl.admit(L0, bs)
    assert c0 % bs == 0 and 0 <= c0 <= L0
    if L0:
        assert abs(c0 - osh.optimum(A, B, C_cpu, C_gpu, L0) * L0) <= bs / 2 + 1e-9
    n = 3000
    max_err = 0.0
    for _ in range(n):
        ctl.route(D)
        target = osh.optimum(A, B, C_cpu, C_gpu, ctl.L) * ctl.L
        max_err = max(max_err, abs(ctl.c - target))
    # the admission rounding (<= bs/2) decays into the batch bound after a few batches
    assert max_err <= max(D, bs) / 2 + 1e-6
    assert abs(ctl.c - osh.optimum(A, B, C_cpu, C_gpu, ctl.L) * ctl.L) <= D / 2 + 1e-6
    p = osh.converged(A, B)
    assert abs(ctl.cpu_batches / n - p) <= (max(D, bs) + abs(C_gpu - C_cpu) / (A + B)) / (n * D) + 1.0 / n


def test_cost_tracking_recovers_A_exactly_and_follows_a_change():
    # dyadic values: every sum and product below is exact in float64
    A_true, C_cpu, W = 0.375, 96.0, 8
    ctl = osh.Controller(2.0, 1.0, C_cpu, 0.0, window=W)
    ctl.admit(1024, 64)
    for i in range(W - 1):
        ctl.observe(A_true * (256 + 64 * i) + C_cpu, 256 + 64 * i)
    ctl.route(64)
    assert ctl.A == 2.0  # window not yet full: calibrated value kept
    ctl.observe(A_true * 512 + C_cpu, 512)
    ctl.route(64)
    assert ctl.A == A_true
    A_new = 1.25
    for i in range(W - 1):
        ctl.observe(A_new * (128 + 32 * i) + C_cpu, 128 + 32 * i)
        ctl.route(64)
        assert ctl.A != A_new  # an old sample is still in the window
    ctl.observe(A_new * 64 + C_cpu, 64)
    ctl.route(64)
    assert ctl.A == A_new


def test_cost_tracking_ignores_empty_and_nonpositive_windows():
    ctl = osh.Controller(2.0, 1.0, 50.0, 0.0, window=2)
    ctl.admit(0, 64)
    ctl.observe(10.0, 0.0)
    ctl.observe(10.0, 0.0)
    ctl.route(64)
    assert ctl.A == 2.0          # no CPU tokens in the window
    ctl.observe(20.0, 10.0)
    ctl.observe(20.0, 10.0)      # (40 - 100) / 20 < 0: overhead over-estimated
    ctl.route(64)
    assert ctl.A == 2.0


def test_line_fit_pins():
    x = np.array([1024, 2048, 4096, 8192, 16384], np.float64)
    assert osh.fit_line(x, 0.5 * x + 30.0) == pytest.approx((0.5, 30.0), rel=1e-13)
    rng = np.random.default_rng(3)
    y = 2.5e-7 * x + 4e-5 + rng.normal(0, 1e-6, x.shape)
    slope, icpt = np.polyfit(x, y, 1)
    assert osh.fit_line(x, y) == pytest.approx((slope, icpt), rel=1e-9)


def test_plants_fail_the_pins():
    """A dropped overhead term or a swapped A / B in Eq. 2 breaks the Eq. 1 balance pin."""
    A, B, C_cpu, C_gpu, L = 2.0, 1.0, 10.0, 400.0, 300.0
    wrong = [B / (A + B), A / (A + B) + (C_gpu - C_cpu) / ((A + B) * L),
             B / (A + B) + (C_cpu - C_gpu) / ((A + B) * L)]
    for r in wrong:
        t_cpu, t_gpu = osh.step_latencies(r, L, A, B, C_cpu, C_gpu)
        assert abs(t_cpu - t_gpu) > 1.0


# ---------------------------------------------------------------- library vs oracle


@pytest.mark.parametrize("model", _models(7, 60))
def test_library_optimum_matches_oracle(model):
    A, B, C_cpu, C_gpu, L = model
    assert share_optimum(A, B, C_cpu, C_gpu, L) == osh.optimum(A, B, C_cpu, C_gpu, L)


def test_library_fit_matches_oracle():
    rng = np.random.default_rng(11)
    x = rng.uniform(100, 1e5, 37)
    y = 3e-7 * x + 1e-4 + rng.normal(0, 1e-6, x.shape)
    assert share_fit(x, y) == pytest.approx(osh.fit_line(x, y), rel=1e-10)
    assert share_fit([1, 2], [5, 9]) == pytest.approx((4.0, 1.0), rel=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_library_controller_matches_oracle(seed):
    """Same admission, same A after every refresh, and the same routing decision for every
    batch, over a run with noisy CPU latencies and a drift of A halfway."""
    rng = random.Random(500 + seed)
    A0, B = rng.uniform(0.5, 3.0), rng.uniform(0.2, 3.0)
    C_cpu, C_gpu = rng.uniform(0, 500), rng.uniform(0, 500)
    W, D, bs = rng.choice([1, 4, 32, 256]), rng.choice([64, 256]), 64
    lib = ShareController(A0, B, C_cpu, C_gpu, window=W)
    ora = osh.Controller(A0, B, C_cpu, C_gpu, W)
    L0 = rng.randrange(0, 50000)
    assert lib.admit(L0, bs) == ora.admit(L0, bs)
    A_true = A0 * rng.uniform(0.5, 1.5)
    for step in range(1500):
        if step == 750:
            A_true *= rng.uniform(0.4, 2.5)
        n = float(ora.c)
        t = A_true * n + C_cpu + rng.gauss(0, 5.0)
        t = max(t, 0.0)
        lib.observe(t, n)
        ora.observe(t, n)
        if step % 3 == 0:
            assert lib.route(D) == ora.route(D)
            s = lib.state()
            assert s["cpu_cost"] == ora.A
            assert s["cpu_tokens"] == ora.c and s["placed_tokens"] == ora.L
            assert s["cpu_batches"] == ora.cpu_batches and s["batches"] == ora.batches
    s = lib.state()
    assert s["converged"] == osh.converged(ora.A, B)
    assert s["target_share"] == osh.optimum(ora.A, B, C_cpu, C_gpu, ora.L)
    assert s["samples"] == min(W, 1500)


def test_library_exact_ties_go_to_the_gpu():
    # A = B, no overheads: r = 1/2 exactly; after admit(0) the first 64-token batch has
    # target 32 = c + D/2, an exact tie
    lib = ShareController(1.0, 1.0)
    ora = osh.Controller(1.0, 1.0, 0.0, 0.0, 256)
    lib.admit(0, 64)
    ora.admit(0, 64)
    got = [lib.route(64) for _ in range(8)]
    assert got == [ora.route(64) for _ in range(8)]
    assert got == [False, True] * 4


def test_library_share_validation():
    with pytest.raises(KvattnError) as e:
        share_optimum(-1.0, 1.0, 0, 0, 10)
    assert e.value.status == _lib.E_INVAL
    with pytest.raises(KvattnError):
        share_optimum(0.0, 0.0, 0, 0, 10)
    with pytest.raises(KvattnError):
        share_optimum(1.0, 1.0, 0, 0, 0.0)
    with pytest.raises(KvattnError):
        share_optimum(1.0, float("nan"), 0, 0, 5.0)
    with pytest.raises(KvattnError):
        share_fit([3, 3, 3], [1, 2, 3])
    with pytest.raises(KvattnError):
        ShareController(1.0, 1.0, window=0)
    c = ShareController(1.0, 1.0)
    with pytest.raises(KvattnError) as e:
        c.route(64)
    assert e.value.status == _lib.E_STATE
    with pytest.raises(KvattnError) as e:
        c.observe(1.0, 1.0)
    assert e.value.status == _lib.E_STATE
    c.admit(100, 64)
    with pytest.raises(KvattnError) as e:
        c.admit(100, 64)
    assert e.value.status == _lib.E_STATE
    with pytest.raises(KvattnError):
        c.route(0)
    with pytest.raises(KvattnError):
        c.observe(-1.0, 3.0)
