"""Tier selection on the GPU vs the oracle: bit-exact index lists."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from tests.spax_testlib import log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gpu_plan(x16: np.ndarray, kf: int, ka: int):
    import torch
    import activation_sparse_decode_token_amd as spax
    n = x16.shape[0]
    xd = to_dev(x16)
    F = torch.full((max(kf, 1),), -7, dtype=torch.int32, device=xd.device)
    A = torch.full((max(ka, 1),), -7, dtype=torch.int32, device=xd.device)
    spax.plan_tiers(xd, n, kf, ka, F, A)
    torch.cuda.synchronize()
    return to_host(F)[:kf], to_host(A)[:ka], to_host(F)[kf:], to_host(A)[ka:]


def _check(x16, kf, ka, label):
    F, A, Fpad, Apad = _gpu_plan(x16, kf, ka)
    oF, oA = O.plan_tiers(x16, kf, ka)
    assert np.array_equal(F, oF), f"{label}: full list differs"
    assert np.array_equal(A, oA), f"{label}: approx list differs"
    # nothing written past the lists
    assert np.all(Fpad == -7) and np.all(Apad == -7), f"{label}: wrote past the end"


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 100, 1000, 1024, 4095, 4096, 4097, 8192, 11008,
                               16385, 28672, 32768, 32769, 65536])
def test_plan_random_laplace(n):
    log(f"plan random n={n}")
    x = WL.laplace_fp16(900, 0, "x", n % 997, n)
    rs = np.random.default_rng(n)
    counts = {(0, 0), (n, 0), (0, n), (n // 3, n // 3), (1, 0), (0, 1)}
    for _ in range(4):
        kf = int(rs.integers(0, n + 1))
        counts.add((kf, int(rs.integers(0, n - kf + 1))))
    for kf, ka in sorted(counts):
        if kf + ka <= n:
            _check(x, kf, ka, f"n={n} kf={kf} ka={ka}")


@pytest.mark.parametrize("n", [5, 300, 5000, 30000])
def test_plan_ties(n):
    log(f"plan ties n={n}")
    rs = np.random.default_rng(11 + n)
    cases = {
        "all-equal": np.full(n, -1.5, dtype=np.float16),
        "signed-zeros": rs.choice(np.array([0.0, -0.0], dtype=np.float16), n),
        "small-alphabet": rs.choice(np.array([0, -0.0, 1, -1, 2, -2, 0.5], dtype=np.float16), n),
        "two-valued": rs.choice(np.array([3.0, -3.0, 0.25], dtype=np.float16), n),
        "inf-nan": rs.choice(np.array([np.inf, -np.inf, np.nan, 1.0, -2.0, 0.0],
                                      dtype=np.float16), n),
        "subnormal": (rs.integers(-3, 4, n) * 2.0 ** -24).astype(np.float16),
    }
    for name, x in cases.items():
        for kf, ka in [(n // 4, n // 4), (n // 2, 0), (1, n - 1), (n - 1, 1), (n // 3, n // 2)]:
            _check(x, kf, ka, f"{name} n={n} kf={kf} ka={ka}")


def test_plan_config_inputs():
    for cfg, n, split in [(1, 1024, WL.CONFIGS[1].splits[0]), (2, 4096, WL.CONFIGS[2].splits[0]),
                          (3, 4096, WL.CONFIGS[3].splits[1]), (3, 11008, WL.CONFIGS[3].splits[2]),
                          (4, 11008, WL.CONFIGS[4].splits[0]), (5, 8192, WL.CONFIGS[5].splits[0]),
                          (5, 28672, WL.CONFIGS[5].splits[0])]:
        kf, ka = WL.tier_counts(n, split)
        for tok in range(3):
            x = WL.laplace_fp16(cfg, 0, "x", tok, n)
            _check(x, kf, ka, f"config {cfg} n={n} token {tok}")
    log("plan config inputs ok")
