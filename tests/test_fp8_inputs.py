"""FP8 (OCP e4m3) inputs on the CPU: the decode the oracle's dequantization
relies on, pinned against the format's own definition, and the per-head
quantization recipe of the seeded inputs."""
import math

import numpy as np
import torch

import workloads
from workloads import Workload


def e4m3_by_definition(code: int) -> float:
    """OCP 8-bit floating point, E4M3: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the all-ones
    exponent with mantissa 7 is NaN (no infinities)."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_matches_the_format_definition():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.array([e4m3_by_definition(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert want[~nan].max() == 448.0 and want[1] == 2.0 ** -9


def test_e4m3_rounding_is_to_nearest_even():
    """The fp32 -> e4m3 conversion used for the inputs rounds to the nearest
    representable value, ties to the even code (brute force over all codes)."""
    vals = np.array([e4m3_by_definition(c) for c in range(128)])   # non-negative codes
    finite = ~np.isnan(vals)
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(0, 448, 4000), rng.uniform(0, 2.0 ** -5, 2000),
                        (vals[finite][:-1] + vals[finite][1:]) / 2]).astype(np.float32)
    got = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(int)
    codes = np.nonzero(finite)[0]
    for xi, gi in zip(x.astype(np.float64), got):
        d = np.abs(vals[codes] - xi)
        best = codes[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert gi == want, (xi, gi, want)


def test_quantize_recipe_maps_each_head_max_to_448():
    w = Workload("fp8", 2, 3, 257, 128, "bf16", causal=True, seed=12)
    q8, k8, v8, dq, dk, dv = workloads.draw_fp8(w)
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.H, w.N, w.d), dtype=torch.float32, generator=g)
    assert q8.dtype == torch.float8_e4m3fn and dq.dtype == torch.float32 and dq.shape == (2, 3)
    amax8 = q8.to(torch.float32).abs().amax(dim=(2, 3))
    assert torch.equal(amax8, torch.full_like(amax8, 448.0))
    deq = workloads.dequantize(q8, dq)
    # relative rounding error of e4m3: at most 2^-4 for normals, 2^-10 * descale
    # absolute below the smallest normal
    err = (deq - q.double()).abs()
    bound = torch.maximum(q.double().abs() * 2.0 ** -4, dq.double()[:, :, None, None] * 2.0 ** -10)
    assert bool((err <= bound * (1 + 1e-12)).all())
