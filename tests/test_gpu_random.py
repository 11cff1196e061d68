"""Seeded random sweep through every entry point, against the CPU oracle.

Each case draws a shape (1 to 64 rows, 1 to 200003 columns), a dtype, a value
scale and a mix of special entries (-inf runs, all -inf rows, NaN, +-80
outliers, copied maxima for ties), and sometimes a base pointer that is only
element-aligned.  The forward, the 3-pass baseline, the logsumexp, the
split-row forward (random slice count) and its no-allocation form, the
unshifted baseline (on inputs whose exponentials stay finite in fp32), and,
for inputs without NaN, the top-K (random K and slice count) and the
selection must each meet the parity bars.  ONORM_RANDOM_CASES sets the number
of cases (48 by default).
"""
import os

import numpy as np
import pytest

import workloads
from gpu_util import TOPK_PROB_ABS, assert_parity, say, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = int(os.environ.get("ONORM_RANDOM_CASES", "48"))
COLS = [1, 2, 3, 5, 8, 17, 63, 64, 100, 127, 255, 511, 1000, 2047, 4096, 4099, 8193, 16384, 32000, 40000, 65536,
        65537, 81920, 131072, 200003]


@pytest.fixture(scope="module")
def ons():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_normalizer_amd
    return online_normalizer_amd


def draw_case(rng: np.random.Generator):
    cols = int(rng.choice(COLS))
    rows = int(rng.choice([1, 2, 3, 7, 16, 33, 64]))
    while rows * cols > (1 << 22) and rows > 1:
        rows //= 2
    x = (rng.standard_normal((rows, cols)) * rng.choice([0.01, 1.0, 5.0, 30.0])).astype(np.float32)
    if rng.random() < 0.3:
        x[rng.random((rows, cols)) < 0.2] = -np.inf
    if rng.random() < 0.15:
        x[int(rng.integers(rows))] = -np.inf
    if rng.random() < 0.2:
        r = int(rng.integers(rows))
        x[r, rng.integers(cols, size=max(1, cols // 1000))] = rng.choice([-80.0, 80.0])
    if rng.random() < 0.2 and cols > 1:  # copies of a row's maximum (ties at the top)
        r = int(rng.integers(rows))
        x[r, rng.integers(cols, size=3)] = np.max(x[r])
    nan = rng.random() < 0.1
    if nan:
        x[int(rng.integers(rows)), int(rng.integers(cols))] = np.nan
    bf16 = bool(rng.random() < 0.4)
    misaligned = bool(rng.random() < 0.25)
    return x, bf16, misaligned, nan


def to_device_at(x: np.ndarray, misaligned: bool):
    """A contiguous device copy of x; with misaligned=True its base sits one
    element past an allocation's start (element-aligned only)."""
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else torch.from_numpy(x)
    if not misaligned:
        return t.cuda()
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    d = buf[1:].view(t.shape)
    d.copy_(t.cuda())
    return d


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case(ons, oracle_lib, case):
    rng = np.random.Generator(np.random.PCG64(9000 + case))
    x32, bf16, misaligned, nan = draw_case(rng)
    x = workloads.f32_to_bf16_bits(x32) if bf16 else x32
    rows, cols = x.shape
    what = f"case {case}: rows={rows} cols={cols} bf16={bf16} misaligned={misaligned} nan={nan}"
    ref = oracle_lib.softmax(x, threads=8)
    lse_ref = oracle_lib.logsumexp(x, threads=8)
    xd = to_device_at(x, misaligned)

    say(f"{what}: forward, safe, lse")
    y = ons.os_softmax_forward(xd)
    s3 = ons.safe_softmax_forward(xd)
    y2, lse = ons.os_softmax_forward_lse(xd, write_y=bool(rng.random() < 0.5))
    torch.cuda.synchronize()
    assert_parity(to_host(y), ref, bf16, f"{what} forward")
    assert_parity(to_host(s3), ref, bf16, f"{what} safe")
    if y2 is not None:
        assert torch.equal(y2.view(torch.int16 if bf16 else torch.int32), y.view(torch.int16 if bf16 else torch.int32))
    lse = to_host(lse).astype(np.float64)
    assert np.array_equal(np.isnan(lse), np.isnan(lse_ref)) and np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= 1e-5 + 2.0 ** -22 * np.abs(lse_ref[fin])), what

    S = int(rng.choice([1, 2, 3, 7, 16, 64, 256]))
    say(f"{what}: split forward S={S}, and on the static scratch")
    ys = ons.os_softmax_forward_split(xd, splits=S)
    Sn = min(S, 16)
    yn = ons.os_softmax_forward_split_noalloc(xd, splits=Sn) if rows * Sn * 8 <= ons.OS_STATIC_SCRATCH_BYTES else None
    torch.cuda.synchronize()
    assert_parity(to_host(ys), ref, bf16, f"{what} split S={S}")
    if yn is not None:
        assert_parity(to_host(yn), ref, bf16, f"{what} split on the static scratch S={Sn}")

    # the unshifted form, where no e^x overflows or underflows to zero sum in fp32
    finite = x32[np.isfinite(x32)]
    if not nan and finite.size and float(finite.max()) < 80.0 and float(finite.min()) > -80.0:
        say(f"{what}: naive")
        yv = ons.naive_softmax_forward(xd)
        torch.cuda.synchronize()
        rn = oracle_lib.naive_softmax(x, threads=8)
        assert_parity(to_host(yv), rn, bf16, f"{what} naive")

    if not nan:
        K = int(rng.integers(1, min(cols, 32) + 1))
        St = int(rng.choice([1, 1, 2, 5, 16]))
        say(f"{what}: top-K K={K} splits={St}")
        p, i = ons.os_softmax_topk(xd, K, splits=St)
        torch.cuda.synchronize()
        pr, ir = oracle_lib.topk(x, K, threads=8)
        assert np.array_equal(to_host(i), ir), f"{what} top-K K={K} S={St}: indices differ"
        p = to_host(p).astype(np.float64)
        assert np.array_equal(np.isnan(p), np.isnan(pr))
        ok = ~np.isnan(pr)
        assert np.max(np.abs(p[ok] - pr[ok]), initial=0.0) <= TOPK_PROB_ABS, what
        say(f"{what}: selection K={K}")
        sv, si = ons.os_topk_select(xd, K)
        torch.cuda.synchronize()
        vr, jr = oracle_lib.topk_select(x, K, threads=8)
        assert np.array_equal(to_host(si), jr), f"{what} selection K={K}: indices differ"
        assert np.array_equal(to_host(sv).astype(np.float64), vr), f"{what} selection K={K}: values differ"
