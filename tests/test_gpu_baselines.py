"""GPU parity of the comparison baselines, through the C ABI, against the CPU
oracle: the unshifted two-pass softmax (naive_softmax_forward) and the top-K
selection over values (os_topk_select), and the unfused Softmax -> TopK
pipelines the fused top-K is compared with.

Bars as for the forward and the top-K: fp32 max |err| <= 2e-6 and per-row
|sum - 1| <= 1e-5, bf16 max relative error <= 8e-3; selection indices and
values exact (the values are copies of the input entries)."""
import numpy as np
import pytest

import workloads
from gpu_util import TOPK_PROB_ABS, assert_parity, say, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ons():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_normalizer_amd
    return online_normalizer_amd


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def bf16_bits(x32):
    return workloads.f32_to_bf16_bits(x32)


# -- the unshifted softmax (paper summary, section 2) ------------------------------

# row lengths through every dispatch class: several rows per wavefront, one
# wavefront, one workgroup, and the streaming kernel past the resident limit
NAIVE_COLS = [1, 3, 100, 128, 129, 1000, 2048, 4097, 8193, 32000, 32001, 70000, 100003]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_naive_softmax(ons, orc, bf16):
    """Inputs whose e^x is finite and normal in fp32 (N(0, 2^2) and U(-10, 10))."""
    for cols in NAIVE_COLS:
        rows = max(3, min(300, (1 << 21) // cols))
        say(f"naive softmax bf16={bf16} rows={rows} cols={cols}")
        x32 = workloads.normal(rows, cols, seed=cols + 5, scale=2.0)
        x32[1::2] = workloads.uniform(rows // 2, cols, seed=cols + 6, lo=-10.0, hi=10.0)
        x32[0, cols // 2] = -np.inf          # adds e^{-inf} = 0
        x = bf16_bits(x32) if bf16 else x32
        y = ons.naive_softmax_forward(to_device(x))
        torch.cuda.synchronize()
        assert_parity(to_host(y), orc.naive_softmax(x), bf16, f"naive cols={cols}")


def test_naive_softmax_full_workloads(ons, orc):
    """The LM-logit rows of workload 2 (entries of +-80 keep e^x finite in fp32)
    and the short rows of workload 4 (first 2^20 rows), in the launch geometry
    the benchmark compares."""
    for n, rows in ((2, None), (4, 1 << 20)):
        x = workloads.config(n) if rows is None else workloads.config(n, 0, rows)
        say(f"naive softmax workload {n} rows={x.shape[0]}")
        y = ons.naive_softmax_forward(to_device(x))
        torch.cuda.synchronize()
        assert_parity(to_host(y), orc.naive_softmax(x, threads=16), False, f"naive workload {n}")


def test_naive_softmax_overflows_where_online_does_not(ons, orc):
    """The failure the page warns of: e^100 is +inf in fp32, so the unshifted
    form gives NaN for that entry and 0 for the rest, while the online
    forward matches the oracle's (safe) softmax."""
    x = workloads.normal(4, 500, seed=9, scale=2.0)
    x[:, 123] = 100.0
    xd = to_device(x)
    yn = to_host(ons.naive_softmax_forward(xd))
    yo = to_host(ons.os_softmax_forward(xd))
    torch.cuda.synchronize()
    assert np.all(np.isnan(yn[:, 123])) and np.all(yn[:, :123] == 0.0)
    assert_parity(yo, orc.softmax(x), False, "online forward next to the overflow")


# -- top-K selection over values ----------------------------------------------------

def check_select(ons, orc, x: np.ndarray, K: int, what: str, nan_rows=None):
    say(f"select {what} rows={x.shape[0]} cols={x.shape[1]} K={K}")
    v, i = ons.os_topk_select(to_device(np.ascontiguousarray(x)), K)
    torch.cuda.synchronize()
    v, i = to_host(v).astype(np.float64), to_host(i)
    vr, ir = orc.topk_select(x, K, threads=8)
    if nan_rows is not None:
        inan = np.sort(i[nan_rows], axis=1)
        assert np.all((inan >= 0) & (inan < x.shape[1])) and np.all(inan[:, 1:] != inan[:, :-1]), what
        keep = np.ones(x.shape[0], dtype=bool)
        keep[nan_rows] = False
        v, i, vr, ir = v[keep], i[keep], vr[keep], ir[keep]
    bad = np.argwhere(i != ir)
    assert bad.size == 0, f"{what}: first index mismatch at {bad[:3].tolist()}"
    assert np.array_equal(v, vr), f"{what}: selected values differ"


@pytest.mark.parametrize("K", [1, 8, 17, 32])
def test_topk_select(ons, orc, K):
    rng = np.random.Generator(np.random.PCG64(40 + K))
    for cols in [K, K + 3, 63, 1000, 4099, 32000, 128256]:
        if cols < K:
            continue
        rows = 256 if cols >= 32000 else 40
        x = workloads.normal(rows, cols, seed=cols * 3 + K, scale=3.0)
        x[::4] = rng.integers(-3, 4, size=x[::4].shape)        # heavy ties
        x[1, :] = -np.inf                                       # only -inf: columns by index
        x[2, cols // 2:] = -np.inf
        x[3, :] = -1.0
        x[3, [0, cols - 1]] = [-0.0, 0.0]                       # -0.0 ties +0.0
        check_select(ons, orc, x, K, f"K={K}")
        check_select(ons, orc, bf16_bits(x), K, f"bf16 K={K}")
        if cols > 1:
            check_select(ons, orc, x[:, 1:], min(K, cols - 1), f"unaligned K={K}")


def test_topk_select_nan_rows(ons, orc):
    x = workloads.normal(8, 5000, seed=3, scale=3.0)
    x[0, 77] = np.nan
    x[1, :] = np.nan
    x[2, :] = -np.inf
    x[2, 4] = np.nan
    check_select(ons, orc, x, 8, "NaN rows", nan_rows=np.arange(3))


# -- the unfused pipelines of the fusion comparison -----------------------------------

def test_unfused_pipelines_workload5(ons, orc):
    """Softmax written out, then selection over the probabilities (the paper
    summary's unfused Online / Safe Softmax + TopK, section 4), on the full
    top-K workload.  Distinct logits may round to equal fp32 probabilities, and
    the selection then orders them by column, so the pipelines need not give
    the fused kernel's order: each rank's probability must be the oracle's
    within the bound, every selected column must carry that probability in the
    oracle's softmax, and the columns must be distinct."""
    x = workloads.config(5)
    K = workloads.TOPK_K
    pr1, ir1 = orc.topk(x, K + 1, threads=16)
    pr, ir = pr1[:, :K], ir1[:, :K]
    # rows whose K + 1 best probabilities are pairwise farther apart than the
    # two sides' errors: there the fp32 probabilities keep the logits' order
    separated = (np.abs(np.diff(pr1, axis=1)) > 2 * TOPK_PROB_ABS).all(axis=1)
    y_ref = orc.softmax(x, threads=16)
    xd = to_device(x)
    for name, fwd in (("online", ons.os_softmax_forward), ("safe", ons.safe_softmax_forward)):
        say(f"unfused {name} pipeline on workload 5")
        y = fwd(xd)
        v, i = ons.os_topk_select(y, K)
        torch.cuda.synchronize()
        v, i = to_host(v).astype(np.float64), to_host(i)
        assert np.max(np.abs(v - pr)) <= TOPK_PROB_ABS, name
        assert np.max(np.abs(np.take_along_axis(y_ref, i.astype(np.int64), axis=1) - pr)) <= TOPK_PROB_ABS, name
        srt = np.sort(i, axis=1)
        assert np.all(srt[:, 1:] != srt[:, :-1]), name
        # where the probabilities are separated, the columns are the fused ones
        assert np.array_equal(i[separated], ir[separated]), name
    assert separated.sum() >= 200  # most rows; the rest hold duplicated maxima


# -- the exponential-rate microbenchmark -----------------------------------------------

@pytest.mark.parametrize("chains", [1, 8])
def test_bench_exp_computes_its_recurrence(ons, chains):
    """Every lane's result is the recurrence v <- 2^v / 2 - 1/2 run `iters`
    times from its start value (numpy in float64; the hardware exponential is
    within a few ulp, and the map contracts, so errors stay ~1e-6)."""
    wgs, iters = 3, 50
    out = torch.full((wgs * 256,), np.nan, dtype=torch.float32, device="cuda")
    say(f"os_bench_exp chains={chains}")
    ons.os_bench_exp(out, wgs, iters, chains)
    torch.cuda.synchronize()
    gid = np.arange(wgs * 256)
    v = np.stack([(gid & 255) / 1024.0 + c / 64.0 - 0.25 for c in range(chains)])
    for _ in range(iters):
        v = np.exp2(v) * 0.5 - 0.5
    ref = v.sum(axis=0)
    assert np.max(np.abs(to_host(out).astype(np.float64) - ref)) <= 1e-5 * chains


def test_device_read_sums(ons):
    """The read reference reads every byte: its per-wave sums add up to the sum
    of the input (small integers, exact in fp32), also with a partial last tile."""
    for n in (4, 1 << 20, (1 << 22) + 12, 10 << 20):
        src = torch.arange(n, device="cuda", dtype=torch.int64).remainder(7).float()
        sink = torch.zeros(4 * 2048, device="cuda")
        say(f"os_device_read {n * 4} bytes")
        ons.os_device_read(src, sink)
        torch.cuda.synchronize()
        assert float(sink.double().sum()) == float(src.double().sum())
