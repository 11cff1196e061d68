"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars: fp32 max |err| <= 2e-6 and per-row |sum - 1| <= 1e-5; bf16 max relative
error <= 8e-3; top-K indices bit-exact under (value desc, index asc), top-K
probabilities within 2e-6.  NaN must appear exactly where the oracle has NaN.
"""
import math

import numpy as np
import pytest

import workloads
from gpu_util import (FP32_MAX_ABS, FP32_ROW_SUM, TOPK_PROB_ABS, assert_fp32_parity, assert_parity, say, to_device,
                      to_host)

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


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    return workloads.f32_to_bf16_bits(x32)


def device_at(x: np.ndarray, shift: int, guard: float = 7.0):
    """A contiguous device copy of x whose first element lies `shift` elements
    past a 256-byte aligned allocation, with `guard`-valued elements around it."""
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else torch.from_numpy(x)
    buf = torch.full((t.numel() + shift + 16,), guard, dtype=t.dtype, device="cuda")
    d = buf[shift:shift + t.numel()].view(t.shape)
    d.copy_(t.cuda())
    return d


def guards_intact(t, shift: int, guard: float = 7.0) -> bool:
    """True when the elements around the view made by device_at still hold `guard`."""
    base = t.untyped_storage()
    flat = torch.empty(0, dtype=t.dtype, device=t.device).set_(base, 0, (base.nbytes() // t.element_size(),))
    head = flat[:shift]
    tail = flat[shift + t.numel():]
    return bool((head == guard).all()) and bool((tail == guard).all())


def run_forward(ons, x: np.ndarray, **kw):
    xd = to_device(x)
    if "lanes" in kw:
        y = ons.os_softmax_forward_tuned(xd, kw["lanes"], kw.get("vecs", 0), kw.get("grid", 0))
    elif kw.get("safe"):
        y = ons.safe_softmax_forward(xd)
    else:
        y = ons.os_softmax_forward(xd)
    torch.cuda.synchronize()
    return to_host(y)


# -- the pages' worked examples --------------------------------------------------

def test_two_shard_example(ons, orc):
    say("two-shard row [1,2,3]")
    x = workloads.two_shard_row()
    y = run_forward(ons, x)
    assert_fp32_parity(y, orc.softmax(x), "two-shard")
    m, d = ons.os_softmax_stats(to_device(x))
    torch.cuda.synchronize()
    assert float(m[0]) == 3.0
    assert abs(float(d[0]) - (1.0 + math.exp(-1.0) + math.exp(-2.0))) <= 2e-7
    # each shard's state on the GPU, merged by the oracle's operator
    ma, da = ons.os_softmax_stats(to_device(np.array([[1.0, 2.0]], dtype=np.float32)))
    mb, db = ons.os_softmax_stats(to_device(np.array([[3.0]], dtype=np.float32)))
    torch.cuda.synchronize()
    assert float(ma[0]) == 2.0 and abs(float(da[0]) - 1.367879) <= 1e-6
    assert float(mb[0]) == 3.0 and float(db[0]) == 1.0
    mab, dab = orc.combine((float(ma[0]), float(da[0])), (float(mb[0]), float(db[0])))
    assert mab == 3.0 and abs(dab - 1.503214) <= 1e-6


def test_lesson_mock_vector(ons, orc):
    say("mock vector")
    x = workloads.mock_row()
    assert_fp32_parity(run_forward(ons, x), orc.softmax(x), "mock")


def test_config1(ons, orc):
    say("config 1: 64x1024 fp32")
    x = workloads.config(1)
    assert_fp32_parity(run_forward(ons, x), orc.softmax(x), "config1")


# -- every kernel shape, ragged and unaligned tails ---------------------------------

SHAPES = [(lanes, vecs) for lanes in (4, 8, 16, 32) for vecs in (1, 2, 4)] + \
    [(lanes, vecs) for lanes in (64, 128, 256, 512, 1024) for vecs in (1, 2, 4, 8)] + \
    [(256, 5), (512, 5), (512, 6), (1024, 5), (1024, 6), (1024, 7), (1024, 16)]


# (1024 x 16 is built for fp32 only)
SHAPE_CASES = [(lanes, vecs, bf16) for bf16 in (False, True) for lanes, vecs in SHAPES
               if not (bf16 and (lanes, vecs) == (1024, 16))]


@pytest.mark.parametrize("lanes,vecs,bf16", SHAPE_CASES,
                         ids=[f"{'bf16' if b else 'f32'}-{a}x{v}" for a, v, b in SHAPE_CASES])
def test_every_resident_shape(ons, orc, lanes, vecs, bf16):
    vec = 8 if bf16 else 4
    cap = lanes * vecs * vec
    # aligned rows may fill the shape; a row that is not 16-byte aligned may
    # span one more 16-byte block, so it fits when cols + vec - 1 <= cap
    cases = {cap, cap - vec, cap - vec + 1, max(1, cap // 2 + 3), max(1, cap // 3)}
    for cols in sorted(c for c in cases if c + (0 if c % vec == 0 else vec - 1) <= cap):
        rows = 37
        say(f"resident {lanes}x{vecs} bf16={bf16} rows={rows} cols={cols}")
        x32 = workloads.normal(rows, cols, seed=cols * 7 + lanes, scale=2.0)
        x = bf16_bits(x32) if bf16 else x32
        y = run_forward(ons, x, lanes=lanes, vecs=vecs)
        assert_parity(y, orc.softmax(x), bf16, f"{lanes}x{vecs} cols={cols}")
    # the longest row the shape holds from an element-aligned base
    cols = cap - vec + 1
    say(f"resident {lanes}x{vecs} bf16={bf16} cols={cols} from an element-aligned base")
    x32 = workloads.normal(9, cols, seed=cols + 3 * lanes, scale=2.0)
    x = bf16_bits(x32) if bf16 else x32
    xin = device_at(x, 1)
    y = ons.os_softmax_forward_tuned(xin, lanes, vecs)
    torch.cuda.synchronize()
    assert_parity(to_host(y), orc.softmax(x), bf16, f"{lanes}x{vecs} cols={cols} shifted")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_auto_dispatch_edge_columns(ons, orc, bf16):
    cols_list = [1, 2, 3, 5, 7, 8, 9, 31, 32, 33, 63, 64, 65, 127, 128, 129, 257, 1000, 1023, 1024, 1025,
                 2047, 2048, 2049, 4097, 8191, 8193, 16385, 26001, 28000, 32000, 32768, 32769, 53001, 56000, 65536,
                 65537, 100003]
    for cols in cols_list:
        rows = 19 if cols < 20000 else 5
        say(f"auto bf16={bf16} rows={rows} cols={cols}")
        x32 = workloads.normal(rows, cols, seed=1000 + cols, scale=3.0)
        x = bf16_bits(x32) if bf16 else x32
        ref = orc.softmax(x)
        assert_parity(run_forward(ons, x), ref, bf16, f"auto cols={cols}")
        assert_parity(run_forward(ons, x, safe=True), ref, bf16, f"safe cols={cols}")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_auto_plan_dense_lengths(ons, orc, bf16):
    """Every row length up to 600 slots (2400 fp32, 4800 bf16 entries; every
    third length past the first 200), so every entry of the automatic plan,
    direct or read through LDS, and every switch between them runs, on
    aligned and element-aligned bases."""
    vec = 8 if bf16 else 4
    lengths = list(range(1, 200)) + list(range(200, 600 * vec + 1, 3))
    for cols in lengths:
        rows = 5
        x32 = workloads.normal(rows, cols, seed=cols * 3 + bf16, scale=3.0)
        x = bf16_bits(x32) if bf16 else x32
        ref = orc.softmax(x)
        for si in ((0, 1) if cols % vec else (0,)):
            say(f"dense lengths bf16={bf16} rows={rows} cols={cols} in+{si}")
            xin = device_at(x, si)
            y = ons.os_softmax_forward(xin)
            torch.cuda.synchronize()
            assert_parity(to_host(y), ref, bf16, f"auto cols={cols} in+{si}")


@pytest.mark.parametrize("cols,rows", [(32000, 1024), (8000, 2048)], ids=["1024x8", "512x8"])
def test_dense_small_batches(ons, orc, cols, rows):
    """fp32 rows on 8-vector shapes: batches of up to two rounds of
    workgroups take the kernel held to 64 VGPRs, one row more takes the
    default one; the two must agree bit for bit, and with the oracle."""
    say(f"dense fp32 rows={rows}/{rows + 1} cols={cols}")
    x = workloads.normal(rows + 1, cols, seed=cols + rows, scale=2.0)
    y_big = run_forward(ons, x)
    y_small = run_forward(ons, x[:rows])
    assert np.array_equal(y_small.view(np.uint32), y_big[:rows].view(np.uint32)), "dense and default kernels differ"
    pick = np.r_[0:4, rows // 2, rows - 3:rows + 1]
    assert_parity(y_big[pick], orc.softmax(x[pick]), False, f"dense cols={cols}")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_streaming_two_pass(ons, orc, bf16):
    for rows, cols in [(3, 1), (5, 100), (7, 4096), (9, 32000), (3, 200001), (2, 1 << 20)]:
        say(f"stream bf16={bf16} rows={rows} cols={cols}")
        x32 = workloads.normal(rows, cols, seed=cols + 5, scale=2.0)
        x = bf16_bits(x32) if bf16 else x32
        assert_parity(run_forward(ons, x, lanes=0), orc.softmax(x), bf16, f"stream cols={cols}")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_hybrid_long_rows(ons, orc, bf16):
    """Aligned rows past the register-resident plans (up to 262144 columns) take the
    hybrid kernel: the first 1024 x VPL vectors stay in registers (fp32: 32768,
    49152 or 65536 elements by row length; bf16: 57344), the next 32768 (fp32)
    or 65536 (bf16) stream once and are kept in LDS, the rest stream twice;
    lengths at and just past the end of the LDS copy for each register part.
    Rows put the maximum in the streamed part only, make the first 65536
    entries (or all but the last 5) -inf, or hold NaN / +inf / only -inf."""
    for rows, cols in ((3, 65544), (17, 100000), (5, 128256), (2, 200000), (2, 262144), (3, 98304), (3, 98308),
                       (3, 122880), (3, 122888), (5, 32772), (5, 49152), (5, 65536), (3, 81920), (3, 81924),
                       (3, 110000), (3, 110004)):
        x32 = workloads.normal(rows, cols, seed=cols + 3, scale=3.0)
        x32[0, cols - 5] = 90.0                 # the row maximum, in the streamed part
        if rows > 2:
            x32[1, :min(65536, cols - 5)] = -np.inf  # nothing in the register part
            x32[2, 70000 % cols] = np.nan
        if rows > 4:
            x32[3, :] = -np.inf
            x32[4, 100] = np.inf
        x = bf16_bits(x32) if bf16 else x32
        ref = orc.softmax(x, threads=8)
        say(f"hybrid bf16={bf16} rows={rows} cols={cols}")
        assert_parity(run_forward(ons, x), ref, bf16, f"hybrid cols={cols}")
        assert_parity(run_forward(ons, x, lanes=0), ref, bf16, f"stream cols={cols}")
        xd = to_device(x)
        m, d = ons.os_softmax_stats(xd)
        _, lse = ons.os_softmax_forward_lse(xd, write_y=False)
        y = ons.os_softmax_forward(xd)
        yi = ons.os_softmax_forward(xd, out=xd)  # in place
        torch.cuda.synchronize()
        assert torch.equal(bits(yi), bits(y))
        mo, do = orc.stats(x, threads=8)
        m, d = to_host(m).astype(np.float64), to_host(d).astype(np.float64)
        fin = np.isfinite(do) & (do > 0)
        assert np.array_equal(m[fin], mo[fin]) and np.max(np.abs(d[fin] - do[fin]) / do[fin], initial=0.0) <= 1e-5
        lo = orc.logsumexp(x, threads=8)
        lse = to_host(lse).astype(np.float64)
        assert np.array_equal(np.isnan(lse), np.isnan(lo)) and np.array_equal(np.isneginf(lse), np.isneginf(lo))
        f = np.isfinite(lo)
        assert np.all(np.abs(lse[f] - lo[f]) <= lse_tol(lo[f]))


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_safe_three_pass(ons, orc, bf16):
    for rows, cols in [(3, 1), (11, 33), (7, 4096), (9, 32000), (3, 200001)]:
        say(f"safe3 bf16={bf16} rows={rows} cols={cols}")
        x32 = workloads.normal(rows, cols, seed=cols + 9, scale=2.0)
        x = bf16_bits(x32) if bf16 else x32
        assert_parity(run_forward(ons, x, safe=True), orc.softmax(x), bf16, f"safe cols={cols}")


def test_grid_stride_with_few_blocks(ons, orc):
    """Few workgroups striding over many rows (LDS slot reuse across rows)."""
    for lanes, vecs, cols in [(1024, 8, 30000), (256, 8, 7000), (8, 4, 128), (64, 4, 1024)]:
        say(f"grid-stride {lanes}x{vecs} cols={cols}")
        x = workloads.normal(301, cols, seed=cols + 1, scale=2.0)
        y = run_forward(ons, x, lanes=lanes, vecs=vecs, grid=3)
        assert_fp32_parity(y, orc.softmax(x), f"grid=3 {lanes}x{vecs}")
    say("grid-stride stream")
    x = workloads.normal(33, 70000, seed=3, scale=2.0)
    assert_fp32_parity(run_forward(ons, x, lanes=0, grid=2), orc.softmax(x), "stream grid=2")


def test_many_rows_cap_the_grid(ons):
    """More rows than a single launch can hold threads for: the grid is capped
    and the kernels stride over the rest (cols = 1, so every output is 1)."""
    rows = 40_000_000
    x = torch.randn(rows, 1, device="cuda")
    for kw in ({"lanes": 0}, {"safe": True}, {}):
        say(f"many rows {rows}x1 {kw}")
        if "lanes" in kw:
            y = ons.os_softmax_forward_tuned(x, 0, 0)
        elif kw:
            y = ons.safe_softmax_forward(x)
        else:
            y = ons.os_softmax_forward(x)
        torch.cuda.synchronize()
        assert bool((y == 1.0).all()), kw


def test_misaligned_base_and_in_place(ons, orc):
    x = workloads.normal(23, 1024, seed=77, scale=2.0)
    ref = orc.softmax(x)
    say("misaligned base pointer")
    flat = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
    flat[1:] = torch.from_numpy(x.reshape(-1)).cuda()
    xin = flat[1:].view(23, 1024)
    out_flat = torch.zeros(x.size + 3, dtype=torch.float32, device="cuda")
    yout = out_flat[3:].view(23, 1024)
    ons.os_softmax_forward(xin, out=yout)
    torch.cuda.synchronize()
    assert_fp32_parity(to_host(yout), ref, "misaligned")
    say("in place")
    xd = to_device(x)
    ons.os_softmax_forward(xd, out=xd)
    torch.cuda.synchronize()
    assert_fp32_parity(to_host(xd), ref, "in-place")
    xd = to_device(x)
    ons.safe_softmax_forward(xd, out=xd)
    torch.cuda.synchronize()
    assert_fp32_parity(to_host(xd), ref, "in-place safe")


# 5, 31, 63, 127, 129, 255, 511 and 1023 (bf16) take multi-row shapes that read
# the rows through LDS; 1001 (bf16) and 1023 (fp32) keep direct loads
UNALIGNED_COLS = [1, 3, 5, 31, 63, 127, 129, 255, 511, 1001, 1023, 2047, 4099, 32001, 50257, 65535, 65537, 100003,
                  262147]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_unaligned_rows_every_path(ons, orc, bf16):
    """Rows that are not 16-byte aligned (odd lengths, element-aligned bases,
    input and output at different offsets) through every forward entry point,
    the safe baseline and the top-K: parity, and no store outside the output."""
    shifts = [(0, 0), (1, 1), (1, 3), (2, 0), (0, 1)] + ([(3, 5), (7, 7)] if bf16 else [(3, 3)])
    for cols in UNALIGNED_COLS:
        rows = 37 if cols < 5000 else (7 if cols < 100000 else 3)
        x32 = workloads.normal(rows, cols, seed=7 * cols + bf16, scale=3.0)
        x = bf16_bits(x32) if bf16 else x32
        ref = orc.softmax(x)
        lse_ref = orc.logsumexp(x, threads=8)
        for si, so in shifts:
            what = f"bf16={bf16} rows={rows} cols={cols} in+{si} out+{so}"
            say(f"unaligned forward/safe/lse/split {what}")
            xin = device_at(x, si)
            for name, call in (("forward", lambda o: ons.os_softmax_forward(xin, out=o)),
                               ("safe", lambda o: ons.safe_softmax_forward(xin, out=o)),
                               ("lse", lambda o: ons.os_softmax_forward_lse(xin, out=o)),
                               ("split3", lambda o: ons.os_softmax_forward_split(xin, splits=3, out=o)),
                               ("split-plan", lambda o: ons.os_softmax_forward_split(xin, out=o))):
                out = device_at(np.zeros_like(x), so)
                r = call(out)
                torch.cuda.synchronize()
                assert_parity(to_host(out), ref, bf16, f"{name} {what}")
                assert guards_intact(out, so), f"{name} {what}: a store landed outside the output"
                if name == "lse":
                    L = to_host(r[1]).astype(np.float64)
                    assert np.all(np.abs(L - lse_ref) <= lse_tol(lse_ref)), what
            assert guards_intact(xin, si), f"{what}: the input was written"
        say(f"unaligned in place / stats / top-K bf16={bf16} cols={cols}")
        for si in (1, 3):
            xd = device_at(x, si)
            ons.os_softmax_forward(xd, out=xd)
            torch.cuda.synchronize()
            assert_parity(to_host(xd), ref, bf16, f"in place +{si} cols={cols}")
            assert guards_intact(xd, si)
            xd = device_at(x, si)
            ons.os_softmax_forward_split(xd, splits=2, out=xd)
            torch.cuda.synchronize()
            assert_parity(to_host(xd), ref, bf16, f"split in place +{si} cols={cols}")
            xd = device_at(x, si)
            m, d = ons.os_softmax_stats(xd)
            torch.cuda.synchronize()
            m_ref, d_ref = orc.stats(x)
            assert np.array_equal(to_host(m).astype(np.float64), m_ref), f"stats m +{si} cols={cols}"
            assert np.max(np.abs(to_host(d) - d_ref) / d_ref) <= 1e-5, f"stats d +{si} cols={cols}"
            K = min(cols, 8)
            for splits in (1, 3):
                p, i = ons.os_softmax_topk(xd, K, splits=splits)
                torch.cuda.synchronize()
                pr, ir = orc.topk(x, K, threads=8)
                assert np.array_equal(to_host(i), ir), f"top-{K} +{si} S={splits} cols={cols}: indices"
                assert np.max(np.abs(to_host(p) - pr)) <= TOPK_PROB_ABS, f"top-{K} +{si} cols={cols}"


@pytest.mark.parametrize("cols", [6, 63, 127, 128, 1024, 32000, 70000])
def test_special_values(ons, orc, cols):
    """-inf entries give 0; rows with +inf, NaN, or only -inf give NaN rows."""
    x = workloads.normal(8, cols, seed=cols, scale=2.0)
    x[0, ::3] = -np.inf
    x[1, :] = -np.inf
    x[2, cols // 2] = np.inf
    x[3, cols - 1] = np.nan
    x[4, 0] = 80.0
    x[4, cols - 1] = 80.0
    x[5, :] = -np.inf
    x[5, cols - 1] = -3.0e38
    x[6, :] = 0.0
    ref = orc.softmax(x)
    for kw in ({}, {"safe": True}, {"lanes": 0}):
        say(f"special values cols={cols} {kw}")
        assert_fp32_parity(run_forward(ons, x, **kw), ref, f"special {kw}")
    say(f"special values stats cols={cols}")
    m, d = ons.os_softmax_stats(to_device(x))
    torch.cuda.synchronize()
    m, d = to_host(m), to_host(d)
    assert m[1] == -np.inf and d[1] == 0.0  # identity state of an all -inf row
    assert m[5] == np.float32(-3.0e38) and d[5] == 1.0


def test_shift_invariance_is_bitwise(ons):
    """Exact shifts (grid values, +64) give bitwise identical outputs on every path."""
    for cols, kw in [(128, {}), (1024, {}), (32000, {}), (5000, {"lanes": 0}), (300, {"safe": True}),
                     (1000, {"lanes": 64, "vecs": 4})]:
        say(f"shift invariance cols={cols} {kw}")
        x = workloads.grid_values(17, cols, seed=cols)
        y0 = run_forward(ons, x, **kw)
        y1 = run_forward(ons, x + np.float32(64.0), **kw)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def test_deterministic(ons):
    x = to_device(workloads.config(2, 0, 512))
    say("determinism")
    a = ons.os_softmax_forward(x)
    b = ons.os_softmax_forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_graph_replays_match_eager(ons):
    """The forward (aligned rows, unaligned rows with direct, LDS-assembled
    and LDS-read stores, and long rows with their LDS copy), the baseline, the
    top-K (tiled, short-row on 32 and 64 entries per lane, bf16 short-row on
    packed entries, and split over two launches) and the split forward
    captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    x = to_device(workloads.config(2, 0, 512))
    xt = to_device(workloads.config(5, 0, 8))
    say("graph capture")
    y_ref = ons.os_softmax_forward(x)
    s_ref = ons.safe_softmax_forward(x)
    p_ref, i_ref = ons.os_softmax_topk(xt, 8)
    xs = to_device(workloads.normal(4, 100003, seed=9, scale=3.0))
    ws = torch.empty(ons.os_softmax_forward_workspace_bytes(4, 8), dtype=torch.uint8, device="cuda")
    sp_ref = ons.os_softmax_forward_split(xs, splits=8, workspace=ws)
    # the split top-K (two launches), the short-row top-K, and unaligned and long-row forwards
    xk = to_device(workloads.normal(16, 128256, seed=10, scale=3.0))
    wk = torch.empty(ons.os_softmax_topk_workspace_bytes(16, 8, 4), dtype=torch.uint8, device="cuda")
    pk_ref, ik_ref = ons.os_softmax_topk_ex(xk, 8, 4, wk)
    xw = to_device(workloads.normal(4200, 512, seed=11, scale=3.0))
    pw_ref, iw_ref = ons.os_softmax_topk_ex(xw, 8, 1, None)
    xb = to_device(bf16_bits(workloads.normal(4200, 512, seed=15, scale=3.0)))    # bf16, packed entries
    pb_ref, ib_ref = ons.os_softmax_topk_ex(xb, 8, 1, None)
    xv = to_device(workloads.normal(16384, 512, seed=16, scale=3.0))              # 64 entries per lane
    pv_ref, iv_ref = ons.os_softmax_topk_ex(xv, 32, 1, None)
    xu = to_device(workloads.normal(64, 50257, seed=12, scale=3.0))
    yu_ref = ons.os_softmax_forward(xu)
    x1 = to_device(workloads.normal(5000, 127, seed=13, scale=3.0))   # read through LDS
    x2 = to_device(workloads.normal(3000, 501, seed=14, scale=3.0))   # stores assembled in LDS
    y1_ref, y2_ref, yk_ref = ons.os_softmax_forward(x1), ons.os_softmax_forward(x2), ons.os_softmax_forward(xk)
    torch.cuda.synchronize()
    y = torch.empty_like(x)
    s3 = torch.empty_like(x)
    sp = torch.empty_like(xs)
    yu = torch.empty_like(xu)
    y1, y2, yk = torch.empty_like(x1), torch.empty_like(x2), torch.empty_like(xk)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ons.os_softmax_forward(x, out=y)
        ons.safe_softmax_forward(x, out=s3)
        p, i = ons.os_softmax_topk(xt, 8)
        ons.os_softmax_forward_split(xs, splits=8, out=sp, workspace=ws)
        pk, ik = ons.os_softmax_topk_ex(xk, 8, 4, wk)
        pw, iw = ons.os_softmax_topk_ex(xw, 8, 1, None)
        pb, ib = ons.os_softmax_topk_ex(xb, 8, 1, None)
        pv, iv = ons.os_softmax_topk_ex(xv, 32, 1, None)
        ons.os_softmax_forward(xu, out=yu)
        ons.os_softmax_forward(x1, out=y1)
        ons.os_softmax_forward(x2, out=y2)
        ons.os_softmax_forward(xk, out=yk)
    for rep in range(4):
        for t in (y, s3, p, i, sp, pk, ik, pw, iw, pb, ib, pv, iv, yu, y1, y2, yk):
            t.zero_()
        junk = ons.os_softmax_forward(torch.randn(64, 1000, device="cuda"))  # eager work between replays
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), rep
        assert torch.equal(s3.view(torch.int32), s_ref.view(torch.int32)), rep
        assert torch.equal(p, p_ref) and torch.equal(i, i_ref), rep
        assert torch.equal(sp.view(torch.int32), sp_ref.view(torch.int32)), rep
        assert torch.equal(pk, pk_ref) and torch.equal(ik, ik_ref), rep
        assert torch.equal(pw, pw_ref) and torch.equal(iw, iw_ref), rep
        assert torch.equal(pb, pb_ref) and torch.equal(ib, ib_ref), rep
        assert torch.equal(pv, pv_ref) and torch.equal(iv, iv_ref), rep
        assert torch.equal(yu.view(torch.int32), yu_ref.view(torch.int32)), rep
        for got, want in ((y1, y1_ref), (y2, y2_ref), (yk, yk_ref)):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), rep
        del junk


def test_graph_replays_more_entries(ons):
    """The naive two-pass forward, the value selection, the split forward on
    the library's static scratch, and the attention forward (full and causal,
    with a ragged key tail) captured in one HIP graph: every replay, with eager
    calls of the same entry points on other inputs between replays, equals the
    eager result bit for bit."""
    x = to_device(workloads.config(2, 0, 256))
    xs = to_device(workloads.normal(8, 100003, seed=21, scale=3.0))
    xt = to_device(bf16_bits(workloads.normal(64, 32000, seed=22, scale=3.0)))
    q, k, v = (to_device(a) for a in workloads.attention_qkv(4, 320, 320, 128, 23))
    say("graph capture (naive, select, no-alloc split, attention)")
    n_ref = ons.naive_softmax_forward(x)
    sv_ref, si_ref = ons.os_topk_select(xt, 8)
    ns_ref = ons.os_softmax_forward_split_noalloc(xs, splits=8)
    o_ref, l_ref = ons.os_attention_forward(q, k, v)
    oc_ref, lc_ref = ons.os_attention_forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    n, ns = torch.empty_like(x), torch.empty_like(xs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ons.naive_softmax_forward(x, out=n)
        sv, si = ons.os_topk_select(xt, 8)
        ons.os_softmax_forward_split_noalloc(xs, splits=8, out=ns)
        o, l = ons.os_attention_forward(q, k, v)
        oc, lc = ons.os_attention_forward(q, k, v, causal=True)
    other = to_device(workloads.normal(4, 70001, seed=24, scale=3.0))
    for rep in range(4):
        for t in (n, sv, si, ns, o, l, oc, lc):
            t.zero_()
        # eager calls between replays, the no-allocation one on the same static scratch
        junk = [ons.os_softmax_forward_split_noalloc(other, splits=4), ons.naive_softmax_forward(other),
                ons.os_attention_forward(k, q, v)]
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(n.view(torch.int32), n_ref.view(torch.int32)), rep
        assert torch.equal(sv, sv_ref) and torch.equal(si, si_ref), rep
        assert torch.equal(ns.view(torch.int32), ns_ref.view(torch.int32)), rep
        for got, want in ((o, o_ref), (oc, oc_ref)):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), rep
        for got, want in ((l, l_ref), (lc, lc_ref)):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), rep
        del junk


def test_binding_rejects_bad_outputs(ons):
    """Caller-supplied outputs and workspaces of the wrong shape, dtype or
    layout are refused by the binding before any launch (the library writes
    rows * K entries through their pointers)."""
    x = to_device(workloads.normal(16, 1000, seed=31, scale=3.0))
    say("binding output checks")
    good_v = torch.empty(16, 8, device="cuda")
    good_i = torch.empty(16, 8, dtype=torch.int32, device="cuda")
    bad = [
        dict(vals=torch.empty(16, 4, device="cuda")),                        # too few columns
        dict(vals=torch.empty(8, 8, device="cuda")),                         # too few rows
        dict(idx=torch.empty(16, 8, dtype=torch.int64, device="cuda")),      # wrong dtype
        dict(idx=torch.empty(8, 16, dtype=torch.int32, device="cuda").t()),  # not contiguous
        dict(vals=torch.empty(16, 8)),                                       # host memory
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            ons.os_topk_select(x, 8, **kw)
        kwp = {"probs" if k == "vals" else k: v for k, v in kw.items()}
        with pytest.raises(ValueError):
            ons.os_softmax_topk_ex(x, 8, 1, None, **kwp)
    with pytest.raises(ValueError):
        ons.os_softmax_forward_split(x, splits=2, workspace=torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ons.os_device_copy(x.t(), torch.empty_like(x))
    v, i = ons.os_topk_select(x, 8, good_v, good_i)
    p, j = ons.os_softmax_topk_ex(x, 8, 1, None, torch.empty_like(good_v), torch.empty_like(good_i))
    torch.cuda.synchronize()
    assert v.data_ptr() == good_v.data_ptr() and torch.equal(i, j)


def test_stats_invariants(ons, orc):
    """1 <= d <= N (up to fp32 rounding), m is the exact row maximum, d matches the oracle."""
    for n in (1, 2, 4):
        x = workloads.config(n, 0, 256)
        say(f"stats config {n}")
        m, d = ons.os_softmax_stats(to_device(x))
        torch.cuda.synchronize()
        m, d = to_host(m).astype(np.float64), to_host(d).astype(np.float64)
        mo, do = orc.stats(x)
        N = x.shape[1]
        assert np.array_equal(m, mo)
        assert np.all(d >= 1.0) and np.all(d <= N * (1 + N * 2.0 ** -24))
        assert np.max(np.abs(d - do) / do) <= 1e-5
    xb = workloads.config(3, 0, 256)
    m, d = ons.os_softmax_stats(to_device(xb))
    torch.cuda.synchronize()
    mo, do = orc.stats(xb)
    assert np.array_equal(to_host(m).astype(np.float64), mo)
    assert np.max(np.abs(to_host(d) - do) / do) <= 1e-5


# -- split-row forward ---------------------------------------------------------------

def run_split(ons, x: np.ndarray, splits, ws=None):
    xd = to_device(x)
    y = ons.os_softmax_forward_split(xd, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_split_forward(ons, orc, bf16):
    """Slices of every size class, ragged last slices, more slices than vectors
    (empty trailing slices), unaligned rows, and splits 1..256."""
    cases = [(3, 1, 4), (5, 7, 16), (4, 100, 3), (7, 4096, 2), (3, 4097, 5), (2, 32000, 16), (5, 32003, 7),
             (3, 65536, 8), (2, 200001, 16), (2, 1 << 20, 16), (1, 1 << 20, 3), (2, 300007, 100),
             (1, 1 << 20, 256), (2, 5000, 256)]
    for rows, cols, S in cases:
        say(f"split forward bf16={bf16} rows={rows} cols={cols} S={S}")
        x32 = workloads.normal(rows, cols, seed=cols + S, scale=3.0)
        x32[0, cols - 1] = 60.0
        x = bf16_bits(x32) if bf16 else x32
        assert_parity(run_split(ons, x, S), orc.softmax(x), bf16, f"split rows={rows} cols={cols} S={S}")


def test_split_forward_plan_and_specials(ons, orc):
    """The planned split on a small batch of long rows; special-value rows; in place; determinism."""
    x = workloads.normal(8, 70000, seed=5, scale=2.0)
    x[0, ::3] = -np.inf
    x[1, :] = -np.inf
    x[2, 50000] = np.inf
    x[3, 69999] = np.nan
    x[4, 0] = 80.0
    x[4, 69999] = 80.0
    x[5, :] = -np.inf
    x[5, 12345] = -3.0e38
    S = ons.os_forward_split_plan(8, 70000)
    say(f"split specials S={S}")
    assert S > 1
    ref = orc.softmax(x)
    assert_fp32_parity(run_split(ons, x, None), ref, "split specials (plan)")
    for S in (2, 16):
        assert_fp32_parity(run_split(ons, x, S), ref, f"split specials S={S}")
    xd = to_device(x)
    y1 = ons.os_softmax_forward_split(xd, splits=8)
    y2 = ons.os_softmax_forward_split(xd, splits=8)
    y3 = ons.os_softmax_forward_split(xd, splits=8, out=xd)  # in place
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert y3.data_ptr() == xd.data_ptr() and torch.equal(xd.view(torch.int32), y1.view(torch.int32))


def test_split_launches_past_the_grid_cap(ons, orc):
    """More (row, slice) units than one launch's 2^31 threads hold: the split
    kernels stride over the rest (forward: 35.8M one-wave units; top-K: 4.8M
    512-thread units; top-K merge: 34M rows at one per wavefront)."""
    x = workloads.normal(140000, 4, seed=140, scale=3.0)
    say("split forward past the grid cap: 140000 rows x 256 slices")
    assert_fp32_parity(run_split(ons, x, 256), orc.softmax(x, threads=8), "split forward, grid stride")
    xt = workloads.normal(300000, 32, seed=300, scale=3.0)
    say("split top-K past the grid cap: 300000 rows x 16 slices")
    p, i = ons.os_softmax_topk(to_device(xt), 1, splits=16)
    torch.cuda.synchronize()
    pr, ir = orc.topk(xt, 1, threads=8)
    assert np.array_equal(to_host(i), ir)
    assert np.max(np.abs(to_host(p).astype(np.float64) - pr)) <= TOPK_PROB_ABS
    # the split top-K's merge launch (one row per wavefront) past its own cap:
    # more than 4 x 2^31 / 256 rows
    xm = workloads.normal(34_000_000, 2, seed=34, scale=3.0)
    say("split top-K merge past the grid cap: 34M rows x 2 slices")
    p, i = ons.os_softmax_topk(to_device(xm), 1, splits=2)
    torch.cuda.synchronize()
    pr, ir = orc.topk(xm, 1, threads=16)
    assert np.array_equal(to_host(i), ir)
    assert np.max(np.abs(to_host(p).astype(np.float64) - pr)) <= TOPK_PROB_ABS


def test_maximum_row_length(ons, orc):
    """One row of the longest length the library takes (OS_MAX_COLS = 2^28
    entries: 1 GiB in fp32, 512 MiB in bf16), through the forward (one
    workgroup streaming the row) and the planned split forward, every output
    against the oracle in blocks of 2^24, and the fp32 row's sum."""
    n = 1 << 28
    x32 = workloads.normal(1, n, seed=28, scale=3.0)
    x32[0, n - 7] = 40.0  # the maximum near the end: every earlier part is rescaled
    for bf16 in (False, True):
        x = bf16_bits(x32) if bf16 else x32
        ref = orc.softmax(x)[0]
        xd = to_device(x)
        for name in ("forward", "split forward"):
            say(f"maximum row length 2^28, bf16={bf16}, {name}")
            y = ons.os_softmax_forward(xd) if name == "forward" else ons.os_softmax_forward_split(xd)
            torch.cuda.synchronize()
            yh = to_host(y)[0]
            del y
            blk = 1 << 24
            for b0 in range(0, n, blk):
                got, want = yh[b0:b0 + blk], ref[b0:b0 + blk]
                if bf16:
                    assert_parity(got[None], want[None], True, f"{name} bf16 block {b0}")
                else:
                    err = float(np.max(np.abs(got.astype(np.float64) - want)))
                    assert err <= FP32_MAX_ABS, f"{name} block {b0}: max abs error {err:.3e}"
            if not bf16:
                total = float(np.sum(yh, dtype=np.float64))
                assert abs(total - 1.0) <= FP32_ROW_SUM, f"{name}: row sum {total}"
            del yh
        del xd, ref


def test_split_forward_reuses_workspace(ons, orc):
    """A caller workspace filled with junk needs no initialisation; back-to-back calls reuse it."""
    ws = torch.full((ons.os_softmax_forward_workspace_bytes(4, 64),), 0x7F, dtype=torch.uint8, device="cuda")
    for cols, S in ((70001, 16), (300000, 64), (90000, 3)):
        x = workloads.normal(4, cols, seed=cols, scale=2.0)
        say(f"split workspace reuse cols={cols} S={S}")
        assert_fp32_parity(run_split(ons, x, S, ws), orc.softmax(x), f"split ws cols={cols}")


# -- logsumexp alongside the forward ------------------------------------------------

def lse_tol(ref: np.ndarray) -> np.ndarray:
    """Bound on |L - L_oracle| for L = m + ln d in fp32.  m is exact.  d's relative
    error stays below about 4e-6: up to 64 sequential fp32 additions per lane
    plus the merge tree (about 74 * 2^-24), with each e^{x-m} within a few ulp.
    So ln d is off by about that much in absolute terms, plus about 1 ulp from
    the base-2 logarithm.  The final fused m + log2(d) * ln 2 rounds once, by
    at most 2^-24 |L|.  Allow 1e-5 absolute plus 2^-22 |L|."""
    return 1e-5 + 2.0 ** -22 * np.abs(ref)


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def check_lse(ons, orc, x: np.ndarray, what: str, write_y: bool = True, rows=None):
    say(f"lse {what} rows={x.shape[0]} cols={x.shape[1]} write_y={write_y}")
    xd = to_device(np.ascontiguousarray(x))
    y, L = ons.os_softmax_forward_lse(xd, write_y=write_y)
    torch.cuda.synchronize()
    L = to_host(L).astype(np.float64)
    if rows is not None:
        L, ref = L[rows], orc.logsumexp(np.ascontiguousarray(x[rows]), threads=16)
    else:
        ref = orc.logsumexp(x, threads=16)
    assert np.array_equal(np.isnan(L), np.isnan(ref)), what
    assert np.array_equal(np.isneginf(L), np.isneginf(ref)), what
    fin = np.isfinite(ref)
    err = np.abs(L[fin] - ref[fin])
    assert np.all(err <= lse_tol(ref[fin])), f"{what}: max |L - ref| = {err.max()}"
    if write_y:
        y_plain = ons.os_softmax_forward(xd)  # same kernels: y must not change
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_plain)), what
    else:
        assert y is None


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_stats_and_lse_dense_lengths(ons, orc, bf16):
    """The row statistics and the logsumexp (with and without y) take the
    forward's automatic plan: every row length up to 64 slots and every
    seventh up to 600, aligned and from an element-aligned base, against the
    oracle (m exact, d within 1e-5 relative, L within lse_tol, y bitwise the
    forward's)."""
    vec = 8 if bf16 else 4
    lengths = list(range(1, 64 * vec + 1)) + list(range(64 * vec + 1, 600 * vec + 1, 7))
    for cols in lengths:
        rows = 5
        x32 = workloads.normal(rows, cols, seed=cols * 5 + 11 + bf16, scale=3.0)
        x = bf16_bits(x32) if bf16 else x32
        m_ref, d_ref = orc.stats(x)
        L_ref = orc.logsumexp(x, threads=8)
        for si in ((0, 1) if cols % vec else (0,)):
            say(f"stats/lse dense lengths bf16={bf16} rows={rows} cols={cols} in+{si}")
            xin = device_at(x, si)
            m, d = ons.os_softmax_stats(xin)
            y, L = ons.os_softmax_forward_lse(xin)
            y_plain = ons.os_softmax_forward(xin)
            torch.cuda.synchronize()
            what = f"bf16={bf16} cols={cols} in+{si}"
            assert np.array_equal(to_host(m).astype(np.float64), m_ref), what
            assert np.max(np.abs(to_host(d) - d_ref) / d_ref) <= 1e-5, what
            assert np.all(np.abs(to_host(L).astype(np.float64) - L_ref) <= lse_tol(L_ref)), what
            assert torch.equal(bits(y), bits(y_plain)), what


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_lse_every_plan_bucket(ons, orc, bf16):
    for cols in [1, 3, 8, 33, 128, 129, 1000, 2048, 4097, 8193, 32000, 65536, 65537, 200001]:
        rows = 13 if cols < 20000 else 4
        x32 = workloads.normal(rows, cols, seed=7000 + cols, scale=4.0)
        x32[0, cols // 2] = 80.0
        x = bf16_bits(x32) if bf16 else x32
        check_lse(ons, orc, x, f"bf16={bf16} cols={cols}")
        check_lse(ons, orc, x, f"bf16={bf16} cols={cols}", write_y=False)


def test_lse_special_rows(ons, orc):
    """-inf rows give -inf, NaN / +inf rows NaN, one element gives x, N equal entries a + ln N."""
    for cols in (6, 1024, 32000, 70000):
        x = workloads.normal(8, cols, seed=cols + 1, scale=2.0)
        x[0, ::3] = -np.inf
        x[1, :] = -np.inf
        x[2, cols // 3] = np.inf
        x[3, cols - 1] = np.nan
        x[4, :] = 0.375
        x[5, :] = -np.inf
        x[5, 1] = -3.0e38
        x[6, :] = -80.0
        x[7, :] = -np.inf
        x[7, cols // 2] = np.nan                # NaN beside nothing but -inf
        check_lse(ons, orc, x, f"special cols={cols}")
        _, L = ons.os_softmax_forward_lse(to_device(x), write_y=False)
        torch.cuda.synchronize()
        L = to_host(L)
        assert L[1] == -np.inf and np.isnan(L[2]) and np.isnan(L[3]) and np.isnan(L[7])
        m, d = ons.os_softmax_stats(to_device(x))
        torch.cuda.synchronize()
        m, d = to_host(m), to_host(d)
        assert m[7] == -np.inf and np.isnan(d[7]) and m[1] == -np.inf and d[1] == 0.0
        assert L[5] == np.float32(-3.0e38)  # one finite entry: L = x exactly
        assert abs(float(L[4]) - (0.375 + math.log(cols))) <= lse_tol(np.array(0.375 + math.log(cols)))
    x = workloads.normal(5, 1, seed=2, scale=30.0)
    _, L = ons.os_softmax_forward_lse(to_device(x), write_y=False)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(L), x[:, 0])  # cols = 1: L = x exactly
    _, L = ons.os_softmax_forward_lse(torch.empty((3, 0), device="cuda"), write_y=False)
    torch.cuda.synchronize()
    assert to_host(L).tolist() == [-np.inf] * 3  # empty rows


def test_lse_in_place(ons):
    x = workloads.normal(37, 4096, seed=77, scale=3.0)
    xd = to_device(x)
    y_ref, L_ref = ons.os_softmax_forward_lse(to_device(x))
    y, L = ons.os_softmax_forward_lse(xd, out=xd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    assert torch.equal(bits(xd), bits(y_ref)) and torch.equal(bits(L), bits(L_ref))


@pytest.mark.parametrize("n", [2, 3, 4])
def test_lse_full_configs(ons, orc, n):
    """Full-size workloads in the forward's launch configuration, every row."""
    check_lse(ons, orc, workloads.config(n), f"config{n}")


# -- fused softmax + top-K ---------------------------------------------------------

def check_topk(ons, orc, x: np.ndarray, K: int, what: str, splits=None, nan_rows=None):
    """Indices bit-exact and probabilities within the bound.  Rows listed in
    nan_rows hold a NaN: their probabilities must be NaN, and their indices K
    distinct columns of the row (which ones is unspecified)."""
    say(f"topk {what} rows={x.shape[0]} cols={x.shape[1]} K={K} splits={splits}")
    xd = to_device(np.ascontiguousarray(x))
    p, i = ons.os_softmax_topk(xd, K, splits=splits)
    torch.cuda.synchronize()
    pr, ir = orc.topk(x, K, threads=8)
    i = to_host(i)
    if nan_rows is not None:
        inan = i[nan_rows]
        assert np.all((inan >= 0) & (inan < x.shape[1])), f"{what}: a NaN row's index is outside the row"
        srt = np.sort(inan, axis=1)
        assert np.all(srt[:, 1:] != srt[:, :-1]), f"{what}: a NaN row repeats an index"
        i[nan_rows] = ir[nan_rows]
        assert np.all(np.isnan(pr[nan_rows])), "the oracle gives NaN probabilities for rows holding NaN"
    bad = np.argwhere(i != ir)
    assert bad.size == 0, f"{what}: first index mismatch at {bad[:3].tolist()}: {i[bad[0][0]]} vs {ir[bad[0][0]]}"
    p = to_host(p).astype(np.float64)
    finite = ~np.isnan(pr)
    assert np.array_equal(np.isnan(p), np.isnan(pr))
    assert np.max(np.abs(p[finite] - pr[finite]), initial=0.0) <= TOPK_PROB_ABS, what


@pytest.mark.parametrize("K", [1, 2, 8, 17, 32])
def test_topk_small_and_ragged(ons, orc, K):
    rng = np.random.Generator(np.random.PCG64(K))
    for cols in [K, K + 1, K + 3, 63, 100, 1023, 4096, 4099, 65537]:
        if cols < K:
            continue
        x = workloads.normal(13, cols, seed=cols * 31 + K, scale=3.0)
        check_topk(ons, orc, x, K, f"normal K={K}")
        xi = rng.integers(-3, 4, size=(13, cols)).astype(np.float32)  # heavy ties
        check_topk(ons, orc, xi, K, f"ties K={K}")


def test_topk_special_rows(ons, orc):
    cols = 5000
    x = workloads.normal(8, cols, seed=5, scale=3.0)
    x[0, :] = 1.25                      # all equal: lowest indices win
    x[1, ::2] = -np.inf                 # half -inf
    x[2, :] = -np.inf
    x[2, [7, 4000, 4999]] = [1.0, 1.0, -2.0]  # fewer finite entries than K: -inf fill by index
    x[3, 10] = -0.0
    x[3, 11] = 0.0
    x[3, :10] = -5.0
    x[4, [0, 4999, 2500]] = 50.0        # triple tie at the top
    x[5, 4090:4100] = 40.0              # ties straddling ranks 8 and 9
    check_topk(ons, orc, x, 8, "special rows")
    check_topk(ons, orc, x[:, 1:4999], 8, "unaligned cols")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_topk_nan_rows(ons, orc, bf16):
    """Rows holding NaN, through the tiled kernel (long rows, split and not)
    and the short-row kernel: NaN probabilities and K distinct in-row indices,
    also where fewer than K entries are numbers."""
    for rows, cols, K, splits in [(12, 5000, 8, None), (12, 5000, 32, None), (12, 128256, 8, 4),
                                  (4096, 100, 8, None), (4096, 100, 1, None), (300, 40, 16, None)]:
        x32 = workloads.normal(rows, cols, seed=cols + K, scale=3.0)
        x32[0, cols // 2] = np.nan                      # one NaN among numbers
        x32[1, :] = np.nan                              # only NaN
        x32[2, :] = -np.inf                             # NaN among -inf
        x32[2, [0, cols - 1]] = np.nan
        x32[3, :] = np.nan                              # fewer numbers than K
        x32[3, [1, cols // 3]] = [2.0, -1.0]
        x32[4, ::2] = np.nan                            # every other entry NaN
        x32[5, cols - 1] = np.nan                       # NaN in the last column
        x = bf16_bits(x32) if bf16 else x32
        nan_rows = np.arange(6)
        check_topk(ons, orc, x, K, f"NaN rows bf16={bf16}", splits=splits, nan_rows=nan_rows)


# batches that the width table maps to 1, 2, 4, 8 and 16 waves per row (and,
# for K = 32, the cap of 2 K parts per wave), each with heavy ties
TOPK_WIDTH_CASES = [(4200, 512, 8), (1024, 512, 8), (64, 2048, 8), (64, 8192, 8), (64, 32000, 8),
                    (64, 512, 32), (1024, 2048, 32), (300, 600, 17)]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_topk_every_width(ons, orc, bf16):
    for rows, cols, K in TOPK_WIDTH_CASES:
        x32 = workloads.normal(rows, cols, seed=rows + cols + K, scale=3.0)
        x32[::5, cols // 3: cols // 3 + 2 * K] = 7.5  # ties across the K-th rank
        x = bf16_bits(x32) if bf16 else x32
        check_topk(ons, orc, x, K, f"width case bf16={bf16}")


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_topk_rows_mostly_neg_inf(ons, orc, bf16):
    """Rows with fewer entries above -inf than K, or only a few: the -inf fill
    goes by index, and the bound stays -inf through the first tiles."""
    for rows, cols, K in [(256, 32000, 8), (64, 5000, 32), (300, 700, 13), (40, 128256, 8)]:
        x32 = workloads.normal(rows, cols, seed=cols + K, scale=2.0)
        x32[:, 5:] = -np.inf                            # 5 entries above -inf in every row
        x32[1::3, : cols // 2] = -np.inf                # then some rows with one late block
        x32[1::3, cols - 100:] = 1.0
        x32[2::7, :] = -np.inf                          # and rows of -inf only
        x = bf16_bits(x32) if bf16 else x32
        check_topk(ons, orc, x, K, f"mostly -inf bf16={bf16}")


# batches the short-row (register-resident) top-K serves: many rows of up to
# 2048 columns, rows of <= 64 columns at any batch; K up to 32
TOPK_ROWS_CASES = [(16384, 100, 32), (16384, 512, 8), (20000, 1000, 2), (2000, 60, 16), (300, 16, 8), (5000, 127, 2),
                   (16384, 255, 32), (64, 5, 5), (9000, 1000, 16), (5000, 300, 8), (3000, 100, 16), (1500, 128, 8),
                   (3000, 500, 4), (10000, 512, 32), (100, 16, 16), (5000, 2000, 2), (3000, 2048, 4),
                   (300, 1500, 1),
                   # 64 entries per lane: many rows with K = 32
                   (16384, 512, 32), (40000, 200, 32), (8192, 1000, 32), (16384, 300, 32), (8192, 1000, 16)]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_topk_short_rows(ons, orc, bf16):
    rng = np.random.Generator(np.random.PCG64(77 + bf16))
    for rows, cols, K in TOPK_ROWS_CASES:
        x32 = workloads.normal(rows, cols, seed=rows * 3 + cols, scale=3.0)
        x32[::3] = rng.integers(-2, 3, size=x32[::3].shape)     # heavy ties
        x32[1::7, cols // 2:] = -np.inf                          # half -inf
        x32[2::11, :] = -np.inf                                  # only -inf
        x32[4::13, cols - 1] = 20.0                              # the best at the row end
        x32[6::19] = -1.0                                        # -0.0 ties +0.0: lower index first
        x32[6::19, [0, cols - 1]] = [-0.0, 0.0]
        x32[5::17, cols // 3] = np.nan                           # NaN rows: probabilities NaN
        x = bf16_bits(x32) if bf16 else x32
        nan_rows = np.arange(5, rows, 17)
        check_topk(ons, orc, x, K, f"short rows bf16={bf16}", nan_rows=nan_rows)
        # one column fewer: rows that are no longer 16-byte aligned
        check_topk(ons, orc, x[:, 1:], min(K, cols - 1), f"short rows shifted bf16={bf16}",
                   nan_rows=nan_rows if cols // 3 >= 1 else None)


def test_topk_many_rows(ons, orc):
    """Enough rows for the 8-wave-per-row launch, with ties and a ragged K."""
    x = workloads.normal(1500, 3001, seed=99, scale=3.0)
    x[::7, 100:140] = 9.5
    check_topk(ons, orc, x, 8, "many rows")
    check_topk(ons, orc, x[:, :3000], 13, "many rows aligned K=13")


@pytest.mark.parametrize("splits", [2, 3, 4, 16])
def test_topk_split_rows(ons, orc, splits):
    """Rows split over several workgroups: empty and ragged slices, ties across
    slices, unaligned rows, both launch widths."""
    rng = np.random.Generator(np.random.PCG64(splits))
    x = workloads.normal(40, 20000, seed=7 + splits, scale=3.0)
    x[3, :] = 2.0
    x[4, [5, 9000, 19999]] = 30.0
    x[5, ::2] = -np.inf
    check_topk(ons, orc, x, 8, f"split {splits}", splits=splits)
    check_topk(ons, orc, x[:, 1:19998], 17, f"split {splits} unaligned", splits=splits)
    xi = rng.integers(-3, 4, size=(9, 100)).astype(np.float32)
    check_topk(ons, orc, xi, 8, f"split {splits} short rows", splits=splits)
    xm = workloads.normal(1100, 3000, seed=3, scale=3.0)
    check_topk(ons, orc, xm, 8, f"split {splits} many rows", splits=splits)
    xl = workloads.normal(12, 70001, seed=11, scale=3.0)  # slices span several tiles
    xl[2, [0, 35000, 70000]] = 25.0
    check_topk(ons, orc, xl, 8, f"split {splits} long rows", splits=splits)


def test_topk_maximum_row_length(ons, orc):
    """Top-32 of one row of OS_MAX_COLS = 2^28 fp32 entries (1 GiB), one
    workgroup and the planned split.  The oracle's full sort of such a row is
    out of reach, so the result is checked by properties that fix it: 32
    distinct in-row columns whose values rank first under (value desc, index
    asc) -- fewer than 32 entries lie above the 32nd value, and every entry
    equal to it that is not selected has a higher column than the selected
    ones -- and probabilities e^{x - m} / d from the oracle's (m, d) of the row.
    A planted duplicate of the maximum exercises the tie rule."""
    n, K = 1 << 28, 32
    x = workloads.normal(1, n, seed=2828, scale=3.0)
    x[0, n - 11] = 40.0   # far above the row's natural maximum (about 19)
    x[0, 12345] = 40.0    # a tie at the top: the lower column ranks first
    x[0, n - 2] = 39.5
    m, d = orc.stats(x)
    xd = to_device(x)
    row = x[0]
    for splits in (1, None):
        say(f"top-K maximum row length 2^28, K={K}, splits={splits}")
        p, i = ons.os_softmax_topk(xd, K, splits=splits)
        torch.cuda.synchronize()
        i = to_host(i)[0].astype(np.int64)
        p = to_host(p)[0].astype(np.float64)
        assert np.all((i >= 0) & (i < n)) and np.unique(i).size == K
        vals = row[i]
        assert i[0] == 12345 and i[1] == n - 11 and i[2] == n - 2
        order_ok = (vals[:-1] > vals[1:]) | ((vals[:-1] == vals[1:]) & (i[:-1] < i[1:]))
        assert np.all(order_ok), "selected entries are not in (value desc, index asc) order"
        vk = vals[-1]
        assert int(np.count_nonzero(row > vk)) < K
        ties = np.flatnonzero(row == vk)
        chosen = np.sort(i[vals == vk])
        assert np.array_equal(ties[:chosen.size], chosen), "a lower column equal to the K-th value was skipped"
        want = np.exp(vals.astype(np.float64) - m[0]) / d[0]
        assert float(np.max(np.abs(p - want))) <= TOPK_PROB_ABS
    del xd


def test_topk_split_reuses_workspace(ons):
    """Back-to-back split calls on one (uninitialised) workspace give identical results."""
    x = to_device(workloads.config(5, 0, 64))
    say("topk split reuse")
    ws = torch.full((ons.os_softmax_topk_workspace_bytes(64, 8, 4),), 0xAB, dtype=torch.uint8, device="cuda")
    a = ons.os_softmax_topk_split(x, 8, 4, ws)
    b = ons.os_softmax_topk_split(x, 8, 4, ws)
    c = ons.os_softmax_topk(x, 8, splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[1], c[1])
    assert torch.equal(a[0], b[0])
    assert float((a[0] - c[0]).abs().max()) <= 1e-6


def test_topk_bf16(ons, orc):
    """bf16 logits (many exact ties after rounding): ragged rows, every K class, splits, an
    element-aligned base, all-equal and mostly -inf rows."""
    rng = np.random.Generator(np.random.PCG64(88))
    for rows, cols in ((7, 1000), (5, 4093), (3, 65536 + 8), (2, 200003)):
        x32 = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
        x32[0, :] = 1.25
        if rows > 2:
            x32[2, :] = -np.inf
            x32[2, rng.integers(cols, size=3)] = 0.5
        x = bf16_bits(x32)
        for K in (1, 8, 13, 32):
            for splits in (1, 3):
                say(f"topk bf16 rows={rows} cols={cols} K={K} splits={splits}")
                p, i = ons.os_softmax_topk(to_device(x), K, splits=splits)
                torch.cuda.synchronize()
                pr, ir = orc.topk(x, K, threads=8)
                assert np.array_equal(to_host(i), ir), f"bf16 cols={cols} K={K} S={splits}"
                p = to_host(p).astype(np.float64)
                assert np.array_equal(np.isnan(p), np.isnan(pr))
                ok = ~np.isnan(pr)
                assert np.max(np.abs(p[ok] - pr[ok]), initial=0.0) <= TOPK_PROB_ABS
    # an element-aligned (not 16-byte aligned) base
    x = bf16_bits((rng.standard_normal((4, 3001)) * 0.1).astype(np.float32))
    buf = torch.empty(x.size + 1, dtype=torch.bfloat16, device="cuda")
    xd = buf[1:].view(4, 3001)
    xd.copy_(to_device(x))
    say("topk bf16 misaligned base")
    p, i = ons.os_softmax_topk(xd, 8)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(i), orc.topk(x, 8)[1])


def test_topk_bf16_full_size(ons, orc):
    """Workload 5's logits rounded to bf16, in the launch the plan picks."""
    x = bf16_bits(workloads.config(5))
    say("topk bf16 full 256x128256")
    p, i = ons.os_softmax_topk(to_device(x), workloads.TOPK_K)
    torch.cuda.synchronize()
    pr, ir = orc.topk(x, workloads.TOPK_K, threads=16)
    assert np.array_equal(to_host(i), ir)
    assert np.max(np.abs(to_host(p).astype(np.float64) - pr)) <= TOPK_PROB_ABS


def test_topk_matches_forward(ons):
    """The fused probabilities equal the full softmax at the selected indices."""
    x = workloads.config(5, 0, 16)
    xd = to_device(x)
    say("topk vs forward")
    p, i = ons.os_softmax_topk(xd, 8)
    y = ons.os_softmax_forward(xd)
    torch.cuda.synchronize()
    yi = torch.gather(y, 1, i.long())
    assert float((yi - p).abs().max()) <= 2e-6


def test_copy_references(ons):
    """Both bandwidth references copy exactly, including ragged rows."""
    for rows, cols in ((4096, 32000), (3, 4), (17, 32768), (5, 1000)):
        say(f"copy references {rows}x{cols}")
        x = torch.randn(rows, cols, device="cuda")
        y = torch.zeros_like(x)
        ons.os_device_copy_rows(x, y)
        y2 = torch.zeros_like(x)
        ons.os_device_copy(x, y2)
        torch.cuda.synchronize()
        assert torch.equal(x, y) and torch.equal(x, y2)
    # past the tiled copy's grid cap (2^31 threads = 2^23 tiles of 4 KiB): 32 GiB + 3 tiles
    n = ((1 << 35) + 3 * 4096) // 4
    say("tiled copy past the grid cap: 32 GiB + 12 KiB")
    a = torch.empty(n, dtype=torch.int32, device="cuda")
    a[: 1 << 20].random_()
    a[-(1 << 20):].random_()
    b = torch.zeros_like(a)
    ons.os_device_copy(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a[: 1 << 20], b[: 1 << 20]) and torch.equal(a[-(1 << 20):], b[-(1 << 20):])
    del a, b
    torch.cuda.empty_cache()


# -- full-size configurations, in the launch configuration the benchmark times -------

def test_config2_full(ons, orc):
    say("config 2 full: 4096x32000 fp32")
    x = workloads.config(2)
    y = run_forward(ons, x)
    ref = orc.softmax(x, threads=16)
    assert_fp32_parity(y, ref, "config2")


def compare_in_row_blocks(orc, x: np.ndarray, y, bf16: bool, what: str, block_elems: int = 1 << 25):
    """Every row of a full-size output against the oracle, in row blocks that
    bound host memory (the oracle's double output of a block is 256 MiB)."""
    rows, cols = x.shape
    step = max(1, block_elems // cols)
    worst = 0.0
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        worst = max(worst, assert_parity(to_host(y[r0:r1]), orc.softmax(x[r0:r1], threads=16), bf16,
                                         f"{what} rows {r0}..{r1 - 1}"))
    return worst


def test_config3_full(ons, orc):
    say("config 3 full: 524288x2048 bf16")
    x = workloads.config(3)
    xd = to_device(x)
    y = ons.os_softmax_forward(xd)
    torch.cuda.synchronize()
    del xd
    # every row: its bf16 outputs sum to 1 within the rounding of 2048 outputs
    s = y.float().sum(dim=1)
    assert float((s - 1).abs().max()) <= 2.0 ** -8 + 1e-5  # |sum of rounding errors| <= u_bf16 * sum(y)
    # every element of every row against the oracle
    compare_in_row_blocks(orc, x, y, True, "config3")


def test_config4_full(ons, orc):
    say("config 4 full: 8388608x128 fp32")
    x = workloads.config(4)
    xd = to_device(x)
    y = ons.os_softmax_forward(xd)
    torch.cuda.synchronize()
    del xd
    # every element of every row against the oracle, and every row's sum
    compare_in_row_blocks(orc, x, y, False, "config4")


def test_config5_topk_full(ons, orc):
    x = workloads.config(5)
    check_topk(ons, orc, x, workloads.TOPK_K, "config5")  # the benchmark's launch (planned split)
    check_topk(ons, orc, x, workloads.TOPK_K, "config5 one workgroup per row", splits=1)
