"""The no-allocation split forward (os_softmax_forward_split_noalloc), called
through the C ABI, against the split forward with a caller's workspace
(os_softmax_forward_split) on the same inputs: the same kernels, so the
outputs must be bitwise equal, and both within the parity bar of the oracle.
Two calls in a row, the second smaller, then a call that fills the static
scratch exactly (rows * splits * 8 == OS_STATIC_SCRATCH_BYTES)."""
import numpy as np
import pytest

import workloads
from gpu_util import assert_parity, say, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ons():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_normalizer_amd
    return online_normalizer_amd


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def run_pair(ons, orc, x: np.ndarray, splits: int, what: str):
    bf16 = x.dtype == np.uint16
    xd = to_device(x)
    rows, cols = x.shape
    out_static = torch.empty_like(xd)
    say(f"no-alloc {what}: rows={rows} cols={cols} bf16={bf16} splits={splits}")
    before = torch.cuda.memory_allocated()
    ons.os_softmax_forward_split_noalloc(xd, splits=splits, out=out_static)
    assert torch.cuda.memory_allocated() == before, "the no-allocation call allocated through torch"
    ws = torch.empty(max(256, ons.os_softmax_forward_workspace_bytes(rows, splits)), dtype=torch.uint8, device="cuda")
    out_ws = ons.os_softmax_forward_split(xd, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(out_static), bits(out_ws)), f"{what}: differs from the workspace entry point"
    assert_parity(to_host(out_static), orc.softmax(x, threads=16), bf16, what)


def test_noalloc_matches_workspace_entry_point(ons, oracle_lib):
    # first call: 64 rows of a 128256-entry vocabulary, planned split
    x1 = workloads.normal(64, 128256, seed=11, scale=3.0)
    s1 = ons.os_forward_split_plan(64, 128256)
    assert s1 > 1
    run_pair(ons, oracle_lib, x1, s1, "first call")
    # second call, smaller: bf16 rows that are not 16-byte aligned, more slices
    # per row but fewer states than the first call left in the scratch
    x2 = workloads.f32_to_bf16_bits(workloads.normal(5, 100001, seed=12, scale=2.0))
    run_pair(ons, oracle_lib, x2, 16, "second, smaller call")
    assert 5 * 16 < 64 * s1


def test_noalloc_fills_the_scratch_exactly(ons, oracle_lib):
    cap = ons.OS_STATIC_SCRATCH_BYTES // 8          # slice states the scratch holds
    rows, splits = cap // 256, 256
    assert rows * splits * 8 == ons.OS_STATIC_SCRATCH_BYTES
    x = workloads.normal(rows, 65537, seed=13, scale=3.0)
    run_pair(ons, oracle_lib, x, splits, "full scratch")
    xd = to_device(x[:1])
    with pytest.raises(ons.OnlineSoftmaxError):
        big = torch.empty((rows + 1, 1), dtype=torch.float32, device="cuda")
        ons.os_softmax_forward_split_noalloc(big, splits=splits)  # one row too many: rejected, nothing launched
    del xd
