"""GPU parity of the attention forward (os_attention_forward), through the C
ABI, against the oracle's definition O = softmax(scale Q K^T) V with its
per-row logsumexp, on seeded bf16 inputs.

Bar, derived from the arithmetic (no tolerance is stated for this path):
  - O: the kernel rounds each weight e^{(s - m) scale} to bf16 before the
    second product (relative error <= 2^-9 per weight, so <= 2^-9 * sum_j
    a_j |V_j| on an output), accumulates in fp32 (error ~1e-4 relative at
    most) and rounds O to bf16 (2^-9 |O|):
        |O - O_ref| <= 2^-8 * (sum_j a_j |V_j| + |O_ref|)     (2x margin).
  - L = m scale + ln l: the fp32 dot products of the first product are off by
    at most 128 * 2^-24 * sum_c |q_c k_c| before the scale, and l by at most
    nk * 2^-24 relative (fp32 summation) plus a few ulp of exp2:
        |L - L_ref| <= scale * 128 * 2^-24 * max_j sum_c |q_c k_c| + 2 nk 2^-24
                       + 2^-22 |L_ref| + 1e-6.
"""
import math
import os

import numpy as np
import pytest

import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ons():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_normalizer_amd
    return online_normalizer_amd


def dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def wide(bits: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def check(ons, orc, q, k, v, causal: bool, what: str, scale=None, threads: int = 16):
    heads, nq, d = q.shape
    nk = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    say(f"attention {what}: heads={heads} nq={nq} nk={nk} causal={causal}")
    O, L = ons.os_attention_forward(dev(q), dev(k), dev(v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    O = O.float().cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    Or, Lr, Oa = orc.attention(q, k, v, scale, causal=causal, threads=threads, want_abs=True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), what
    err = np.abs(O - Or) - 2.0 ** -8 * (Oa + np.abs(Or))
    assert float(err.max()) <= 0.0, f"{what}: O off by {float(np.abs(O - Or).max()):.3e} beyond the bound"
    # the logsumexp bound needs max_j sum_c |q_c k_c| per row
    qa, ka = np.abs(wide(q)), np.abs(wide(k))
    dots = np.einsum("hic,hjc->hij", qa, ka)
    if causal:
        dots = np.where(np.tril(np.ones((nq, nk), dtype=bool)), dots, 0.0)
    bound_s = scale * d * 2.0 ** -24 * dots.max(axis=2)
    tol = bound_s + 2 * nk * 2.0 ** -24 + 2.0 ** -22 * np.abs(Lr) + 1e-6
    assert np.all(np.abs(L - Lr) <= tol), f"{what}: L off by {float(np.abs(L - Lr).max()):.3e}"
    return float(np.abs(O - Or).max()), float(np.abs(L - Lr).max())


# query and key lengths around the tile sizes (128 query rows per workgroup,
# 32 per wave, 64 keys per tile): one row, ragged tails, exact multiples
SHAPES = [(1, 1), (1, 64), (31, 63), (127, 64), (128, 64), (129, 65), (200, 300), (64, 1), (256, 128), (257, 130),
          (513, 70)]


@pytest.mark.parametrize("nq,nk", SHAPES, ids=[f"{a}x{b}" for a, b in SHAPES])
def test_attention_small(ons, oracle_lib, nq, nk):
    q, k, v = workloads.attention_qkv(3, nq, nk, 128, seed=2000 + nq * 7 + nk)
    check(ons, oracle_lib, q, k, v, False, f"{nq}x{nk}")


@pytest.mark.parametrize("n", [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 383, 385, 600])
def test_attention_causal(ons, oracle_lib, n):
    q, k, v = workloads.attention_qkv(3, n, n, 128, seed=3000 + n)
    check(ons, oracle_lib, q, k, v, True, f"causal n={n}")


RANDOM_CASES = int(os.environ.get("ONORM_RANDOM_ATTN_CASES", "24"))


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_attention_random(ons, oracle_lib, case):
    """A seeded random draw of heads (1-4), query and key lengths around the
    tile sizes, the causal mask and the scale (ONORM_RANDOM_ATTN_CASES sets the
    number of cases, 24 by default)."""
    rng = np.random.Generator(np.random.PCG64(77000 + case))
    heads = int(rng.integers(1, 5))
    causal = bool(rng.random() < 0.4)
    nq = int(rng.choice([1, 2, 31, 32, 33, 63, 64, 65, 127, 200, 255, 256, 257, 300, 511, 513, 700]))
    nk = nq if causal else int(rng.choice([1, 3, 63, 64, 65, 100, 128, 129, 255, 256, 300, 640, 1000]))
    scale = float(rng.choice([1.0 / math.sqrt(128), 0.01, 0.3, 1.0]))
    q, k, v = workloads.attention_qkv(heads, nq, nk, 128, seed=77000 + 3 * case)
    check(ons, oracle_lib, q, k, v, causal, f"random case {case} (scale {scale})", scale=scale, threads=4)


def test_attention_special_inputs(ons, oracle_lib):
    """Large logits (scale 1, |q.k| up to ~hundreds: exercises the running
    maximum's rescaling), equal keys (uniform weights), and a key that wins
    every row late in the sequence."""
    q, k, v = workloads.attention_qkv(2, 150, 260, 128, seed=4000)
    check(ons, oracle_lib, q, k, v, False, "scale 1", scale=1.0)
    keq = np.ascontiguousarray(np.broadcast_to(k[:, :1], k.shape))
    check(ons, oracle_lib, q, keq, v, False, "equal keys")
    kl = k.copy()
    kl[:, 250] = workloads.f32_to_bf16_bits(np.sign(workloads.bf16_bits_to_f32(q[:, 0])) * 3.0)
    check(ons, oracle_lib, q, kl, v, False, "late winning key")


def test_attention_rising_maximum(ons, oracle_lib):
    """Rows whose maximum rises by more than 8 in log2 units every two or
    three key tiles, interleaved with rows whose maximum is their first key:
    in one wavefront some rows move their running maximum (and rescale) while
    the others keep theirs."""
    heads, n, d = 2, 700, 128
    rng = np.random.default_rng(4300)
    qf = rng.standard_normal((heads, n, d)) * 0.01
    qf[:, 0::2, 0] = 1.0
    qf[:, 1::2, 0] = -1.0
    kf = rng.standard_normal((heads, n, d)) * 0.01
    kf[:, :, 0] = np.arange(n) * 0.04  # logits of the even rows grow by 2.56 a tile, ~3.7 in log2 units
    vf = rng.standard_normal((heads, n, d))
    q, k, v = (workloads.f32_to_bf16_bits(x.astype(np.float32)) for x in (qf, kf, vf))
    check(ons, oracle_lib, q, k, v, False, "rising maximum", scale=1.0)
    check(ons, oracle_lib, q, k, v, True, "rising maximum, causal", scale=1.0)


def test_attention_in_place_and_deterministic(ons):
    q, k, v = workloads.attention_qkv(2, 300, 300, 128, seed=5000)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o1, l1 = ons.os_attention_forward(qd, kd, vd)
    o2, l2 = ons.os_attention_forward(qd, kd, vd)
    o3, _ = ons.os_attention_forward(qd, kd, vd, out=qd)  # o == q
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert o3.data_ptr() == qd.data_ptr() and torch.equal(qd.view(torch.int16), o1.view(torch.int16))


def test_attention_longest_key_sequence(ons, oracle_lib):
    """The longest key sequence the library takes (OS_ATTN_MAX_SEQ = 2^22
    keys: 1 GiB of K and of V for one head) against a few query rows, every
    output against the oracle (with the bound of the module docstring, the
    dot-product term taken as max|k| * sum|q|)."""
    nk = 1 << 22
    q, k, v = workloads.attention_qkv(1, 5, nk, 128, seed=4200)
    scale = 1.0 / math.sqrt(128)
    say(f"attention: 1 head, 5 queries, {nk} keys")
    O, L = ons.os_attention_forward(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    O = O.float().cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    Or, Lr, Oa = oracle_lib.attention(q, k, v, scale, want_abs=True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    err = np.abs(O - Or) - 2.0 ** -8 * (Oa + np.abs(Or))
    assert float(err.max()) <= 0.0, f"O off by {float(np.abs(O - Or).max()):.3e} beyond the bound"
    bound_s = scale * 128 * 2.0 ** -24 * np.abs(wide(q)).sum(axis=2) * float(np.abs(wide(k)).max())
    tol = bound_s + 2 * nk * 2.0 ** -24 + 2.0 ** -22 * np.abs(Lr) + 1e-6
    assert np.all(np.abs(L - Lr) <= tol), f"L off by {float(np.abs(L - Lr).max())}"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_attention_workload_full(ons, oracle_lib, causal):
    """The attention workload (256 heads x 2048 x 128, bf16) in the launch the
    benchmark times, every output against the oracle."""
    q, k, v = workloads.attention_workload()
    heads = q.shape[0]
    say(f"attention workload causal={causal}")
    O, L = ons.os_attention_forward(dev(q), dev(k), dev(v), causal=causal)
    torch.cuda.synchronize()
    O = O.float().cpu().numpy()
    L = L.cpu().numpy()
    scale = 1.0 / math.sqrt(128)
    for h0 in range(0, heads, 32):  # in head blocks: bounded host memory
        sl = slice(h0, h0 + 32)
        Or, Lr, Oa = oracle_lib.attention(q[sl], k[sl], v[sl], scale, causal=causal, threads=16, want_abs=True)
        err = np.abs(O[sl].astype(np.float64) - Or) - 2.0 ** -8 * (Oa + np.abs(Or))
        assert float(err.max()) <= 0.0, f"heads {h0}..: O beyond the bound"
        # the L bound of the module docstring, with sum_c |q_c k_c| <= max|k| * sum_c |q_c|
        bound_s = scale * 128 * 2.0 ** -24 * np.abs(wide(q[sl])).sum(axis=2) * np.abs(wide(k[sl])).max(axis=(1, 2))[:, None]
        tol = bound_s + 2 * k.shape[1] * 2.0 ** -24 + 2.0 ** -22 * np.abs(Lr) + 1e-6
        assert np.all(np.abs(L[sl] - Lr) <= tol), f"heads {h0}..: L off by {float(np.abs(L[sl] - Lr).max())}"
