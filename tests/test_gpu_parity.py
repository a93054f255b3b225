"""HIP path vs the fp64 oracle on small and edge shapes, element by element.

Every output element is compared; shapes span several 128-row query blocks
and 64-key tiles with ragged tails, both dtypes, both head dims, both masks.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from oracle import attention_ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, N, D, dtype, qk_spread=1.0, exact_scores=False):
    """q, k, v ~ N(0,1) (q and k times qk_spread), rounded to dtype, as float32 values.

    exact_scores: q and k rounded to multiples of 1/16 within [-4, 4], so every
    product q_d k_d (a multiple of 2^-8 below 16 in magnitude) and every partial
    sum over D <= 128 of them (below 2^11) is exactly representable in fp32 (and
    bf16 holds the inputs exactly): the scores carry no rounding, and with a
    power-of-two scale neither do the scaled scores."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((3, B, H, N, D)).astype(np.float32)
    x[:2] *= np.float32(qk_spread)
    if exact_scores:
        x[:2] = np.clip(np.round(x[:2] * 16.0), -64, 64) / np.float32(16.0)
    if dtype == "bf16":
        x = fi.bf16_round(x)
    return x


def _check(x, dtype, causal, scale, what):
    B, H, N, D = x.shape[1:]
    q, k, v = (gu.to_device_values(x[i], dtype) for i in range(3))
    gu.log(f"[gpu] {what}: B={B} H={H} N={N} D={D} {dtype} causal={causal} scale={scale}")
    o, lse = gu.run(q, k, v, causal, scale)
    o_ref = np.empty((B, H, N, D))
    l_ref = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o_ref[b, h], l_ref[b, h] = attention_ref(x[0, b, h], x[1, b, h], x[2, b, h], causal, scale)
    err = gu.errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    gu.assert_within(err, dtype, what)
    return o, lse


EDGE_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(N, causal, D, dtype):
    x = _inputs(N * 4 + D + causal, 1, 2, N, D, dtype)
    _check(x, dtype, causal, 1 / math.sqrt(D), f"edge N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_worked_example_padded(dtype):
    """The hand-worked two-key case, zero-padded to D=64 (zero columns change no
    score and give zero outputs)."""
    x = np.zeros((3, 1, 1, 2, 64), dtype=np.float32)
    x[0, 0, 0, 0, 0] = math.log(3.0)
    x[1, 0, 0, 1, 0] = 1.0
    x[2, 0, 0, :, 0] = [4.0, 8.0]
    if dtype == "bf16":
        x = fi.bf16_round(x)
    for causal in (False, True):
        o, lse = _check(x, dtype, causal, 1.0, f"worked example causal={causal}")
        o = o.float().cpu().numpy()[0, 0]
        assert np.all(o[:, 1:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_score_shift_beyond_exp_range(dtype):
    """Every score of a row shifted by +1000: exp without the running max would
    overflow; O is unchanged and LSE moves by 1000.  The other columns give
    exactly representable scores (see _inputs), so the fp32 scores near 8000 are
    exact and the contract's bounds apply unchanged."""
    N, D = 300, 64
    x = _inputs(8, 1, 1, N, D, "f32", exact_scores=True)
    x[0, 0, 0, :, D - 1] = 8000.0   # q's last column
    x[1, 0, 0, :, D - 1] = 1.0      # k's last column -> +1000 at scale 1/8
    if dtype == "bf16":
        x = fi.bf16_round(x)
    for causal in (False, True):
        _check(x, dtype, causal, 0.125, f"shift +1000 causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
def test_unusual_scales(scale, dtype):
    """Exactly representable scores (see _inputs) at scales -1/8, 0 and 2 (powers
    of two): the contract's bounds apply unchanged."""
    x = _inputs(77, 1, 2, 200, 64, dtype, exact_scores=True)
    for causal in (False, True):
        _check(x, dtype, causal, scale, f"scale={scale} causal={causal}")


def test_peaked_spread():
    """Q and K times 4 (as in the peaked workload): near one-hot rows stress the running max."""
    x = _inputs(5, 1, 4, 777, 128, "bf16", qk_spread=4.0)
    _check(x, "bf16", True, 1 / math.sqrt(128), "peaked x4 N=777")
    _check(x, "bf16", False, 1 / math.sqrt(128), "peaked x4 N=777 noncausal")


def test_aliased_inputs_q_equals_k_equals_v():
    """q = k = v in one buffer (the pages' benchmark clones q into k and v)."""
    x = _inputs(11, 1, 2, 333, 128, "bf16")
    q = gu.to_device_values(x[0], "bf16")
    o, lse = gu.run(q, q, q, True, 1 / math.sqrt(128))
    o_ref = np.empty((1, 2, 333, 128))
    l_ref = np.empty((1, 2, 333))
    for h in range(2):
        o_ref[0, h], l_ref[0, h] = attention_ref(x[0, 0, h], x[0, 0, h], x[0, 0, h], True, 1 / math.sqrt(128))
    gu.assert_within(gu.errors(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref), "bf16", "q=k=v")


def test_every_output_written_and_deterministic():
    """NaN-filled outputs are fully overwritten; two runs agree bit for bit."""
    import exact_attention_65_amd as fa
    x = _inputs(3, 2, 3, 517, 128, "bf16")
    q, k, v = (gu.to_device_values(x[i], "bf16") for i in range(3))
    for causal in (False, True):
        outs = []
        for _ in range(2):
            o = torch.full_like(q, float("nan"))
            lse = torch.full((2, 3, 517), float("nan"), device=q.device)
            fa.attention_forward(q, k, v, causal=causal, out=o, lse=lse)
            torch.cuda.synchronize()
            assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
            outs.append((o.clone(), lse.clone()))
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
        assert torch.equal(outs[0][1], outs[1][1])


def test_non_default_stream():
    x = _inputs(21, 1, 2, 640, 128, "bf16")
    q, k, v = (gu.to_device_values(x[i], "bf16") for i in range(3))
    ref_o, ref_l = gu.run(q, k, v, False, 1 / math.sqrt(128))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = gu.run(q, k, v, False, 1 / math.sqrt(128), stream=s)
    s.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(lse, ref_l)


def test_status_errors_on_device():
    import exact_attention_65_amd as fa
    q = torch.zeros(1, 1, 64, 80, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.attention_forward(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 64, device="cuda")
    # o aliasing q
    with pytest.raises(fa.FaError) as e:
        fa.attention_forward(q, q, q, out=q, lse=lse)
    assert e.value.status == fa.FA_ERR_ALIASING
    # misaligned view
    big = torch.zeros(1 + 64 * 64, dtype=torch.bfloat16, device="cuda")
    qm = big[1:].view(1, 1, 64, 64)
    with pytest.raises(fa.FaError) as e:
        fa.attention_forward(qm, qm, qm, out=o, lse=lse)
    assert e.value.status == fa.FA_ERR_MISALIGNED


def test_binding_rejects_bad_output_tensors():
    """Outputs, gradients and workspaces handed to the torch helpers are checked
    before any launch: a wrong shape, dtype, device or layout raises ValueError."""
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 64, dtype=torch.float32, device="cuda")
    bad_outs = [torch.zeros(1, 2, 63, 64, dtype=torch.bfloat16, device="cuda"),   # too small
                torch.zeros(1, 2, 64, 64, dtype=torch.float16, device="cuda"),    # wrong dtype
                torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16),                  # host memory
                torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda").transpose(2, 3)]
    for o in bad_outs:
        with pytest.raises(ValueError):
            fa.attention_forward(q, q, q, out=o)
        with pytest.raises(ValueError):
            fa.attention_forward_split(q, q, q, out=o, n_splits=2)
    with pytest.raises(ValueError):
        fa.attention_forward(q, q, q, lse=torch.zeros(1, 2, 63, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.attention_forward_split(q, q, q, n_splits=2,
                                   workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        fa.attention_backward(q, q, q, q, lse, q, dq=bad_outs[0])
    with pytest.raises(ValueError):
        fa.attention_backward(q, q, q, q, lse, q, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
