"""fa_fwd_fp8 against the fp64 oracle of the dequantised inputs
(oracle.attention_fp8_ref).

Tolerance (tests/error_models.py, fixed before measuring): the bf16 contract
(max |dO| <= 2e-2, mean |dO| <= 2e-3, |dLSE| <= 1e-3), which covers the
roundings fa_fwd shares with the bf16 path (V widened to bf16 exactly, P and O
rounded to bf16), plus the score error of the scaled FP8 matrix instruction,
whose sums are not specified to fp32 accuracy: under the stated assumption that
each 64-product sum is accurate to 2^-10 of the sum of its products'
magnitudes, row i's scores are off by at most E_i, which moves LSE_i by at
most E_i and O_id by at most 2 E_i max_j |v_jd|.  Both terms are computed per
row from the inputs; the tests log the largest error / bound ratios.
"""
import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
import fa_inputs.fp8 as f8
from oracle import attention_fp8_ref, attention_ref, mx_dequantize
from tests import error_models as em
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _inputs(w):
    return [f8.full_mx(w, t) for t in (fi.T_Q, fi.T_K, fi.T_V)]


def _run(inp, causal, scale, out=None, lse=None):
    (q, qs), (k, ks), (v, vs) = inp
    o, l = fa.attention_forward_fp8(_dev(q), _dev(qs), _dev(k), _dev(ks), _dev(v), _dev(vs), causal=causal,
                                    scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


def _compare(inp, o, lse, heads, causal, scale, what, rows_for=None):
    (q, qs), (k, ks), (v, vs) = inp
    tol = gu.TOL["bf16"]
    worst = dict(o_ratio=0.0, lse_ratio=0.0, o_max=0.0, lse_max=0.0)
    mean_err, mean_bound, n_el = 0.0, 0.0, 0
    for b, h in heads:
        rows = None if rows_for is None else rows_for(h)
        o_ref, lse_ref = attention_fp8_ref(q[b, h], qs[b, h], k[b, h], ks[b, h], v[b, h], vs[b, h], causal, scale,
                                           rows=rows)
        qd, kd, vd = (mx_dequantize(c[b, h], sc[b, h]) for c, sc in ((q, qs), (k, ks), (v, vs)))
        e_row, o_term = em.fp8_row_terms(qd, kd, vd, causal, scale, rows=rows)
        og = o[b, h].float().cpu().numpy()
        lg = lse[b, h].cpu().numpy()
        if rows is not None:
            og, lg = og[rows], lg[rows]
        assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), f"{what} (b={b}, h={h}): non-finite output"
        do = np.abs(og.astype(np.float64) - o_ref)
        dl = np.abs(lg.astype(np.float64) - lse_ref)
        worst["o_ratio"] = max(worst["o_ratio"], float((do / (tol["o_max"] + o_term)).max()))
        worst["lse_ratio"] = max(worst["lse_ratio"], float((dl / (tol["lse"] + e_row)).max()))
        worst["o_max"] = max(worst["o_max"], float(do.max()))
        worst["lse_max"] = max(worst["lse_max"], float(dl.max()))
        mean_err += float(do.sum())
        mean_bound += float((tol["o_mean"] + o_term).sum())
        n_el += do.size
    worst["o_mean_ratio"] = mean_err / mean_bound
    gu.record(dict(case=what, dtype="fp8", **worst))
    gu.log(f"  {what}: max|dO|={worst['o_max']:.3e} (err/bound {worst['o_ratio']:.3f}) "
           f"max|dLSE|={worst['lse_max']:.3e} (err/bound {worst['lse_ratio']:.3f}) "
           f"mean err/bound {worst['o_mean_ratio']:.3f}")
    assert worst["o_ratio"] <= 1.0, f"{what}: |dO| above its bound ({worst['o_ratio']:.3f} x)"
    assert worst["lse_ratio"] <= 1.0, f"{what}: |dLSE| above its bound ({worst['lse_ratio']:.3f} x)"
    assert worst["o_mean_ratio"] <= 1.0, f"{what}: mean |dO| above its bound ({worst['o_mean_ratio']:.3f} x)"


SMALL_N = [1, 17, 64, 65, 128, 129, 200, 333, 1000]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SMALL_N)
def test_fp8_small_shapes(N, causal, D):
    w = fi.Workload(f"fp8_n{N}_d{D}", 800 + 4 * SMALL_N.index(N) + D // 64, 1, 2, N, D, "fp8", causal)
    gu.log(f"[gpu] fp8 N={N} D={D} causal={causal}")
    inp = _inputs(w)
    o, lse = _run(inp, causal, w.scale)
    _compare(inp, o, lse, [(0, 0), (0, 1)], causal, w.scale, f"{w.name} causal={causal}")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.3])
def test_fp8_other_scales(scale):
    w = fi.Workload("fp8_scale_n300_d128", 850, 1, 2, 300, 128, "fp8", True)
    inp = _inputs(w)
    o, lse = _run(inp, True, scale)
    _compare(inp, o, lse, [(0, 0), (0, 1)], True, scale, f"{w.name} scale={scale}")


@pytest.mark.parametrize("D", [128, 256])
def test_fp8_block_scales_vary(D):
    """Scale codes drawn independently per block over a wide range: every
    block's scale must reach the right products (at D = 256 each converting
    lane's values span two V blocks)."""
    w = fi.Workload(f"fp8_wide_n257_d{D}", 851, 1, 2, 257, D, "fp8", False)
    inp = _inputs(w)
    g = np.random.default_rng(851)
    # Q, K block scales over 2^-12 .. 2^-4 (scores of order one at scale 2^-7),
    # V block scales over 2^-17 .. 2^6 (O errors are judged relative to V's RMS)
    ranges = ((115, 124), (115, 124), (110, 134))
    out = [(codes, g.integers(lo, hi, sc.shape).astype(np.uint8)) for (codes, sc), (lo, hi) in zip(inp, ranges)]
    o, lse = _run(out, False, 2.0 ** -7)
    # V values span 2^23 here, so no single absolute bound fits every output;
    # each element is bounded by the bf16 error model instead (tests/
    # error_models.py): the weights are normalised by their own rounded sum, so
    # each carries at most 2u relative error (u = 2^-8), O is rounded once more
    # (u |O|), and the FP8 score term adds 2 E_i max_j |v_jd|; times KAPPA
    u = em.U16["bf16"]
    for hh in range(2):
        qd, kd, vd = (mx_dequantize(c[0, hh], sc[0, hh]) for c, sc in out)
        o_ref, lse_ref = attention_ref(qd, kd, vd, False, 2.0 ** -7)
        wabs, _ = attention_ref(qd, kd, np.abs(vd), False, 2.0 ** -7)
        e_row, o_term = em.fp8_row_terms(qd, kd, vd, False, 2.0 ** -7)
        err = np.abs(o[0, hh].float().cpu().numpy() - o_ref)
        bound = em.KAPPA * (2 * u * wabs + u * np.abs(o_ref)) + o_term + 1e-30
        ratio = float((err / bound).max())
        dl = np.abs(lse[0, hh].cpu().numpy() - lse_ref)
        lratio = float((dl / (1e-3 + e_row)).max())
        gu.log(f"  {w.name} head {hh}: max |dO| / bound = {ratio:.3f}, max |dLSE| / bound = {lratio:.3f}")
        assert ratio <= 1.0, f"{w.name} head {hh}: error above the bf16 error-model bound ({ratio:.3f})"
        assert lratio <= 1.0, f"{w.name} head {hh}: LSE error above its bound ({lratio:.3f})"


@pytest.mark.parametrize("D", [128, 256])
def test_fp8_peaked_scores(D):
    w = fi.Workload(f"fp8_peaked_n512_d{D}", 852, 1, 4, 512, D, "fp8", True, fi.PEAKED)
    inp = _inputs(w)
    o, lse = _run(inp, True, w.scale)
    _compare(inp, o, lse, [(0, h) for h in range(4)], True, w.scale, w.name)


@pytest.mark.parametrize("D", [128, 256])
def test_fp8_outputs_written_and_deterministic(D):
    w = fi.Workload(f"fp8_canary_n999_d{D}", 853, 2, 3, 999, D, "fp8", True)
    inp = _inputs(w)
    runs = []
    for _ in range(2):
        o = torch.full((2, 3, 999, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((2, 3, 999), float("nan"), device="cuda")
        _run(inp, True, w.scale, out=o, lse=lse)
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        runs.append((o.clone(), lse.clone()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("w", fi.FP8_WORKLOADS, ids=lambda w: w.name)
def test_fp8_full_size_workload(w):
    """The FP8 workloads in the benchmark's launch configuration: every head,
    every row."""
    gu.log(f"[gpu] fp8 workload {w.name}")
    inp = _inputs(w)
    o, lse = _run(inp, w.causal, w.scale)
    _compare(inp, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)], w.causal, w.scale,
             w.name + " all rows")
