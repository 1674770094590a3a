"""Seeded random shapes through the bf16 forward, split-KV and backward paths,
against the fp64 oracle at the same tolerances as the hand-picked cases.

Each case draws B, the GQA ratio, Hkv, ragged Nq and Nk (one row up to a few
tiles, Nq > Nk included), d, causal and a split count from a fixed seed, so
the planner's choices (waves per workgroup, packed heads, key ranges) and the
kernels' edge handling meet combinations no hand-picked case names.
"""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_backward_fp64, attention_fp64
from tests.gpu_util import compare, out_to_f64, to_device, to_f64
from tests.test_backward import compare_grad, run_backward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


def draw(i):
    r = np.random.default_rng(np.random.SeedSequence([4242, i]))
    B = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 4, 8]))
    Hkv = int(r.integers(1, 4))
    Nq = int(r.choice([1, 2, 7, 31, 33, 64, 65, 100, 190, 257]))
    Nk = int(r.choice([1, 5, 63, 64, 65, 129, 200, 333, 700]))
    d = int(r.choice([64, 128, 256]))
    causal = bool(r.integers(0, 2))
    nsplit = int(r.choice([0, 1, 2, 3, 5]))
    return B, G * Hkv, Hkv, Nq, Nk, d, causal, nsplit


CASES = [draw(i) for i in range(24)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_random_shape_forward_and_split(api, case):
    B, Hq, Hkv, Nq, Nk, d, causal, nsplit = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    x = gen.make_inputs(w, (51, sum(case)))
    print(f"case: random forward {w.name} nsplit={nsplit}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o, lse = api.attention(q, k, v, causal=causal)
    o2, lse2 = api.attention_splitkv(q, k, v, causal=causal, nsplit=nsplit)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_fp64(*(to_f64(x[t], "bf16") for t in "qkv"), w.softmax_scale, causal)
    compare(out_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, what=w.name)
    compare(out_to_f64(o2), lse2.cpu().numpy().astype(np.float64), o_ref, lse_ref, what=w.name + " split")


@pytest.mark.parametrize("case", CASES[:16], ids=lambda c: "x".join(map(str, c)))
def test_random_shape_backward(api, case):
    B, Hq, Hkv, Nq, Nk, d, causal, _ = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    x = gen.make_inputs(w, (52, sum(case)))
    do_bits = gen.make_dout(w, (52, sum(case)))
    print(f"case: random backward {w.name}", flush=True)
    dq, dk, dv = run_backward(api, w, x, do_bits)
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    dof = to_f64(do_bits, "bf16")
    rq, rk, rv = attention_backward_fp64(qf, kf, vf, dof, w.softmax_scale, causal)
    if Nk == 1:
        # one key: dQ and dK are exactly 0 and the kernels leave rounding noise
        # of at most scale d 2^-24 max|dO.V| max|K| per dQ element (the bound
        # of the single-key case, summed over the Nq rows for dK)
        bound = w.softmax_scale * d * 2.0 ** -24 * np.abs(dof * vf[:, np.repeat(np.arange(Hkv), Hq // Hkv)]) \
            .sum(axis=-1).max() * np.abs(kf).max()
        assert (rq == 0).all() and (rk == 0).all()
        assert np.abs(dq).max() <= bound, (np.abs(dq).max(), bound)
        assert np.abs(dk).max() <= Nq * (Hq // Hkv) * bound * np.abs(qf).max() / np.abs(kf).max()
    else:
        compare_grad(dq, rq, f"{w.name} dQ")
        compare_grad(dk, rk, f"{w.name} dK")
    compare_grad(dv, rv, f"{w.name} dV")


@pytest.mark.parametrize("case", CASES[:16], ids=lambda c: "x".join(map(str, c)))
def test_random_shape_fp8(api, case):
    """The same drawn shapes through fa_fp8_prepare (with the rotation) and
    fa_fwd_fp8, against the fp64 oracle on exactly the e4m3 values the GPU
    consumed: cosine >= 0.999, rows with no key O = 0 and LSE = -inf, the LSE
    within the per-row bound of the fp8 MFMA's grouped sums."""
    from tests.test_fp8 import check_lse_against_dequantised, cosine, dequantise_gpu, score_error_bound
    B, Hq, Hkv, Nq, Nk, d, causal, _ = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, dtype="fp8", causal=causal)
    x = gen.make_inputs(w, (53, sum(case)))
    print(f"case: random fp8 {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    signs = torch.from_numpy(x["signs"]).cuda()
    o, lse, prep = api.attention_fp8(q, k, v, causal=causal, scale=w.softmax_scale, signs=signs)
    torch.cuda.synchronize()
    o, lse = out_to_f64(o), lse.cpu().numpy().astype(np.float64)
    qq, kq, vq = dequantise_gpu(prep["q8"].cpu().numpy(), prep["k8"].cpu().numpy(), prep["v8t"].cpu().numpy(),
                                prep["descale"].cpu().numpy().astype(np.float64), Nk, w.softmax_scale)
    o_q, lse_q = attention_fp64(qq, kq, vq, w.softmax_scale, causal)
    assert np.isfinite(o).all()
    none = np.isneginf(lse_q)
    assert (o[none] == 0).all()
    if (~none).any():
        assert cosine(o[~none], o_q[~none]) >= 0.999, cosine(o[~none], o_q[~none])
    check_lse_against_dequantised(lse, lse_q, score_error_bound(qq, kq, w.softmax_scale), w.name)
