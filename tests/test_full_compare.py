"""The whole-tensor comparison used by the large GPU parity tests, on the CPU:
per-head statistics gathered over a process pool equal the same statistics
taken directly over the whole tensor."""
import numpy as np

from exact_attention_07_amd import gen
from oracle import attention_fp64
from oracle.formats import bf16_bits_to_f64
from tests.full_compare import compare_all_heads, compare_fp8_all_heads


def _direct(o, o_ref):
    e = o - o_ref
    return dict(max_abs=np.abs(e).max(), mean_abs=np.abs(e).mean(), rmse=np.sqrt((e * e).mean()),
                cosine=(o * o_ref).sum() / np.sqrt((o * o).sum() * (o_ref * o_ref).sum()))


def test_pool_statistics_equal_direct_statistics():
    w = gen.workload(2, 4, 2, 40, 70, 64, causal=True)
    x = gen.make_inputs(w, (11,))
    q, k, v = (bf16_bits_to_f64(x[t]) for t in "qkv")
    o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, True)
    rng = np.random.default_rng(3)
    # a planted error of known size in one element, plus small noise elsewhere
    o_bad = o_ref + 1e-4 * rng.standard_normal(o_ref.shape)
    o_bad[1, 3, 17, 5] += 0.25
    lse_bad = lse_ref + 1e-6
    lse_bad[0, 2, 9] += 0.01
    for workers in (1, 2):
        st = compare_all_heads(x["q"], x["k"], x["v"], w.softmax_scale, True,
                               {"exact": (o_ref, lse_ref), "bad": (o_bad, lse_bad)}, workers=workers)
        assert st["exact"]["max_abs"] == 0.0 and st["exact"]["lse_max_abs"] == 0.0
        assert abs(st["exact"]["cosine"] - 1.0) < 1e-12
        ref = _direct(o_bad, o_ref)
        for key, val in ref.items():
            assert abs(st["bad"][key] - val) <= 1e-12 * max(1.0, abs(val)), (key, st["bad"][key], val)
        assert abs(st["bad"]["lse_max_abs"] - (0.01 + 1e-6)) < 1e-9
        assert st["bad"]["n"] == o_ref.size and st["bad"]["nonfinite"] == 0
        assert st["bad"]["lse_inf_mismatch"] == 0


def test_pool_flags_nonfinite_and_missing_infinities():
    w = gen.workload(1, 2, 1, 8, 4, 64, causal=True)   # Nq > Nk: rows without keys, LSE = -inf
    x = gen.make_inputs(w, (12,))
    q, k, v = (bf16_bits_to_f64(x[t]) for t in "qkv")
    o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, True)
    assert np.isneginf(lse_ref).any()
    o_nan = o_ref.copy()
    o_nan[0, 1, 7, 3] = np.nan
    lse_fin = np.where(np.isneginf(lse_ref), 0.0, lse_ref)
    st = compare_all_heads(x["q"], x["k"], x["v"], w.softmax_scale, True,
                           {"nan": (o_nan, lse_ref), "fin": (o_ref, lse_fin)}, workers=1)
    assert st["nan"]["nonfinite"] == 1
    assert st["fin"]["lse_inf_mismatch"] == int(np.isneginf(lse_ref).sum())


def test_fp8_pool_separates_format_error_from_kernel_error():
    """With an 'output' equal to the exact attention of the dequantised codes
    (rounded to bf16), the kernel-error statistics are at bf16 rounding level
    and the format-error statistics equal a direct computation."""
    from oracle import fp8 as ofp8
    from oracle.formats import e4m3_decode
    w = gen.workload(1, 3, 3, 50, 90, 64, dtype="fp8", outlier_prob=0.01)
    x = gen.make_inputs(w, (13,))
    q, k, v = (bf16_bits_to_f64(x[t]) for t in "qkv")
    prep = ofp8.prepare(q, k, v, x["signs"], w.softmax_scale)
    qd, kd, vd = ofp8.dequantised(prep)
    o_deq, _ = attention_fp64(qd, kd, vd, w.softmax_scale, False)
    o_true, _ = attention_fp64(q, k, v, w.softmax_scale, False)
    o_bits = gen.f32_to_bf16_bits(o_deq.astype(np.float32))
    v8 = np.ascontiguousarray(np.swapaxes(prep["v8t"], 2, 3))
    sq, sk, sv = prep["scales"]
    st = compare_fp8_all_heads(x["q"], x["k"], x["v"], w.softmax_scale,
                               {"r": (o_bits, prep["q8"], prep["k8"], v8, (sq / prep["c0"], sk, sv))}, workers=2)["r"]
    assert st["gpu_deq"]["max_abs"] <= 2.0 ** -8 * np.abs(o_deq).max()
    assert st["gpu_deq"]["cosine"] > 0.99999
    ref = _direct(o_deq, o_true)
    for key, val in ref.items():
        assert abs(st["deq_true"][key] - val) <= 1e-12 * max(1.0, abs(val)), (key, st["deq_true"][key], val)
    np.testing.assert_allclose(e4m3_decode(prep["q8"]) * (sq / prep["c0"]), qd, rtol=1e-15, atol=0)
