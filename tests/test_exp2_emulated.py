"""GPU tests of fa_fwd_exp2_emulated (through the C ABI): fa_fwd with a
quarter or a half of the exponentials computed by the FMA-pipe polynomial
("FlashAttention-4震撼发布：性能再攀新高", second algorithmic improvement).

* Against the fp64 oracle at the bf16 bars, on ragged shapes (several tiles,
  ragged tails, GQA, MQA, one query, one key, rows that see no key, packed
  GQA heads), d = 64 and 128, causal and not.
* Against fa_fwd on the same inputs: each probability differs by at most
  the polynomial's relative error (7.5e-5) before both round it to bf16,
  which can move it by one bf16 step (2^-7 relative), so
  |O_emu - O_fwd| <= 2^-7 sum_j p_ij |v_jc| / sum_j p_ij + bf16 rounding of
  both outputs (2 x 2^-9 |O|); the LSE uses the fp32 probabilities and
  moves by at most ln(1 + 7.5e-5) plus fp32 rounding.
* Rows that see no key give O = 0 and LSE = -inf exactly; the workload of
  the benchmark (causal GQA B2 Hq32 Hkv8 N8192 d128) on sampled rows.
"""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64, attention_rows_fp64
from tests.gpu_util import compare, out_to_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [
    # B, Hq, Hkv, Nq, Nk
    (2, 4, 2, 200, 333),
    (1, 8, 1, 130, 130),
    (1, 3, 3, 1, 77),
    (1, 2, 1, 70, 1),
    (1, 2, 2, 150, 40),     # Nq > Nk: causal rows with no visible key
    (2, 8, 2, 1, 300),      # decoding: GQA heads packed into one wave
    (2, 32, 4, 8, 200),     # packed over two waves
    (2, 16, 4, 1024, 1024), # enough workgroups for the 8-wave d = 128 kernel
]


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


def _run(api, fn, w, x, quarters=None):
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    if quarters is None:
        fn(q, k, v, o, lse, w.softmax_scale, w.causal)
    else:
        fn(q, k, v, o, lse, w.softmax_scale, w.causal, quarters)
    torch.cuda.synchronize()
    return out_to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("quarters", [1, 2])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_against_the_oracle_and_fa_fwd(api, shape, d, causal, quarters):
    B, Hq, Hkv, Nq, Nk = shape
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", causal=causal)
    x = gen.make_inputs(w, (sum(shape), d, causal, 2))
    print(f"case: exp2 emulated {quarters}/4 {w.name}", flush=True)
    o, lse = _run(api, api.fa_fwd_exp2_emulated, w, x, quarters)
    q, k, v = (to_f64(x[t], "bf16") for t in "qkv")
    o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, causal)
    compare(o, lse, o_ref, lse_ref, what=w.name)
    # against fa_fwd
    o_f, lse_f = _run(api, api.fa_fwd, w, x)
    acc, _ = attention_fp64(q, k, np.abs(v), w.softmax_scale, causal)
    tol = 2.0 ** -7 * acc + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    err = np.abs(o - o_f)
    assert (err <= tol).all(), f"max excess {(err - tol).max():.3e}"
    none = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), none)
    assert (o[none] == 0).all()
    le = np.abs(lse[~none] - lse_f[~none])
    assert (le <= 1e-4 + 2e-6 * np.abs(lse_f[~none])).all(), le.max()


def test_benchmark_workload_sampled_rows(api):
    w, x = gen.make_config(3)
    print(f"case: exp2 emulated 2/4 {w.name}", flush=True)
    o, lse = _run(api, api.fa_fwd_exp2_emulated, w, x, 2)
    rng = np.random.default_rng(7)
    rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.Nq - 1)]
    rows += [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Nq))) for _ in range(30)]
    q, k, v = (to_f64(x[t], "bf16") for t in "qkv")
    o_ref, lse_ref = attention_rows_fp64(q, k, v, w.softmax_scale, True, rows)
    got = np.stack([o[b, h, i] for b, h, i in rows])
    got_l = np.array([lse[b, h, i] for b, h, i in rows])
    compare(got, got_l, o_ref, lse_ref, what=w.name)


def test_deterministic(api):
    w = gen.workload(1, 8, 2, 300, 300, 128, causal=True)
    x = gen.make_inputs(w, (5,))
    a, la = _run(api, api.fa_fwd_exp2_emulated, w, x, 1)
    b, lb = _run(api, api.fa_fwd_exp2_emulated, w, x, 1)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_rejected_arguments(api):
    w = gen.workload(1, 2, 2, 64, 64, 256)
    x = gen.make_inputs(w, (1,))
    with pytest.raises(api.FaError) as e:
        _run(api, api.fa_fwd_exp2_emulated, w, x, 1)
    assert e.value.status == 3
    w = gen.workload(1, 2, 2, 64, 64, 128)
    x = gen.make_inputs(w, (1,))
    for bad in (0, 3):
        with pytest.raises(api.FaError) as e:
            _run(api, api.fa_fwd_exp2_emulated, w, x, bad)
        assert e.value.status == 8
