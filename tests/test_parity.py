"""GPU parity: libfa.so (through its C ABI) against the fp64 oracle.

Small and ragged shapes are compared element by element in full.  The large
standing workloads are compared in full too, in the launch configuration the
benchmark uses, with the oracle computed one (b, h) head at a time over a
pool of host processes; a quicker check on sampled rows is kept beside it.
"""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64, attention_rows_fp64
from tests.gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, LSE_ABS, compare, out_to_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


def _run(api, w, x):
    q, k, v = (to_device(x[t], w.dtype) for t in "qkv")
    o, lse = api.attention(q, k, v, causal=w.causal, scale=w.softmax_scale)
    torch.cuda.synchronize()
    return out_to_f64(o), lse.cpu().numpy().astype(np.float64)


def _full_check(api, w, x, **tol):
    print(f"case: {w.name}", flush=True)
    o, lse = _run(api, w, x)
    q, k, v = (to_f64(x[t], w.dtype) for t in "qkv")
    o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, w.causal)
    return compare(o, lse, o_ref, lse_ref, what=w.name, **tol)


# ---------------------------------------------------------------- standing workloads
def test_tiny_fp32_single_head(api):
    w, x = gen.make_config(1)
    _full_check(api, w, x)
    # the fp32 path splits operands into bf16 hi+lo: about 2^-16 relative per product
    _full_check(api, w, x, max_abs=1e-4, mean_abs=1e-5, lse_abs=1e-4)


def test_gpt2_small_causal(api):
    w, x = gen.make_config(2)
    _full_check(api, w, x)


def _sampled_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.Nq - 1), (0, w.Hq - 1, 63), (w.B - 1, 0, 64), (0, 1, w.Nq // 2)]
    while len(rows) < n:
        rows.append((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Nq))))
    return rows


@pytest.mark.parametrize("cfg", [3, 4])
def test_large_workloads_sampled(api, cfg):
    w, x = gen.make_config(cfg)
    print(f"case: {w.name}", flush=True)
    o, lse = _run(api, w, x)
    rows = _sampled_rows(w, 40, cfg)
    q, k, v = (to_f64(x[t], w.dtype) for t in "qkv")
    o_ref, lse_ref = attention_rows_fp64(q, k, v, w.softmax_scale, w.causal, rows)
    got_o = np.stack([o[b, h, i] for b, h, i in rows])
    got_l = np.array([lse[b, h, i] for b, h, i in rows])
    compare(got_o, got_l, o_ref, lse_ref, what=w.name)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("cfg", [3, 4])
def test_large_workloads_every_element(api, cfg):
    """The whole output of the standing workload against the oracle: max and
    mean |dO| over all elements and max |dLSE| over all rows, with the oracle
    computed one (b, h) head per task over the host's cores."""
    from tests.full_compare import compare_all_heads, pool_size
    w, x = gen.make_config(cfg)
    print(f"case: {w.name} (every element, {pool_size()} host workers)", flush=True)
    q, k, v = (to_device(x[t], w.dtype) for t in "qkv")
    o, lse = api.attention(q, k, v, causal=w.causal, scale=w.softmax_scale)
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    lse_h = lse.cpu().numpy()
    del q, k, v, o, lse
    st = compare_all_heads(x["q"], x["k"], x["v"], w.softmax_scale, w.causal, {"o": (o_bits, lse_h)})["o"]
    print(f"{w.name}: max|dO| {st['max_abs']:.3e} mean|dO| {st['mean_abs']:.3e} rmse {st['rmse']:.3e} "
          f"max|dLSE| {st['lse_max_abs']:.3e} over {st['n']} elements", flush=True)
    assert st["nonfinite"] == 0 and st["lse_inf_mismatch"] == 0
    assert st["max_abs"] <= BF16_MAX_ABS, st
    assert st["mean_abs"] <= BF16_MEAN_ABS, st
    assert st["lse_max_abs"] <= LSE_ABS, st


# ---------------------------------------------------------------- ragged shapes and edge cases
SHAPES = [
    # B, Hq, Hkv, Nq, Nk
    (2, 4, 2, 200, 333),     # several tiles, ragged tails, GQA 2
    (1, 8, 1, 130, 130),     # MQA
    (1, 6, 2, 257, 257),     # GQA 3 (one head per workgroup)
    (1, 3, 3, 1, 77),        # a single query
    (1, 2, 1, 70, 1),        # a single key
    (1, 2, 2, 150, 40),      # Nq > Nk: causal rows with no visible key
    (1, 4, 4, 64, 64),       # exactly one tile
    # G * Nq <= 32: the GQA group's heads share one wave's query columns (bf16)
    (2, 8, 2, 1, 300),       # decoding, GQA 4: 4 of 32 columns
    (1, 32, 1, 1, 200),      # 32 heads in one wave
    (3, 6, 2, 10, 100),      # 3 heads x 10 rows
    (1, 4, 2, 16, 70),       # 2 heads x 16 rows: every column
    (1, 8, 2, 7, 5),         # Nq > Nk: causal rows with no visible key
    # more heads than one wave's columns hold: packed over several waves
    (2, 32, 4, 8, 200),      # 8 heads x 8 rows: two waves
    (1, 24, 2, 10, 150),     # 12 heads x 10 rows: four waves of 3 heads
]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(api, shape, d, causal, dtype):
    B, Hq, Hkv, Nq, Nk = shape
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, dtype=dtype, causal=causal)
    x = gen.make_inputs(w, (sum(shape), d, causal))
    tol = {} if dtype == "bf16" else dict(max_abs=1e-4, mean_abs=1e-5, lse_abs=1e-4)
    _full_check(api, w, x, **tol)


# ---------------------------------------------------------------- closed forms and hygiene on the GPU
def test_causal_first_row_is_exactly_first_value_row(api):
    w = gen.workload(2, 4, 2, 96, 96, 128, causal=True)
    x = gen.make_inputs(w, (1,))
    o, lse = _run(api, w, x)
    v = to_f64(x["v"], "bf16")
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(o[b, h, 0], v[b, h // 2, 0])


def test_identical_keys_give_mean_of_values(api):
    w = gen.workload(1, 2, 2, 100, 300, 64)
    x = gen.make_inputs(w, (2,))
    x["k"] = np.repeat(x["k"][:, :, :1], 300, axis=2)
    o, lse = _run(api, w, x)
    v = to_f64(x["v"], "bf16")
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=2e-2)


def test_deterministic(api):
    w, x = gen.make_config(2)
    q, k, v = (to_device(x[t], w.dtype) for t in "qkv")
    o1, l1 = api.attention(q, k, v, causal=True)
    o2, l2 = api.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_writes_stay_inside_outputs(api):
    w = gen.workload(1, 2, 1, 77, 50, 128, causal=True)
    x = gen.make_inputs(w, (3,))
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    n = q.numel()
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((2 * 77 + 64,), 7.0, dtype=torch.float32, device="cuda")
    o = buf[:n].view(q.shape)
    lse = lbuf[:2 * 77].view(1, 2, 77)
    api.fa_fwd(q, k, v, o, lse, 1 / np.sqrt(128), True)
    torch.cuda.synchronize()
    assert (buf[n:] == 7.0).all() and (lbuf[2 * 77:] == 7.0).all()


def test_status_errors_raise(api):
    q = torch.zeros(1, 2, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.FaError) as e:
        api.fa_fwd(q, q, q, torch.empty_like(q), None, 0.1, False)
    assert e.value.status == 3        # head dimension 96


# ---------------------------------------------------------------- large grids (eight-wave workgroups at d = 128)
def _edge_rows(w, rng, n):
    """Rows at the ends of query blocks, tails and random positions."""
    rows = []
    for i in (0, 31, 32, 63, 64, 127, 128, w.Nq // 2, w.Nq - 64, w.Nq - 2, w.Nq - 1):
        if 0 <= i < w.Nq:
            rows.append((int(rng.integers(w.B)), int(rng.integers(w.Hq)), i))
    while len(rows) < n:
        rows.append((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Nq))))
    return rows


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1999, 1999), (2000, 2500), (2047, 1100)])
def test_large_grid_ragged(api, nq, nk, causal):
    # >= 1024 workgroups of 8 waves: the launch configuration of the long-context workloads
    w = gen.workload(2, 64, 16, nq, nk, 128, causal=causal)
    x = gen.make_inputs(w, (nq, nk, int(causal)))
    print(f"case: {w.name}", flush=True)
    o, lse = _run(api, w, x)
    rows = _edge_rows(w, np.random.default_rng(nq + nk), 48)
    q, k, v = (to_f64(x[t], w.dtype) for t in "qkv")
    o_ref, lse_ref = attention_rows_fp64(q, k, v, w.softmax_scale, w.causal, rows)
    got_o = np.stack([o[b, h, i] for b, h, i in rows])
    got_l = np.array([lse[b, h, i] for b, h, i in rows])
    compare(got_o, got_l, o_ref, lse_ref, what=w.name)
    assert np.isfinite(o).all()
    if causal and nq > nk:
        # queries that see no key (i + nk - nq < 0): O = 0, LSE = -inf
        assert (o[:, :, : nq - nk] == 0).all() and np.isneginf(lse[:, :, : nq - nk]).all()


PERSISTENT = [
    # B, Hq, Hkv, N, d, causal: work items of the plan
    (1, 36, 9, 14600, 128, True),    # 2061 items of 8 waves
    (1, 36, 9, 7300, 128, False),    # 1035
    (1, 7, 7, 4990, 256, True),      # 273 items of 4 waves
    (3, 12, 6, 2000, 256, False),    # 576
    (4, 10, 5, 1900, 64, True),      # 600 items of 4 waves, two workgroups per CU
    (3, 12, 12, 1900, 128, True),    # 540
]


@pytest.mark.parametrize("case", PERSISTENT, ids=lambda c: "x".join(map(str, c)))
def test_persistent_grid_covers_every_row(api, case):
    """The kernels that hold a whole CU per workgroup (8 waves at d = 128, 4
    at d = 256) run grids with more work items than CUs as one persistent
    workgroup per CU, each taking items in rounds; the causal 4-wave kernels at
    d = 64 and 128 do so with two workgroups per CU.  Item counts here are not
    multiples of the grid (most not of 8): O and LSE start as NaN and must be
    written everywhere, and sampled rows (block ends, the tail, random) match
    the oracle."""
    B, Hq, Hkv, n, d, causal = case
    w = gen.workload(B, Hq, Hkv, n, n, d, causal=causal)
    x = gen.make_inputs(w, (n, int(causal), 77))
    print(f"case: persistent grid {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device="cuda")
    api.fa_fwd(q, k, v, o, lse, w.softmax_scale, causal)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), "rows left unwritten"
    of, lf = out_to_f64(o), lse.cpu().numpy().astype(np.float64)
    rows = _edge_rows(w, np.random.default_rng(n), 48)
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    o_ref, lse_ref = attention_rows_fp64(qf, kf, vf, w.softmax_scale, causal, rows)
    compare(np.stack([of[b, h, i] for b, h, i in rows]), np.array([lf[b, h, i] for b, h, i in rows]),
            o_ref, lse_ref, what=w.name)


def test_concurrent_host_threads_on_separate_streams(api):
    """Several host threads call fa_fwd at once, each on its own stream, on
    shapes that take persistent and one-item grids (the library keeps a
    per-device CU-count cache that every launch reads); every result matches
    the oracle."""
    import threading
    cases = [gen.workload(2, 8, 2, 640, 640, 128, causal=True),
             gen.workload(1, 4, 4, 512, 700, 256),
             gen.workload(2, 6, 3, 300, 300, 64, causal=True),
             gen.workload(1, 16, 4, 1024, 1024, 128, causal=True),
             gen.workload(3, 4, 1, 200, 520, 128)]
    xs = [gen.make_inputs(w, (77, i)) for i, w in enumerate(cases)]
    results, errors = [None] * len(cases), []
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            w, x = cases[i], xs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                q, k, v = (to_device(x[t], "bf16") for t in "qkv")
                o = torch.empty_like(q)
                lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
            s.synchronize()
            start.wait(timeout=60)
            for _ in range(4):
                api.fa_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, s)
            s.synchronize()
            results[i] = (out_to_f64(o), lse.cpu().numpy().astype(np.float64))
        except Exception as e:  # noqa: BLE001
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=90)
    assert not errors, errors
    for (w, x), (o, lse) in zip(zip(cases, xs), results):
        q, k, v = (to_f64(x[t], "bf16") for t in "qkv")
        o_ref, lse_ref = attention_fp64(q, k, v, w.softmax_scale, w.causal)
        compare(o, lse, o_ref, lse_ref, what=w.name)
