"""GPU parity of fa_bwd (dQ, dK, dV) against the fp64 oracle's gradients.

The HIP path runs fa_fwd (O, LSE) and then fa_bwd on seeded bf16 inputs;
the oracle differentiates the definition in fp64 on the same bf16 values
(attention_backward_fp64).  Shapes cover MHA, GQA and MQA, causal and not,
head dimensions 64, 128 and 256, ragged query and key counts spanning
several tiles, rows that see no key (causal with Nq > Nk), a single query
row, and a GQA head group at the full long-context size.

Tolerance (bf16 arithmetic, unit roundoff u = 2^-9): P and dS enter their
products rounded to bf16 (relative error u per term), D is formed from the
bf16 O (error u |dO||O| per row), and each gradient is rounded to bf16
(u relative).  The products are accumulated in fp32.  With random-sign terms
these errors add in quadrature, so the root-mean-square error of a gradient
stays a small multiple of u times its root-mean-square value, and the largest
error a small multiple of u times its largest magnitude:
    rms|g - g_ref| <= 2^-7 rms|g_ref|,   max|g - g_ref| <= 2^-6 max|g_ref|
(4u and 8u; measured: rms 1.1u - 1.4u, max at most 3u on these shapes).
Sharper softmax rows (large scores) weaken this for dQ and dK: dS = P (dP - D)
then cancels, and the rounding of O to bf16 inside D stops being small
against it.  The case with outlier channels measures that effect and takes
twice the bounds (there the exact gradient with D formed from bf16(O) alone
is 3.5u from the true one in rms for dQ).
"""
import math

import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_backward_fp64
from tests.gpu_util import out_to_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RMS_REL = 2.0 ** -7
MAX_REL = 2.0 ** -6


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


def compare_grad(g, ref, what, rms_rel=RMS_REL, max_rel=MAX_REL):
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    err = np.abs(g - ref)
    rms_ref = math.sqrt(float(np.mean(ref * ref)))
    max_ref = float(np.abs(ref).max())
    rms_err = math.sqrt(float(np.mean(err * err)))
    print(f"  {what}: rms err / rms ref = {rms_err / max(rms_ref, 1e-300):.2e}, "
          f"max err / max ref = {err.max() / max(max_ref, 1e-300):.2e}", flush=True)
    if max_ref == 0.0:
        assert err.max() == 0.0, f"{what}: nonzero gradient where the reference is 0"
        return
    assert rms_err <= rms_rel * rms_ref, f"{what}: rms err {rms_err:.3e} > {rms_rel} x rms ref {rms_ref:.3e}"
    assert err.max() <= max_rel * max_ref, f"{what}: max err {err.max():.3e} > {max_rel} x max ref {max_ref:.3e}"


def run_backward(api, w, x, do_bits):
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    do = to_device(do_bits, "bf16")
    o, lse = api.attention(q, k, v, causal=w.causal, scale=w.softmax_scale)
    dq, dk, dv = api.attention_backward(q, k, v, o, lse, do, causal=w.causal, scale=w.softmax_scale)
    torch.cuda.synchronize()
    return out_to_f64(dq), out_to_f64(dk), out_to_f64(dv)


def check(api, w, seed, rms_rel=RMS_REL, max_rel=MAX_REL):
    x = gen.make_inputs(w, seed)
    do_bits = gen.make_dout(w, seed)
    print(f"case: backward {w.name}", flush=True)
    dq, dk, dv = run_backward(api, w, x, do_bits)
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    rq, rk, rv = attention_backward_fp64(qf, kf, vf, to_f64(do_bits, "bf16"), w.softmax_scale, w.causal)
    compare_grad(dq, rq, f"{w.name} dQ", rms_rel, max_rel)
    compare_grad(dk, rk, f"{w.name} dK", rms_rel, max_rel)
    compare_grad(dv, rv, f"{w.name} dV", rms_rel, max_rel)


CASES = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 2, 2, 64, 64, 128),       # one tile each way
    (1, 4, 2, 300, 300, 128),     # GQA 2, ragged, several tiles
    (2, 8, 2, 257, 200, 128),     # GQA 4, Nq > Nk
    (1, 4, 1, 150, 333, 128),     # MQA, Nq < Nk
    (1, 3, 3, 129, 700, 64),      # d = 64
    (2, 4, 2, 190, 190, 64),      # d = 64, GQA
    (1, 2, 1, 100, 260, 256),     # d = 256, MQA
    (1, 2, 2, 1, 500, 128),       # a single query row
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_backward_matches_the_oracle(api, case, causal):
    B, Hq, Hkv, Nq, Nk, d = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    check(api, w, (sum(case), int(causal), 21))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_single_key(api, causal):
    """One key: every visible row's softmax is the constant 1, so dQ and dK
    are exactly 0 and dV is the sum of dO over the rows that see the key.
    The kernels reach the zeros as dP - D with D formed from the bf16 O (here
    O = V exactly, D accumulated in a different order than dP), so dQ and dK
    carry rounding noise bounded by scale |dP - D| max|K| <= scale * d * 2^-24
    max_i sum_c |dO_ic V_c| max|K| per element (fp32 accumulation of d
    exact products); dV is checked like the other cases."""
    w = gen.workload(1, 2, 2, 500, 1, 64, causal=causal)
    x = gen.make_inputs(w, (25, int(causal)))
    do_bits = gen.make_dout(w, (25, int(causal)))
    dq, dk, dv = run_backward(api, w, x, do_bits)
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    dof = to_f64(do_bits, "bf16")
    rq, rk, rv = attention_backward_fp64(qf, kf, vf, dof, w.softmax_scale, causal)
    assert (rq == 0).all() and (rk == 0).all()
    bound = w.softmax_scale * 64 * 2.0 ** -24 * np.abs(dof * vf).sum(axis=-1).max() * np.abs(kf).max()
    assert np.abs(dq).max() <= bound, (np.abs(dq).max(), bound)
    # dK sums dS Q over the rows: at most 500 rows of such noise times max|Q| / max|K|
    assert np.abs(dk).max() <= 500 * bound * np.abs(qf).max() / np.abs(kf).max()
    compare_grad(dv, rv, "dV")


def test_backward_outlier_channels(api):
    # a few feature channels of Q and K eight times larger (sharper softmax
    # rows): twice the bounds, for the reason given at the top
    w = gen.workload(1, 4, 2, 256, 256, 256, causal=False, outlier_channel_frac=0.02)
    check(api, w, (22,), 2 * RMS_REL, 2 * MAX_REL)


def test_backward_rows_without_keys_get_zero_dq(api):
    # causal with Nq > Nk: the first Nq - Nk rows see no key; their dQ is 0 and
    # they add nothing to dK, dV
    w = gen.workload(1, 2, 1, 130, 40, 128, causal=True)
    x = gen.make_inputs(w, (23,))
    do_bits = gen.make_dout(w, (23,))
    dq, dk, dv = run_backward(api, w, x, do_bits)
    assert (dq[:, :, : 130 - 40] == 0).all()
    qf, kf, vf = (to_f64(x[t], "bf16") for t in "qkv")
    rq, rk, rv = attention_backward_fp64(qf, kf, vf, to_f64(do_bits, "bf16"), w.softmax_scale, True)
    compare_grad(dk, rk, "dK")
    compare_grad(dv, rv, "dV")


def test_backward_full_size_head_group(api):
    """The long-context GQA shape (B2 Hq32 Hkv8 N8192 d128, causal) in the
    launch configuration of the full problem; the oracle checks one head group
    (batch 1, key/value head 5 and its 4 query heads), sliced from the same
    inputs."""
    w, x = gen.make_config(3)
    do_bits = gen.make_dout(w, (3,))
    print(f"case: backward full size {w.name}", flush=True)
    dq, dk, dv = run_backward(api, w, x, do_bits)
    b, hk, G = 1, 5, w.Hq // w.Hkv
    hs = slice(hk * G, hk * G + G)
    qf = to_f64(x["q"][b:b + 1, hs], "bf16")
    kf = to_f64(x["k"][b:b + 1, hk:hk + 1], "bf16")
    vf = to_f64(x["v"][b:b + 1, hk:hk + 1], "bf16")
    dof = to_f64(do_bits[b:b + 1, hs], "bf16")
    rq, rk, rv = attention_backward_fp64(qf, kf, vf, dof, w.softmax_scale, True)
    compare_grad(dq[b:b + 1, hs], rq, "full dQ")
    compare_grad(dk[b:b + 1, hk:hk + 1], rk, "full dK")
    compare_grad(dv[b:b + 1, hk:hk + 1], rv, "full dV")


def test_backward_agrees_with_torch_autograd_on_the_cpu(api):
    """A second reference for the same quantity: autograd of the plain fp64
    attention formula on the CPU (the products of the definition), on one
    small GQA case."""
    w = gen.workload(1, 4, 2, 96, 130, 64, causal=True)
    x = gen.make_inputs(w, (24,))
    do_bits = gen.make_dout(w, (24,))
    dq, dk, dv = run_backward(api, w, x, do_bits)
    q, k, v = (torch.from_numpy(to_f64(x[t], "bf16")).requires_grad_() for t in "qkv")
    do = torch.from_numpy(to_f64(do_bits, "bf16"))
    kr, vr = k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1)
    s = (q @ kr.transpose(-1, -2)) * w.softmax_scale
    i = torch.arange(96)[:, None]
    j = torch.arange(130)[None, :]
    s = s.masked_fill(j > i + (130 - 96), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    o.backward(do)
    compare_grad(dq, q.grad.numpy(), "autograd dQ")
    compare_grad(dk, k.grad.numpy(), "autograd dK")
    compare_grad(dv, v.grad.numpy(), "autograd dV")


def test_backward_stages_equal_the_whole(api):
    """fa_bwd_dq followed by fa_bwd_dkdv writes exactly what fa_bwd writes."""
    w = gen.workload(2, 8, 2, 200, 333, 128, causal=True)
    x = gen.make_inputs(w, (26,))
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    do = to_device(gen.make_dout(w, (26,)), "bf16")
    o, lse = api.attention(q, k, v, causal=True)
    dq1, dk1, dv1 = api.attention_backward(q, k, v, o, lse, do, causal=True)
    nbytes = api.bwd_workspace_size(2, 8, 2, 200, 333, 128, True)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    api.fa_bwd_dq(q, k, v, o, lse, do, dq2, w.softmax_scale, True, ws)
    api.fa_bwd_dkdv(q, k, v, o, lse, do, dk2, dv2, w.softmax_scale, True, ws)
    torch.cuda.synchronize()
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the workspace starts with (LSE log2 e, D) per row (partial sums of the
    # split heads, G = 4 here, follow them)
    pairs = ws[: 2 * 8 * 200 * 2].view(2, 8, 200, 2).cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(pairs[..., 0], lse.cpu().numpy() * math.log2(math.e), rtol=1e-6)
    d_ref = (do.float() * o.float()).sum(-1).cpu().numpy()
    np.testing.assert_allclose(pairs[..., 1], d_ref, rtol=1e-4, atol=1e-4)


# Grids large enough that the planner picks the multi-wave workgroups (at
# least 512 dK/dV workgroups, 1024 dQ workgroups where possible): d = 64 with
# 4-wave, 64-key-per-wave dK/dV workgroups; d = 256 with 2-wave ones; d = 128
# with 4-wave ones (8 would leave fewer than 512).  The kernels run the whole
# problem; the oracle checks the gradients of one head group.
LARGE = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (4, 32, 16, 2000, 2000, 64, True),
    (2, 16, 8, 2048, 2048, 256, False),
    (2, 16, 8, 1000, 4000, 128, True),
]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "x".join(map(str, c)))
def test_backward_large_grids_one_head_group(api, case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    x = gen.make_inputs(w, (27, sum(case[:6])))
    do_bits = gen.make_dout(w, (27, sum(case[:6])))
    print(f"case: backward large grid {w.name}", flush=True)
    dq, dk, dv = run_backward(api, w, x, do_bits)
    b, hk, G = B - 1, Hkv - 1, Hq // Hkv
    hs = slice(hk * G, hk * G + G)
    rq, rk, rv = attention_backward_fp64(to_f64(x["q"][b:b + 1, hs], "bf16"), to_f64(x["k"][b:b + 1, hk:hk + 1], "bf16"),
                                         to_f64(x["v"][b:b + 1, hk:hk + 1], "bf16"),
                                         to_f64(do_bits[b:b + 1, hs], "bf16"), w.softmax_scale, causal)
    compare_grad(dq[b:b + 1, hs], rq, f"{w.name} dQ")
    compare_grad(dk[b:b + 1, hk:hk + 1], rk, f"{w.name} dK")
    compare_grad(dv[b:b + 1, hk:hk + 1], rv, f"{w.name} dV")


# Few key/value heads (MQA and small-batch GQA): too few (group, key block)
# pairs to fill the GPU, so the G query heads of every group are split into
# parts whose fp32 partial sums of dK and dV are added by a second kernel.
# Whole problems against the oracle.
HEAD_SPLIT = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 16, 1, 2048, 2048, 128, True),
    (2, 8, 1, 1000, 1500, 64, False),
    (1, 12, 2, 700, 900, 256, True),
    (1, 6, 3, 500, 700, 128, False),
]


@pytest.mark.parametrize("case", HEAD_SPLIT, ids=lambda c: "x".join(map(str, c)))
def test_backward_with_split_heads(api, case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, causal=causal)
    check(api, w, (28, sum(case[:6])))


@pytest.mark.parametrize("B,Hq,Hkv,n,causal", [(1, 36, 9, 14600, True), (1, 36, 9, 7300, False), (8, 16, 16, 2048, True)],
                         ids=["causal_2061_items", "noncausal_1035_items", "causal_4wave_2048_items"])
def test_backward_persistent_dq_covers_every_row(api, B, Hq, Hkv, n, causal):
    """The dQ kernel of eight-wave d = 128 plans with more work items than CUs
    runs as a persistent grid (one workgroup per CU, taking items in rounds),
    and so does the causal four-wave one up to 4096 rows, two workgroups per
    CU.  At 2061 and 1035 items (not multiples of 8) and at 2048 four-wave
    items dQ starts as NaN and must be written everywhere.  Sampled rows of
    several heads match the oracle: a row's dQ depends only on its own Q and
    dO rows and on the keys it sees, so the oracle runs on that row and those
    keys alone."""
    w = gen.workload(B, Hq, Hkv, n, n, 128, causal=causal)
    x = gen.make_inputs(w, (n, int(causal), 78))
    do_bits = gen.make_dout(w, (n, int(causal), 78))
    print(f"case: backward persistent dQ {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    do = to_device(do_bits, "bf16")
    o, lse = api.attention(q, k, v, causal=causal, scale=w.softmax_scale)
    dq = torch.full_like(q, float("nan"))
    nbytes = api.bwd_workspace_size(B, Hq, Hkv, n, n, 128, causal)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device="cuda")
    api.fa_bwd_dq(q, k, v, o, lse, do, dq, w.softmax_scale, causal, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(dq).any().item(), "dQ rows left unwritten"
    dqf = out_to_f64(dq)
    rng = np.random.default_rng(n)
    got, ref = [], []
    b = B - 1
    for h in (0, Hq // 3, Hq - 1):
        hk = h // (Hq // Hkv)
        for i in [0, 63, 64, 255, 256, n // 2, n - 1] + [int(r) for r in rng.integers(0, n, 5)]:
            nk = i + 1 if causal else n
            rq, _, _ = attention_backward_fp64(
                to_f64(x["q"][b:b + 1, h:h + 1, i:i + 1], "bf16"), to_f64(x["k"][b:b + 1, hk:hk + 1, :nk], "bf16"),
                to_f64(x["v"][b:b + 1, hk:hk + 1, :nk], "bf16"), to_f64(do_bits[b:b + 1, h:h + 1, i:i + 1], "bf16"),
                w.softmax_scale, False)
            got.append(dqf[b, h, i])
            ref.append(rq[0, 0, 0])
    compare_grad(np.array(got), np.array(ref), f"{w.name} dQ rows")


@pytest.mark.parametrize("case", [(8, 32, 8, 2048, 128, True), (11, 28, 7, 1700, 128, False),
                                  (4, 16, 16, 2048, 256, True), (6, 16, 8, 1500, 256, False),
                                  (4, 16, 16, 2048, 64, True), (2, 32, 8, 4096, 64, True),
                                  (1, 32, 32, 2048, 128, True), (1, 32, 32, 2048, 128, False),
                                  (4, 16, 16, 2048, 64, False)],
                         ids=["d128_causal_512_items", "d128_noncausal_539_items", "d256_causal_1024_items",
                              "d256_noncausal_576_items", "d64_causal_512_items", "d64_causal_2048_items_head_parts",
                              "d128_4wave_causal_512_items", "d128_4wave_noncausal", "d64_4wave_noncausal"])
def test_backward_persistent_dkdv_covers_every_key(api, case):
    """Up to 4096 query rows, the dK/dV kernels that fill a CU with one or two
    workgroups (8 or 4 waves at d = 128, 4 at d = 256 and 64, 2 at d = 64) run as
    persistent grids when the plan has at least two key blocks per workgroup
    (here 512 to 2048 items, one count not a multiple of 8, one plan with the
    query heads split into parts); so do the dQ kernels at d = 128 and 256.
    dQ, dK and dV start as NaN and must be written everywhere; one head
    group's gradients match the oracle."""
    B, Hq, Hkv, N, d, causal = case
    w = gen.workload(B, Hq, Hkv, N, N, d, causal=causal)
    x = gen.make_inputs(w, (N, int(causal), 79))
    do_bits = gen.make_dout(w, (N, int(causal), 79))
    print(f"case: backward persistent dK/dV {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    do = to_device(do_bits, "bf16")
    o, lse = api.attention(q, k, v, causal=causal, scale=w.softmax_scale)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    nbytes = api.bwd_workspace_size(B, Hq, Hkv, N, N, d, causal)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device="cuda")
    api.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, w.softmax_scale, causal, ws)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert not torch.isnan(t).any().item(), f"{name} left unwritten"
    b, hk, G = B - 1, Hkv - 1, Hq // Hkv
    hs = slice(hk * G, hk * G + G)
    rq, rk, rv = attention_backward_fp64(to_f64(x["q"][b:b + 1, hs], "bf16"), to_f64(x["k"][b:b + 1, hk:hk + 1], "bf16"),
                                         to_f64(x["v"][b:b + 1, hk:hk + 1], "bf16"),
                                         to_f64(do_bits[b:b + 1, hs], "bf16"), w.softmax_scale, causal)
    compare_grad(out_to_f64(dq)[b:b + 1, hs], rq, f"{w.name} dQ")
    compare_grad(out_to_f64(dk)[b:b + 1, hk:hk + 1], rk, f"{w.name} dK")
    compare_grad(out_to_f64(dv)[b:b + 1, hk:hk + 1], rv, f"{w.name} dV")
