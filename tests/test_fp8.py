"""GPU tests of the fp8 path, fa_fp8_prepare and fa_fwd_fp8 (through the C ABI), against the oracle.

* The GPU's e4m3 conversion equals the oracle's codec on every finite code
  and on every rounding midpoint (ties to even).
* The prepared codes and scales equal the oracle's preparation, except at
  near-ties, where the fp32 arithmetic of the GPU may pick the other one of
  the two neighbouring e4m3 values.
* Attention on inputs whose probabilities are exact powers of two (integer
  logits with scale = ln 2, operands on a scaled e4m3 grid, power-of-two
  scales) is compared element by element: the only errors left are the
  grouped sums inside the fp8 MFMA, the fp32 accumulation and the bf16
  rounding of O.
* On random inputs: cosine >= 0.99 against the fp64 oracle on the unquantised
  bf16 source (the accuracy bar of the fp8 path), and the LSE against the
  oracle on the dequantised codes.
* The fp8 workload at full size on sampled rows, with and without the
  rotation (the errors of both are printed).
"""
import numpy as np
import pytest

from exact_attention_07_amd import gen
from oracle import attention_fp64, attention_rows_fp64
from oracle import fp8 as ofp8
from oracle.formats import bf16_bits_to_f64, e4m3_decode, e4m3_decode_table, e4m3_encode_rne
from tests.gpu_util import out_to_f64, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FP8_COSINE = 0.99


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_07_amd import api as a
    a.lib()
    return a


# ---------------------------------------------------------------- helpers
def key_order(v8t):
    """V^T codes [.., d, Nkp] from the stored order back to key order.

    Stored order (fa.h): within each block of 64 keys, key 32a + 8g + 4h + r
    sits at position 32h + 16a + 4g + r.
    """
    kk = np.arange(64)
    pos = 32 * ((kk >> 2) & 1) + 16 * (kk >> 5) + 4 * ((kk >> 3) & 3) + (kk & 3)
    j = np.arange(v8t.shape[-1])
    return v8t[..., (j // 64) * 64 + pos[j % 64]]


def e4m3_step(t):
    """Spacing of the e4m3 grid at |t| (subnormal spacing 2^-9 below 2^-6)."""
    a = np.abs(np.asarray(t, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def bf16_from_f64(a):
    bits = gen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    assert np.array_equal(bf16_bits_to_f64(bits), np.asarray(a, dtype=np.float64)), "not exact in bf16"
    return bits


def run_prepare(api, q, k, v, signs=None, descale=None, amax_ws=None, scale=None):
    """fa_fp8_prepare on device bf16 tensors; returns host copies (q8, k8, v8t, descale)."""
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    q8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    k8 = torch.empty(k.shape, dtype=torch.uint8, device="cuda")
    v8t = torch.full((B, Hkv, d, api.padded_keys(Nk)), 0x55, dtype=torch.uint8, device="cuda")
    descale = torch.empty(3, dtype=torch.float32, device="cuda") if descale is None else descale
    amax_ws = torch.full((3,), 12345, dtype=torch.int32, device="cuda") if amax_ws is None else amax_ws
    api.fa_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs, scale)
    torch.cuda.synchronize()
    return q8.cpu().numpy(), k8.cpu().numpy(), v8t.cpu().numpy(), descale.cpu().numpy().astype(np.float64)


def gpu_c0(scale):
    """The factor fa_fp8_prepare folds into Q: scale (passed as fp32) times
    log2(e), rounded to fp32."""
    return float(np.float32(float(np.float32(scale)) * np.log2(np.e)))


def dequantise_gpu(q8, k8, v8t, descale, nk, scale):
    """fp64 Q, K, V that the GPU codes stand for (V back in [B, Hkv, Nk, d]);
    the Q codes carry c0, which is divided out."""
    q = e4m3_decode(q8) * (descale[0] / gpu_c0(scale))
    k = e4m3_decode(k8) * descale[1]
    v = np.swapaxes(e4m3_decode(key_order(v8t)[..., :nk]) * descale[2], 2, 3)
    return q, k, v


def check_codes(codes, exact_values, scale, what):
    """GPU codes against the fp64 values they quantise (with the GPU's scale):
    every code is the round-to-nearest-even code of t = value/scale, except
    where t lies within 2^-20 (|t| + |row of t|_2) of a midpoint between two
    e4m3 values: there the fp32 arithmetic of the GPU (the scale, and the
    rotation, whose rounding error is a small multiple of 2^-24 times the row
    norm) may land on either side or on the tie itself, and the code must be
    one of the two neighbours."""
    t = np.asarray(exact_values, dtype=np.float64) / scale
    g = e4m3_decode(codes)
    assert np.isfinite(g).all(), f"{what}: NaN code"
    ref = e4m3_encode_rne(t)
    r = e4m3_decode(ref)
    differ = ~((ref == codes) | ((r == 0) & (g == 0)))
    if differ.any():
        row_norm = np.broadcast_to(np.linalg.norm(t, axis=-1, keepdims=True), t.shape)
        td, gd, rd = t[differ], g[differ], r[differ]
        mid = (gd + rd) / 2
        near_tie = np.abs(td - mid) <= 2.0 ** -20 * (np.abs(td) + row_norm[differ])
        neighbours = np.abs(gd - rd) <= e4m3_step(np.minimum(np.abs(gd), np.abs(rd))) * (1 + 1e-12)
        bad = ~(near_tie & neighbours)
        assert not bad.any(), (f"{what}: {int(bad.sum())} codes differ from round-to-nearest-even away from a tie, "
                               f"e.g. value {td[bad][0]!r} -> {gd[bad][0]!r} (expected {rd[bad][0]!r})")
    return float(differ.mean())


def cosine(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# ---------------------------------------------------------------- e4m3 conversion
def test_e4m3_conversion_matches_the_codec(api):
    """Every finite e4m3 value and every midpoint between neighbours, through
    the V quantisation with scale 1 (the tensor's amax is 448)."""
    table = e4m3_decode_table()
    finite = table[~np.isnan(table)]
    grid = np.sort(table[:0x7F])
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([finite, mids, -mids, [448.0]])
    nk, d = 16, 64
    v = np.zeros(nk * d)
    v[:vals.size] = vals
    v = v.reshape(1, 1, nk, d)
    qk = np.zeros((1, 1, nk, d), dtype=np.uint16)
    qk[..., 0] = 0x3f80  # 1.0
    q8, k8, v8t, descale = run_prepare(api, to_device(qk, "bf16"), to_device(qk, "bf16"),
                                       to_device(bf16_from_f64(v), "bf16"))
    assert descale[2] == 1.0
    codes = np.swapaxes(key_order(v8t)[..., :nk], 2, 3)
    ref = e4m3_encode_rne(v)
    zero = e4m3_decode(ref) == 0
    np.testing.assert_array_equal(np.where(zero, 0, codes), np.where(zero, 0, ref))
    # zeros may carry either sign bit, never another code
    assert np.isin(codes[zero], [0x00, 0x80]).all()


# ---------------------------------------------------------------- preparation
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("rotate", [False, True])
def test_prepare_matches_the_oracle(api, d, rotate):
    B, Hq, Hkv, Nq, Nk = 2, 4, 2, 100, 77
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, dtype="fp8", outlier_prob=0.01)
    x = gen.make_inputs(w, (d, int(rotate)))
    print(f"case: prepare {w.name} rotate={rotate}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    signs = torch.from_numpy(x["signs"]).cuda() if rotate else None
    ws = torch.full((3,), -1, dtype=torch.int32, device="cuda")
    ds = torch.empty(3, dtype=torch.float32, device="cuda")
    scale = 0.7 / np.sqrt(d)
    # a first call on 4x larger tensors leaves a larger amax in the workspace:
    # the second call must not see it
    run_prepare(api, q * 4, k * 4, v * 4, signs, ds, ws, scale)
    q8, k8, v8t, descale = run_prepare(api, q, k, v, signs, ds, ws, scale)
    qf, kf, vf = (bf16_bits_to_f64(x[t]) for t in "qkv")
    ref = ofp8.prepare(qf, kf, vf, x["signs"] if rotate else None, scale)
    # s_q and s_k are powers of two (equal unless the fp32 and fp64 amax
    # straddle one, which these inputs do not), s_v amax / 448
    for s in descale[:2]:
        assert np.frexp(s)[0] == 0.5, descale
    np.testing.assert_array_equal(descale[:2], ref["scales"][:2])
    np.testing.assert_allclose(descale[2], ref["scales"][2], rtol=2 ** -23)
    check_codes(q8, gpu_c0(scale) * ref["qr"], descale[0], "Q")
    check_codes(k8, ref["kr"], descale[1], "K")
    vk = key_order(v8t)
    check_codes(np.swapaxes(vk[..., :Nk], 2, 3), vf, descale[2], "V")
    assert (vk[..., Nk:] == 0).all(), "padding keys of V^T must be zero"


# ---------------------------------------------------------------- attention with exact probabilities
SHAPES = [
    # B, Hq, Hkv, Nq, Nk
    (2, 4, 2, 200, 333),     # several tiles, ragged tails, GQA 2
    (1, 8, 1, 130, 130),     # MQA
    (1, 6, 2, 257, 257),     # GQA 3
    (1, 3, 3, 1, 77),        # a single query
    (1, 2, 1, 70, 1),        # a single key
    (1, 2, 2, 150, 40),      # Nq > Nk: causal rows with no visible key
    (1, 4, 4, 64, 64),       # exactly one tile
]


def integer_logit_inputs(B, Hq, Hkv, Nq, Nk, d, seed):
    """Q, K with integer dot products spread over at most 8 per row, V on a
    scaled e4m3 grid; each tensor's largest magnitude is 7, so every scale
    is 7/448 = 2^-6 and the codes are 64 x the values.

    Q rows have four entries of +-1 in columns 1..d-1, K entries are in
    {-1, 0, 1}: q.k lies in [-4, 4].  Column 0 is zero except Q[0,0,Nq-1,0]
    = K[0,0,0,0] = 7, which makes key 0 dominate that one query row.  With
    scale = ln 2 every probability the kernel uses is 2^(integer) in
    [2^-8, 2^8] (masked keys 0; in the dominated row the other keys fall
    below the e4m3 range), exactly representable in e4m3.  The factor
    c0 = scale * log2(e) that the Q codes carry is 1 in fp32 for this scale,
    so the Q scale stays 2^-6.  All code products
    of Q K^T are multiples of 64 * 64, far above the granularity of the fp8
    MFMA's grouped sums, so the logits are exact.
    """
    rng = np.random.default_rng(seed)
    q = np.zeros((B, Hq, Nq, d))
    cols = np.argsort(rng.random((B, Hq, Nq, d - 1)), axis=-1)[..., :4] + 1
    np.put_along_axis(q, cols, rng.choice([-1.0, 1.0], size=cols.shape), axis=-1)
    k = rng.integers(-1, 2, size=(B, Hkv, Nk, d)).astype(np.float64)
    k[..., 0] = 0.0
    q[0, 0, Nq - 1, 0] = 7.0
    k[0, 0, 0, 0] = 7.0
    v = e4m3_decode(e4m3_encode_rne(64.0 * np.clip(rng.standard_normal((B, Hkv, Nk, d)), -6.5, 6.5))) / 64.0
    v[0, 0, 0, 0] = 7.0
    return q, k, v


# Many query blocks over a ragged key range: non-causal workgroups take their
# key tiles in an order rotated by their query block, so the partial last
# tile falls in the middle of most workgroups' loops.
ROTATED_SHAPES = [(1, 2, 2, 1024, 1000), (1, 4, 4, 2048, 2000)]


# gfx950's fp8 MFMA adds each group of 8 consecutive products of a lane with
# the bits below 2^(e-14) of every product dropped, e the exponent of the
# group's largest product: at most 8 * 2^-13 = 2^-10 of that product per group
MFMA_FP8_GROUP_REL = 2.0 ** -10


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_probabilities_elementwise(api, shape, d, causal):
    B, Hq, Hkv, Nq, Nk = shape
    print(f"case: exact-probability fp8 {shape} d={d} causal={causal}", flush=True)
    q, k, v = integer_logit_inputs(B, Hq, Hkv, Nq, Nk, d, (sum(shape), d, causal))
    scale = float(np.float32(np.log(2.0)))
    qd, kd, vd = (to_device(bf16_from_f64(t), "bf16") for t in (q, k, v))
    o, lse, prep = api.attention_fp8(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(prep["descale"].cpu().numpy(), [2.0 ** -6] * 3)
    o, lse = out_to_f64(o), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = attention_fp64(q, k, v, scale, causal)
    acc, _ = attention_fp64(q, k, np.abs(v), scale, causal)     # sum_j p_ij |v_jc|
    # bf16 rounding of O (2^-9 relative, doubled for the fp32 reciprocal), the
    # grouped sums of P V inside the MFMA, and the fp32 sums over at most
    # Nk + 64 terms of O and of l
    tol = 2.0 ** -8 * np.abs(o_ref) + (MFMA_FP8_GROUP_REL + 2 * (Nk + 64) * 2.0 ** -24) * acc
    err = np.abs(o - o_ref)
    assert (err <= tol).all(), f"max excess {(err - tol).max():.3e}, max |dO| {err.max():.3e}"
    inf_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), inf_ref)
    le = np.abs(lse[~inf_ref] - lse_ref[~inf_ref])
    assert (le <= 4e-7 * np.abs(lse_ref[~inf_ref]) + 1e-5).all(), f"max |dLSE| {le.max():.3e}"


@pytest.mark.parametrize("shape", ROTATED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_probabilities_rotated_key_order(api, shape):
    test_exact_probabilities_elementwise(api, shape, 128, False)


def test_fp8_mfma_group_sum_granularity(api):
    """The in-group precision the tolerance above assumes, seen through the
    LSE of single-key attention (one key: l = 1 and LSE = ln2 * q.k with
    scale = ln 2).  A product of 448 * 448 drops a product of magnitude
    below 2^(17-14) = 8 in the same group of 8, keeps one of 8, and keeps
    any product in another group exactly."""
    scale = float(np.float32(np.log(2.0)))

    def gpu_dot(qr, kr):
        d = qr.size
        q = np.zeros((1, 1, 1, d)); k = np.zeros((1, 1, 1, d)); v = np.zeros((1, 1, 1, d))
        q[0, 0, 0], k[0, 0, 0] = qr, kr
        v[0, 0, 0, 0] = 1.0
        _, lse, prep = api.attention_fp8(*(to_device(bf16_from_f64(t), "bf16") for t in (q, k, v)),
                                         causal=False, scale=scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(prep["descale"].cpu().numpy()[:2], [1.0, 1.0])
        return float(lse.cpu()[0, 0, 0]) / scale

    def case(small, col):
        qr, kr = np.zeros(64), np.zeros(64)
        qr[0], kr[0] = 448.0, 448.0
        qr[col], kr[col] = small, 1.0
        return gpu_dot(qr, kr) - (448.0 * 448.0 + small)

    assert abs(case(4.0, 1) + 4.0) < 0.05       # dropped
    assert abs(case(-4.0, 1) - 4.0) < 0.05      # dropped (either sign)
    assert abs(case(8.0, 1)) < 0.05             # kept
    assert abs(case(1.0, 8)) < 0.05             # another group: kept


# ---------------------------------------------------------------- random inputs
def score_error_bound(q, k, scale):
    """Per query row, a bound on |S_gpu - S| over its keys from the grouped
    sums of the fp8 MFMA: at most MFMA_FP8_GROUP_REL of the largest product
    of every group of 8 consecutive channels (q, k: the dequantised
    operands, [B, H, N, d] and [B, Hkv, Nk, d])."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            kk = np.abs(k[b, h // (Hq // Hkv)]).reshape(-1, d // 8, 8)
            for i0 in range(0, Nq, 64):
                qq = np.abs(q[b, h, i0:i0 + 64]).reshape(-1, 1, d // 8, 8)
                out[b, h, i0:i0 + 64] = (qq * kk[None]).max(axis=-1).sum(axis=-1).max(axis=-1)
    return MFMA_FP8_GROUP_REL * scale * out


def check_lse_against_dequantised(lse, lse_q, bound, what):
    """The LSE comes from fp32 probabilities, so against the oracle on the
    dequantised codes it differs only by the score errors (the LSE moves at
    most by the largest score error of its row) and fp32 rounding."""
    inf_ref = np.isneginf(lse_q)
    np.testing.assert_array_equal(np.isneginf(lse), inf_ref, err_msg=what)
    ok = ~inf_ref
    le = np.abs(lse[ok] - lse_q[ok])
    tol = 1e-5 + 2e-6 * np.abs(lse_q[ok]) + bound[ok]
    assert (le <= tol).all(), f"{what}: max |dLSE| {le.max():.3e}, max excess {(le - tol).max():.3e}"


def run_fp8(api, x, w, rotate):
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    signs = torch.from_numpy(x["signs"]).cuda() if rotate else None
    o, lse, prep = api.attention_fp8(q, k, v, causal=w.causal, scale=w.softmax_scale, signs=signs)
    torch.cuda.synchronize()
    deq = dequantise_gpu(prep["q8"].cpu().numpy(), prep["k8"].cpu().numpy(), prep["v8t"].cpu().numpy(),
                         prep["descale"].cpu().numpy().astype(np.float64), w.Nk, w.softmax_scale)
    return out_to_f64(o), lse.cpu().numpy().astype(np.float64), deq


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_inputs_against_the_oracle(api, shape, d, causal):
    B, Hq, Hkv, Nq, Nk = shape
    w = gen.workload(B, Hq, Hkv, Nq, Nk, d, dtype="fp8", causal=causal)
    x = gen.make_inputs(w, (sum(shape), d, int(causal), 8))
    print(f"case: fp8 {w.name}", flush=True)
    o, lse, (qq, kq, vq) = run_fp8(api, x, w, rotate=True)
    assert np.isfinite(o).all()
    qf, kf, vf = (bf16_bits_to_f64(x[t]) for t in "qkv")
    o_true, _ = attention_fp64(qf, kf, vf, w.softmax_scale, causal)
    c = cosine(o, o_true)
    assert c >= FP8_COSINE, f"cosine {c:.5f}"
    o_q, lse_q = attention_fp64(qq, kq, vq, w.softmax_scale, causal)
    check_lse_against_dequantised(lse, lse_q, score_error_bound(qq, kq, w.softmax_scale), w.name)
    cq = cosine(o, o_q)
    assert cq >= 0.999, f"cosine against the dequantised oracle {cq:.6f}"


FP8_PERSISTENT = [
    # B, Hq, Hkv, N, d, causal: more work items than the persistent grid holds
    (4, 16, 16, 2050, 128, True),    # two workgroups per CU, items not a multiple of the grid
    (3, 12, 4, 4000, 64, True),
    (2, 16, 8, 2000, 256, True),     # one workgroup per CU
    (2, 16, 16, 2000, 256, False),
]


@pytest.mark.parametrize("case", FP8_PERSISTENT, ids=lambda c: "x".join(map(str, c)))
def test_persistent_grid_covers_every_row(api, case):
    """The causal 4-wave fp8 kernels and the non-causal d = 256 one run grids
    with more work items than fit the GPU at once as persistent workgroups
    taking items in rounds.  O and LSE start as NaN and must be written
    everywhere; sampled rows (block ends, the tail, random) match the oracle
    on the dequantised codes (cosine, and the LSE within the per-row bound)."""
    B, Hq, Hkv, n, d, causal = case
    w = gen.workload(B, Hq, Hkv, n, n, d, dtype="fp8", causal=causal)
    x = gen.make_inputs(w, (n, d, int(causal), 78))
    print(f"case: fp8 persistent grid {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    o, lse, prep = api.attention_fp8(q, k, v, causal=causal, scale=w.softmax_scale)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    api.fa_fwd_fp8(prep["q8"], prep["k8"], prep["v8t"], prep["descale"], o, lse, causal)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), "rows left unwritten"
    of, lf = out_to_f64(o), lse.cpu().numpy().astype(np.float64)
    qq, kq, vq = dequantise_gpu(prep["q8"].cpu().numpy(), prep["k8"].cpu().numpy(), prep["v8t"].cpu().numpy(),
                                prep["descale"].cpu().numpy().astype(np.float64), n, w.softmax_scale)
    rng = np.random.default_rng(n)
    rows = [(0, 0, 0), (B - 1, Hq - 1, n - 1), (0, Hq - 1, 127), (B - 1, 0, 128), (0, 1, n - 2)]
    rows += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(n))) for _ in range(35)]
    o_q, lse_q = attention_rows_fp64(qq, kq, vq, w.softmax_scale, causal, rows)
    got = np.stack([of[b, h, i] for b, h, i in rows])
    assert cosine(got, o_q) >= 0.999, cosine(got, o_q)
    g = Hq // Hkv
    bound = np.array([score_error_bound(qq[b:b + 1, h:h + 1, i:i + 1], kq[b:b + 1, h // g:h // g + 1],
                                        w.softmax_scale)[0, 0, 0] for b, h, i in rows])
    check_lse_against_dequantised(np.array([lf[b, h, i] for b, h, i in rows]), lse_q, bound, w.name)


def fp8_errors(o, o_true):
    err = o - o_true
    return dict(cos=cosine(o, o_true), rmse=float(np.sqrt((err ** 2).mean())), maxabs=float(np.abs(err).max()))


def test_outliers_rotated_and_unrotated(api):
    """Q and K with +-50 outliers (p = 0.001), 4 heads of 2048 queries: both
    runs against the fp64 oracle on the bf16 source, errors printed; the
    rotated run meets the cosine bar."""
    w = gen.workload(1, 4, 4, 2048, 2048, 128, dtype="fp8", outlier_prob=0.001)
    x = gen.make_inputs(w, (2048, 128, 5))
    print(f"case: fp8 {w.name}", flush=True)
    qf, kf, vf = (bf16_bits_to_f64(x[t]) for t in "qkv")
    o_true, _ = attention_fp64(qf, kf, vf, w.softmax_scale, False)
    rep = {}
    for rotate in (True, False):
        o, lse, (qq, kq, vq) = run_fp8(api, x, w, rotate)
        rep[rotate] = fp8_errors(o, o_true)
        _, lse_q = attention_fp64(qq, kq, vq, w.softmax_scale, False)
        check_lse_against_dequantised(lse, lse_q, score_error_bound(qq, kq, w.softmax_scale),
                                      f"rotate={rotate}")
    for rotate, r in rep.items():
        print(f"fp8 {'rotated' if rotate else 'unrotated'}: cosine {r['cos']:.6f} rmse {r['rmse']:.3e} "
              f"max|err| {r['maxabs']:.3e}", flush=True)
    assert rep[True]["cos"] >= FP8_COSINE


def test_fp8_deterministic_and_writes_stay_inside_outputs(api):
    w = gen.workload(1, 2, 1, 77, 50, 128, dtype="fp8", causal=True)
    x = gen.make_inputs(w, (3,))
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    _, _, prep = api.attention_fp8(q, k, v, causal=True)
    n = q.numel()
    outs = []
    for _ in range(2):
        buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
        lbuf = torch.full((2 * 77 + 64,), 7.0, dtype=torch.float32, device="cuda")
        o = buf[:n].view(q.shape)
        lse = lbuf[:2 * 77].view(1, 2, 77)
        api.fa_fwd_fp8(prep["q8"], prep["k8"], prep["v8t"], prep["descale"], o, lse, True)
        torch.cuda.synchronize()
        assert (buf[n:] == 7.0).all() and (lbuf[2 * 77:] == 7.0).all()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- the fp8 workload at full size
def test_fp8_workload_sampled_rows(api):
    w, x = gen.make_config(5)
    print(f"case: {w.name}", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    signs = torch.from_numpy(x["signs"]).cuda()
    qf, kf, vf = (bf16_bits_to_f64(x[t]) for t in "qkv")
    rng = np.random.default_rng(5)
    rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.Nq - 1), (1, 7, w.Nq // 2)]
    rows += [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Nq))) for _ in range(45)]
    o_true, _ = attention_rows_fp64(qf, kf, vf, w.softmax_scale, False, rows)
    del qf, kf, vf
    report = {}
    for rotate in (True, False):
        o, lse, prep = api.attention_fp8(q, k, v, causal=False, scale=w.softmax_scale,
                                         signs=signs if rotate else None)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all()
        got = np.stack([out_to_f64(o[b, h, i]) for b, h, i in rows])
        got_l = np.array([float(lse[b, h, i]) for b, h, i in rows])
        report[rotate] = fp8_errors(got, o_true)
        # LSE against the oracle on the dequantised codes of the sampled rows
        qq, kq, vq = dequantise_gpu(prep["q8"].cpu().numpy(), prep["k8"].cpu().numpy(), prep["v8t"].cpu().numpy(),
                                    prep["descale"].cpu().numpy().astype(np.float64), w.Nk, w.softmax_scale)
        _, lse_q = attention_rows_fp64(qq, kq, vq, w.softmax_scale, False, rows)
        g = w.Hq // w.Hkv
        bound = np.array([score_error_bound(qq[b:b + 1, h:h + 1, i:i + 1], kq[b:b + 1, h // g:h // g + 1],
                                            w.softmax_scale)[0, 0, 0] for b, h, i in rows])
        report[rotate]["lse"] = (got_l, lse_q, bound)
        del o, lse, prep, qq, kq, vq
    for rotate, r in report.items():
        print(f"fp8 {'rotated' if rotate else 'unrotated'}: cosine {r['cos']:.6f} rmse {r['rmse']:.3e} "
              f"max|err| {r['maxabs']:.3e}", flush=True)
    print(f"rmse ratio unrotated/rotated: {report[False]['rmse'] / report[True]['rmse']:.3f}", flush=True)
    for rotate, r in report.items():
        check_lse_against_dequantised(*r["lse"], f"rotate={rotate}")
    assert report[True]["cos"] >= FP8_COSINE


def test_fp8_workload_every_element(api):
    """The fp8 workload's whole output, rotated and unrotated, on every
    element against two fp64 oracles: on the unquantised bf16 source (the
    accuracy of the fp8 path: cosine, RMSE, max |error|) and on exactly the
    e4m3 values the GPU consumed (the kernel's own error).

    Bars: the kernel's output against the oracle on its own dequantised
    inputs has cosine >= 0.999; against the source, the unrotated run meets
    the fp8 accuracy bar (cosine >= 0.99) and each run loses at most 3e-4 of
    cosine beyond what the e4m3 inputs alone lose (the exact attention of
    the dequantised Q, K, V).  On this input the rotated run's e4m3 inputs
    alone reach only about 0.9899, below 0.99: its outliers are exactly +-50,
    the per-tensor amax, which e4m3 represents exactly unrotated while the
    rotation spreads them into inexact values; that is a property of the
    format on this data, not of the kernel, and is reported, not asserted.
    The oracle runs one (b, h) head per task over the host's cores."""
    from tests.full_compare import compare_fp8_all_heads, pool_size
    w, x = gen.make_config(5)
    print(f"case: {w.name} (every element, {pool_size()} host workers)", flush=True)
    q, k, v = (to_device(x[t], "bf16") for t in "qkv")
    signs = torch.from_numpy(x["signs"]).cuda()
    runs = {}
    for rotate in (True, False):
        o, lse, prep = api.attention_fp8(q, k, v, causal=False, scale=w.softmax_scale,
                                         signs=signs if rotate else None)
        torch.cuda.synchronize()
        v8 = np.ascontiguousarray(np.swapaxes(key_order(prep["v8t"].cpu().numpy())[..., :w.Nk], 2, 3))
        runs["rotated" if rotate else "unrotated"] = (
            o.view(torch.int16).cpu().numpy().view(np.uint16), prep["q8"].cpu().numpy(), prep["k8"].cpu().numpy(),
            v8, prep["descale"].cpu().numpy().astype(np.float64) / [gpu_c0(w.softmax_scale), 1.0, 1.0])
        del o, lse, prep
    del q, k, v
    st = compare_fp8_all_heads(x["q"], x["k"], x["v"], w.softmax_scale, runs)
    for nm, r in st.items():
        for key, what in (("gpu_true", "GPU vs source oracle"), ("deq_true", "e4m3 inputs alone"),
                          ("gpu_deq", "GPU vs dequantised oracle")):
            a = r[key]
            print(f"fp8 {nm}, {what}: cosine {a['cosine']:.6f} rmse {a['rmse']:.4e} max|err| {a['max_abs']:.4e} "
                  f"mean|err| {a['mean_abs']:.4e}", flush=True)
    print(f"rmse ratio unrotated/rotated (GPU vs source): "
          f"{st['unrotated']['gpu_true']['rmse'] / st['rotated']['gpu_true']['rmse']:.4f}", flush=True)
    for nm, r in st.items():
        assert r["gpu_true"]["nonfinite"] == 0, nm
        assert r["gpu_deq"]["cosine"] >= 0.999, (nm, r["gpu_deq"])
        assert r["gpu_true"]["cosine"] >= r["deq_true"]["cosine"] - 3e-4, (nm, r)
    assert st["unrotated"]["gpu_true"]["cosine"] >= FP8_COSINE, st["unrotated"]
