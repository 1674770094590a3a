"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Every check below comes from the definition's mathematics (closed forms,
invariants, special cases), from hand-derived worked examples under
tests/golden/, from brute force written differently (pure Python, no max
shift), or from an independent library implementation (torch's float8 and
bfloat16 conversions).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_backward_fp64, attention_fp64, attention_keys_fp64, attention_rows_fp64, merge_fp64,
                    online_fp64, formats, fp8)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- worked examples
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    o_ref = np.array(case["o"], dtype=np.float64)
    lse_ref = np.array([[[float(x) for x in h] for h in b] for b in case["lse"]])
    o, lse = attention_fp64(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)
    o2, lse2, _ = online_fp64(q, k, v, case["scale"], case["causal"], bc=1, tau=0.0)
    np.testing.assert_allclose(o2, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse_ref, rtol=0, atol=1e-14)
    B, H, N, _ = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(N)]
    o3, lse3 = attention_rows_fp64(q, k, v, case["scale"], case["causal"], rows)
    np.testing.assert_allclose(o3, o_ref.reshape(-1, o_ref.shape[-1]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse3, lse_ref.reshape(-1), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, scale, causal):
    """Pure-Python softmax attention: exp without max shift, explicit sums."""
    B, HQ, NQ, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    HKV, NK = len(k[0]), len(k[0][0])
    o = [[[[0.0] * D for _ in range(NQ)] for _ in range(HQ)] for _ in range(B)]
    lse = [[[-math.inf] * NQ for _ in range(HQ)] for _ in range(B)]
    for b in range(B):
        for h in range(HQ):
            g = h * HKV // HQ          # query head h belongs to the (h*Hkv/Hq)-th key/value group
            for i in range(NQ):
                w = []
                for j in range(NK):
                    if causal and j - (NK - NQ) > i:
                        continue
                    dot = 0.0
                    for t in range(D):
                        dot += q[b][h][i][t] * k[b][g][j][t]
                    w.append((j, math.exp(scale * dot)))
                if not w:
                    continue
                z = sum(x for _, x in w)
                lse[b][h][i] = math.log(z)
                for t in range(D):
                    o[b][h][i][t] = sum(x * v[b][g][j][t] for j, x in w) / z
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 5, 7, 3), (2, 4, 2, 6, 6, 4), (1, 3, 1, 8, 5, 8), (1, 2, 2, 3, 8, 2), (2, 6, 3, 7, 7, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(shape, causal):
    B, HQ, HKV, NQ, NK, D = shape
    rng = np.random.default_rng(sum(shape) + causal)
    q, k, v = _rand(rng, B, HQ, NQ, D), _rand(rng, B, HKV, NK, D), _rand(rng, B, HKV, NK, D)
    scale = 0.7
    o_b, lse_b = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    o, lse = attention_fp64(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lse_b))
    fin = np.isfinite(lse_b)
    np.testing.assert_allclose(lse[fin], lse_b[fin], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_its_value_row():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 2, 3, 9, 16), _rand(rng, 2, 3, 1, 16), _rand(rng, 2, 3, 1, 16)
    o, lse = attention_fp64(q, k, v, 0.25, False)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    np.testing.assert_allclose(lse, 0.25 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), rtol=1e-14, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    nk = 13
    q, v = _rand(rng, 1, 2, 5, 8), _rand(rng, 1, 2, nk, 8)
    k = np.repeat(_rand(rng, 1, 2, 1, 8), nk, axis=2)
    o, lse = attention_fp64(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]) + math.log(nk), atol=1e-13)


def test_rows_of_p_sum_to_one_and_are_nonnegative():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 11, 8), _rand(rng, 1, 1, 17, 8), _rand(rng, 1, 1, 17, 8)
    for causal in (False, True):
        _, _, ps = attention_fp64(q * 3, k * 3, v, 0.3, causal, return_p=True)
        for p in ps:
            assert (p >= 0).all()
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15 * 17)


def test_constant_logit_shift_leaves_output_and_shifts_lse():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4)
    scale, shift = 0.8, 3.25
    q2 = np.concatenate([q, np.full((1, 1, 6, 1), shift / scale)], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, 9, 1))], axis=-1)
    o1, l1 = attention_fp64(q, k, v, scale, False)
    o2, l2 = attention_fp64(q2, k2, v, scale, False)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + shift, atol=1e-13)


def test_dominant_logit_selects_one_value_row():
    rng = np.random.default_rng(5)
    nk, d = 10, 8
    q, k, v = _rand(rng, 1, 1, 1, d), _rand(rng, 1, 1, nk, d), _rand(rng, 1, 1, nk, d)
    jstar = 6
    k[0, 0, jstar] = 60.0 * q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0])   # q.k_j* = 60
    k[0, 0, np.arange(nk) != jstar] *= 0.1
    s = (k[0, 0] @ q[0, 0, 0])
    gap = s[jstar] - np.max(np.delete(s, jstar))
    assert gap >= 50
    o, _ = attention_fp64(q, k, v, 1.0, False)
    bound = 2 * (nk - 1) * math.exp(-gap) * np.abs(v).max()
    assert np.abs(o[0, 0, 0] - v[0, 0, jstar]).max() <= bound + 1e-15


def test_linear_in_v_and_constant_v():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 2, 7, 8), _rand(rng, 1, 2, 12, 8), _rand(rng, 1, 2, 12, 8)
    for causal in (False, True):
        o, _ = attention_fp64(q, k, v, 0.4, causal)
        o2, _ = attention_fp64(q, k, -2.5 * v + 1.75, 0.4, causal)
        np.testing.assert_allclose(o2, -2.5 * o + 1.75, atol=1e-13)
        o1, _ = attention_fp64(q, k, np.ones_like(v), 0.4, causal)
        np.testing.assert_allclose(o1, 1.0, atol=1e-15)


def test_causal_first_row_is_first_value_row():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 2, 2, 9, 8), _rand(rng, 2, 2, 9, 8), _rand(rng, 2, 2, 9, 8)
    o, lse = attention_fp64(q, k, v, 0.35, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.35 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)
    # row i equals non-causal attention over keys 0..i
    for i in (1, 4, 8):
        oi, li = attention_fp64(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.35, False)
        np.testing.assert_allclose(o[:, :, i:i + 1], oi, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i:i + 1], li, atol=1e-14)


def test_one_by_one_causal_equals_noncausal():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 1, 4), _rand(rng, 1, 1, 1, 4)
    a = attention_fp64(q, k, v, 1.0, True)
    b = attention_fp64(q, k, v, 1.0, False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (6, 3)])
def test_gqa_equals_mha_with_repeated_kv_heads(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    q, k, v = _rand(rng, 2, hq, 5, 8), _rand(rng, 2, hkv, 7, 8), _rand(rng, 2, hkv, 7, 8)
    g = hq // hkv
    for causal in (False, True):
        o, lse = attention_fp64(q, k, v, 0.5, causal)
        o2, lse2 = attention_fp64(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.5, causal)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)


def test_rows_variant_matches_full_on_ragged_sample():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 2, 4, 19, 8), _rand(rng, 2, 2, 23, 8), _rand(rng, 2, 2, 23, 8)
    for causal in (False, True):
        o, lse = attention_fp64(q, k, v, 0.3, causal)
        rows = [(1, 3, 18), (0, 0, 0), (0, 2, 7), (1, 1, 11)]
        o2, lse2 = attention_rows_fp64(q, k, v, 0.3, causal, rows)
        for r, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(o2[r], o[b, h, i], atol=1e-14)
            np.testing.assert_allclose(lse2[r], lse[b, h, i], atol=1e-14)


# ---------------------------------------------------------------- online softmax (exactness claim)
@pytest.mark.parametrize("bc", [1, 3, 16])
@pytest.mark.parametrize("tau", [0.0, 8.0, 1e9])
@pytest.mark.parametrize("group", [1, 4])
def test_online_equals_two_pass(bc, tau, group):
    rng = np.random.default_rng(bc * 100 + int(min(tau, 99)) + group)
    B, HQ, HKV, NQ, NK, D = 1, 4, 2, 9, 21, 8
    q, k, v = _rand(rng, B, HQ, NQ, D), _rand(rng, B, HKV, NK, D), _rand(rng, B, HKV, NK, D)
    # logits that keep increasing along the keys force the running maximum to move
    k = k + (np.arange(NK)[None, None, :, None] * 0.9) * np.sign(q.mean(axis=(1, 2)))[:, None, None, :]
    for causal in (False, True):
        for nq in (NQ, 4):            # nq < nk exercises bottom-right alignment
            o, lse = attention_fp64(q[:, :, :nq], k, v, 0.6, causal)
            o2, lse2, _ = online_fp64(q[:, :, :nq], k, v, 0.6, causal, bc=bc, tau=tau, group=group)
            np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_online_fully_masked_rows():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 1, 1, 7, 4), _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 3, 4)
    o, lse = attention_fp64(q, k, v, 1.0, True)
    o2, lse2, _ = online_fp64(q, k, v, 1.0, True, bc=2, tau=8.0, group=4)
    assert np.isneginf(lse[0, 0, :4]).all() and (o[0, 0, :4] == 0).all()
    np.testing.assert_array_equal(np.isneginf(lse2), np.isneginf(lse))
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2[np.isfinite(lse)], lse[np.isfinite(lse)], atol=1e-13)


def test_online_rescale_counts():
    # one query, keys whose logits grow by 1 (log2 units) per key: block maxima grow each block
    nk = 16
    q = np.ones((1, 1, 1, 1))
    k = (np.arange(nk, dtype=np.float64) * math.log(2.0)).reshape(1, 1, nk, 1)
    v = np.ones((1, 1, nk, 1))
    _, _, (ev0, dec0) = online_fp64(q, k, v, 1.0, False, bc=2, tau=0.0)
    assert (ev0, dec0) == (7, 7)           # every block after the first rescales
    _, _, (ev8, dec8) = online_fp64(q, k, v, 1.0, False, bc=2, tau=8.0)
    assert dec8 == 7 and ev8 == 1          # growth passes 8 only once (at key 9, then m_ref=9 and 15-9 <= 8)
    _, _, (evi, _) = online_fp64(q, k, v, 1.0, False, bc=2, tau=1e9)
    assert evi == 0


# ---------------------------------------------------------------- number formats
def test_bf16_decode_known_patterns():
    got = formats.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3EAA], dtype=np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.0 and np.signbit(got[3]) and np.isposinf(got[4])
    assert got[5] == 0.33203125


def test_e4m3_known_codes():
    t = formats.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x07] == 7 * 2.0 ** -9 and t[0x01] == 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and t[0x00] == 0.0 and t[0x80] == 0.0
    assert t[0x40] == 2.0 and t[0x44] == 3.0 and t[0x30] == 0.5
    finite = t[:0x7F]
    assert (np.diff(finite) > 0).all()       # codes 0x00..0x7E are strictly increasing


def test_e4m3_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = formats.e4m3_decode(codes)
    back = formats.e4m3_encode_rne(vals)
    np.testing.assert_array_equal(back[codes != 0x80], codes[codes != 0x80])
    pos = formats.e4m3_decode_table()[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    enc = formats.e4m3_encode_rne(mids)
    assert (enc % 2 == 0).all()              # ties go to the even code
    assert formats.e4m3_encode_rne(np.array([1e6, -500.0]))[0] == 0x7E


def test_e4m3_matches_torch_float8():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(20000) * 0.01,
                        (formats.e4m3_decode_table()[:0x7E] + formats.e4m3_decode_table()[1:0x7F]) / 2])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.e4m3_encode_rne(x)
    same = (got == ref) | ((got & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all()


# ---------------------------------------------------------------- Hadamard rotation (FlashAttention-3 FP8 step)
@pytest.mark.parametrize("d", [1, 2, 8, 64, 128, 256])
def test_sylvester_hadamard_is_orthogonal_in_integers(d):
    h = fp8.sylvester_hadamard(d)
    assert set(np.unique(h)) <= {-1, 1}
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))


def test_rotation_leaves_qk_and_attention_unchanged():
    rng = np.random.default_rng(12)
    d = 64
    signs = rng.integers(0, 2, d) * 2 - 1.0
    m = fp8.rotation(signs)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-15)
    q, k, v = _rand(rng, 1, 2, 6, d), _rand(rng, 1, 2, 9, d), _rand(rng, 1, 2, 9, d)
    np.testing.assert_allclose((q @ m) @ np.swapaxes(k @ m, 2, 3), q @ np.swapaxes(k, 2, 3), rtol=1e-12, atol=1e-12)
    o1, l1 = attention_fp64(q, k, v, 0.125, False)
    o2, l2 = attention_fp64(q @ m, k @ m, v, 0.125, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_rotation_spreads_an_outlier_channel():
    d = 128
    x = np.zeros((1, d)); x[0, 5] = 50.0
    y = x @ fp8.rotation(np.ones(d))
    np.testing.assert_allclose(np.abs(y), 50.0 / math.sqrt(d), rtol=1e-14)


def test_quantise_per_tensor():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 5, 7)) * 4
    codes, s = fp8.quantise(x)
    deq = formats.e4m3_decode(codes) * s
    assert abs(np.abs(deq).max() - np.abs(x).max()) <= 1e-12 * np.abs(x).max()
    # |x/s - decode(code)| is at most half a code step of the decoded magnitude's binade
    r = x / s
    step = np.where(np.abs(r) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -6))) - 3))
    assert (np.abs(r - formats.e4m3_decode(codes)) <= step / 2 + 1e-12).all()
    z, s0 = fp8.quantise(np.zeros(4))
    assert s0 == 1.0 and (formats.e4m3_decode(z) == 0).all()


@pytest.mark.parametrize("amax", [448.0, 447.0, 449.0, 1.0, 3.5, 2.0 ** -20, 7e5])
def test_quantise_power_of_two_scale(amax):
    # the scale is a power of two s with amax / s in (224, 448]; a tensor whose
    # amax is 448 times a power of two gets exactly that power
    x = np.array([0.25 * amax, -amax, 0.0])
    codes, s = fp8.quantise(x, pow2=True)
    m, e = math.frexp(s)
    assert m == 0.5
    assert 224.0 < amax / s <= 448.0
    if amax == 448.0:
        assert s == 1.0
    deq = formats.e4m3_decode(codes) * s
    assert abs(deq[1] + amax) <= amax * 2.0 ** -4   # within half a step of the top binade
    assert deq[2] == 0.0


def test_prepare_layouts_and_product():
    rng = np.random.default_rng(14)
    d = 16
    q, k, v = _rand(rng, 1, 2, 5, d), _rand(rng, 1, 1, 6, d), _rand(rng, 1, 1, 6, d)
    signs = rng.integers(0, 2, d) * 2 - 1.0
    p = fp8.prepare(q, k, v, signs, scale=0.3)
    assert p["q8"].shape == q.shape and p["k8"].shape == k.shape and p["v8t"].shape == (1, 1, d, 6)
    assert abs(p["c0"] - 0.3 / math.log(2.0)) <= 1e-15
    # the query codes carry c0: decode(q8) * s_q approximates c0 * (rotated Q)
    qc = formats.e4m3_decode(p["q8"]) * p["scales"][0]
    assert np.abs(qc - p["c0"] * p["qr"]).max() <= p["c0"] * np.abs(p["qr"]).max() / 16
    qd, kd, vd = fp8.dequantised(p)
    assert vd.shape == v.shape
    # quantised rotated product approximates the unrotated product
    exact = q[0, 0] @ k[0, 0].T
    approx = qd[0, 0] @ kd[0, 0].T
    assert np.abs(approx - exact).max() < 0.25 * np.abs(exact).max()
    assert np.abs(vd - v).max() <= np.abs(v).max() / 16


# ---------------------------------------------------------------- attention split over key ranges
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,cuts", [(7, 19, (0, 5, 6, 19)), (12, 12, (0, 4, 8, 12)), (20, 9, (0, 3, 9)),
                                        (1, 33, (0, 11, 22, 33)), (5, 40, (0, 40))])
def test_merge_of_key_ranges_equals_full_attention(causal, nq, nk, cuts):
    rng = np.random.default_rng(nq * 100 + nk)
    q = rng.standard_normal((2, 4, nq, 8)) * 2
    k = rng.standard_normal((2, 2, nk, 8))
    v = rng.standard_normal((2, 2, nk, 5))
    o, lse = attention_fp64(q, k, v, 0.4, causal)
    parts = [attention_keys_fp64(q, k, v, 0.4, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = merge_fp64([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_array_equal(np.isneginf(lm), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lm[fin], lse[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
    # the merge does not depend on the order of the parts
    om2, lm2 = merge_fp64([p[0] for p in parts[::-1]], [p[1] for p in parts[::-1]])
    np.testing.assert_allclose(om2, om, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lm2), np.isneginf(lm))


def test_merge_closed_forms():
    o1 = np.array([[1.0, 2.0]]); o2 = np.array([[3.0, -2.0]])
    # equal weights: the mean, lse + ln 2
    o, l = merge_fp64([o1, o2], [np.array([0.5]), np.array([0.5])])
    np.testing.assert_allclose(o, [[2.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(l, [0.5 + math.log(2.0)], atol=1e-15)
    # weights e^1 : e^0
    o, l = merge_fp64([o1, o2], [np.array([1.0]), np.array([0.0])])
    w = math.e / (math.e + 1.0)
    np.testing.assert_allclose(o, w * o1 + (1 - w) * o2, atol=1e-15)
    np.testing.assert_allclose(l, [math.log(math.e + 1.0)], atol=1e-15)
    # a part that saw no key does not count; all empty -> 0, -inf
    o, l = merge_fp64([o1, np.zeros_like(o1)], [np.array([0.25]), np.array([-np.inf])])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(l, [0.25], atol=1e-15)
    o, l = merge_fp64([np.zeros_like(o1)] * 3, [np.array([-np.inf])] * 3)
    assert (o == 0).all() and np.isneginf(l).all()


def test_key_range_single_key_is_its_value_row():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 4, 6)); k = rng.standard_normal((1, 1, 10, 6)); v = rng.standard_normal((1, 1, 10, 6))
    o, l = attention_keys_fp64(q, k, v, 0.3, False, 7, 8)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 7], (4, 6)), atol=1e-15)
    np.testing.assert_allclose(l[0, 0], 0.3 * (q[0, 0] @ k[0, 0, 7]), atol=1e-14)


# ---------------------------------------------------------------- gradients
def _loss(q, k, v, do, scale, causal):
    o, _ = attention_fp64(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 7, 4), (2, 4, 2, 6, 6, 3), (1, 3, 3, 7, 4, 5)],
                         ids=["mha", "gqa", "nq_gt_nk"])
def test_backward_matches_finite_differences(shape, causal):
    B, HQ, HKV, NQ, NK, D = shape
    rng = np.random.default_rng(sum(shape) + 7 * causal)
    q = rng.standard_normal((B, HQ, NQ, D))
    k = rng.standard_normal((B, HKV, NK, D))
    v = rng.standard_normal((B, HKV, NK, D))
    do = rng.standard_normal((B, HQ, NQ, D))
    scale = 0.7
    dq, dk, dv = attention_backward_fp64(q, k, v, do, scale, causal)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7, err_msg=f"d{name}")


def test_backward_single_key_and_delta_identity():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 2, 5, 4)); k = rng.standard_normal((1, 1, 1, 4)); v = rng.standard_normal((1, 1, 1, 4))
    do = rng.standard_normal((1, 2, 5, 4))
    dq, dk, dv = attention_backward_fp64(q, k, v, do, 0.5, False)
    # one key: P = 1 everywhere, so the scores do not matter and dV is the sum of dO over all rows and heads
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0, 0], do.sum(axis=(0, 1, 2)), atol=1e-13)
    # D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic (used by the kernels): rows of dS sum to zero
    q = rng.standard_normal((1, 1, 6, 3)); k = rng.standard_normal((1, 1, 9, 3)); v = rng.standard_normal((1, 1, 9, 3))
    do = rng.standard_normal((1, 1, 6, 3))
    dq, dk, dv = attention_backward_fp64(q, k, v, do, 0.9, True)
    o, _ = attention_fp64(q, k, v, 0.9, True)
    p_list = attention_fp64(q, k, v, 0.9, True, return_p=True)[2]
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((p_list[0] * dp).sum(axis=1), (do[0, 0] * o[0, 0]).sum(axis=1), atol=1e-13)


def test_backward_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 6, 3)); k = rng.standard_normal((2, 2, 8, 3)); v = rng.standard_normal((2, 2, 8, 3))
    do = rng.standard_normal((2, 4, 6, 3))
    dq, dk, dv = attention_backward_fp64(q, k, v, do, 0.6, True)
    dq2, dk2, dv2 = attention_backward_fp64(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), do, 0.6, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 2, 8, 3).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 2, 8, 3).sum(axis=2), atol=1e-13)
