"""The seeded input generator: determinism, encodings and the workload structure."""
import numpy as np
import pytest

from exact_attention_07_amd import gen


def test_bf16_encoder_matches_torch_and_ties():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    hi = rng.integers(0, 1 << 16, size=50000, dtype=np.uint32)
    ties = (hi << 16) | 0x8000                  # exactly halfway between two bf16 values
    rand = rng.integers(0, 1 << 32, size=50000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([ties, rand, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gen.f32_to_bf16_bits(x), ref)


def test_seeded_and_distinct():
    w = gen.workload(1, 2, 1, 33, 47, 64)
    a = gen.make_inputs(w, (5,))
    b = gen.make_inputs(w, (5,))
    c = gen.make_inputs(w, (6,))
    for t in ("q", "k", "v"):
        np.testing.assert_array_equal(a[t], b[t])
        assert not np.array_equal(a[t], c[t])
    assert not np.array_equal(a["k"], a["v"])
    assert a["q"].shape == (1, 2, 33, 64) and a["k"].shape == (1, 1, 47, 64) and a["q"].dtype == np.uint16


def test_standing_workloads_shapes_and_flops():
    w3 = gen.CONFIGS[3]
    assert (w3.B, w3.Hq, w3.Hkv, w3.Nq, w3.Nk, w3.d, w3.causal) == (2, 32, 8, 8192, 8192, 128, True)
    assert w3.flops() == 4 * 2 * 32 * 8192 * 8192 * 128 / 2
    assert gen.CONFIGS[1].softmax_scale == 1 / 8 and gen.CONFIGS[1].dtype == "f32"
    w1, x1 = gen.make_config(1)
    assert x1["q"].dtype == np.float32 and x1["q"].shape == (1, 1, 128, 64)
    assert abs(float(x1["q"].std()) - 1) < 0.05


def test_outlier_channels_shared_by_q_and_k():
    w = gen.workload(1, 2, 2, 64, 64, 256, outlier_channel_frac=0.005)
    x = gen.make_inputs(w, (4,))
    ch = x["outlier_channels"]
    assert len(ch) == 1
    q = (x["q"].astype(np.uint32) << 16).view(np.float32)
    k = (x["k"].astype(np.uint32) << 16).view(np.float32)
    other = [c for c in range(256) if c != ch[0]]
    for t in (q, k):
        assert 5 < np.abs(t[..., ch[0]]).mean() / np.abs(t[..., other]).mean() < 11


def test_fp8_outliers_and_signs():
    w = gen.workload(1, 2, 2, 512, 512, 128, dtype="fp8", outlier_prob=0.001)
    x = gen.make_inputs(w, (3,))
    q = (x["q"].astype(np.uint32) << 16).view(np.float32)
    n = np.count_nonzero(np.abs(q) == 50.0)
    expect = q.size * 0.001
    assert abs(n - expect) < 5 * np.sqrt(expect)
    assert set(np.unique(x["signs"])) == {-1.0, 1.0} and x["signs"].shape == (128,)
